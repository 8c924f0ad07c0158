"""The CPU side under AddressSanitizer and UndefinedBehaviorSanitizer: the oracle built with gcc's
sanitizers runs its pins, and the host half of the HIP library built with clang's runs the ABI
tests (argument validation, split planning, workspace sizing; no kernel is launched).  Each
suite runs in a child process that preloads the matching sanitizer runtime; any report fails
the child, and with it this test."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _run(args, env_extra, timeout=600):
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=1", UBSAN_OPTIONS="halt_on_error=1",
               **env_extra)
    res = subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider", *args], cwd=ROOT,
                         env=env, capture_output=True, text=True, timeout=timeout)
    tail = (res.stdout + res.stderr)[-3000:]
    assert res.returncode == 0, tail
    assert "AddressSanitizer" not in tail and "runtime error" not in tail, tail
    return tail


def test_oracle_pins_under_asan_and_ubsan():
    import oracle
    lib = oracle.build(sanitize=True)
    libasan = subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True, text=True).stdout.strip()
    libubsan = subprocess.run(["gcc", "-print-file-name=libubsan.so"], capture_output=True, text=True).stdout.strip()
    if not os.path.exists(libasan):
        pytest.skip("gcc's libasan is not installed")
    out = _run(["tests/test_oracle_pins.py", "tests/test_oracle_mutations.py::test_unmodified_oracle_passes_the_battery"],
               {"LD_PRELOAD": f"{libasan}:{libubsan}", "KVQ_ORACLE_LIB": lib})
    assert " passed" in out


def test_host_library_under_asan_and_ubsan():
    from long_context_decode_flash_amd import build as B
    lib = B.SANITIZED_LIB
    srcs = [os.path.join(B.CSRC, s) for s in B.SOURCES]
    if not os.path.exists(lib) or os.path.getmtime(lib) < max(os.path.getmtime(s) for s in srcs):
        B.build(sanitize=True)
    out = _run(["tests/test_abi.py"], {"LD_PRELOAD": B.asan_runtime(), "KVQ_LIB": lib})
    assert " passed" in out

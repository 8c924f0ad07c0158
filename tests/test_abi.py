"""The C-ABI library on the CPU: it loads, exports every symbol include/kvq.h declares, and its
host-side logic (sizes, split planning, argument validation) behaves as documented.  No call
here reaches a kernel launch: every invalid call returns before any HIP call."""
import ctypes
import os
import re
import subprocess

import pytest

from long_context_decode_flash_amd import build as B
from long_context_decode_flash_amd import kvq

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(kvq.LIB_PATH):
        B.build()
    return kvq.lib()


def declared_functions():
    names = []
    for h in sorted(os.listdir(os.path.join(ROOT, "include"))):
        if h.endswith(".h"):
            text = open(os.path.join(ROOT, "include", h)).read()
            text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
            names += re.findall(r"^\s*[A-Za-z_][\w \*]*?\b(kvq_\w+)\s*\(", text, flags=re.M)
    return sorted(set(names))


def test_library_exports_every_declared_symbol(lib):
    names = declared_functions()
    assert {"kvq_append", "kvq_decode_attn"} <= set(names)
    out = subprocess.run(["nm", "-D", "--defined-only", kvq.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = set(re.findall(r"\bT (kvq_\w+)", out))
    missing = [n for n in names if n not in exported]
    assert not missing, missing
    for n in names:
        assert getattr(lib, n) is not None


def test_block_bytes(lib):
    assert kvq.block_bytes(64, 256) == 25728
    assert kvq.block_bytes(16, 64) == 1632
    assert kvq.block_bytes(32, 128) == 32 * (128 + 2 + 64 + 8)
    for bad in ((64, 96), (48, 256), (8, 64), (512, 64), (0, 64)):
        assert kvq.block_bytes(*bad) == 0


def test_split_plan(lib):
    # headline: 2 sequences x 4 KV heads x 92,160 tokens
    s = kvq.decode_num_splits(2, 4, 92160)
    nblk = 92160 // 32
    bps = -(-nblk // s)
    assert s * bps >= nblk and (s - 1) * bps < nblk
    assert 128 <= 8 * s <= 512
    # explicit requests are clamped to the number of 32-token blocks
    assert kvq.decode_num_splits(1, 1, 100, 3) == 2  # 4 blocks, 2 per split
    assert kvq.decode_num_splits(1, 1, 100, 1000) == 4
    assert kvq.decode_num_splits(1, 1, 1, 0) == 1
    assert kvq.decode_num_splits(1, 1, 100, 0) == 1  # one block per wave of one workgroup
    # every planned split starts inside the context
    for n_seq, hkv, L, req in ((1, 4, 262144, 0), (1, 1, 512, 0), (3, 2, 1001, 7), (1, 4, 8192, 0)):
        s = kvq.decode_num_splits(n_seq, hkv, L, req)
        nblk = -(-L // 32)
        bps = -(-nblk // s)
        assert (s - 1) * bps < nblk <= s * bps
    with pytest.raises(kvq.KVQError):
        kvq.decode_num_splits(0, 4, 100)
    with pytest.raises(kvq.KVQError):
        kvq.decode_num_splits(1, 4, 100, -1)


def test_split_plan_by_format(lib):
    # the 4-bit-V format takes the plan whose busiest wave has the fewest 32-token blocks (32
    # splits: 90 blocks, 23 for the busiest of 4 waves); the 8-bit-V formats, bandwidth-bound,
    # keep 240 workgroups with 24 blocks per wave
    assert kvq.decode_num_splits(2, 4, 92160, kv_format=0) == 32
    assert kvq.decode_num_splits(2, 4, 92160) == 32
    for fmt in (1, 2):
        assert kvq.decode_num_splits(2, 4, 92160, kv_format=fmt) == 30
    # the workspace query covers every format's plan
    for fmt in (0, 1, 2):
        s = kvq.decode_num_splits(2, 4, 92160, kv_format=fmt)
        assert kvq.decode_workspace_bytes(2, 1, 24, 4, 256, 92160) >= 2 * 4 * s * 6 * (256 + 2) * 4
    # shapes where both models agree
    for fmt in (0, 1, 2):
        assert kvq.decode_num_splits(1, 4, 262144, n_rows=4, kv_format=fmt) == 64
        assert kvq.decode_num_splits(1, 4, 65536, kv_format=fmt) == 64
    # a windowed plan is that of the window's span (a window may start inside a block: 31 more
    # tokens), in each format
    for fmt in (0, 1, 2):
        assert kvq.decode_num_splits(2, 4, 92160, n_rows=1, window=65536, kv_format=fmt) == \
            kvq.decode_num_splits(2, 4, 65536 + 31, kv_format=fmt)
    # a request is the same in every format; an unknown format is refused
    assert kvq.decode_num_splits(2, 4, 92160, 17, kv_format=1) == 17
    with pytest.raises(kvq.KVQError):
        kvq.decode_num_splits(2, 4, 92160, kv_format=7)


def test_workspace_size(lib):
    s = kvq.decode_num_splits(2, 4, 92160)
    assert kvq.decode_workspace_bytes(2, 1, 24, 4, 256, 92160) == 2 * 4 * s * 6 * (256 + 2) * 4
    # (max, sum) entries per unit are padded to an even count
    s3 = kvq.decode_num_splits(1, 1, 4096, 3)
    assert kvq.decode_workspace_bytes(1, 1, 1, 1, 64, 4096, 3) == s3 * 64 * 4 + (s3 + 1) // 2 * 16
    # one split writes the output directly and needs only a token workspace
    assert kvq.decode_workspace_bytes(1, 1, 4, 1, 64, 100) == 16
    assert kvq.decode_workspace_bytes(2, 1, 24, 5, 256, 92160) == 0  # heads not divisible
    assert kvq.decode_workspace_bytes(2, 1, 24, 4, 100, 92160) == 0


P = ctypes.c_void_p
FAKE = ctypes.c_void_p(0x100000)  # aligned, never dereferenced: validation fails first


def append_rc(lib, pool=FAKE, num_pages=4, page_size=16, hkv=1, d=64, k=FAKE, v=FAKE,
              slots=FAKE, n_tok=1):
    return lib.kvq_append(pool, num_pages, page_size, hkv, d, k, v, slots, n_tok, None)


def test_append_validation(lib):
    assert append_rc(lib, pool=None) == kvq.KVQ_ERR_ARG
    assert append_rc(lib, num_pages=0) == kvq.KVQ_ERR_ARG
    assert append_rc(lib, hkv=0) == kvq.KVQ_ERR_ARG
    assert append_rc(lib, d=96) == kvq.KVQ_ERR_UNSUPPORTED
    assert append_rc(lib, page_size=24) == kvq.KVQ_ERR_UNSUPPORTED
    assert append_rc(lib, page_size=512) == kvq.KVQ_ERR_UNSUPPORTED
    assert append_rc(lib, n_tok=-1) == kvq.KVQ_ERR_ARG
    assert append_rc(lib, k=None) == kvq.KVQ_ERR_ARG
    assert append_rc(lib, slots=None) == kvq.KVQ_ERR_ARG
    assert append_rc(lib, pool=ctypes.c_void_p(0x100004)) == kvq.KVQ_ERR_ARG  # misaligned
    assert append_rc(lib, n_tok=0) == kvq.KVQ_OK  # nothing to do, nothing enqueued


def test_kv_formats(lib):
    """K8/V4, K8/V8 and fp8 block sizes (fp8 has the K8/V8 layout); an unknown format is
    refused before any HIP call."""
    assert lib.kvq_block_bytes_fmt(kvq.KVQ_FORMAT_K8V4, 64, 256) == 64 * (256 + 2 + 128 + 16)
    assert lib.kvq_block_bytes_fmt(kvq.KVQ_FORMAT_K8V8, 64, 256) == 64 * (2 * 256 + 2 + 16)
    assert lib.kvq_block_bytes_fmt(kvq.KVQ_FORMAT_K8V8, 16, 64) == 16 * (2 * 64 + 2 + 4)
    assert lib.kvq_block_bytes(64, 256) == lib.kvq_block_bytes_fmt(kvq.KVQ_FORMAT_K8V4, 64, 256)
    for P, D in ((64, 256), (16, 64), (32, 128)):
        assert lib.kvq_block_bytes_fmt(kvq.KVQ_FORMAT_FP8, P, D) == \
            lib.kvq_block_bytes_fmt(kvq.KVQ_FORMAT_K8V8, P, D)
    assert lib.kvq_block_bytes_fmt(3, 64, 256) == 0
    assert lib.kvq_block_bytes_fmt(-1, 64, 256) == 0
    assert lib.kvq_append_fmt(3, FAKE, 4, 16, 1, 64, FAKE, FAKE, FAKE, 1, None) == \
        kvq.KVQ_ERR_UNSUPPORTED
    assert lib.kvq_append_fmt(kvq.KVQ_FORMAT_FP8, FAKE, 4, 16, 1, 64, FAKE, FAKE, FAKE, 0,
                              None) == kvq.KVQ_OK
    assert lib.kvq_append_fmt(kvq.KVQ_FORMAT_K8V8, FAKE, 4, 16, 1, 64, FAKE, FAKE, FAKE, 0,
                              None) == kvq.KVQ_OK
    assert lib.kvq_decode_attn_fmt(7, FAKE, 8, 16, 2, 64, FAKE, FAKE, FAKE, 1, 1, 4, 8, 100,
                                   0.0, 0, FAKE, None, FAKE, 1 << 30, None) == \
        kvq.KVQ_ERR_UNSUPPORTED
    assert lib.kvq_decode_step_fmt(7, FAKE, 8, 16, 2, 64, None, None, 0, FAKE, FAKE, FAKE, 1, 1,
                                   4, 8, 100, 0.0, 0, FAKE, None, FAKE, 1 << 30, None) == \
        kvq.KVQ_ERR_UNSUPPORTED


def decode_rc(lib, **kw):
    a = dict(pool=FAKE, num_pages=8, page_size=16, hkv=2, d=64, q=FAKE, pt=FAKE, sl=FAKE,
             n_seq=1, n_rows=1, hq=4, max_pages=8, max_seq_len=100, scale=0.0, splits=0,
             out=FAKE, lse=None, ws=FAKE, ws_bytes=1 << 30)
    a.update(kw)
    return lib.kvq_decode_attn(a["pool"], a["num_pages"], a["page_size"], a["hkv"], a["d"],
                               a["q"], a["pt"], a["sl"], a["n_seq"], a["n_rows"], a["hq"],
                               a["max_pages"], a["max_seq_len"], a["scale"], a["splits"],
                               a["out"], a["lse"], a["ws"], a["ws_bytes"], None)


def test_decode_validation(lib):
    E = kvq
    assert decode_rc(lib, pool=None) == E.KVQ_ERR_ARG
    assert decode_rc(lib, q=None) == E.KVQ_ERR_ARG
    assert decode_rc(lib, pt=None) == E.KVQ_ERR_ARG
    assert decode_rc(lib, sl=None) == E.KVQ_ERR_ARG
    assert decode_rc(lib, out=None) == E.KVQ_ERR_ARG
    assert decode_rc(lib, d=32) == E.KVQ_ERR_UNSUPPORTED
    assert decode_rc(lib, page_size=17) == E.KVQ_ERR_UNSUPPORTED
    assert decode_rc(lib, n_rows=0) == E.KVQ_ERR_UNSUPPORTED
    assert decode_rc(lib, n_rows=5) == E.KVQ_ERR_UNSUPPORTED
    assert decode_rc(lib, hq=5) == E.KVQ_ERR_ARG                  # not a multiple of hkv
    assert decode_rc(lib, hq=2 * 33) == E.KVQ_ERR_UNSUPPORTED      # 33 rows per KV head
    assert decode_rc(lib, hq=2 * 9, n_rows=4) == E.KVQ_ERR_UNSUPPORTED
    assert decode_rc(lib, max_seq_len=129) == E.KVQ_ERR_ARG       # beyond the page table
    assert decode_rc(lib, max_seq_len=0) == E.KVQ_ERR_ARG
    assert decode_rc(lib, n_seq=0) == E.KVQ_ERR_ARG
    assert decode_rc(lib, splits=-1) == E.KVQ_ERR_ARG
    assert decode_rc(lib, scale=float("nan")) == E.KVQ_ERR_ARG
    assert decode_rc(lib, scale=float("inf")) == E.KVQ_ERR_ARG
    assert decode_rc(lib, ws=None) == E.KVQ_ERR_WORKSPACE
    need = kvq.decode_workspace_bytes(1, 1, 4, 2, 64, 100)
    assert decode_rc(lib, ws_bytes=need - 1) == E.KVQ_ERR_WORKSPACE
    assert decode_rc(lib, q=ctypes.c_void_p(0x100002)) == E.KVQ_ERR_ARG


def test_decode_rejects_misaligned_out(lib):
    """out is written with 16-byte stores: a misaligned pointer is refused on the host."""
    assert decode_rc(lib, out=ctypes.c_void_p(0x100004)) == kvq.KVQ_ERR_ARG
    assert step_rc(lib, out=ctypes.c_void_p(0x100008)) == kvq.KVQ_ERR_ARG


def noalloc_rc(lib, **kw):
    a = dict(fmt=0, pool=FAKE, num_pages=8, page_size=16, hkv=2, d=64, k=None, v=None, n_new=0,
             q=FAKE, pt=FAKE, sl=FAKE, n_seq=1, n_rows=1, hq=4, max_pages=8, max_seq_len=100,
             scale=0.0, splits=0, out=FAKE, lse=None)
    a.update(kw)
    return lib.kvq_decode_step_noalloc(a["fmt"], a["pool"], a["num_pages"], a["page_size"],
                                       a["hkv"], a["d"], a["k"], a["v"], a["n_new"], a["q"],
                                       a["pt"], a["sl"], a["n_seq"], a["n_rows"], a["hq"],
                                       a["max_pages"], a["max_seq_len"], a["scale"], a["splits"],
                                       a["out"], a["lse"], None)


def test_noalloc_validation(lib):
    """kvq_decode_step_noalloc checks its arguments as kvq_decode_step does, and refuses a call
    whose partials exceed the static scratch with KVQ_ERR_SCRATCH; all before any HIP call."""
    E = kvq
    assert noalloc_rc(lib, pool=None) == E.KVQ_ERR_ARG
    assert noalloc_rc(lib, q=None) == E.KVQ_ERR_ARG
    assert noalloc_rc(lib, out=ctypes.c_void_p(0x100004)) == E.KVQ_ERR_ARG
    assert noalloc_rc(lib, d=96) == E.KVQ_ERR_UNSUPPORTED
    assert noalloc_rc(lib, fmt=5) == E.KVQ_ERR_UNSUPPORTED
    assert noalloc_rc(lib, n_new=-1) == E.KVQ_ERR_ARG
    assert noalloc_rc(lib, n_new=2) == E.KVQ_ERR_ARG  # k_new / v_new missing
    assert noalloc_rc(lib, n_new=E.KVQ_MAX_STEP_TOKENS + 1, k=FAKE, v=FAKE) == E.KVQ_ERR_ARG
    # 32 sequences x 8 KV heads x 128 splits x 32 rows x D 256: far past 16 MiB
    big = dict(n_seq=32, hkv=8, hq=64, n_rows=4, d=256, page_size=64, num_pages=1 << 16,
               max_pages=4096, max_seq_len=1 << 18, splits=128)
    need = kvq.decode_workspace_bytes(32, 4, 64, 8, 256, 1 << 18, 128)
    assert need > E.KVQ_NOALLOC_SCRATCH_BYTES
    assert noalloc_rc(lib, **big) == E.KVQ_ERR_SCRATCH
    assert "static" in kvq.strerror(E.KVQ_ERR_SCRATCH)
    # every automatic plan of the benchmark's workloads fits
    for n_seq, hkv, hq, R, L in ((1, 1, 4, 1, 512), (1, 4, 24, 1, 8192), (1, 4, 24, 1, 65536),
                                 (2, 4, 24, 1, 92160), (1, 4, 24, 4, 262144), (1, 8, 256, 1, 1 << 20)):
        assert kvq.decode_workspace_bytes(n_seq, R, hq, hkv, 256, L) <= E.KVQ_NOALLOC_SCRATCH_BYTES


def test_strerror(lib):
    for code in (0, -1, -2, -3, -4, 7):
        assert isinstance(kvq.strerror(code), str) and kvq.strerror(code)


def test_binding_fails_loudly_without_the_library(monkeypatch, tmp_path):
    monkeypatch.setattr(kvq, "_lib", None)
    monkeypatch.setattr(kvq, "LIB_PATH", str(tmp_path / "missing.so"))
    with pytest.raises(RuntimeError, match="not built"):
        kvq.lib()


def step_rc(lib, **kw):
    a = dict(pool=FAKE, num_pages=8, page_size=16, hkv=2, d=64, k=FAKE, v=FAKE, n_new=1, q=FAKE,
             pt=FAKE, sl=FAKE, n_seq=1, n_rows=1, hq=4, max_pages=8, max_seq_len=100, scale=0.0,
             splits=0, out=FAKE, lse=None, ws=FAKE, ws_bytes=1 << 30)
    a.update(kw)
    return lib.kvq_decode_step(a["pool"], a["num_pages"], a["page_size"], a["hkv"], a["d"],
                               a["k"], a["v"], a["n_new"], a["q"], a["pt"], a["sl"], a["n_seq"],
                               a["n_rows"], a["hq"], a["max_pages"], a["max_seq_len"], a["scale"],
                               a["splits"], a["out"], a["lse"], a["ws"], a["ws_bytes"], None)


def test_decode_step_validation(lib):
    assert step_rc(lib, n_new=-1) == kvq.KVQ_ERR_ARG
    assert step_rc(lib, n_new=kvq.KVQ_MAX_STEP_TOKENS + 1) == kvq.KVQ_ERR_ARG
    assert step_rc(lib, k=None) == kvq.KVQ_ERR_ARG
    assert step_rc(lib, v=None) == kvq.KVQ_ERR_ARG
    # the decode checks apply as for kvq_decode_attn
    assert step_rc(lib, pool=None) == kvq.KVQ_ERR_ARG
    assert step_rc(lib, d=32) == kvq.KVQ_ERR_UNSUPPORTED
    assert step_rc(lib, ws=None) == kvq.KVQ_ERR_WORKSPACE


def win_rc(lib, step=False, **kw):
    a = dict(fmt=0, pool=FAKE, num_pages=8, page_size=16, hkv=2, d=64, k=FAKE, v=FAKE, n_new=1,
             q=FAKE, pt=FAKE, sl=FAKE, n_seq=1, n_rows=1, hq=4, max_pages=8, max_seq_len=100,
             window=40, ring=0, scale=0.0, splits=0, out=FAKE, lse=None, ws=FAKE,
             ws_bytes=1 << 30)
    a.update(kw)
    tail = (a["n_seq"], a["n_rows"], a["hq"], a["max_pages"], a["max_seq_len"], a["window"],
            a["ring"], a["scale"], a["splits"], a["out"], a["lse"], a["ws"], a["ws_bytes"], None)
    if step:
        return lib.kvq_decode_step_win(a["fmt"], a["pool"], a["num_pages"], a["page_size"],
                                       a["hkv"], a["d"], a["k"], a["v"], a["n_new"], a["q"],
                                       a["pt"], a["sl"], *tail)
    return lib.kvq_decode_attn_win(a["fmt"], a["pool"], a["num_pages"], a["page_size"], a["hkv"],
                                   a["d"], a["q"], a["pt"], a["sl"], *tail)


def test_window_ring_validation(lib):
    E = kvq
    for step in (False, True):
        assert win_rc(lib, step, window=-1) == E.KVQ_ERR_ARG
        assert win_rc(lib, step, ring=-1) == E.KVQ_ERR_ARG
        assert win_rc(lib, step, window=0, ring=4) == E.KVQ_ERR_ARG     # a ring needs a window
        assert win_rc(lib, step, ring=9) == E.KVQ_ERR_ARG               # more than the table
        # 40 + 1 - 1 tokens at any offset in 16-token pages touch up to 4 pages
        assert win_rc(lib, step, ring=3) == E.KVQ_ERR_ARG
        # 50 + 4 - 1 tokens touch up to 5 pages (an offset of 15 plus 53 tokens)
        assert win_rc(lib, step, ring=4, n_rows=4, window=50) == E.KVQ_ERR_ARG
        assert win_rc(lib, step, ring=5, n_rows=4, window=50, ws=None) == E.KVQ_ERR_WORKSPACE
        # a ring lets positions run past the page table: the call gets as far as the workspace
        assert win_rc(lib, step, ring=4, max_seq_len=1 << 20, ws=None) == E.KVQ_ERR_WORKSPACE
        # without a ring the page table must hold max_seq_len
        assert win_rc(lib, step, max_seq_len=129) == E.KVQ_ERR_ARG
        assert win_rc(lib, step, fmt=7) == E.KVQ_ERR_UNSUPPORTED
    # a fused step appends only tokens some row sees
    assert win_rc(lib, True, window=4, n_rows=2, n_new=6) == E.KVQ_ERR_ARG
    assert win_rc(lib, True, window=4, n_rows=2, n_new=5, ws=None) == E.KVQ_ERR_WORKSPACE


def test_window_split_plan(lib):
    # a window plans its pieces over W + n_rows - 1 tokens plus one block, not the context
    for window, n_rows, msl in ((4096, 1, 1 << 20), (65536, 4, 262144), (100, 1, 50)):
        span = min(window + n_rows - 1 + 31, msl)
        assert kvq.decode_num_splits(2, 4, msl, n_rows=n_rows, window=window) == \
            kvq.decode_num_splits(2, 4, span)
        assert kvq.decode_workspace_bytes(2, n_rows, 24, 4, 256, msl, window=window) == \
            kvq.decode_workspace_bytes(2, n_rows, 24, 4, 256, span)
    assert lib.kvq_decode_num_splits_win(1, 4, 1000, 1, -1, 0) == kvq.KVQ_ERR_ARG
    assert lib.kvq_decode_workspace_bytes_win(1, 1, 4, 4, 64, 1000, -1, 0) == 0


def prefill_rc(lib, **kw):
    a = dict(fmt=0, pool=FAKE, num_pages=8, page_size=16, hkv=2, d=64, q=FAKE, pt=FAKE, sl=FAKE,
             n_seq=1, chunk=10, hq=4, max_pages=8, max_seq_len=100, scale=0.0, splits=0,
             out=FAKE, lse=None, ws=FAKE, ws_bytes=1 << 30)
    a.update(kw)
    return lib.kvq_prefill_attn(a["fmt"], a["pool"], a["num_pages"], a["page_size"], a["hkv"],
                                a["d"], a["q"], a["pt"], a["sl"], a["n_seq"], a["chunk"], a["hq"],
                                a["max_pages"], a["max_seq_len"], a["scale"], a["splits"],
                                a["out"], a["lse"], a["ws"], a["ws_bytes"], None)


def test_prefill_validation(lib):
    """Every argument error of kvq_prefill_attn is found on the host (FAKE pointers are never
    dereferenced)."""
    E = kvq
    assert prefill_rc(lib, pool=None) == E.KVQ_ERR_ARG
    assert prefill_rc(lib, q=None) == E.KVQ_ERR_ARG
    assert prefill_rc(lib, out=None) == E.KVQ_ERR_ARG
    assert prefill_rc(lib, fmt=3) == E.KVQ_ERR_UNSUPPORTED
    assert prefill_rc(lib, d=96) == E.KVQ_ERR_UNSUPPORTED
    assert prefill_rc(lib, chunk=0) == E.KVQ_ERR_ARG
    assert prefill_rc(lib, chunk=E.KVQ_MAX_CHUNK + 1) == E.KVQ_ERR_UNSUPPORTED
    assert prefill_rc(lib, hq=5) == E.KVQ_ERR_ARG
    assert prefill_rc(lib, hkv=1, hq=16, chunk=8192) == E.KVQ_ERR_UNSUPPORTED  # 131072 rows
    assert prefill_rc(lib, max_seq_len=129) == E.KVQ_ERR_ARG
    assert prefill_rc(lib, splits=-1) == E.KVQ_ERR_ARG
    assert prefill_rc(lib, scale=float("nan")) == E.KVQ_ERR_ARG
    assert prefill_rc(lib, ws=None) == E.KVQ_ERR_WORKSPACE
    need = kvq.prefill_workspace_bytes(1, 10, 4, 2, 64, 100)
    assert need > 0
    assert prefill_rc(lib, ws_bytes=need - 1) == E.KVQ_ERR_WORKSPACE
    assert prefill_rc(lib, q=ctypes.c_void_p(0x100002)) == E.KVQ_ERR_ARG
    assert prefill_rc(lib, out=ctypes.c_void_p(0x100004)) == E.KVQ_ERR_ARG


def test_prefill_split_plan(lib):
    """The prefill plan fills the 256 CUs in whole rounds where it can: the 1,024-position chunk
    of two 92,160-token sequences (4 KV heads, 6 query heads each) has 2 x 4 x 24 tiles of 256
    rows, and four pieces per tile make 768 workgroups (3 rounds); the workspace holds each
    piece's partials."""
    s = kvq.prefill_num_splits(2, 1024, 24, 4, 92160)
    assert s == 4 and (2 * 4 * 24 * s) % 256 == 0
    nblk = 92160 // 32
    assert kvq.prefill_num_splits(1, 1024, 24, 4, 92160, 3) == 3
    assert kvq.prefill_num_splits(1, 1, 1, 1, 64) == 1  # too few blocks to split
    ws = kvq.prefill_workspace_bytes(2, 1024, 24, 4, 256, 92160)
    rows = 1024 * 6
    assert ws >= 8 * s * rows * 256 * 4 + 8 * s * rows * 8
    assert kvq.prefill_workspace_bytes(1, 0, 4, 2, 64, 100) == 0
    assert nblk > 0


def test_grids_beyond_32_bit_work_items_are_refused(lib):
    """A call whose attention or merge grid would count 2^32 work-items or more is refused on
    the host (HIP's grid limit), instead of launching a truncated grid."""
    E = kvq
    # decode: 2^24 units (sequences x KV heads) of one split: 2^24 x 256 threads
    assert decode_rc(lib, n_seq=1 << 16, hkv=256, hq=256, num_pages=1 << 10, splits=1) == \
        E.KVQ_ERR_UNSUPPORTED
    # one sequence fewer passes the grid check and stops at the (missing) workspace
    assert decode_rc(lib, n_seq=(1 << 16) - 1, hkv=256, hq=256, num_pages=1 << 10, splits=1,
                     ws=None) == E.KVQ_ERR_WORKSPACE
    # append: one 256-thread workgroup per 16 tokens and KV head: 2^20 groups x 16 heads x 256
    assert append_rc(lib, hkv=16, n_tok=1 << 24, num_pages=1 << 10) == E.KVQ_ERR_UNSUPPORTED
    assert append_rc(lib, hkv=16, n_tok=(1 << 24) - 15, num_pages=1 << 10) == E.KVQ_ERR_UNSUPPORTED
    # decode merge: 2^18 units x 2 splits: 256 merge workgroups of 64 lanes per unit
    assert decode_rc(lib, n_seq=1 << 16, hkv=4, hq=128, d=256, page_size=64, num_pages=64,
                     max_pages=8, max_seq_len=400, splits=2) == E.KVQ_ERR_UNSUPPORTED
    # prefill merge: 128 units x 65,536 rows x 64 dims-of-4 / 8 items x 64 lanes = 2^32
    assert prefill_rc(lib, n_seq=32, hkv=4, hq=32, d=256, chunk=8192, page_size=64,
                      num_pages=1 << 14, max_pages=256, max_seq_len=16384, splits=2) == \
        E.KVQ_ERR_UNSUPPORTED
    # the same with one piece has no merge launch and passes the grid check
    assert prefill_rc(lib, n_seq=32, hkv=4, hq=32, d=256, chunk=8192, page_size=64,
                      num_pages=1 << 14, max_pages=256, max_seq_len=16384, splits=1,
                      ws=None) == E.KVQ_ERR_WORKSPACE


def test_probe_validation(lib):
    """The measurement probes refuse bad arguments on the host, before any HIP call."""
    E = kvq
    P = ctypes.c_void_p
    buf = P(1 << 20)
    sink = P(4096)
    f = lib.kvq_probe_stream_read
    assert f(None, 4096, 0, 1, sink, None) == E.KVQ_ERR_ARG
    assert f(buf, 4095, 0, 1, sink, None) == E.KVQ_ERR_ARG          # not a multiple of 4 KB
    assert f(P((1 << 20) + 16), 4096, 0, 1, sink, None) == E.KVQ_ERR_ARG  # not 4 KB aligned
    assert f(buf, 4096, 3, 1, sink, None) == E.KVQ_ERR_ARG          # no such load form
    assert f(buf, 4096, 0, 0, sink, None) == E.KVQ_ERR_ARG
    assert f(buf, 4096, 0, (1 << 20) + 1, sink, None) == E.KVQ_ERR_ARG
    assert f(buf, 4096, 0, 1, None, None) == E.KVQ_ERR_ARG
    g = lib.kvq_probe_clock
    out = P(1 << 20)
    assert g(None, 1, 100, None, None) == E.KVQ_ERR_ARG
    assert g(P((1 << 20) + 4), 1, 100, None, None) == E.KVQ_ERR_ARG  # not 8-byte aligned
    assert g(out, 0, 100, None, None) == E.KVQ_ERR_ARG
    assert g(out, 4097, 100, None, None) == E.KVQ_ERR_ARG
    assert g(out, 1, 0, None, None) == E.KVQ_ERR_ARG
    assert g(out, 1, 10000001, None, None) == E.KVQ_ERR_ARG
    assert g(None, 0, 0, None, None) == E.KVQ_ERR_ARG  # the rate query needs somewhere to write


def test_debug_errors_entry(lib):
    """kvq_debug_errors is a KVQ_DEBUG-build feature: the normal build refuses it; the debug
    build exports every declared symbol and refuses a NULL output before any HIP call."""
    E = kvq
    v = ctypes.c_uint32(0)
    assert lib.kvq_debug_errors(ctypes.byref(v), 1, None) == E.KVQ_ERR_UNSUPPORTED
    if not os.path.exists(B.DEBUG_LIB):
        B.build(debug=True)
    out = subprocess.run(["nm", "-D", "--defined-only", B.DEBUG_LIB], capture_output=True,
                         text=True, check=True).stdout
    exported = set(re.findall(r"\bT (kvq_\w+)", out))
    assert not [n for n in declared_functions() if n not in exported]
    dbg = ctypes.CDLL(B.DEBUG_LIB)
    dbg.kvq_debug_errors.argtypes = [ctypes.c_void_p, ctypes.c_int32, ctypes.c_void_p]
    assert dbg.kvq_debug_errors(None, 1, None) == E.KVQ_ERR_ARG

"""CPU oracle for the paged K8/V4 (and K8/V8) cache and its decode attention.

TEST INFRASTRUCTURE ONLY: the tests, ``__graft_entry__.smoke()`` and the benchmark's
``cpu_baseline`` leg are the only callers.  The product path never imports this package.

The arithmetic lives in ``kvq_oracle.c`` (plain C, fp64 attention, fp32-defined quantizer);
this module builds it with gcc when needed and marshals numpy arrays through ctypes.  It
imports nothing from the HIP library's package and shares no code with it.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
SOURCE = os.path.join(_HERE, "kvq_oracle.c")
_SO = os.path.join(_HERE, "liboracle.so")
_lock = threading.Lock()

CFLAGS = ["-O2", "-std=c11", "-fopenmp", "-ffp-contract=off", "-fno-fast-math",
          "-fPIC", "-shared", "-Wall"]


SANITIZED_SO = os.path.join(_HERE, "liboracle_san.so")
SANITIZE_FLAGS = ["-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
                  "-fno-omit-frame-pointer", "-g"]


def build(force: bool = False, source: str = SOURCE, out: str = _SO, sanitize: bool = False) -> str:
    """Compile the oracle C source into a shared library (gcc). Returns the library path.
    sanitize: AddressSanitizer + UndefinedBehaviorSanitizer build (liboracle_san.so), for a
    process that preloads gcc's libasan."""
    if sanitize and out == _SO:
        out = SANITIZED_SO
    if force or not os.path.exists(out) or os.path.getmtime(out) < os.path.getmtime(source):
        tmp = out + ".tmp%d" % os.getpid()
        flags = CFLAGS + (SANITIZE_FLAGS if sanitize else [])
        subprocess.check_call(["gcc", *flags, "-o", tmp, source, "-lm"])
        os.replace(tmp, out)
    return out


def _declare(lib):
    P = ctypes.c_void_p
    I = ctypes.c_int
    lib.kvq_oracle_fp16_to_double.argtypes = [ctypes.c_uint16]
    lib.kvq_oracle_fp16_to_double.restype = ctypes.c_double
    lib.kvq_oracle_fp16_from_double.argtypes = [ctypes.c_double]
    lib.kvq_oracle_fp16_from_double.restype = ctypes.c_uint16
    lib.kvq_oracle_quantize_group.argtypes = [P, I, I, P, P]
    lib.kvq_oracle_quantize_group.restype = None
    lib.kvq_oracle_block_bytes_fmt.argtypes = [I, I, I]
    lib.kvq_oracle_block_bytes_fmt.restype = ctypes.c_size_t
    lib.kvq_oracle_format_offset_fmt.argtypes = [I, I, I, I, I, I, ctypes.POINTER(ctypes.c_int)]
    lib.kvq_oracle_format_offset_fmt.restype = ctypes.c_longlong
    lib.kvq_oracle_append_fmt.argtypes = [P, I, I, I, I, I, P, P, P, I]
    lib.kvq_oracle_append_fmt.restype = None
    lib.kvq_oracle_read_slot_fmt.argtypes = [P, I, I, I, I, I, I, I, P, P, P, P]
    lib.kvq_oracle_read_slot_fmt.restype = None
    lib.kvq_oracle_append_kf.argtypes = [P, I, I, I, I, I, P, P, P, I]
    lib.kvq_oracle_append_kf.restype = None
    lib.kvq_oracle_decode_attn_kf.argtypes = [P, I, I, I, I, I, I, I, P, P, P, I, I, I, I,
                                              ctypes.c_double, P, I, P, P]
    lib.kvq_oracle_decode_attn_kf.restype = None
    lib.kvq_oracle_attn_weights_kf.argtypes = [P, I, I, I, I, I, I, I, P, P, P, I, I, I,
                                               ctypes.c_double, I, I, I, P]
    lib.kvq_oracle_attn_weights_kf.restype = I
    lib.kvq_oracle_e4m3_to_double.argtypes = [ctypes.c_uint8]
    lib.kvq_oracle_e4m3_to_double.restype = ctypes.c_double
    lib.kvq_oracle_e4m3_from_float.argtypes = [ctypes.c_float]
    lib.kvq_oracle_e4m3_from_float.restype = ctypes.c_uint8
    lib.kvq_oracle_quantize_group_f8.argtypes = [P, I, P, P]
    lib.kvq_oracle_quantize_group_f8.restype = None
    lib.kvq_oracle_num_threads.argtypes = []
    lib.kvq_oracle_num_threads.restype = I
    lib.kvq_oracle_set_num_threads.argtypes = [I]
    lib.kvq_oracle_set_num_threads.restype = None
    return lib


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


# KV formats as the library header numbers them: 0 K8/V4, 1 K8/V8, 2 fp8 (e4m3 K and V in the
# K8/V8 layout).  Calls take either vbits (4 or 8: the integer formats) or kv_format.
FMT_K8V4, FMT_K8V8, FMT_FP8 = 0, 1, 2


def _fmt(vbits, kv_format):
    kf = (1 if vbits == 8 else 0) if kv_format is None else int(kv_format)
    return (4 if kf == 0 else 8), kf


class Oracle:
    """The oracle's entry points bound to one compiled library (the default build, or a
    variant a test compiled from modified source)."""

    def __init__(self, lib_path: str):
        self.lib = _declare(ctypes.CDLL(lib_path))

    def num_threads(self) -> int:
        return self.lib.kvq_oracle_num_threads()

    def set_num_threads(self, n: int) -> None:
        self.lib.kvq_oracle_set_num_threads(int(n))

    def fp16_to_double(self, bits: int) -> float:
        return self.lib.kvq_oracle_fp16_to_double(int(bits))

    def fp16_from_double(self, x: float) -> int:
        return int(self.lib.kvq_oracle_fp16_from_double(float(x)))

    def quantize_group(self, x, qmax: int):
        """Quantize one scale group (fp32 values). Returns (int8 codes, fp16 scale bits)."""
        x = _c(x, np.float32)
        codes = np.zeros(x.size, np.int8)
        sb = np.zeros(1, np.uint16)
        self.lib.kvq_oracle_quantize_group(_ptr(x), x.size, int(qmax), _ptr(codes), _ptr(sb))
        return codes, int(sb[0])

    def e4m3_to_double(self, code: int) -> float:
        return self.lib.kvq_oracle_e4m3_to_double(int(code))

    def e4m3_from_float(self, y: float) -> int:
        return int(self.lib.kvq_oracle_e4m3_from_float(float(y)))

    def quantize_group_f8(self, x):
        """fp8 scale group (fp32 values). Returns (uint8 E4M3 codes, fp16 scale bits)."""
        x = _c(x, np.float32)
        codes = np.zeros(x.size, np.uint8)
        sb = np.zeros(1, np.uint16)
        self.lib.kvq_oracle_quantize_group_f8(_ptr(x), x.size, _ptr(codes), _ptr(sb))
        return codes, int(sb[0])

    # vbits: bits per V code, 4 (K8/V4, the default) or 8 (K8/V8 and fp8)
    def block_bytes(self, page_size: int, head_dim: int, vbits: int = 4) -> int:
        return int(self.lib.kvq_oracle_block_bytes_fmt(page_size, head_dim, vbits))

    def pool_bytes(self, num_pages: int, page_size: int, num_kv_heads: int,
                   head_dim: int, vbits: int = 4) -> int:
        return num_pages * num_kv_heads * self.block_bytes(page_size, head_dim, vbits)

    def format_offset(self, what: int, page_size: int, head_dim: int, slot: int, index: int,
                      vbits: int = 4):
        """(byte offset within a block, aux) for what = 0 K code, 1 K scale, 2 V code
        (aux = 1 for the high nibble of a 4-bit code), 3 V scale (index = scale group)."""
        aux = ctypes.c_int(0)
        off = self.lib.kvq_oracle_format_offset_fmt(what, page_size, head_dim, vbits, slot, index,
                                                    ctypes.byref(aux))
        return int(off), int(aux.value)

    def append(self, pool: np.ndarray, num_pages: int, page_size: int, num_kv_heads: int,
               head_dim: int, k, v, slot_mapping, vbits: int = 4, kv_format=None) -> None:
        """Quantize tokens k, v (fp32 [n_tok][Hkv][D]) into ``pool`` (uint8, in place)."""
        vbits, kf = _fmt(vbits, kv_format)
        assert pool.dtype == np.uint8 and pool.flags.c_contiguous
        assert pool.size >= self.pool_bytes(num_pages, page_size, num_kv_heads, head_dim, vbits)
        k = _c(k, np.float32)
        v = _c(v, np.float32)
        slots = _c(slot_mapping, np.int32)
        n_tok = slots.size
        assert k.size == n_tok * num_kv_heads * head_dim and v.size == k.size
        self.lib.kvq_oracle_append_kf(_ptr(pool), num_pages, page_size, num_kv_heads, head_dim,
                                      kf, _ptr(k), _ptr(v), _ptr(slots), n_tok)

    def new_pool(self, num_pages: int, page_size: int, num_kv_heads: int, head_dim: int,
                 vbits: int = 4):
        return np.zeros(self.pool_bytes(num_pages, page_size, num_kv_heads, head_dim, vbits),
                        np.uint8)

    def read_slot(self, pool: np.ndarray, page_size: int, num_kv_heads: int, head_dim: int,
                  page: int, slot: int, head: int, vbits: int = 4):
        """Codes and scale bits stored for one (page, slot, KV head)."""
        kc = np.zeros(head_dim, np.int8)
        vc = np.zeros(head_dim, np.int8)
        ks = np.zeros(1, np.uint16)
        vs = np.zeros(head_dim // 32, np.uint16)
        self.lib.kvq_oracle_read_slot_fmt(_ptr(pool), page_size, num_kv_heads, head_dim, vbits,
                                          page, slot, head, _ptr(kc), _ptr(ks), _ptr(vc), _ptr(vs))
        return kc, int(ks[0]), vc, vs

    def decode_attn(self, pool: np.ndarray, num_pages: int, page_size: int, num_kv_heads: int,
                    head_dim: int, q_bits, page_table, seq_lens, n_rows: int, n_q_heads: int,
                    softmax_scale: float = 0.0, select=None, vbits: int = 4, window: int = 0,
                    ring_pages: int = 0, kv_format=None):
        """fp64 attention. ``q_bits``: uint16 fp16 bits [n_seq][n_rows][Hq][D].

        Returns (out, lse): with ``select`` None, out is [n_seq][n_rows][Hq][D] and lse
        [n_seq][n_rows][Hq]; with ``select`` a list of (b, i, hq), out is [len][D], lse [len].
        ``window`` > 0: row i sees only the last ``window`` tokens up to its own position;
        ``ring_pages`` > 0: logical page n lives in page-table entry n mod ``ring_pages``.
        """
        vbits, kf = _fmt(vbits, kv_format)
        q = _c(q_bits, np.uint16)
        pt = _c(page_table, np.int32)
        sl = _c(seq_lens, np.int32)
        n_seq = sl.size
        max_pages = pt.size // n_seq
        assert pt.size == n_seq * max_pages
        assert q.size == n_seq * n_rows * n_q_heads * head_dim
        if select is None:
            count = n_seq * n_rows * n_q_heads
            sel = None
        else:
            sel = _c(np.asarray(select).reshape(-1, 3), np.int32)
            count = sel.shape[0]
        out = np.zeros((count, head_dim), np.float64)
        lse = np.zeros(count, np.float64)
        self.lib.kvq_oracle_decode_attn_kf(_ptr(pool), num_pages, page_size, num_kv_heads,
                                            head_dim, kf, window, ring_pages, _ptr(q), _ptr(pt),
                                            _ptr(sl), n_seq, n_rows, n_q_heads, max_pages,
                                            float(softmax_scale),
                                            None if sel is None else _ptr(sel), count, _ptr(out),
                                            _ptr(lse))
        if select is None:
            return (out.reshape(n_seq, n_rows, n_q_heads, head_dim),
                    lse.reshape(n_seq, n_rows, n_q_heads))
        return out, lse

    def attn_weights(self, pool: np.ndarray, num_pages: int, page_size: int,
                     num_kv_heads: int, head_dim: int, q_bits, page_table, seq_lens,
                     n_rows: int, n_q_heads: int, b: int, i: int, hq: int,
                     softmax_scale: float = 0.0, vbits: int = 4, window: int = 0,
                     ring_pages: int = 0, kv_format=None):
        """Softmax weights over the L tokens of sequence b for query row i, head hq."""
        vbits, kf = _fmt(vbits, kv_format)
        q = _c(q_bits, np.uint16)
        pt = _c(page_table, np.int32)
        sl = _c(seq_lens, np.int32)
        max_pages = pt.size // sl.size
        w = np.zeros(max(int(sl[b]), 1), np.float64)
        n = self.lib.kvq_oracle_attn_weights_kf(_ptr(pool), num_pages, page_size, num_kv_heads,
                                                 head_dim, kf, window, ring_pages, _ptr(q),
                                                 _ptr(pt), _ptr(sl), n_rows, n_q_heads, max_pages,
                                                 float(softmax_scale), b, i, hq, _ptr(w))
        return w, n


_default = None


def default() -> Oracle:
    """The oracle built from kvq_oracle.c (compiled on first use if needed)."""
    global _default
    with _lock:
        if _default is None:
            # KVQ_ORACLE_LIB names another build of the same source (the sanitizer build)
            _default = Oracle(os.environ.get("KVQ_ORACLE_LIB") or build())
        return _default


def __getattr__(name):
    # module-level access to the default oracle's methods: oracle.decode_attn(...), ...
    if name.startswith("_"):
        raise AttributeError(name)
    return getattr(default(), name)

"""Python binding of ``libkvq.so`` (include/kvq.h): argument marshalling only.

Every step of the path runs in the library's HIP kernels; torch provides device memory and the
stream.  There is no fallback: without the built library every call raises.
"""
from __future__ import annotations

import ctypes
import os
import threading
from dataclasses import dataclass

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
# KVQ_LIB names another build of the same library (the sanitizer build of the CPU tests)
LIB_PATH = os.environ.get("KVQ_LIB") or os.path.join(_HERE, "libkvq.so")

KVQ_OK = 0
KVQ_ERR_ARG = -1
KVQ_ERR_UNSUPPORTED = -2
KVQ_ERR_WORKSPACE = -3
KVQ_ERR_HIP = -4
KVQ_ERR_SCRATCH = -5
KVQ_NOALLOC_SCRATCH_BYTES = 16 << 20  # the static split scratch of kvq_decode_step_noalloc
KVQ_MAX_STEP_TOKENS = 64
KVQ_FORMAT_K8V4 = 0  # 4-bit V codes
KVQ_FORMAT_K8V8 = 1  # 8-bit V codes
KVQ_FORMAT_FP8 = 2   # K and V as OCP e4m3 codes, the 8-bit V layout
KVQ_MAX_CHUNK = 8192  # chunked prefill: positions per chunk
FORMATS = {"k8v4": KVQ_FORMAT_K8V4, "k8v8": KVQ_FORMAT_K8V8, "fp8": KVQ_FORMAT_FP8}

_lock = threading.Lock()
_lib = None


class KVQError(RuntimeError):
    def __init__(self, code: int, where: str):
        self.code = code
        super().__init__(f"{where}: {strerror(code)} (code {code})")


def lib():
    """The loaded library (raises if it has not been built)."""
    global _lib
    with _lock:
        if _lib is not None:
            return _lib
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is not built; run `python -m long_context_decode_flash_amd.build` "
                "(hipcc, gfx950). There is no CPU fallback.")
        L = ctypes.CDLL(LIB_PATH)
        P = ctypes.c_void_p
        I = ctypes.c_int32
        L.kvq_block_bytes.argtypes = [I, I]
        L.kvq_block_bytes.restype = ctypes.c_size_t
        L.kvq_strerror.argtypes = [ctypes.c_int]
        L.kvq_strerror.restype = ctypes.c_char_p
        L.kvq_decode_num_splits.argtypes = [I, I, I, I]
        L.kvq_decode_num_splits.restype = I
        L.kvq_decode_workspace_bytes.argtypes = [I, I, I, I, I, I, I]
        L.kvq_decode_workspace_bytes.restype = ctypes.c_size_t
        L.kvq_append.argtypes = [P, I, I, I, I, P, P, P, I, P]
        L.kvq_append.restype = ctypes.c_int
        L.kvq_decode_attn.argtypes = [P, I, I, I, I, P, P, P, I, I, I, I, I, ctypes.c_float, I,
                                      P, P, P, ctypes.c_size_t, P]
        L.kvq_decode_attn.restype = ctypes.c_int
        L.kvq_decode_step.argtypes = [P, I, I, I, I, P, P, I, P, P, P, I, I, I, I, I,
                                      ctypes.c_float, I, P, P, P, ctypes.c_size_t, P]
        L.kvq_decode_step.restype = ctypes.c_int
        L.kvq_block_bytes_fmt.argtypes = [I, I, I]
        L.kvq_block_bytes_fmt.restype = ctypes.c_size_t
        L.kvq_append_fmt.argtypes = [I] + L.kvq_append.argtypes
        L.kvq_append_fmt.restype = ctypes.c_int
        L.kvq_decode_attn_fmt.argtypes = [I] + L.kvq_decode_attn.argtypes
        L.kvq_decode_attn_fmt.restype = ctypes.c_int
        L.kvq_decode_step_fmt.argtypes = [I] + L.kvq_decode_step.argtypes
        L.kvq_decode_step_fmt.restype = ctypes.c_int
        # sliding window over ring pages: (window, ring_pages) after max_seq_len
        at = L.kvq_decode_attn_fmt.argtypes
        L.kvq_decode_attn_win.argtypes = at[:14] + [I, I] + at[14:]
        L.kvq_decode_attn_win.restype = ctypes.c_int
        st = L.kvq_decode_step_fmt.argtypes
        L.kvq_decode_step_win.argtypes = st[:17] + [I, I] + st[17:]
        L.kvq_decode_step_win.restype = ctypes.c_int
        # the step without a workspace: the step_fmt arguments minus (workspace, bytes)
        L.kvq_decode_step_noalloc.argtypes = st[:-3] + [P]
        L.kvq_decode_step_noalloc.restype = ctypes.c_int
        L.kvq_decode_num_splits_win.argtypes = [I, I, I, I, I, I]
        L.kvq_decode_num_splits_win.restype = I
        L.kvq_decode_num_splits_fmt.argtypes = [I, I, I, I, I, I, I]
        L.kvq_decode_num_splits_fmt.restype = I
        L.kvq_decode_workspace_bytes_win.argtypes = [I, I, I, I, I, I, I, I]
        L.kvq_decode_workspace_bytes_win.restype = ctypes.c_size_t
        # chunked prefill: the decode_attn_fmt arguments with chunk in place of n_rows
        L.kvq_prefill_attn.argtypes = L.kvq_decode_attn_fmt.argtypes
        L.kvq_prefill_attn.restype = ctypes.c_int
        L.kvq_prefill_num_splits.argtypes = [I, I, I, I, I, I]
        L.kvq_prefill_num_splits.restype = I
        L.kvq_prefill_workspace_bytes.argtypes = [I, I, I, I, I, I, I]
        L.kvq_prefill_workspace_bytes.restype = ctypes.c_size_t
        L.kvq_probe_stream_read.argtypes = [P, ctypes.c_size_t, I, I, P, P]
        L.kvq_probe_stream_read.restype = ctypes.c_int
        L.kvq_probe_clock.argtypes = [P, I, ctypes.c_uint32, ctypes.POINTER(ctypes.c_int32), P]
        L.kvq_probe_clock.restype = ctypes.c_int
        L.kvq_debug_errors.argtypes = [ctypes.POINTER(ctypes.c_uint32), I, P]
        L.kvq_debug_errors.restype = ctypes.c_int
        _lib = L
        return L


def strerror(code: int) -> str:
    return lib().kvq_strerror(int(code)).decode()


def block_bytes(page_size: int, head_dim: int, kv_format: int = KVQ_FORMAT_K8V4) -> int:
    return int(lib().kvq_block_bytes_fmt(kv_format, page_size, head_dim))


def pool_bytes(num_pages: int, page_size: int, num_kv_heads: int, head_dim: int,
               kv_format: int = KVQ_FORMAT_K8V4) -> int:
    return num_pages * num_kv_heads * block_bytes(page_size, head_dim, kv_format)


def decode_num_splits(n_seq: int, num_kv_heads: int, max_seq_len: int,
                      num_splits: int = 0, *, n_rows: int = 1, window: int = 0,
                      kv_format: int = KVQ_FORMAT_K8V4) -> int:
    r = int(lib().kvq_decode_num_splits_fmt(kv_format, n_seq, num_kv_heads, max_seq_len, n_rows,
                                             window, num_splits))
    if r < 0:
        raise KVQError(r, "kvq_decode_num_splits_fmt")
    return r


def decode_workspace_bytes(n_seq: int, n_rows: int, n_q_heads: int, num_kv_heads: int,
                           head_dim: int, max_seq_len: int, num_splits: int = 0, *,
                           window: int = 0) -> int:
    if window:
        return int(lib().kvq_decode_workspace_bytes_win(n_seq, n_rows, n_q_heads, num_kv_heads,
                                                         head_dim, max_seq_len, window,
                                                         num_splits))
    return int(lib().kvq_decode_workspace_bytes(n_seq, n_rows, n_q_heads, num_kv_heads,
                                                 head_dim, max_seq_len, num_splits))


def _attn_fn(window: int, ring_pages: int):
    """The decode entry point for these window / ring arguments, and a function that inserts
    them into an argument tuple of the plain (format) call."""
    if window or ring_pages:
        return (lib().kvq_decode_attn_win,
                lambda a: a[:14] + (int(window), int(ring_pages)) + a[14:])
    return lib().kvq_decode_attn_fmt, lambda a: a


def _step_fn(window: int, ring_pages: int):
    if window or ring_pages:
        return (lib().kvq_decode_step_win,
                lambda a: a[:17] + (int(window), int(ring_pages)) + a[17:])
    return lib().kvq_decode_step_fmt, lambda a: a


def _stream_ptr(stream) -> int:
    if stream is None:
        stream = torch.cuda.current_stream()
    return int(stream.cuda_stream) if hasattr(stream, "cuda_stream") else int(stream)


def _dev(t: torch.Tensor, name: str, dtype: torch.dtype | None = None) -> int:
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t.data_ptr()


@dataclass
class PagedCache:
    """A caller-owned pool tensor (uint8, on the GPU), its geometry and its KV format."""
    pool: torch.Tensor
    num_pages: int
    page_size: int
    num_kv_heads: int
    head_dim: int
    kv_format: int = KVQ_FORMAT_K8V4

    @staticmethod
    def allocate(num_pages: int, page_size: int, num_kv_heads: int, head_dim: int,
                 device="cuda", kv_format: int = KVQ_FORMAT_K8V4) -> "PagedCache":
        n = pool_bytes(num_pages, page_size, num_kv_heads, head_dim, kv_format)
        if n == 0:
            raise KVQError(KVQ_ERR_UNSUPPORTED, "PagedCache.allocate")
        pool = torch.zeros(n, dtype=torch.uint8, device=device)
        return PagedCache(pool, num_pages, page_size, num_kv_heads, head_dim, kv_format)

    def append(self, k, v, slot_mapping, stream=None) -> None:
        append(self, k, v, slot_mapping, stream=stream)

    def decode_attn(self, q, page_table, seq_lens, max_seq_len: int, **kw):
        return decode_attn(self, q, page_table, seq_lens, max_seq_len, **kw)


def append(cache: PagedCache, k: torch.Tensor, v: torch.Tensor, slot_mapping: torch.Tensor,
           stream=None) -> None:
    """kvq_append: quantize k, v (fp32 [n_tok][Hkv][D]) into their slots of ``cache``."""
    n_tok = slot_mapping.numel()
    shape = (n_tok, cache.num_kv_heads, cache.head_dim)
    if tuple(k.shape) != shape or tuple(v.shape) != shape:
        raise ValueError(f"k and v must be {shape}")
    rc = lib().kvq_append_fmt(
        cache.kv_format, _dev(cache.pool, "pool", torch.uint8), cache.num_pages, cache.page_size,
        cache.num_kv_heads, cache.head_dim, _dev(k, "k", torch.float32),
        _dev(v, "v", torch.float32), _dev(slot_mapping, "slot_mapping", torch.int32), n_tok,
        _stream_ptr(stream))
    if rc != KVQ_OK:
        raise KVQError(rc, "kvq_append")


def decode_attn(cache: PagedCache, q: torch.Tensor, page_table: torch.Tensor,
                seq_lens: torch.Tensor, max_seq_len: int, *, softmax_scale: float = 0.0,
                num_splits: int = 0, out: torch.Tensor | None = None, want_lse: bool = True,
                lse: torch.Tensor | None = None, workspace: torch.Tensor | None = None,
                stream=None, window: int = 0, ring_pages: int = 0):
    """kvq_decode_attn. q: fp16 [n_seq][n_rows][Hq][D]; page_table: int32 [n_seq][max_pages];
    seq_lens: int32 [n_seq]. Returns (out fp32 [n_seq][n_rows][Hq][D], lse or None).
    ``window`` / ``ring_pages`` > 0 select kvq_decode_attn_win (sliding window, ring pages)."""
    if q.dim() != 4 or q.shape[3] != cache.head_dim:
        raise ValueError("q must be [n_seq][n_rows][n_q_heads][head_dim]")
    n_seq, n_rows, n_q_heads, D = (int(x) for x in q.shape)
    if page_table.dim() != 2 or page_table.shape[0] != n_seq:
        raise ValueError("page_table must be [n_seq][max_pages_per_seq]")
    if seq_lens.numel() != n_seq:
        raise ValueError("seq_lens must have n_seq entries")
    dev = q.device
    if out is None:
        out = torch.empty((n_seq, n_rows, n_q_heads, D), dtype=torch.float32, device=dev)
    if want_lse and lse is None:
        lse = torch.empty((n_seq, n_rows, n_q_heads), dtype=torch.float32, device=dev)
    need = decode_workspace_bytes(n_seq, n_rows, n_q_heads, cache.num_kv_heads, D, max_seq_len,
                                  num_splits, window=window)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=dev)
    fn, ins = _attn_fn(window, ring_pages)
    rc = fn(*ins((
        cache.kv_format, _dev(cache.pool, "pool", torch.uint8), cache.num_pages, cache.page_size,
        cache.num_kv_heads, D, _dev(q, "q", torch.float16),
        _dev(page_table, "page_table", torch.int32), _dev(seq_lens, "seq_lens", torch.int32),
        n_seq, n_rows, n_q_heads, int(page_table.shape[1]), int(max_seq_len),
        float(softmax_scale), int(num_splits), _dev(out, "out", torch.float32),
        _dev(lse, "lse", torch.float32) if lse is not None else None,
        _dev(workspace, "workspace", torch.uint8), workspace.numel(), _stream_ptr(stream))))
    if rc != KVQ_OK:
        raise KVQError(rc, "kvq_decode_attn")
    return out, lse


def prefill_num_splits(n_seq: int, chunk: int, n_q_heads: int, num_kv_heads: int,
                       max_seq_len: int, num_splits: int = 0) -> int:
    r = int(lib().kvq_prefill_num_splits(n_seq, chunk, n_q_heads, num_kv_heads, max_seq_len,
                                         num_splits))
    if r < 0:
        raise KVQError(r, "kvq_prefill_num_splits")
    return r


def prefill_workspace_bytes(n_seq: int, chunk: int, n_q_heads: int, num_kv_heads: int,
                            head_dim: int, max_seq_len: int, num_splits: int = 0) -> int:
    return int(lib().kvq_prefill_workspace_bytes(n_seq, chunk, n_q_heads, num_kv_heads, head_dim,
                                                 max_seq_len, num_splits))


def _prefill_args(cache, q, page_table, seq_lens, max_seq_len, out, lse, workspace,
                  softmax_scale, num_splits, stream):
    if q.dim() != 4 or q.shape[3] != cache.head_dim:
        raise ValueError("q must be [n_seq][chunk][n_q_heads][head_dim]")
    n_seq, chunk, n_q_heads, D = (int(x) for x in q.shape)
    if tuple(out.shape) != (n_seq, chunk, n_q_heads, D):
        raise ValueError("out must be [n_seq][chunk][n_q_heads][head_dim]")
    if page_table.dim() != 2 or page_table.shape[0] != n_seq or seq_lens.numel() != n_seq:
        raise ValueError("page_table must be [n_seq][max_pages_per_seq], seq_lens [n_seq]")
    return (cache.kv_format, _dev(cache.pool, "pool", torch.uint8), cache.num_pages,
            cache.page_size, cache.num_kv_heads, D, _dev(q, "q", torch.float16),
            _dev(page_table, "page_table", torch.int32), _dev(seq_lens, "seq_lens", torch.int32),
            n_seq, chunk, n_q_heads, int(page_table.shape[1]), int(max_seq_len),
            float(softmax_scale), int(num_splits), _dev(out, "out", torch.float32),
            _dev(lse, "lse", torch.float32) if lse is not None else None,
            _dev(workspace, "workspace", torch.uint8), workspace.numel(), _stream_ptr(stream))


def prefill_attn(cache: PagedCache, q: torch.Tensor, page_table: torch.Tensor,
                 seq_lens: torch.Tensor, max_seq_len: int, *, softmax_scale: float = 0.0,
                 num_splits: int = 0, out: torch.Tensor | None = None, want_lse: bool = True,
                 lse: torch.Tensor | None = None, workspace: torch.Tensor | None = None,
                 stream=None):
    """kvq_prefill_attn: the chunk (the last ``chunk`` tokens of each sequence, already
    appended) attends causally to the cache. q: fp16 [n_seq][chunk][Hq][D]. Returns (out fp32
    [n_seq][chunk][Hq][D], lse or None)."""
    n_seq, chunk, n_q_heads, D = (int(x) for x in q.shape)
    dev = q.device
    if out is None:
        out = torch.empty((n_seq, chunk, n_q_heads, D), dtype=torch.float32, device=dev)
    if want_lse and lse is None:
        lse = torch.empty((n_seq, chunk, n_q_heads), dtype=torch.float32, device=dev)
    if workspace is None:
        need = prefill_workspace_bytes(n_seq, chunk, n_q_heads, cache.num_kv_heads, D,
                                       max_seq_len, num_splits)
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=dev)
    rc = lib().kvq_prefill_attn(*_prefill_args(cache, q, page_table, seq_lens, max_seq_len, out,
                                               lse, workspace, softmax_scale, num_splits, stream))
    if rc != KVQ_OK:
        raise KVQError(rc, "kvq_prefill_attn")
    return out, lse


def prepare_prefill(cache: PagedCache, q: torch.Tensor, page_table: torch.Tensor,
                    seq_lens: torch.Tensor, max_seq_len: int, out: torch.Tensor,
                    lse: torch.Tensor | None, workspace: torch.Tensor, *,
                    softmax_scale: float = 0.0, num_splits: int = 0, stream=None):
    """Marshal the arguments of one kvq_prefill_attn once; the returned callable re-issues it."""
    args = _prefill_args(cache, q, page_table, seq_lens, max_seq_len, out, lse, workspace,
                         softmax_scale, num_splits, stream)
    fn = lib().kvq_prefill_attn

    def call():
        rc = fn(*args)
        if rc != KVQ_OK:
            raise KVQError(rc, "kvq_prefill_attn")
    return call


def _step_args(cache, k_new, v_new, q, page_table, seq_lens, max_seq_len, out, lse, workspace,
               softmax_scale, num_splits, stream):
    n_seq, n_rows, n_q_heads, D = (int(x) for x in q.shape)
    if D != cache.head_dim or tuple(out.shape) != (n_seq, n_rows, n_q_heads, D):
        raise ValueError("q / out shapes do not match the cache")
    if k_new is None or k_new.numel() == 0:
        n_new, kp, vp = 0, None, None
    else:
        n_new = int(k_new.shape[1])
        shape = (n_seq, n_new, cache.num_kv_heads, D)
        if tuple(k_new.shape) != shape or tuple(v_new.shape) != shape:
            raise ValueError(f"k_new and v_new must be {shape}")
        kp, vp = _dev(k_new, "k_new", torch.float32), _dev(v_new, "v_new", torch.float32)
    return (cache.kv_format, _dev(cache.pool, "pool", torch.uint8), cache.num_pages, cache.page_size,
            cache.num_kv_heads, D, kp, vp, n_new, _dev(q, "q", torch.float16),
            _dev(page_table, "page_table", torch.int32), _dev(seq_lens, "seq_lens", torch.int32),
            n_seq, n_rows, n_q_heads, int(page_table.shape[1]), int(max_seq_len),
            float(softmax_scale), int(num_splits), _dev(out, "out", torch.float32),
            _dev(lse, "lse", torch.float32) if lse is not None else None,
            _dev(workspace, "workspace", torch.uint8) if workspace is not None else None,
            workspace.numel() if workspace is not None else 0, _stream_ptr(stream))


def decode_step_noalloc(cache: PagedCache, k_new: torch.Tensor | None, v_new: torch.Tensor | None,
                        q: torch.Tensor, page_table: torch.Tensor, seq_lens: torch.Tensor,
                        max_seq_len: int, *, softmax_scale: float = 0.0, num_splits: int = 0,
                        out: torch.Tensor | None = None, want_lse: bool = True,
                        lse: torch.Tensor | None = None, stream=None):
    """kvq_decode_step_noalloc: kvq_decode_step (format of the cache) with the split partials in
    the library's static device array instead of a workspace.  The C call allocates nothing;
    this wrapper allocates ``out`` / ``lse`` only when they are not given."""
    n_seq, n_rows, n_q_heads, D = (int(x) for x in q.shape)
    dev = q.device
    if out is None:
        out = torch.empty((n_seq, n_rows, n_q_heads, D), dtype=torch.float32, device=dev)
    if want_lse and lse is None:
        lse = torch.empty((n_seq, n_rows, n_q_heads), dtype=torch.float32, device=dev)
    args = _step_args(cache, k_new, v_new, q, page_table, seq_lens, max_seq_len, out, lse, None,
                      softmax_scale, num_splits, stream)
    rc = lib().kvq_decode_step_noalloc(*(args[:-3] + args[-1:]))
    if rc != KVQ_OK:
        raise KVQError(rc, "kvq_decode_step_noalloc")
    return out, lse


def decode_step(cache: PagedCache, k_new: torch.Tensor | None, v_new: torch.Tensor | None,
                q: torch.Tensor, page_table: torch.Tensor, seq_lens: torch.Tensor,
                max_seq_len: int, *, softmax_scale: float = 0.0, num_splits: int = 0,
                out: torch.Tensor | None = None, want_lse: bool = True,
                lse: torch.Tensor | None = None, workspace: torch.Tensor | None = None,
                stream=None, window: int = 0, ring_pages: int = 0):
    """kvq_decode_step: append each sequence's newest n_new tokens (k_new, v_new fp32
    [n_seq][n_new][Hkv][D], the last n_new of seq_lens[b]) and attend, in one call.
    Returns (out, lse) as decode_attn (``window`` / ``ring_pages`` as there)."""
    n_seq, n_rows, n_q_heads, D = (int(x) for x in q.shape)
    dev = q.device
    if out is None:
        out = torch.empty((n_seq, n_rows, n_q_heads, D), dtype=torch.float32, device=dev)
    if want_lse and lse is None:
        lse = torch.empty((n_seq, n_rows, n_q_heads), dtype=torch.float32, device=dev)
    if workspace is None:
        need = decode_workspace_bytes(n_seq, n_rows, n_q_heads, cache.num_kv_heads, D,
                                      max_seq_len, num_splits, window=window)
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=dev)
    fn, ins = _step_fn(window, ring_pages)
    rc = fn(*ins(_step_args(cache, k_new, v_new, q, page_table, seq_lens, max_seq_len, out, lse,
                            workspace, softmax_scale, num_splits, stream)))
    if rc != KVQ_OK:
        raise KVQError(rc, "kvq_decode_step")
    return out, lse


def prepare_decode_step(cache: PagedCache, k_new: torch.Tensor | None, v_new: torch.Tensor | None,
                        q: torch.Tensor, page_table: torch.Tensor, seq_lens: torch.Tensor,
                        max_seq_len: int, out: torch.Tensor, lse: torch.Tensor | None,
                        workspace: torch.Tensor, *, softmax_scale: float = 0.0,
                        num_splits: int = 0, stream=None, window: int = 0, ring_pages: int = 0):
    """Marshal the arguments of one kvq_decode_step once; the returned callable re-issues it."""
    fn, ins = _step_fn(window, ring_pages)
    args = ins(_step_args(cache, k_new, v_new, q, page_table, seq_lens, max_seq_len, out, lse,
                          workspace, softmax_scale, num_splits, stream))

    def call():
        rc = fn(*args)
        if rc != KVQ_OK:
            raise KVQError(rc, "kvq_decode_step")
    return call


def prepare_append(cache: PagedCache, k: torch.Tensor, v: torch.Tensor,
                   slot_mapping: torch.Tensor, stream=None):
    """Marshal the arguments of one kvq_append once; the returned callable re-issues it.
    For loops where the per-call Python checks would cost more than the kernel."""
    n_tok = slot_mapping.numel()
    shape = (n_tok, cache.num_kv_heads, cache.head_dim)
    if tuple(k.shape) != shape or tuple(v.shape) != shape:
        raise ValueError(f"k and v must be {shape}")
    args = (cache.kv_format, _dev(cache.pool, "pool", torch.uint8), cache.num_pages,
            cache.page_size, cache.num_kv_heads, cache.head_dim, _dev(k, "k", torch.float32),
            _dev(v, "v", torch.float32), _dev(slot_mapping, "slot_mapping", torch.int32), n_tok,
            _stream_ptr(stream))
    fn = lib().kvq_append_fmt

    def call():
        rc = fn(*args)
        if rc != KVQ_OK:
            raise KVQError(rc, "kvq_append")
    return call


def prepare_decode_attn(cache: PagedCache, q: torch.Tensor, page_table: torch.Tensor,
                        seq_lens: torch.Tensor, max_seq_len: int, out: torch.Tensor,
                        lse: torch.Tensor | None, workspace: torch.Tensor, *,
                        softmax_scale: float = 0.0, num_splits: int = 0, stream=None,
                        window: int = 0, ring_pages: int = 0):
    """Marshal the arguments of one kvq_decode_attn once; the returned callable re-issues it."""
    n_seq, n_rows, n_q_heads, D = (int(x) for x in q.shape)
    if D != cache.head_dim or tuple(out.shape) != (n_seq, n_rows, n_q_heads, D):
        raise ValueError("q / out shapes do not match the cache")
    fn, ins = _attn_fn(window, ring_pages)
    args = ins((cache.kv_format, _dev(cache.pool, "pool", torch.uint8), cache.num_pages,
            cache.page_size, cache.num_kv_heads, D, _dev(q, "q", torch.float16),
            _dev(page_table, "page_table", torch.int32), _dev(seq_lens, "seq_lens", torch.int32),
            n_seq, n_rows, n_q_heads, int(page_table.shape[1]), int(max_seq_len),
            float(softmax_scale), int(num_splits), _dev(out, "out", torch.float32),
            _dev(lse, "lse", torch.float32) if lse is not None else None,
            _dev(workspace, "workspace", torch.uint8), workspace.numel(), _stream_ptr(stream)))

    def call():
        rc = fn(*args)
        if rc != KVQ_OK:
            raise KVQError(rc, "kvq_decode_attn")
    return call


def prepare_stream_probe(buf: torch.Tensor, mode: int, workgroups: int, sink: torch.Tensor,
                         stream=None):
    """kvq_probe_stream_read over all of ``buf`` (uint8, 4 KB-aligned, a multiple of 4 KB):
    the plain streaming read the decode's bandwidth is set against.  Returns a callable that
    re-issues it."""
    args = (_dev(buf, "buf", torch.uint8), buf.numel(), int(mode), int(workgroups),
            _dev(sink, "sink", torch.int32), _stream_ptr(stream))

    def call():
        rc = lib().kvq_probe_stream_read(*args)
        if rc != KVQ_OK:
            raise KVQError(rc, "kvq_probe_stream_read")
    return call


KVQ_DBG_PAGE_ID = 1
KVQ_DBG_SLOT = 2


def debug_errors(clear: bool = True, stream=None) -> int:
    """The range-report word of the KVQ_DEBUG build (KVQ_DBG_PAGE_ID | KVQ_DBG_SLOT bits), after
    waiting for ``stream``; cleared when ``clear``.  Raises KVQError(KVQ_ERR_UNSUPPORTED) when
    the loaded library is not a KVQ_DEBUG build."""
    v = ctypes.c_uint32(0)
    rc = lib().kvq_debug_errors(ctypes.byref(v), 1 if clear else 0, _stream_ptr(stream))
    if rc != KVQ_OK:
        raise KVQError(rc, "kvq_debug_errors")
    return v.value


def clock_counter_khz() -> int:
    """Rate of the GPU's constant-rate counter that kvq_probe_clock sets the shader clock
    against, in kHz (no launch)."""
    khz = ctypes.c_int32(0)
    rc = lib().kvq_probe_clock(None, 0, 0, ctypes.byref(khz), None)
    if rc != KVQ_OK:
        raise KVQError(rc, "kvq_probe_clock")
    return khz.value


def prepare_clock_probe(out: torch.Tensor, spin_ticks: int = 2000, stream=None):
    """kvq_probe_clock with one workgroup per three int64 entries of ``out``: each call of the
    returned callable enqueues a spin of ``spin_ticks`` constant-rate ticks and leaves
    (shader cycles, ticks, XCD) per workgroup in ``out``; shader MHz = cycles / ticks *
    clock_counter_khz() / 1000."""
    if out.dtype != torch.int64 or out.numel() % 3 != 0:
        raise ValueError("out: int64 with 3 entries per workgroup")
    args = (_dev(out, "out", torch.int64), out.numel() // 3, int(spin_ticks), None, _stream_ptr(stream))

    def call():
        rc = lib().kvq_probe_clock(*args)
        if rc != KVQ_OK:
            raise KVQError(rc, "kvq_probe_clock")
    return call

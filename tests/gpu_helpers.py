"""Shared plumbing of the GPU parity tests: run a workload through the HIP library (via the
C ABI binding) and through the CPU oracle, from the same seeded inputs."""
from __future__ import annotations

import functools
import sys

import numpy as np

import oracle
from long_context_decode_flash_amd import workloads as W

TOL_ABS = 2e-3  # attention max-abs bound against the fp64 oracle
TOL_REL = 1e-3  # the same max-abs error, relative to the largest |ref| of the compared outputs
LSE_ABS = 1e-4  # log-sum-exp max-abs bound (natural-log units)


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def torch_mod():
    import torch
    return torch


def kvq():
    from long_context_decode_flash_amd import kvq as _k
    return _k


def to_dev(a: np.ndarray):
    torch = torch_mod()
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


# KV formats: the library's format code and the oracle's bits per V code (fp8 codes use the
# 8-bit V layout)
VBITS = {0: 4, 1: 8, 2: 8}
FORMAT_IDS = {0: "k8v4", 1: "k8v8", 2: "fp8"}


def gpu_cache(inp: W.Inputs, kv_format=0):
    wl = inp.wl
    return kvq().PagedCache.allocate(wl.pool_pages, wl.page_size, wl.num_kv_heads, wl.head_dim,
                                     kv_format=kv_format)


def gpu_append(cache, k, v, slots):
    torch = torch_mod()
    kvq().append(cache, to_dev(k), to_dev(v), to_dev(slots.astype(np.int32)))
    torch.cuda.synchronize()


def gpu_fill(inp: W.Inputs, cache=None, split_step=True, kv_format=0):
    """Fill a pool on the GPU: the cached context, then the step's appended tokens."""
    cache = cache or gpu_cache(inp, kv_format)
    if split_step and inp.wl.n_new and np.all(inp.seq_lens == inp.wl.seq_len):
        gpu_append(cache, *inp.prefill())
        gpu_append(cache, *inp.step_tokens())
    else:
        gpu_append(cache, *inp.all_tokens())
    return cache


def gpu_decode(inp: W.Inputs, cache, num_splits=0, max_seq_len=None, page_table=None,
               softmax_scale=0.0):
    torch = torch_mod()
    wl = inp.wl
    q = to_dev(inp.q_bits).view(torch.float16)
    pt = to_dev(inp.page_table if page_table is None else page_table)
    sl = to_dev(inp.seq_lens)
    msl = int(max_seq_len or max(int(inp.seq_lens.max()), 1))
    out, lse = kvq().decode_attn(cache, q, pt, sl, msl, num_splits=num_splits,
                                 softmax_scale=softmax_scale)
    torch.cuda.synchronize()
    return out.cpu().numpy(), lse.cpu().numpy()


def oracle_fill(inp: W.Inputs, kv_format=0):
    wl = inp.wl
    vb = VBITS[kv_format]
    pool = oracle.new_pool(wl.pool_pages, wl.page_size, wl.num_kv_heads, wl.head_dim, vb)
    if wl.n_new and np.all(inp.seq_lens == wl.seq_len):
        oracle.append(pool, wl.pool_pages, wl.page_size, wl.num_kv_heads, wl.head_dim,
                      *inp.prefill(), kv_format=kv_format)
        oracle.append(pool, wl.pool_pages, wl.page_size, wl.num_kv_heads, wl.head_dim,
                      *inp.step_tokens(), kv_format=kv_format)
    else:
        oracle.append(pool, wl.pool_pages, wl.page_size, wl.num_kv_heads, wl.head_dim,
                      *inp.all_tokens(), kv_format=kv_format)
    return pool


def oracle_decode(inp: W.Inputs, pool, select=None, softmax_scale=0.0, kv_format=0):
    wl = inp.wl
    return oracle.decode_attn(pool, wl.pool_pages, wl.page_size, wl.num_kv_heads, wl.head_dim,
                              inp.q_bits, inp.page_table, inp.seq_lens, wl.n_rows,
                              wl.n_q_heads, softmax_scale=softmax_scale, select=select,
                              kv_format=kv_format)


@functools.lru_cache(maxsize=2)
def full_workload(name: str):
    """(inputs, oracle pool) of a full-size workload, cached across tests."""
    inp = W.generate(W.WORKLOADS[name])
    return inp, oracle_fill(inp)


def assert_close(tag, got, ref, tol_abs=TOL_ABS, tol_rel=TOL_REL):
    """Attention outputs against the oracle, element by element: max-abs within tol_abs and
    within tol_rel of the largest |ref| (at long contexts |out| is only ~sqrt(e/N), so the
    absolute bound alone would be loose)."""
    assert np.all(np.isfinite(got)), f"{tag}: non-finite output"
    mx = report(tag, got, ref)
    scale = float(np.max(np.abs(ref))) if ref.size else 0.0
    assert mx <= tol_abs, f"{tag}: max-abs {mx:.3e} > {tol_abs:g}"
    assert mx <= tol_rel * scale, f"{tag}: max-abs {mx:.3e} > {tol_rel:g} * max|ref| = {tol_rel * scale:.3e}"
    return mx


def assert_lse(tag, got, ref, tol=LSE_ABS):
    """Log-sum-exp: -inf exactly where the oracle has it (a row that sees no token), else
    within tol."""
    fin = np.isfinite(ref)
    assert np.array_equal(fin, np.isfinite(got)), f"{tag}: lse finiteness differs"
    assert np.all(got[~fin] == ref[~fin]), f"{tag}: lse of rows that see nothing"
    err = float(np.max(np.abs(got[fin] - ref[fin]), initial=0.0))
    assert err <= tol, f"{tag}: lse max-abs {err:.3e} > {tol:g}"
    return err


def report(tag, got, ref):
    err = np.abs(got - ref)
    mx = float(np.max(err)) if err.size else 0.0
    scale = float(np.max(np.abs(ref))) if ref.size else 0.0
    say(f"{tag}: max_abs={mx:.3e} max|ref|={scale:.3e} rel={mx / max(scale, 1e-30):.3e}")
    return mx

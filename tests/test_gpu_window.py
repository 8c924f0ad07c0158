"""Sliding window over ring pages on the GPU (kvq_decode_attn_win / kvq_decode_step_win), against
the CPU oracle's windowed attention on the same seeded inputs: every output of small cases
(several tiles, ragged lengths, MTP rows, windows shorter and longer than the context, ring
tables whose positions run far past the page table), the fused step's pool bytes bit-exact, and
every output row of a 184K-token context under a 64K-token window."""
import numpy as np
import pytest

from long_context_decode_flash_amd import workloads as W
from tests.gpu_helpers import (assert_close, assert_lse, gpu_append, gpu_cache, kvq, oracle,
                               report, say, to_dev, torch_mod, VBITS)

pytestmark = pytest.mark.gpu


def _oracle_pool(inp, k, v, slots, kf):
    wl = inp.wl
    pool = oracle.new_pool(wl.pool_pages, wl.page_size, wl.num_kv_heads, wl.head_dim, VBITS[kf])
    oracle.append(pool, wl.pool_pages, wl.page_size, wl.num_kv_heads, wl.head_dim, k, v, slots,
                  kv_format=kf)
    return pool


def _run(inp, cache, table, window, ring, num_splits=0, msl=None, kv_format=0):
    torch = torch_mod()
    q = to_dev(inp.q_bits).view(torch.float16)
    msl = int(msl or int(inp.seq_lens.max()))
    out, lse = kvq().decode_attn(cache, q, to_dev(table), to_dev(inp.seq_lens), msl,
                                 num_splits=num_splits, window=window, ring_pages=ring)
    torch.cuda.synchronize()
    return out.cpu().numpy(), lse.cpu().numpy()


def _ref(inp, pool, table, window, ring, kf, select=None):
    wl = inp.wl
    return oracle.decode_attn(pool, wl.pool_pages, wl.page_size, wl.num_kv_heads, wl.head_dim,
                              inp.q_bits, table, inp.seq_lens, wl.n_rows, wl.n_q_heads,
                              select=select, kv_format=kf, window=window, ring_pages=ring)


def _check(tag, out, lse, ref_out, ref_lse):
    assert_close(tag, out, ref_out)
    assert_lse(tag, lse, ref_lse)


LINEAR_CASES = [
    # (n_seq, seq_lens, Hkv, Hq, D, P, n_rows, windows)
    (1, (300,), 1, 4, 64, 16, 1, (1, 17, 64, 100, 299, 300, 1000)),
    (2, (777, 205), 2, 12, 128, 32, 4, (1, 33, 128, 500)),
    (2, (1000, 613), 4, 24, 256, 64, 1, (40, 256, 700)),
    (1, (1111,), 4, 24, 256, 64, 4, (3, 96, 1111)),
]


@pytest.mark.parametrize("kv_format", [0, 1, 2], ids=["k8v4", "k8v8", "fp8"])
@pytest.mark.parametrize("case", range(len(LINEAR_CASES)))
def test_window_linear_table_every_output(case, kv_format):
    n_seq, lens, hkv, hq, D, P, R, windows = LINEAR_CASES[case]
    kf = kv_format
    say(f"[window linear] case {case} fmt {kv_format}: lens {lens} D {D} P {P} R {R}")
    inp = W.custom(n_seq=n_seq, seq_lens=lens, num_kv_heads=hkv, n_q_heads=hq, head_dim=D,
                   page_size=P, n_rows=R, seed=300 + case)
    k, v, slots = inp.all_tokens()
    pool = _oracle_pool(inp, k, v, slots, kf)
    cache = gpu_cache(inp, kv_format)
    gpu_append(cache, k, v, slots)
    for window in windows:
        ref_out, ref_lse = _ref(inp, pool, inp.page_table, window, 0, kf)
        for splits in (0, 1, 3):
            out, lse = _run(inp, cache, inp.page_table, window, 0, splits)
            _check(f"case {case} fmt {kv_format} W {window} splits {splits}", out, lse,
                   ref_out, ref_lse)


RING_CASES = [
    # (n_seq, seq_lens, Hkv, Hq, D, P, n_rows, window, ring_pages)
    (1, (5000,), 1, 4, 64, 16, 1, 40, 4),
    (2, (3001, 2222), 2, 12, 128, 32, 4, 100, 5),
    (2, (20000, 7777), 4, 24, 256, 64, 1, 1000, 17),
    (1, (9999,), 4, 24, 256, 64, 4, 63, 3),
]


@pytest.mark.parametrize("kv_format", [0, 1, 2], ids=["k8v4", "k8v8", "fp8"])
@pytest.mark.parametrize("case", range(len(RING_CASES)))
def test_window_ring_every_output(case, kv_format):
    n_seq, lens, hkv, hq, D, P, R, window, ring = RING_CASES[case]
    kf = kv_format
    say(f"[window ring] case {case} fmt {kv_format}: lens {lens} D {D} P {P} R {R} W {window} "
        f"ring {ring}")
    # the pool holds only the rings; positions run far past the ring table
    inp = W.custom(n_seq=n_seq, seq_lens=lens, num_kv_heads=hkv, n_q_heads=hq, head_dim=D,
                   page_size=P, n_rows=R, seed=400 + case)
    table, (k, v, slots) = inp.ring(ring)
    assert int(inp.seq_lens.max()) > table.shape[1] * P
    pool = _oracle_pool(inp, k, v, slots, kf)
    cache = gpu_cache(inp, kv_format)
    gpu_append(cache, k, v, slots)
    ref_out, ref_lse = _ref(inp, pool, table, window, ring, kf)
    for splits in (0, 1, 2):
        out, lse = _run(inp, cache, table, window, ring, splits)
        _check(f"ring case {case} fmt {kv_format} splits {splits}", out, lse, ref_out, ref_lse)


@pytest.mark.parametrize("kv_format", [0, 1, 2], ids=["k8v4", "k8v8", "fp8"])
def test_window_ring_fused_step(kv_format):
    """kvq_decode_step_win on a ring: the step's tokens overwrite the ring slots of tokens a
    ring length earlier; the pool bytes match the oracle's append of the same history, and the
    outputs its windowed attention."""
    torch = torch_mod()
    kf = kv_format
    R, n_new, window, ring, P = 4, 4, 200, 6, 64
    inp = W.custom(n_seq=2, seq_lens=(4099, 1090), num_kv_heads=4, n_q_heads=24, head_dim=256,
                   page_size=P, n_rows=R, seed=511)
    wl = inp.wl
    pre_lens = inp.seq_lens - n_new
    table, (k0, v0, s0) = inp.ring(ring, lens=pre_lens)
    k_new = np.zeros((2, n_new, 4, 256), np.float32)
    v_new = np.zeros_like(k_new)
    ks, vs, ss = [], [], []
    for b in range(2):
        L = int(inp.seq_lens[b])
        k_new[b] = inp.k[b, L - n_new:L]
        v_new[b] = inp.v[b, L - n_new:L]
        ks.append(inp.k[b, L - n_new:L])
        vs.append(inp.v[b, L - n_new:L])
        ss.append(inp.ring_slots(table, ring, b, L - n_new, L))
    pool = _oracle_pool(inp, k0, v0, s0, kf)
    oracle.append(pool, wl.pool_pages, P, 4, 256, np.concatenate(ks), np.concatenate(vs),
                  np.concatenate(ss), kv_format=kf)
    ref_out, ref_lse = _ref(inp, pool, table, window, ring, kf)
    for splits in (0, 1, 3):
        say(f"[window ring step] fmt {kv_format} splits {splits}")
        cache = gpu_cache(inp, kv_format)
        gpu_append(cache, k0, v0, s0)
        q = to_dev(inp.q_bits).view(torch.float16)
        out, lse = kvq().decode_step(cache, to_dev(k_new), to_dev(v_new), q, to_dev(table),
                                     to_dev(inp.seq_lens), int(inp.seq_lens.max()),
                                     num_splits=splits, window=window, ring_pages=ring)
        torch.cuda.synchronize()
        assert np.array_equal(cache.pool.cpu().numpy(), pool), "pool bytes differ"
        _check(f"ring step fmt {kv_format} splits {splits}", out.cpu().numpy(),
               lse.cpu().numpy(), ref_out, ref_lse)


def test_window_full_size_every_row():
    """184K tokens over two sequences (the interleaved-page-table workload), each row under a
    64K-token window: every output row against the oracle."""
    from tests.gpu_helpers import full_workload
    inp, pool = full_workload("ctx184k_c2")
    wl = inp.wl
    cache = gpu_cache(inp)
    gpu_append(cache, *inp.prefill())
    gpu_append(cache, *inp.step_tokens())
    window = 65536
    out, lse = _run(inp, cache, inp.page_table, window, 0, msl=wl.seq_len)
    ref_out, ref_lse = _ref(inp, pool, inp.page_table, window, 0, 0)
    _check("ctx184k_c2 window 65536 every row", out, lse, ref_out, ref_lse)

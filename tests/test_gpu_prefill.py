"""Chunked-prefill attention on the GPU (kvq_prefill_attn) against the CPU oracle: a chunk of C
positions at the end of each context attends causally to the cache, which is the oracle's
attention with n_rows = C.  Every output of small cases (several 128-row tiles, ragged lengths,
a chunk longer than the context, the whole prompt as one chunk, all three KV formats, several
context pieces), unwritten slots full of junk bytes, agreement with the decode call at small
chunks, and sampled rows of the last 1,024-position chunk of the 184K-token workload."""
import numpy as np
import pytest

from long_context_decode_flash_amd import workloads as W
from tests import gpu_helpers as H

pytestmark = pytest.mark.gpu

FMTS = pytest.mark.parametrize("kv_format", [0, 1, 2], ids=["k8v4", "k8v8", "fp8"])

CASES = [
    # (n_seq, seq_lens, Hkv, Hq, D, P, chunk)
    (1, (300,), 1, 4, 64, 16, 40),          # 160 rows: a full and a partial tile
    (2, (777, 205), 2, 12, 128, 32, 50),    # ragged, 300 rows per KV head
    (1, (1500,), 4, 24, 256, 64, 100),      # 600 rows, 5 tiles
    (1, (130,), 2, 12, 256, 64, 130),       # the whole prompt as one chunk
    (2, (20, 61), 1, 4, 64, 16, 30),        # a chunk longer than the first context
    (1, (700,), 2, 16, 128, 128, 33),       # 128-token pages, 8 query heads per KV head
    (1, (1030,), 1, 2, 256, 256, 200),      # 256-token pages, a ragged last page
    (2, (97, 160), 4, 8, 64, 32, 64),       # 32-token pages, two sequences sharing the pool
]


def _prefill(inp, cache, num_splits=0, max_seq_len=None):
    torch = H.torch_mod()
    q = H.to_dev(inp.q_bits).view(torch.float16)
    msl = int(max_seq_len or int(inp.seq_lens.max()))
    out, lse = H.kvq().prefill_attn(cache, q, H.to_dev(inp.page_table), H.to_dev(inp.seq_lens),
                                    msl, num_splits=num_splits)
    torch.cuda.synchronize()
    return out.cpu().numpy(), lse.cpu().numpy()


def _check(tag, out, lse, ref_out, ref_lse):
    H.assert_close(tag, out, ref_out)
    H.assert_lse(tag, lse, ref_lse)


@FMTS
@pytest.mark.parametrize("case", range(len(CASES)))
def test_prefill_every_output(case, kv_format):
    n_seq, lens, hkv, hq, D, P, C = CASES[case]
    H.say(f"[prefill] case {case} fmt {H.FORMAT_IDS[kv_format]}: lens {lens} D {D} P {P} C {C}")
    inp = W.custom(n_seq=n_seq, seq_lens=lens, num_kv_heads=hkv, n_q_heads=hq, head_dim=D,
                   page_size=P, n_rows=C, seed=600 + case)
    cache = H.gpu_cache(inp, kv_format)
    H.gpu_append(cache, *inp.all_tokens())
    pool = H.oracle_fill(inp, kv_format)
    assert np.array_equal(cache.pool.cpu().numpy(), pool)
    ref_out, ref_lse = H.oracle_decode(inp, pool, kv_format=kv_format)
    for splits in (0, 1, 3):
        out, lse = _prefill(inp, cache, splits)
        _check(f"case {case} splits {splits}", out, lse, ref_out, ref_lse)


@FMTS
def test_prefill_unwritten_slots_hold_junk(kv_format):
    """Slots never appended hold 0xFF bytes (NaN scales and E4M3 codes); the ragged context ends
    read them into the staged blocks."""
    torch = H.torch_mod()
    H.say(f"[prefill junk] {H.FORMAT_IDS[kv_format]}")
    inp = W.custom(n_seq=2, seq_lens=(333, 250), num_kv_heads=2, n_q_heads=12, head_dim=256,
                   page_size=64, n_rows=37, seed=650)
    cache = H.gpu_cache(inp, kv_format)
    cache.pool.fill_(0xFF)
    torch.cuda.synchronize()
    H.gpu_append(cache, *inp.all_tokens())
    ref_out, ref_lse = H.oracle_decode(inp, H.oracle_fill(inp, kv_format), kv_format=kv_format)
    for splits in (0, 2):
        out, lse = _prefill(inp, cache, splits)
        _check(f"junk splits {splits}", out, lse, ref_out, ref_lse)


@pytest.mark.parametrize("C", [1, 4])
def test_prefill_matches_decode_at_small_chunks(C):
    """A chunk of C <= 4 positions is a decode step with C query rows: the two kernels agree to
    fp32 rounding."""
    H.say(f"[prefill vs decode] C {C}")
    inp = W.custom(n_seq=2, seq_lens=(900, 417), num_kv_heads=4, n_q_heads=24, head_dim=256,
                   page_size=64, n_rows=C, seed=660 + C)
    cache = H.gpu_cache(inp)
    H.gpu_append(cache, *inp.all_tokens())
    out_p, lse_p = _prefill(inp, cache)
    out_d, lse_d = H.gpu_decode(inp, cache)
    scale = float(np.max(np.abs(out_d)))
    assert float(np.max(np.abs(out_p - out_d))) <= 1e-5 * scale
    np.testing.assert_allclose(lse_p, lse_d, rtol=0, atol=1e-5)


def chunk_queries(n_seq, chunk, n_q_heads, head_dim, seed):
    """fp16 bits of N(0,1) queries for a prefill chunk."""
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((n_seq, chunk, n_q_heads, head_dim), dtype=np.float32)
    return np.ascontiguousarray(q.astype(np.float16).view(np.uint16))


def test_prefill_full_size_sampled_rows():
    """The last 1,024-position chunk of each 92,160-token sequence of the 184K-token pool,
    automatic plan: sampled positions and heads against the oracle."""
    torch = H.torch_mod()
    inp, pool = H.full_workload("ctx184k_c2")
    wl = inp.wl
    C = 1024
    H.say(f"[prefill full] ctx184k_c2 chunk {C}")
    cache = H.gpu_fill(inp)
    q_bits = chunk_queries(wl.n_seq, C, wl.n_q_heads, wl.head_dim, 2024)
    q = H.to_dev(q_bits).view(torch.float16)
    out, lse = H.kvq().prefill_attn(cache, q, H.to_dev(inp.page_table), H.to_dev(inp.seq_lens),
                                    wl.seq_len)
    torch.cuda.synchronize()
    out, lse = out.cpu().numpy(), lse.cpu().numpy()
    sel = [(0, 0, 0), (0, 511, 7), (1, 1023, 23), (1, 300, 12), (0, 1023, 5), (1, 0, 18)]
    ref_out, ref_lse = H.oracle.decode_attn(pool, wl.pool_pages, wl.page_size, wl.num_kv_heads,
                                            wl.head_dim, q_bits, inp.page_table, inp.seq_lens, C,
                                            wl.n_q_heads, select=sel)
    got = np.stack([out[b, i, h] for b, i, h in sel])
    got_lse = np.array([lse[b, i, h] for b, i, h in sel])
    _check("ctx184k_c2 chunk 1024 sampled", got, got_lse, ref_out, ref_lse)

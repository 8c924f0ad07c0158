"""kvq_decode_step_noalloc (split partials in the library's static device array, no workspace)
against kvq_decode_step_fmt with a caller workspace: the same pool bytes and bit-identical
outputs and log-sum-exps on calls in a row, each smaller than the one before, and both within
the oracle's bounds."""
import numpy as np
import pytest

from long_context_decode_flash_amd import workloads as W
from tests import gpu_helpers as H

pytestmark = pytest.mark.gpu

CALLS = [
    # MTP verify rows (24 per KV head, two row blocks), the automatic plan over two sequences,
    # four new tokens appended inside the launch
    (0, dict(n_seq=2, seq_lens=(3000, 1900), num_kv_heads=4, n_q_heads=24, head_dim=256,
             page_size=64, n_rows=4, seed=71), 4, 0),
    # smaller: one sequence, 8 rows per KV head, head_dim 128, three splits (the scratch still
    # holds the first call's partials, which this call must not read)
    (0, dict(n_seq=1, seq_lens=(700,), num_kv_heads=2, n_q_heads=8, head_dim=128, page_size=32,
             n_rows=1, seed=72), 1, 3),
    # smaller still, fp8 codes, one split (the attention kernel writes the output itself)
    (2, dict(n_seq=1, seq_lens=(150,), num_kv_heads=1, n_q_heads=4, head_dim=64, page_size=16,
             n_rows=2, seed=73), 2, 1),
]


def test_noalloc_step_matches_the_workspace_step():
    import torch
    kvq = H.kvq()
    for kv_format, case, n_new, splits in CALLS:
        H.say(f"[noalloc] {H.FORMAT_IDS[kv_format]} {case} n_new {n_new} splits {splits}")
        inp = W.custom(**case)
        pre, _, k_new, v_new = inp.ragged_split(n_new)
        q = H.to_dev(inp.q_bits).view(torch.float16)
        pt, sl = H.to_dev(inp.page_table), H.to_dev(inp.seq_lens)
        msl = int(inp.seq_lens.max())
        kn, vn = H.to_dev(k_new), H.to_dev(v_new)
        a = H.gpu_cache(inp, kv_format)
        H.gpu_append(a, *pre)
        b = H.gpu_cache(inp, kv_format)
        H.gpu_append(b, *pre)
        out_a, lse_a = kvq.decode_step(a, kn, vn, q, pt, sl, msl, num_splits=splits)
        out_b, lse_b = kvq.decode_step_noalloc(b, kn, vn, q, pt, sl, msl, num_splits=splits)
        torch.cuda.synchronize()
        assert torch.equal(a.pool, b.pool), "pool bytes differ"
        assert torch.equal(out_a, out_b), "outputs differ from kvq_decode_step_fmt"
        assert torch.equal(lse_a, lse_b), "lse differs from kvq_decode_step_fmt"
        pool_ref = H.oracle_fill(inp, kv_format)
        assert np.array_equal(b.pool.cpu().numpy(), pool_ref)
        out_r, lse_r = H.oracle_decode(inp, pool_ref, kv_format=kv_format)
        H.assert_close("  out", out_b.cpu().numpy(), out_r)
        H.assert_lse("  lse", lse_b.cpu().numpy(), lse_r)

"""GPU parity: the HIP path (through the C ABI) against the CPU oracle on the same seeded inputs.

Bar: pool bytes (codes and scales) bit-exact; attention max-abs <= 2e-3 against the fp64
oracle and <= 1e-3 of the largest |ref| of the compared outputs, log-sum-exp within 1e-4,
element by element: at sizes the oracle finishes in seconds, and on every output row of the
full-size workloads in the launch configuration the benchmark times.
"""
import numpy as np
import pytest

from long_context_decode_flash_amd import workloads as W
from tests import gpu_helpers as H

pytestmark = pytest.mark.gpu


# ------------------------------------------------------------------ append ---------------

@pytest.mark.parametrize("name", list(W.WORKLOADS))
def test_append_pool_bytes_bit_exact_full_size(name):
    H.say(f"[append bit-exact] {name}")
    inp, pool_ref = H.full_workload(name)
    cache = H.gpu_fill(inp)
    pool = cache.pool.cpu().numpy()
    diff = np.flatnonzero(pool != pool_ref)
    H.say(f"  pool {pool.size} B, differing bytes {diff.size}")
    assert diff.size == 0, f"first differing byte at {diff[:8]}"


def test_append_edge_rows_bit_exact():
    """Zero rows, tiny (subnormal-scale) rows, huge (saturating) rows, exact ties, padding
    slots (-1) and slots past the pool in one call."""
    H.say("[append edge rows]")
    rng = np.random.default_rng(77)
    for P, D, Hkv in ((16, 64, 2), (64, 256, 1), (32, 128, 3)):
        pages = 6
        n = 12
        k = rng.standard_normal((n, Hkv, D)).astype(np.float32)
        v = rng.standard_normal((n, Hkv, D)).astype(np.float32)
        k[0] = 0.0
        v[0] = 0.0
        k[1] *= np.float32(1e-6)
        v[1] *= np.float32(1e-7)
        k[2] *= np.float32(1e7)
        v[2] *= np.float32(1e6)
        k[3] = (np.arange(D) % 17 - 8 + 0.5).astype(np.float32)  # halves: ties under scale 1
        k[3, :, 0] = 127.0
        v[4, :, :] = np.float32(3.5)
        v[4, :, ::32] = np.float32(7.0)
        slots = rng.choice(pages * P, n, replace=False).astype(np.int32)
        slots[5] = -1
        slots[6] = pages * P + 3
        inp_pool = H.oracle.new_pool(pages, P, Hkv, D)
        H.oracle.append(inp_pool, pages, P, Hkv, D, k, v, slots)
        cache = H.kvq().PagedCache.allocate(pages, P, Hkv, D)
        H.gpu_append(cache, k, v, slots)
        got = cache.pool.cpu().numpy()
        assert np.array_equal(got, inp_pool), (P, D, Hkv, np.flatnonzero(got != inp_pool)[:8])


def test_append_fp8_rounding_edges_bit_exact():
    """fp8 codes at the edges of E4M3 rounding, against the oracle's encoder: with a K row's
    absmax 448 the scale is exactly 1, so each value is its own quotient: exact midpoints
    between normal neighbours (ties go to the even mantissa), midpoints between subnormals and
    at the subnormal/normal edge, negative values that round to zero (code 0x80), the largest
    value, and -0.0 itself (code 0x80, the sign of the IEEE quotient); plus zero, tiny and huge
    rows and V groups of mixed magnitudes."""
    H.say("[append fp8 edges]")
    rng = np.random.default_rng(79)
    ties = np.array([1.0625, 1.1875, 1.3125, 3.75 + 0.125, 0.5 * 2.0 ** -9, 1.5 * 2.0 ** -9,
                     7.5 * 2.0 ** -9, 2.0 ** -6 + 2.0 ** -10, 2.0 ** -6 + 3 * 2.0 ** -10, 240.0 + 8.0,
                     416.0 + 8.0, 448.0, 0.25 * 2.0 ** -9, 0.75 * 2.0 ** -9], np.float64)
    for P, D, Hkv in ((16, 64, 2), (64, 256, 1), (32, 128, 3)):
        pages = 6
        n = 12
        k = rng.standard_normal((n, Hkv, D)).astype(np.float32)
        v = rng.standard_normal((n, Hkv, D)).astype(np.float32)
        k[0] = 0.0
        v[0] = 0.0
        k[1] *= np.float32(1e-6)
        v[1] *= np.float32(1e-7)
        k[2] *= np.float32(1e7)
        v[2] *= np.float32(1e6)
        row = np.resize(np.concatenate([ties, -ties]), D).astype(np.float32)
        row[0] = 448.0
        row[1] = -0.0
        k[3] = row
        v[3] = row
        k[7, :, 3::17] = np.float32(-0.0)
        v[7, :, 5::11] = np.float32(-0.0)
        v[4, :, :] = np.float32(3.5)
        v[4, :, ::32] = np.float32(448.0)
        slots = rng.choice(pages * P, n, replace=False).astype(np.int32)
        slots[5] = -1
        slots[6] = pages * P + 3
        ref = H.oracle.new_pool(pages, P, Hkv, D, 8)
        H.oracle.append(ref, pages, P, Hkv, D, k, v, slots, kv_format=2)
        cache = H.kvq().PagedCache.allocate(pages, P, Hkv, D, kv_format=2)
        H.gpu_append(cache, k, v, slots)
        got = cache.pool.cpu().numpy()
        assert np.array_equal(got, ref), (P, D, Hkv, np.flatnonzero(got != ref)[:8])


@pytest.mark.parametrize("kv_format", [0, 1, 2], ids=["k8v4", "k8v8", "fp8"])
def test_append_tile_and_row_paths_bit_exact(kv_format):
    """Groups of 16 tokens that fill one tile in order are written as whole tiles; any other
    group token by token.  One call mixes both: whole tiles, a run starting mid-tile, a tile with
    two slots swapped, a tile with a padding slot, and a short last group."""
    H.say(f"[append tile / row paths] format {kv_format}")
    vb = H.VBITS[kv_format]
    rng = np.random.default_rng(78)
    for P, D, Hkv in ((64, 256, 2), (16, 64, 1), (32, 128, 3)):
        # segments in disjoint 64-slot regions (no slot written twice, whatever the page size);
        # each is one 16-token group of the kernel (groups start at multiples of 16 tokens)
        pages = 12 * 64 // P
        slots = [np.arange(64, 64 + 48)]                        # 3 whole tiles
        slots.append(np.arange(192 + 8, 192 + 24))              # mid-tile start
        sw = np.arange(320, 336)
        sw[[3, 7]] = sw[[7, 3]]
        slots.append(sw)                                        # out of order
        pad = np.arange(384 + 16, 384 + 32)
        pad[5] = -1
        slots.append(pad)                                       # padding inside a tile
        slots.append(np.arange(512, 528))                       # whole tile
        slots.append(np.arange(576, 581))                       # short last group
        slots = np.concatenate(slots).astype(np.int32)
        n = slots.size
        k = rng.standard_normal((n, Hkv, D)).astype(np.float32)
        v = rng.standard_normal((n, Hkv, D)).astype(np.float32)
        k[2] = 0.0
        v[50] *= np.float32(1e-6)
        ref = H.oracle.new_pool(pages, P, Hkv, D, vb)
        H.oracle.append(ref, pages, P, Hkv, D, k, v, slots, kv_format=kv_format)
        cache = H.kvq().PagedCache.allocate(pages, P, Hkv, D, kv_format=kv_format)
        H.gpu_append(cache, k, v, slots)
        got = cache.pool.cpu().numpy()
        assert np.array_equal(got, ref), (P, D, Hkv, np.flatnonzero(got != ref)[:8])


# ------------------------------------------------------------------ decode, small --------

SMALL = [
    W.WORKLOADS["tiny_512"],
    W.scaled(W.WORKLOADS["ctx8k"], 1000),
    W.scaled(W.WORKLOADS["ctx64k_outlier"], 777),
    W.scaled(W.WORKLOADS["ctx184k_c2"], 611),
    W.scaled(W.WORKLOADS["ctx256k_mtp"], 1003),
]


@pytest.mark.parametrize("wl", SMALL, ids=lambda w: w.name)
def test_decode_small_every_output(wl):
    """Every output element at sizes spanning several tiles and a ragged tail."""
    H.say(f"[decode small] {wl.name} L={wl.seq_len}")
    inp = W.generate(wl)
    cache = H.gpu_fill(inp)
    pool_ref = H.oracle_fill(inp)
    assert np.array_equal(cache.pool.cpu().numpy(), pool_ref)
    out, lse = H.gpu_decode(inp, cache)
    out_r, lse_r = H.oracle_decode(inp, pool_ref)
    H.assert_close("  out", out, out_r)
    H.assert_lse("  lse", lse, lse_r)


@pytest.mark.parametrize("case", [
    dict(n_seq=1, seq_lens=(1,), n_rows=1),
    dict(n_seq=1, seq_lens=(4,), n_rows=4),
    dict(n_seq=1, seq_lens=(32,), n_rows=1),
    dict(n_seq=1, seq_lens=(33,), n_rows=2),
    dict(n_seq=1, seq_lens=(16,), n_rows=1),
    dict(n_seq=3, seq_lens=(1, 200, 47), n_rows=1),
    dict(n_seq=2, seq_lens=(2, 129), n_rows=4),   # rows 0-1 of seq 0 see no token
], ids=lambda c: "L" + "-".join(map(str, c["seq_lens"])) + f"_R{c['n_rows']}")
def test_decode_edge_lengths(case):
    H.say(f"[decode edge] {case}")
    inp = W.custom(num_kv_heads=2, n_q_heads=6, head_dim=64, page_size=16, seed=5, **case)
    cache = H.gpu_fill(inp)
    out, lse = H.gpu_decode(inp, cache)
    out_r, lse_r = H.oracle_decode(inp, H.oracle_fill(inp))
    H.assert_close("  out", out, out_r)
    finite = np.isfinite(lse_r)
    assert np.all(out[~finite] == 0)
    H.assert_lse("  lse", lse, lse_r)


@pytest.mark.parametrize("shape", [
    dict(head_dim=64, page_size=16, num_kv_heads=1, n_q_heads=1, n_rows=1),
    dict(head_dim=128, page_size=32, num_kv_heads=2, n_q_heads=16, n_rows=2),
    dict(head_dim=256, page_size=256, num_kv_heads=1, n_q_heads=8, n_rows=4),   # 32 rows
    dict(head_dim=128, page_size=128, num_kv_heads=4, n_q_heads=4, n_rows=3),
    dict(head_dim=256, page_size=16, num_kv_heads=2, n_q_heads=32, n_rows=1),
], ids=lambda s: "D{head_dim}_P{page_size}_G{g}_R{n_rows}".format(
    g=s["n_q_heads"] // s["num_kv_heads"], **s))
def test_decode_shapes(shape):
    H.say(f"[decode shapes] {shape}")
    inp = W.custom(n_seq=2, seq_lens=(531, 300), seed=9, **shape)
    cache = H.gpu_fill(inp)
    out, lse = H.gpu_decode(inp, cache)
    out_r, lse_r = H.oracle_decode(inp, H.oracle_fill(inp))
    H.assert_close("  out", out, out_r)
    H.assert_lse("  lse", lse, lse_r)


@pytest.mark.parametrize("wl", SMALL[1:], ids=lambda w: w.name)
def test_decode_peaked_attention(wl):
    """Queries scaled by 8: attention concentrates on a few tokens, outputs are O(1)."""
    wl = W.scaled(wl, wl.seq_len, name=wl.name + "_peaked", q_scale=8.0)
    H.say(f"[decode peaked] {wl.name}")
    inp = W.generate(wl)
    cache = H.gpu_fill(inp)
    out, lse = H.gpu_decode(inp, cache)
    out_r, lse_r = H.oracle_decode(inp, H.oracle_fill(inp))
    H.assert_close("  out", out, out_r)
    H.assert_lse("  lse", lse, lse_r)


def test_decode_split_count_invariance():
    wl = W.scaled(W.WORKLOADS["ctx184k_c2"], 3001)
    H.say(f"[split invariance] {wl.name}")
    inp = W.generate(wl)
    cache = H.gpu_fill(inp)
    base, lbase = H.gpu_decode(inp, cache, num_splits=1)
    for s in (2, 7, 0, 94):
        out, lse = H.gpu_decode(inp, cache, num_splits=s)
        assert H.report(f"  splits={s}", out, base) <= 1e-5
        np.testing.assert_allclose(lse, lbase, rtol=0, atol=1e-5)


def test_decode_page_permutation_bit_identical():
    wl = W.scaled(W.WORKLOADS["ctx184k_c2"], 2000)
    H.say(f"[page permutation] {wl.name}")
    inp = W.generate(wl)
    out_a, lse_a = H.gpu_decode(inp, H.gpu_fill(inp))
    perm = np.random.default_rng(3).permutation(wl.pool_pages).astype(np.int32)
    inp.page_table = perm[inp.page_table]
    out_b, lse_b = H.gpu_decode(inp, H.gpu_fill(inp))
    assert np.array_equal(out_a, out_b) and np.array_equal(lse_a, lse_b)


def test_decode_mtp_rows_equal_single_row_decodes():
    wl = W.scaled(W.WORKLOADS["ctx256k_mtp"], 1500)
    H.say(f"[mtp rows] {wl.name}")
    inp = W.generate(wl)
    cache = H.gpu_fill(inp)
    L, R = wl.seq_len, wl.n_rows
    out, lse = H.gpu_decode(inp, cache, num_splits=5, max_seq_len=L)
    for i in range(R):
        one = W.generate(wl)
        one.wl = W.scaled(wl, L, n_rows=1, n_new=0)
        one.q_bits = np.ascontiguousarray(inp.q_bits[:, i:i + 1])
        one.seq_lens = np.array([L - R + 1 + i], np.int32)
        one.page_table = inp.page_table
        o1, l1 = H.gpu_decode(one, cache, num_splits=5, max_seq_len=L)
        assert H.report(f"  row {i}", o1[0, 0], out[0, i]) <= 1e-6
        np.testing.assert_allclose(l1[0, 0], lse[0, i], rtol=0, atol=1e-6)


def test_decode_batch_equals_each_sequence_alone():
    inp = W.custom(n_seq=2, seq_lens=(700, 450), num_kv_heads=2, n_q_heads=12, head_dim=256,
                   page_size=64, n_rows=1, seed=12)
    H.say("[batch vs alone]")
    cache = H.gpu_fill(inp)
    out, lse = H.gpu_decode(inp, cache, num_splits=6, max_seq_len=700)
    for b in range(2):
        one = W.custom(n_seq=2, seq_lens=(700, 450), num_kv_heads=2, n_q_heads=12,
                       head_dim=256, page_size=64, n_rows=1, seed=12)
        one.wl = W.scaled(inp.wl, 700, n_seq=1)
        one.q_bits = np.ascontiguousarray(inp.q_bits[b:b + 1])
        one.page_table = np.ascontiguousarray(inp.page_table[b:b + 1])
        one.seq_lens = inp.seq_lens[b:b + 1].copy()
        o1, l1 = H.gpu_decode(one, cache, num_splits=6, max_seq_len=700)
        assert np.array_equal(o1[0], out[b]) and np.array_equal(l1[0], lse[b])


# ------------------------------------------------------------------ K8/V8 and fp8 ----------
# 8-bit V codes (KVQ_FORMAT_K8V8) and E4M3 K and V codes (KVQ_FORMAT_FP8): the same bar, pool
# bytes bit-exact and outputs within 2e-3.

V8_SMALL = SMALL + [W.custom(n_seq=2, seq_lens=(700, 333), num_kv_heads=2, n_q_heads=12,
                             head_dim=128, page_size=32, n_rows=2, seed=61, name="d128").wl,
                    W.custom(n_seq=1, seq_lens=(300,), num_kv_heads=1, n_q_heads=4,
                             head_dim=64, page_size=16, n_rows=1, seed=300, name="d64_ragged").wl]
FMT8 = pytest.mark.parametrize("kv_format", [1, 2], ids=["k8v8", "fp8"])


@FMT8
@pytest.mark.parametrize("wl", V8_SMALL, ids=lambda w: w.name)
def test_v8_decode_small_every_output(wl, kv_format):
    H.say(f"[{H.FORMAT_IDS[kv_format]} small] {wl.name} L={wl.seq_len}")
    inp = W.generate(wl)
    cache = H.gpu_fill(inp, kv_format=kv_format)
    pool_ref = H.oracle_fill(inp, kv_format)
    assert np.array_equal(cache.pool.cpu().numpy(), pool_ref)
    for splits in (0, 3):
        out, lse = H.gpu_decode(inp, cache, num_splits=splits)
        out_r, lse_r = H.oracle_decode(inp, pool_ref, kv_format=kv_format)
        H.assert_close(f"  out (splits {splits})", out, out_r)
        H.assert_lse(f"  lse (splits {splits})", lse, lse_r)


@FMT8
def test_v8_peaked_attention(kv_format):
    """Queries scaled up so the softmax concentrates on few tokens and outputs are O(1)."""
    wl = W.scaled(W.WORKLOADS["ctx184k_c2"], 611, name="c2_611_peaked", q_scale=8.0)
    H.say(f"[{H.FORMAT_IDS[kv_format]} peaked] {wl.name}")
    inp = W.generate(wl)
    cache = H.gpu_fill(inp, kv_format=kv_format)
    pool_ref = H.oracle_fill(inp, kv_format)
    out, lse = H.gpu_decode(inp, cache)
    out_r, lse_r = H.oracle_decode(inp, pool_ref, kv_format=kv_format)
    H.assert_close("  out", out, out_r)
    H.assert_lse("  lse", lse, lse_r)


@FMT8
def test_v8_step_equals_append_then_decode(kv_format):
    """kvq_decode_step in an 8-bit format: the same pool bytes and outputs as kvq_append
    followed by kvq_decode_attn, and the oracle's."""
    import torch
    H.say(f"[{H.FORMAT_IDS[kv_format]} step]")
    kvq = H.kvq()
    inp = W.custom(n_seq=1, seq_lens=(1154,), num_kv_heads=4, n_q_heads=24, head_dim=256,
                   page_size=64, n_rows=4, seed=62)
    wl = inp.wl
    n_new = 4
    pre, new_flat, k_new, v_new = inp.ragged_split(n_new)
    a = H.gpu_cache(inp, kv_format)
    H.gpu_append(a, *pre)
    H.gpu_append(a, *new_flat)
    out_a, lse_a = H.gpu_decode(inp, a, num_splits=7)
    b = H.gpu_cache(inp, kv_format)
    H.gpu_append(b, *pre)
    q = H.to_dev(inp.q_bits).view(torch.float16)
    out_b, lse_b = kvq.decode_step(b, H.to_dev(k_new), H.to_dev(v_new), q, H.to_dev(inp.page_table),
                                   H.to_dev(inp.seq_lens), wl.seq_len, num_splits=7)
    torch.cuda.synchronize()
    assert np.array_equal(a.pool.cpu().numpy(), b.pool.cpu().numpy())
    assert np.array_equal(out_a, out_b.cpu().numpy()) and np.array_equal(lse_a, lse_b.cpu().numpy())
    out_r, _ = H.oracle_decode(inp, H.oracle_fill(inp, kv_format), kv_format=kv_format)
    H.assert_close("  out", out_a, out_r)


@FMT8
def test_v8_full_size_headline(kv_format):
    """The 184K-token two-sequence workload in an 8-bit format with the automatic plan: the
    whole pool bit-exact, every output row against the oracle."""
    H.say(f"[{H.FORMAT_IDS[kv_format]} full] ctx184k_c2")
    inp = W.generate(W.WORKLOADS["ctx184k_c2"])
    pool_ref = H.oracle_fill(inp, kv_format)
    cache = H.gpu_fill(inp, kv_format=kv_format)
    got = cache.pool.cpu().numpy()
    assert np.array_equal(got, pool_ref), np.flatnonzero(got != pool_ref)[:8]
    out, lse = H.gpu_decode(inp, cache)
    out_r, lse_r = H.oracle_decode(inp, pool_ref, kv_format=kv_format)
    H.assert_close("  out", out, out_r)
    H.assert_lse("  lse", lse, lse_r)


@pytest.mark.parametrize("kv_format", [0, 1, 2], ids=["k8v4", "k8v8", "fp8"])
def test_decode_unwritten_slots_hold_junk(kv_format):
    """Slots no token was appended to hold 0xFF bytes (NaN scales, NaN E4M3 codes): the ragged
    ends of the contexts and the slots before a window start read such bytes into the staged
    blocks, and the outputs must still match the oracle's."""
    import torch
    H.say(f"[junk slots] {H.FORMAT_IDS[kv_format]}")
    for lens, D, P, R, hkv, hq in (((300, 77), 256, 64, 4, 4, 24), ((333,), 64, 16, 1, 1, 4),
                                   ((515, 100), 128, 32, 2, 2, 12)):
        inp = W.custom(n_seq=len(lens), seq_lens=lens, num_kv_heads=hkv, n_q_heads=hq,
                       head_dim=D, page_size=P, n_rows=R, seed=90 + D)
        cache = H.gpu_cache(inp, kv_format)
        cache.pool.fill_(0xFF)
        torch.cuda.synchronize()
        k, v, slots = inp.all_tokens()
        H.gpu_append(cache, k, v, slots)
        pool_ref = H.oracle_fill(inp, kv_format)
        for splits in (0, 3):
            out, lse = H.gpu_decode(inp, cache, num_splits=splits)
            out_r, lse_r = H.oracle_decode(inp, pool_ref, kv_format=kv_format)
            H.assert_close(f"  D {D} splits {splits}", out, out_r)
            H.assert_lse(f"  D {D} splits {splits}", lse, lse_r)
        # a window whose start falls inside a block: the slots before it are real tokens here,
        # and the junk beyond the ends is read as above
        q = H.to_dev(inp.q_bits).view(torch.float16)
        for window in (45, 200):
            out, lse = H.kvq().decode_attn(cache, q, H.to_dev(inp.page_table),
                                           H.to_dev(inp.seq_lens), int(max(lens)),
                                           window=window)
            torch.cuda.synchronize()
            wl = inp.wl
            out_r, lse_r = H.oracle.decode_attn(pool_ref, wl.pool_pages, P, hkv, D, inp.q_bits,
                                                inp.page_table, inp.seq_lens, R, hq,
                                                kv_format=kv_format, window=window)
            H.assert_close(f"  D {D} window {window}", out.cpu().numpy(), out_r)
            H.assert_lse(f"  D {D} window {window}", lse.cpu().numpy(), lse_r)


# ------------------------------------------------------------------ decode, full size ----

def _full_step(inp):
    """The benchmark's launch configuration on a full-size workload: the cached context
    appended with kvq_append, then one kvq_decode_step that appends the step's new tokens and
    attends (kvq_decode_attn when the step appends nothing), with the automatic split plan."""
    import torch
    kvq = H.kvq()
    wl = inp.wl
    cache = H.gpu_cache(inp)
    H.gpu_append(cache, *inp.prefill())
    q = H.to_dev(inp.q_bits).view(torch.float16)
    pt, sl = H.to_dev(inp.page_table), H.to_dev(inp.seq_lens)
    if wl.n_new:
        n = wl.seq_len - wl.n_new
        out, lse = kvq.decode_step(cache, H.to_dev(inp.k[:, n:]), H.to_dev(inp.v[:, n:]), q, pt, sl,
                                   wl.seq_len)
    else:
        out, lse = kvq.decode_attn(cache, q, pt, sl, wl.seq_len)
    torch.cuda.synchronize()
    return cache, out.cpu().numpy(), lse.cpu().numpy()


@pytest.mark.parametrize("name", list(W.WORKLOADS))
def test_decode_full_size_every_row(name):
    """Full-size workloads in the configuration the benchmark times: the pool bytes after the
    step bit-exact, and every output row (every sequence, query row and query head) against the
    oracle."""
    H.say(f"[decode full] {name}")
    inp, pool_ref = H.full_workload(name)
    cache, out, lse = _full_step(inp)
    got = cache.pool.cpu().numpy()
    assert np.array_equal(got, pool_ref), np.flatnonzero(got != pool_ref)[:8]
    del got
    out_r, lse_r = H.oracle_decode(inp, pool_ref)
    H.assert_close("  out", out, out_r)
    H.assert_lse("  lse", lse, lse_r)


@pytest.mark.parametrize("name", ["ctx184k_c2", "ctx256k_mtp"])
def test_decode_full_size_peaked_every_row(name):
    """The same full-size steps with the queries scaled by 8 (exact in fp16): the softmax
    concentrates on a few tokens, so outputs are O(1) and rounding errors are not hidden by the
    ~sqrt(e/N) magnitude of a flat average."""
    import copy
    H.say(f"[decode full peaked] {name}")
    inp, pool_ref = H.full_workload(name)
    peaked = copy.copy(inp)
    peaked.q_bits = (inp.q_bits.view(np.float16) * np.float16(8.0)).view(np.uint16)
    assert np.array_equal(peaked.q_bits.view(np.float16) / np.float16(8.0), inp.q_bits.view(np.float16))
    _, out, lse = _full_step(peaked)
    out_r, lse_r = H.oracle_decode(peaked, pool_ref)
    H.assert_close("  out", out, out_r)
    H.assert_lse("  lse", lse, lse_r)
    assert float(np.max(np.abs(out_r))) > 0.3, "the peaked variant should give O(1) outputs"


@pytest.mark.parametrize("kv_format", [0, 2], ids=["k8v4", "fp8"])
def test_out_of_range_page_ids_are_clamped(kv_format):
    """Page-table entries outside [0, num_pages) read the clamped page and are never followed
    (the header's contract), in the decode (several splits, ids in the first and later chunks)
    and in the chunked prefill: outputs equal the oracle's, which clamps the same way."""
    import torch
    H.say(f"[page clamp] {H.FORMAT_IDS[kv_format]}")
    inp = W.custom(n_seq=2, seq_lens=(2200, 700), num_kv_heads=2, n_q_heads=12, head_dim=256,
                   page_size=64, n_rows=2, seed=4243)
    wl = inp.wl
    cache = H.gpu_fill(inp, kv_format=kv_format)
    pool_ref = H.oracle_fill(inp, kv_format)
    bad = inp.page_table.copy()
    bad[0, 1] = -1
    bad[0, 20] = wl.pool_pages + 5
    bad[0, 34] = 2 ** 31 - 1  # the last page of sequence 0
    bad[1, 0] = -(2 ** 31)
    bad[1, 7] = wl.pool_pages
    ref = H.oracle.decode_attn(pool_ref, wl.pool_pages, wl.page_size, wl.num_kv_heads,
                               wl.head_dim, inp.q_bits, bad, inp.seq_lens, wl.n_rows,
                               wl.n_q_heads, kv_format=kv_format)
    for splits in (0, 1, 5):
        out, lse = H.gpu_decode(inp, cache, num_splits=splits, page_table=bad)
        H.assert_close(f"  decode splits {splits}", out, ref[0])
        H.assert_lse(f"  decode splits {splits}", lse, ref[1])
    q = H.to_dev(inp.q_bits).view(torch.float16)
    out, lse = H.kvq().prefill_attn(cache, q, H.to_dev(bad), H.to_dev(inp.seq_lens), 2200)
    torch.cuda.synchronize()
    H.assert_close("  prefill", out.cpu().numpy(), ref[0])
    H.assert_lse("  prefill", lse.cpu().numpy(), ref[1])


def test_decode_rejects_small_workspace():
    import torch
    H.say("[workspace check]")
    inp = W.custom(n_seq=1, seq_lens=(100,), seed=2)
    cache = H.gpu_fill(inp)
    kvq = H.kvq()
    q = H.to_dev(inp.q_bits).view(torch.float16)
    with pytest.raises(kvq.KVQError) as e:
        kvq.decode_attn(cache, q, H.to_dev(inp.page_table), H.to_dev(inp.seq_lens), 100,
                        num_splits=2, workspace=torch.empty(16, dtype=torch.uint8, device="cuda"))
    assert e.value.code == kvq.KVQ_ERR_WORKSPACE


def test_decode_workspace_reused_across_shapes():
    """One workspace, never initialized, serves calls of different shapes in a row: nothing a
    call leaves in it affects the next."""
    import torch
    H.say("[workspace reuse]")
    kvq = H.kvq()
    cases = [
        W.custom(n_seq=2, seq_lens=(900, 333), num_kv_heads=2, n_q_heads=12, head_dim=256,
                 page_size=64, n_rows=1, seed=41),
        W.custom(n_seq=1, seq_lens=(1500,), num_kv_heads=4, n_q_heads=16, head_dim=128,
                 page_size=32, n_rows=4, seed=42),
        W.custom(n_seq=3, seq_lens=(70, 5, 260), num_kv_heads=1, n_q_heads=4, head_dim=64,
                 page_size=16, n_rows=2, seed=43),
    ]
    ws = torch.full((1 << 24,), 0xFF, dtype=torch.uint8, device="cuda")  # NaN bit patterns
    for rep in range(2):
        for splits in (0, 3):
            for inp in cases:
                wl = inp.wl
                cache = H.gpu_fill(inp)
                q = H.to_dev(inp.q_bits).view(torch.float16)
                out, lse = kvq.decode_attn(cache, q, H.to_dev(inp.page_table),
                                           H.to_dev(inp.seq_lens), int(inp.seq_lens.max()),
                                           num_splits=splits, workspace=ws)
                torch.cuda.synchronize()
                out_r, _ = H.oracle_decode(inp, H.oracle_fill(inp))
                H.assert_close(f"  rep {rep} splits {splits} {wl.head_dim}", out.cpu().numpy(), out_r)


# kvq_decode_step (append of each sequence's newest tokens fused into the decode launch) must
# leave the same pool bytes and return the same bits as kvq_append followed by kvq_decode_attn.
STEP_CASES = [
    dict(n_seq=2, seq_lens=(1000, 333), num_kv_heads=2, n_q_heads=12, head_dim=256,
         page_size=64, n_rows=1, n_new=1, splits=0, seed=51),
    # MTP verify: 4 new tokens across a 32-token block edge that is also a split edge (7 splits
    # of 6 blocks over 37 blocks put blocks 35 and 36 in different workgroups)
    dict(n_seq=1, seq_lens=(1154,), num_kv_heads=4, n_q_heads=24, head_dim=256, page_size=64,
         n_rows=4, n_new=4, splits=7, seed=52),
    # ragged, a sequence barely longer than its new tokens, head_dim 64, page 16
    dict(n_seq=3, seq_lens=(70, 5, 260), num_kv_heads=1, n_q_heads=4, head_dim=64,
         page_size=16, n_rows=2, n_new=3, splits=0, seed=53),
    dict(n_seq=1, seq_lens=(500,), num_kv_heads=2, n_q_heads=8, head_dim=128, page_size=32,
         n_rows=1, n_new=0, splits=2, seed=54),
    # one split per context (the attention kernel writes the output itself)
    dict(n_seq=2, seq_lens=(40, 64), num_kv_heads=2, n_q_heads=4, head_dim=128, page_size=16,
         n_rows=1, n_new=2, splits=1, seed=55),
]


@pytest.mark.parametrize("case", STEP_CASES, ids=[f"step{i}" for i in range(len(STEP_CASES))])
def test_decode_step_equals_append_then_decode(case):
    import torch
    kvq = H.kvq()
    c = dict(case)
    n_new, splits = c.pop("n_new"), c.pop("splits")
    H.say(f"[decode_step] {case}")
    inp = W.custom(**c)
    pre, new, k_new, v_new = inp.ragged_split(n_new)
    q = H.to_dev(inp.q_bits).view(torch.float16)
    pt, sl = H.to_dev(inp.page_table), H.to_dev(inp.seq_lens)
    msl = int(inp.seq_lens.max())
    a = H.gpu_cache(inp)
    H.gpu_append(a, *pre)
    H.gpu_append(a, *new)
    out_a, lse_a = kvq.decode_attn(a, q, pt, sl, msl, num_splits=splits)
    b = H.gpu_cache(inp)
    H.gpu_append(b, *pre)
    kn = H.to_dev(k_new) if n_new else None
    vn = H.to_dev(v_new) if n_new else None
    out_b, lse_b = kvq.decode_step(b, kn, vn, q, pt, sl, msl, num_splits=splits)
    torch.cuda.synchronize()
    assert torch.equal(a.pool, b.pool), "pool bytes differ from append + decode"
    assert torch.equal(out_a, out_b) and torch.equal(lse_a, lse_b)
    out_r, lse_r = H.oracle_decode(inp, H.oracle_fill(inp))
    assert np.array_equal(b.pool.cpu().numpy(), H.oracle_fill(inp))
    H.assert_close("  step out", out_b.cpu().numpy(), out_r)
    H.assert_lse("  step lse", lse_b.cpu().numpy(), lse_r)


def test_decode_step_full_size_headline():
    """The 184,320-token two-sequence step through kvq_decode_step: same pool bytes and bits
    as kvq_append + kvq_decode_attn."""
    import torch
    kvq = H.kvq()
    wl = W.WORKLOADS["ctx184k_c2"]
    H.say("[decode_step full size]")
    inp = W.generate(wl)
    k_new = inp.k[:, wl.seq_len - wl.n_new:]
    v_new = inp.v[:, wl.seq_len - wl.n_new:]
    q = H.to_dev(inp.q_bits).view(torch.float16)
    pt, sl = H.to_dev(inp.page_table), H.to_dev(inp.seq_lens)
    a = H.gpu_cache(inp)
    H.gpu_append(a, *inp.prefill())
    b = H.gpu_cache(inp)
    b.pool.copy_(a.pool)
    H.gpu_append(a, *inp.step_tokens())
    out_a, lse_a = kvq.decode_attn(a, q, pt, sl, wl.seq_len)
    out_b, lse_b = kvq.decode_step(b, H.to_dev(k_new), H.to_dev(v_new), q, pt, sl, wl.seq_len)
    torch.cuda.synchronize()
    assert torch.equal(a.pool, b.pool)
    assert torch.equal(out_a, out_b) and torch.equal(lse_a, lse_b)


def test_run_to_run_bit_identical():
    """The same call twice gives the same bytes: the decode step (append + attention, several
    splits), the chunked prefill and the append, with the workspace dirtied in between.  No
    result depends on which workgroup finishes first: splits merge in a fixed order and no
    kernel accumulates through atomics."""
    import torch
    H.say("[run to run]")
    kvq = H.kvq()
    inp = W.custom(n_seq=2, seq_lens=(3000, 1300), num_kv_heads=2, n_q_heads=12, head_dim=256,
                   page_size=64, n_rows=4, seed=515)
    wl = inp.wl
    q = H.to_dev(inp.q_bits).view(torch.float16)
    pt, sl = H.to_dev(inp.page_table), H.to_dev(inp.seq_lens)
    n_new = 4
    k_new = H.to_dev(np.ascontiguousarray(np.stack([inp.k[b, int(L) - n_new:int(L)] for b, L in
                                                    enumerate(inp.seq_lens)])))
    v_new = H.to_dev(np.ascontiguousarray(np.stack([inp.v[b, int(L) - n_new:int(L)] for b, L in
                                                    enumerate(inp.seq_lens)])))
    results = []
    for rep in range(2):
        cache = H.gpu_cache(inp)
        k, v, s = inp.all_tokens()
        keep = np.ones(len(s), bool)  # the step's tokens are appended by the step itself
        off = 0
        for b, L in enumerate(inp.seq_lens):
            keep[off + int(L) - n_new: off + int(L)] = False
            off += int(L)
        H.gpu_append(cache, k[keep], v[keep], s[keep])
        ws = torch.full((kvq.decode_workspace_bytes(wl.n_seq, wl.n_rows, wl.n_q_heads,
                                                    wl.num_kv_heads, wl.head_dim, 3000, 5),),
                        37 + rep, dtype=torch.uint8, device="cuda")
        out, lse = kvq.decode_step(cache, k_new, v_new, q, pt, sl, 3000, workspace=ws, num_splits=5)
        pout, plse = kvq.prefill_attn(cache, q, pt, sl, 3000)
        torch.cuda.synchronize()
        results.append([cache.pool.cpu().numpy(), out.cpu().numpy(), lse.cpu().numpy(),
                        pout.cpu().numpy(), plse.cpu().numpy()])
    for a, b in zip(*results):
        assert np.array_equal(a, b)

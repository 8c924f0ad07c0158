"""Pins of the CPU oracle against things other than itself (no GPU).

Each test ties a part of ``oracle/kvq_oracle.c`` to an independent fact: numpy's IEEE
float16/float32 arithmetic, an argmin over every code, hand-worked fixtures, closed forms of
softmax attention, structural invariants, and a pure-Python brute force on tiny inputs.
"""
import math
import os

import numpy as np
import pytest

import oracle
from tests import brute, pin_battery
from long_context_decode_flash_amd import workloads as W

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ------------------------------------------------------------------ fp16 conversion ------

def test_fp16_decode_all_patterns():
    """Every binary16 bit pattern decodes to numpy's float16 value."""
    o = oracle.default()
    for bits in range(0, 1 << 16, 1):
        ref = np.uint16(bits).view(np.float16)
        got = o.fp16_to_double(bits)
        if np.isnan(ref):
            assert math.isnan(got)
        else:
            assert got == float(ref), hex(bits)


def test_fp16_encode_matches_numpy_rne():
    """Round-to-nearest-even fp32 -> fp16 (normals, subnormals, exact ties, overflow)."""
    o = oracle.default()
    rng = np.random.default_rng(11)
    xs = list((rng.standard_normal(4000) * 10.0 ** rng.integers(-9, 6, 4000)).astype(np.float32))
    # exact ties between neighbouring fp16 values, in the normal and subnormal ranges
    for bits in list(range(0x0001, 0x0400, 37)) + list(range(0x0400, 0x7BFF, 997)):
        a = float(np.uint16(bits).view(np.float16))
        b = float(np.uint16(bits + 1).view(np.float16))
        xs.append(np.float32((a + b) / 2))
    xs += [np.float32(v) for v in (65504.0, 65519.0, 65520.0, 1e9, 2.0 ** -24, 2.0 ** -25,
                                   2.0 ** -25 * 1.0000001, 2.0 ** -14, 0.0, -0.0)]
    for x in xs:
        assert o.fp16_from_double(float(x)) == brute.fp16_bits_np(x), repr(x)
        assert o.fp16_from_double(-float(x)) == brute.fp16_bits_np(-x), repr(x)


# ------------------------------------------------------------------ quantizer ------------

def _codes_and_scale(x, qmax):
    return oracle.default().quantize_group(np.asarray(x, np.float32), qmax)


@pytest.mark.parametrize("qmax,n", [(127, 256), (127, 64), (7, 32)])
def test_quantizer_is_argmin_ties_to_even(qmax, n):
    """Away from near-ties, each code is the argmin over all codes of |x - c*s| with the
    stored fp16 scale; at a quotient within an ulp of a half-integer the code is one of the
    two nearest; the scale is numpy's fp16(fp32(absmax / qmax))."""
    rng = np.random.default_rng(qmax * 1000 + n)
    near_ties = 0
    for trial in range(60):
        x = rng.standard_normal(n).astype(np.float32) * np.float32(10.0 ** rng.integers(-3, 3))
        codes, sb = _codes_and_scale(x, qmax)
        a = np.max(np.abs(x))
        assert sb == brute.fp16_bits_np(np.float32(a) / np.float32(qmax))
        s = brute.fp16_value_np(sb)
        for xi, c in zip(x, codes):
            q = float(xi) / s
            frac = abs(q - math.floor(q) - 0.5)
            if frac < 1e-6 * max(1.0, abs(q)):
                near_ties += 1
                assert int(c) in (math.floor(q), math.ceil(q))
                continue
            assert int(c) == brute.argmin_code(float(xi), s, qmax), (xi, s)
    assert near_ties < 5


def test_quantizer_constructed_exact_ties_go_to_even():
    for qmax in (127, 7):
        s = 0.25  # exact fp16; absmax qmax*s makes the scale exactly 0.25
        vals = [qmax * s] + [(k + 0.5) * s for k in range(-qmax, qmax)]
        vals = vals[:32] if qmax == 7 else vals[:256]
        x = np.array(vals + [0.0] * (32 - len(vals) % 32 if len(vals) % 32 else 0), np.float32)
        codes, sb = _codes_and_scale(x, qmax)
        assert brute.fp16_value_np(sb) == s
        for xi, c in zip(x[1:len(vals)], codes[1:len(vals)]):
            k = math.floor(float(xi) / s)
            expect = k if k % 2 == 0 else k + 1
            assert int(c) == expect, (xi, c)


def test_quantizer_golden_cases():
    """Hand-worked groups: exact ties, a non-representable scale, zero, saturation, subnormal."""
    rows = []
    with open(os.path.join(GOLDEN, "quantizer_cases.txt")) as f:
        for line in f:
            line = line.split("#")[0].strip()
            if not line:
                continue
            qmax, vals, sb, codes = [p.strip() for p in line.split(";")]
            rows.append((int(qmax), [float(v) for v in vals.split()], int(sb, 16),
                         [int(c) for c in codes.split()]))
    assert len(rows) >= 7
    for qmax, vals, sb_ref, codes_ref in rows:
        x = np.zeros(32, np.float32)
        x[:len(vals)] = vals
        codes, sb = _codes_and_scale(x, qmax)
        assert sb == sb_ref, (vals, hex(sb))
        assert list(codes[:len(codes_ref)]) == codes_ref, (vals, codes)
        assert not np.any(codes[len(vals):]), "zeros must stay zero"


def test_quantizer_invariants():
    """Negation negates codes; scaling by 2^k scales the scale by 2^k and keeps the codes;
    |code| <= qmax and the absmax element maps to +-qmax when the scale is normal."""
    rng = np.random.default_rng(5)
    for qmax, n in ((127, 256), (7, 32)):
        for _ in range(40):
            x = rng.standard_normal(n).astype(np.float32)
            c, sb = _codes_and_scale(x, qmax)
            cn, sbn = _codes_and_scale(-x, qmax)
            assert sb == sbn and np.array_equal(cn, -c)
            assert np.all(np.abs(c.astype(int)) <= qmax)
            assert abs(int(c[np.argmax(np.abs(x))])) == qmax
            for k in (-6, -1, 3, 7):
                c2, sb2 = _codes_and_scale(x * np.float32(2.0 ** k), qmax)
                assert np.array_equal(c2, c)
                assert brute.fp16_value_np(sb2) == brute.fp16_value_np(sb) * 2.0 ** k


# ------------------------------------------------------------------ page format ----------

@pytest.mark.parametrize("vbits", [4, 8])
@pytest.mark.parametrize("P,D", [(16, 64), (64, 256), (32, 128), (16, 256), (256, 64)])
def test_format_is_a_bijection(P, D, vbits):
    """Each code, nibble and scale has its own place; the four sections tile the block (4-bit V
    codes two to a byte, 8-bit ones a byte each)."""
    o = oracle.default()
    bb = o.block_bytes(P, D, vbits)
    vbytes = P * D * vbits // 8
    assert bb == P * (D + 2 + D // 16) + vbytes
    k = {o.format_offset(0, P, D, s, d, vbits)[0] for s in range(P) for d in range(D)}
    assert k == set(range(0, P * D))
    ks = {o.format_offset(1, P, D, s, 0, vbits)[0] for s in range(P)}
    assert ks == set(range(P * D, P * D + 2 * P, 2))
    v = {o.format_offset(2, P, D, s, d, vbits) for s in range(P) for d in range(D)}
    v0 = P * D + 2 * P
    nibs = (0, 1) if vbits == 4 else (0,)
    assert v == {(b, nib) for b in range(v0, v0 + vbytes) for nib in nibs}
    vs = {o.format_offset(3, P, D, s, j, vbits)[0] for s in range(P) for j in range(D // 32)}
    vs0 = v0 + vbytes
    assert vs == set(range(vs0, vs0 + 2 * P * D // 32, 2)) and vs0 + 2 * P * D // 32 == bb
    # every byte of one token's codes belongs to that token alone
    owner = {}
    for s in range(P):
        for d in range(D):
            b, _ = o.format_offset(2, P, D, s, d, vbits)
            assert owner.setdefault(b, s) == s


def test_format_golden_offsets():
    o = oracle.default()
    n = 0
    with open(os.path.join(GOLDEN, "format_offsets.txt")) as f:
        for line in f:
            line = line.split("#")[0].strip()
            if not line:
                continue
            lhs, rhs = line.split("->")
            what, P, D, s, idx = (int(x) for x in lhs.split())
            off, nib = (int(x) for x in rhs.split())
            assert o.format_offset(what, P, D, s, idx) == (off, nib), line
            n += 1
    assert n >= 15


@pytest.mark.parametrize("vbits", [4, 8])
def test_append_round_trip_and_touches_only_its_slot(vbits):
    """read_slot returns numpy-quantized codes; bytes of other slots are left as they were."""
    o = oracle.default()
    rng = np.random.default_rng(3)
    for P, D, Hkv in ((16, 64, 1), (64, 256, 2), (32, 128, 3)):
        pages = 5
        pool = rng.integers(0, 256, o.pool_bytes(pages, P, Hkv, D, vbits), dtype=np.uint8)
        before = pool.copy()
        slots = np.array([0, P - 1, 2 * P + 5, 4 * P + 17 % P], np.int32)
        k = rng.standard_normal((len(slots), Hkv, D)).astype(np.float32)
        v = rng.standard_normal((len(slots), Hkv, D)).astype(np.float32)
        o.append(pool, pages, P, Hkv, D, k, v, slots, vbits=vbits)
        touched = np.zeros(pool.size, bool)
        bb = o.block_bytes(P, D, vbits)
        for n, slot in enumerate(slots):
            page, s = divmod(int(slot), P)
            for h in range(Hkv):
                kc, ks, vc, vs = o.read_slot(pool, P, Hkv, D, page, s, h, vbits)
                kc_r, ks_r, vc_r, vs_r = brute.quantize_token_np(k[n, h], v[n, h],
                                                                 127 if vbits == 8 else 7)
                assert np.array_equal(kc, kc_r) and ks == ks_r
                assert np.array_equal(vc, vc_r) and list(vs) == list(vs_r)
                base = (page * Hkv + h) * bb
                for what, count in ((0, D), (1, 1), (2, D), (3, D // 32)):
                    for idx in range(count):
                        off, _ = o.format_offset(what, P, D, s, idx, vbits)
                        touched[base + off] = True
                        if what in (1, 3):
                            touched[base + off + 1] = True
        assert np.array_equal(pool[~touched], before[~touched])


def test_append_skips_out_of_range_slots():
    o = oracle.default()
    P, D, pages = 16, 64, 3
    pool = np.zeros(o.pool_bytes(pages, P, 1, D), np.uint8)
    k = np.ones((3, 1, D), np.float32)
    o.append(pool, pages, P, 1, D, k, k, np.array([-1, pages * P, pages * P + 100], np.int32))
    assert not pool.any()


# ------------------------------------------------------------------ attention ------------

def _fill(o, inp):
    wl = inp.wl
    pool = o.new_pool(wl.pool_pages, wl.page_size, wl.num_kv_heads, wl.head_dim)
    k, v, slots = inp.all_tokens()
    o.append(pool, wl.pool_pages, wl.page_size, wl.num_kv_heads, wl.head_dim, k, v, slots)
    return pool


def _attend(o, inp, pool, scale=0.0, select=None):
    wl = inp.wl
    return o.decode_attn(pool, wl.pool_pages, wl.page_size, wl.num_kv_heads, wl.head_dim,
                         inp.q_bits, inp.page_table, inp.seq_lens, wl.n_rows, wl.n_q_heads,
                         softmax_scale=scale, select=select)


def _brute(inp):
    wl = inp.wl
    n, L, H, D = wl.n_seq, wl.seq_len, wl.num_kv_heads, wl.head_dim
    kc = np.zeros((n, L, H, D), np.int8)
    vc = np.zeros((n, L, H, D), np.int8)
    ks = np.zeros((n, L, H), np.uint16)
    vs = np.zeros((n, L, H, D // 32), np.uint16)
    for b in range(n):
        for t in range(int(inp.seq_lens[b])):
            for h in range(H):
                kc[b, t, h], ks[b, t, h], vc[b, t, h], vs[b, t, h] = brute.quantize_token_np(
                    inp.k[b, t, h], inp.v[b, t, h])
    return brute.attention_brute(inp.q_bits, kc, ks, vc, vs, inp.seq_lens, wl.n_rows,
                                 wl.n_q_heads, H, 1.0 / math.sqrt(D))


@pytest.mark.parametrize("case", [
    dict(n_seq=1, seq_lens=(37,), num_kv_heads=1, n_q_heads=4, head_dim=64, page_size=16,
         n_rows=1),
    dict(n_seq=2, seq_lens=(45, 20), num_kv_heads=2, n_q_heads=6, head_dim=64, page_size=16,
         n_rows=4),
    dict(n_seq=1, seq_lens=(33,), num_kv_heads=1, n_q_heads=2, head_dim=128, page_size=32,
         n_rows=2, k_outliers=True),
])
def test_oracle_matches_pure_python_brute_force(case):
    """Tiny ragged cases with random page order, GQA and the MTP causal mask."""
    inp = W.custom(**case, seed=sum(case["seq_lens"]))
    o = oracle.default()
    pool = _fill(o, inp)
    out, lse = _attend(o, inp, pool)
    out_b, lse_b = _brute(inp)
    np.testing.assert_allclose(out, out_b, rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse, lse_b, rtol=0, atol=1e-11)


def _one_token_values(o, pool, wl, b, t, h, inp):
    page = int(inp.page_table[b, t // wl.page_size])
    kc, ks, vc, vs = o.read_slot(pool, wl.page_size, wl.num_kv_heads, wl.head_dim, page,
                                 t % wl.page_size, h)
    k_hat = kc.astype(float) * brute.fp16_value_np(ks)
    v_hat = vc.astype(float) * np.repeat([brute.fp16_value_np(x) for x in vs], 32)
    return k_hat, v_hat


def test_closed_form_constant_v_returns_v():
    inp = W.custom(n_seq=1, seq_lens=(50,), num_kv_heads=2, n_q_heads=4, head_dim=64,
                   page_size=16, n_rows=1, seed=21)
    inp.v[:] = inp.v[:, :1]  # every token carries token 0's V row
    o = oracle.default()
    pool = _fill(o, inp)
    out, _ = _attend(o, inp, pool)
    for hq in range(4):
        _, v_hat = _one_token_values(o, pool, inp.wl, 0, 0, hq // 2, inp)
        np.testing.assert_allclose(out[0, 0, hq], v_hat, rtol=0, atol=1e-13)


def test_closed_form_single_token():
    inp = W.custom(n_seq=1, seq_lens=(1,), num_kv_heads=1, n_q_heads=3, head_dim=64,
                   page_size=16, n_rows=1, seed=22)
    o = oracle.default()
    pool = _fill(o, inp)
    out, lse = _attend(o, inp, pool)
    k_hat, v_hat = _one_token_values(o, pool, inp.wl, 0, 0, 0, inp)
    for hq in range(3):
        q = inp.q_bits[0, 0, hq].view(np.float16).astype(float)
        np.testing.assert_array_equal(out[0, 0, hq], v_hat)
        assert lse[0, 0, hq] == pytest.approx(q @ k_hat / 8.0, abs=1e-12)


def test_closed_form_zero_query_is_uniform_mean():
    inp = W.custom(n_seq=1, seq_lens=(40,), num_kv_heads=1, n_q_heads=2, head_dim=64,
                   page_size=16, n_rows=1, seed=23)
    inp.q_bits[:] = 0
    o = oracle.default()
    pool = _fill(o, inp)
    out, lse = _attend(o, inp, pool)
    mean = np.mean([_one_token_values(o, pool, inp.wl, 0, t, 0, inp)[1] for t in range(40)], 0)
    np.testing.assert_allclose(out[0, 0, 0], mean, rtol=0, atol=1e-13)
    assert lse[0, 0, 0] == pytest.approx(math.log(40), abs=1e-13)


def test_closed_form_two_tokens_is_a_sigmoid_blend():
    inp = W.custom(n_seq=1, seq_lens=(2,), num_kv_heads=1, n_q_heads=1, head_dim=64,
                   page_size=16, n_rows=1, seed=24)
    o = oracle.default()
    scale = 0.37
    pool = _fill(o, inp)
    out, lse = _attend(o, inp, pool, scale=scale)
    k0, v0 = _one_token_values(o, pool, inp.wl, 0, 0, 0, inp)
    k1, v1 = _one_token_values(o, pool, inp.wl, 0, 1, 0, inp)
    q = inp.q_bits[0, 0, 0].view(np.float16).astype(float)
    z0, z1 = scale * (q @ k0), scale * (q @ k1)
    sig = 1.0 / (1.0 + math.exp(z1 - z0))
    np.testing.assert_allclose(out[0, 0, 0], sig * v0 + (1 - sig) * v1, rtol=0, atol=1e-13)
    assert lse[0, 0, 0] == pytest.approx(max(z0, z1) + math.log1p(math.exp(-abs(z0 - z1))),
                                         abs=1e-12)


def test_closed_form_needle_dominates():
    """A key aligned with the query and scaled up takes (almost) all the weight."""
    inp = W.custom(n_seq=1, seq_lens=(64,), num_kv_heads=1, n_q_heads=1, head_dim=64,
                   page_size=16, n_rows=1, seed=25)
    q = inp.q_bits[0, 0, 0].view(np.float16).astype(np.float32)
    inp.k[0, 29, 0] = q * np.float32(4.0)
    o = oracle.default()
    pool = _fill(o, inp)
    out, _ = _attend(o, inp, pool)
    _, v_needle = _one_token_values(o, pool, inp.wl, 0, 29, 0, inp)
    w, n = o.attn_weights(pool, inp.wl.pool_pages, 16, 1, 64, inp.q_bits, inp.page_table,
                          inp.seq_lens, 1, 1, 0, 0, 0)
    assert n == 64 and w[29] > 0.999999
    np.testing.assert_allclose(out[0, 0, 0], v_needle, rtol=0, atol=1e-5)


def test_weights_sum_to_one_and_respect_the_causal_mask():
    inp = W.custom(n_seq=1, seq_lens=(70,), num_kv_heads=2, n_q_heads=4, head_dim=64,
                   page_size=16, n_rows=4, seed=26)
    o = oracle.default()
    pool = _fill(o, inp)
    for i in range(4):
        w, n = o.attn_weights(pool, inp.wl.pool_pages, 16, 2, 64, inp.q_bits, inp.page_table,
                              inp.seq_lens, 4, 4, 0, i, 3)
        assert n == 70 - 4 + i + 1
        assert abs(w.sum() - 1.0) < 1e-12
        assert np.all(w[n:] == 0) and np.all(w[:n] > 0)


def test_page_order_does_not_change_the_result():
    """Moving pages around the pool (and the page table with them) is bit-identical."""
    inp = W.custom(n_seq=2, seq_lens=(90, 61), num_kv_heads=2, n_q_heads=4, head_dim=64,
                   page_size=16, n_rows=2, extra_pages=5, seed=27)
    o = oracle.default()
    out_a, lse_a = _attend(o, inp, _fill(o, inp))
    perm = np.random.default_rng(1).permutation(inp.wl.pool_pages).astype(np.int32)
    inp.page_table = perm[inp.page_table]
    out_b, lse_b = _attend(o, inp, _fill(o, inp))
    assert np.array_equal(out_a, out_b) and np.array_equal(lse_a, lse_b)


def test_gqa_equals_mha_with_repeated_kv_heads():
    g = W.custom(n_seq=1, seq_lens=(48,), num_kv_heads=2, n_q_heads=6, head_dim=64,
                 page_size=16, n_rows=1, seed=28)
    m = W.custom(n_seq=1, seq_lens=(48,), num_kv_heads=6, n_q_heads=6, head_dim=64,
                 page_size=16, n_rows=1, seed=28)
    m.k[:] = np.repeat(g.k, 3, axis=2)
    m.v[:] = np.repeat(g.v, 3, axis=2)
    m.q_bits[:] = g.q_bits
    m.page_table = g.page_table
    o = oracle.default()
    out_g, lse_g = _attend(o, g, _fill(o, g))
    out_m, lse_m = _attend(o, m, _fill(o, m))
    assert np.array_equal(out_g, out_m) and np.array_equal(lse_g, lse_m)


@pytest.mark.parametrize("R,L", [(4, 75), (40, 100)], ids=["mtp4", "chunk40"])
def test_mtp_row_equals_single_row_decode_at_shorter_length(R, L):
    """Row i of n_rows = R sees exactly what a one-row decode of length L - R + 1 + i sees: the
    MTP verify step (R = 4) and a prefill chunk (R = 40, the chunk's positions)."""
    mtp = W.custom(n_seq=1, seq_lens=(L,), num_kv_heads=1, n_q_heads=2, head_dim=64,
                   page_size=16, n_rows=R, seed=29)
    o = oracle.default()
    pool = _fill(o, mtp)
    out, lse = _attend(o, mtp, pool)
    for i in range(R):
        one = W.custom(n_seq=1, seq_lens=(L,), num_kv_heads=1, n_q_heads=2, head_dim=64,
                       page_size=16, n_rows=1, seed=29)
        one.q_bits = np.ascontiguousarray(mtp.q_bits[:, i:i + 1])
        one.seq_lens = np.array([L - R + 1 + i], np.int32)
        one.page_table = mtp.page_table
        o1, l1 = _attend(o, one, pool)
        assert np.array_equal(o1[0, 0], out[0, i]) and np.array_equal(l1[0, 0], lse[0, i])


def test_batch_equals_each_sequence_alone_and_select_matches_full():
    inp = W.custom(n_seq=2, seq_lens=(55, 30), num_kv_heads=1, n_q_heads=2, head_dim=64,
                   page_size=16, n_rows=1, seed=30)
    o = oracle.default()
    pool = _fill(o, inp)
    out, lse = _attend(o, inp, pool)
    for b in range(2):
        sel = [(b, 0, hq) for hq in range(2)]
        o_s, l_s = _attend(o, inp, pool, select=sel)
        assert np.array_equal(o_s, out[b, 0]) and np.array_equal(l_s, lse[b, 0])


def test_rows_that_see_no_token_give_zero_and_minus_inf():
    inp = W.custom(n_seq=1, seq_lens=(2,), num_kv_heads=1, n_q_heads=1, head_dim=64,
                   page_size=16, n_rows=4, seed=31)
    o = oracle.default()
    out, lse = _attend(o, inp, _fill(o, inp))
    assert np.all(out[0, :2] == 0) and np.all(np.isneginf(lse[0, :2]))
    assert np.all(np.isfinite(lse[0, 2:]))


def test_out_of_range_page_ids_read_the_clamped_page():
    """Page-table entries below 0 read page 0 and entries at or past num_pages read the last
    page (the library header's out-of-range contract), against a pure-Python brute force that
    resolves each clamped page to the tokens the valid table stored there (or to unwritten,
    all-zero slots)."""
    o = oracle.default()
    assert pin_battery.check_page_clamp(o)
    # and the clamp is all there is to it: the same table with the entries clamped by hand
    inp, bad = pin_battery.clamp_case()
    wl = inp.wl
    pool = _fill(o, inp)
    fixed = np.clip(bad, 0, wl.pool_pages - 1).astype(np.int32)
    a = o.decode_attn(pool, wl.pool_pages, wl.page_size, wl.num_kv_heads, wl.head_dim,
                      inp.q_bits, bad, inp.seq_lens, wl.n_rows, wl.n_q_heads)
    b = o.decode_attn(pool, wl.pool_pages, wl.page_size, wl.num_kv_heads, wl.head_dim,
                      inp.q_bits, fixed, inp.seq_lens, wl.n_rows, wl.n_q_heads)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])

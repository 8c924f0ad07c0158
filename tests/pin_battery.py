"""A compact battery of the oracle pins, runnable against any compiled oracle variant.

``run(o)`` returns the names of the checks that fail for oracle ``o``.  The real oracle must
fail none; each mutant in ``test_oracle_mutations.py`` must fail at least one.  The references
(numpy float16, argmin codes, hand-worked fixtures, pure-Python brute force, closed forms) never
come from the oracle under test.
"""
from __future__ import annotations

import functools
import math
import os

import numpy as np

from long_context_decode_flash_amd import workloads as W
from tests import brute

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")

BRUTE_CASES = [
    dict(n_seq=1, seq_lens=(37,), num_kv_heads=1, n_q_heads=4, head_dim=64, page_size=16,
         n_rows=1),
    dict(n_seq=2, seq_lens=(45, 20), num_kv_heads=2, n_q_heads=6, head_dim=64, page_size=16,
         n_rows=4),
    dict(n_seq=1, seq_lens=(33,), num_kv_heads=1, n_q_heads=2, head_dim=128, page_size=32,
         n_rows=2, k_outliers=True),
]


def _case(i):
    c = BRUTE_CASES[i]
    return W.custom(**c, seed=sum(c["seq_lens"]))


@functools.lru_cache(maxsize=None)
def _brute_ref(i, vqmax=7, window=0):
    inp = _case(i)
    wl = inp.wl
    n, L, H, D = wl.n_seq, wl.seq_len, wl.num_kv_heads, wl.head_dim
    f8 = vqmax == "fp8"
    kc = np.zeros((n, L, H, D), np.uint8 if f8 else np.int8)
    vc = np.zeros((n, L, H, D), np.uint8 if f8 else np.int8)
    ks = np.zeros((n, L, H), np.uint16)
    vs = np.zeros((n, L, H, D // 32), np.uint16)
    for b in range(n):
        for t in range(int(inp.seq_lens[b])):
            for h in range(H):
                kc[b, t, h], ks[b, t, h], vc[b, t, h], vs[b, t, h] = brute.quantize_token_np(
                    inp.k[b, t, h], inp.v[b, t, h], vqmax)
    vals = brute.e4m3_values_torch() if f8 else None
    return brute.attention_brute(inp.q_bits, kc, ks, vc, vs, inp.seq_lens, wl.n_rows,
                                 wl.n_q_heads, H, 1.0 / math.sqrt(D), window,
                                 (lambda c: float(vals[int(c)])) if f8 else None)


def _golden_lines(name):
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.split("#")[0].strip()
            if line:
                yield line


def check_fp16(o):
    for bits in range(0, 1 << 16, 7):
        ref = float(np.uint16(bits).view(np.float16))
        got = o.fp16_to_double(bits)
        if not (math.isnan(ref) and math.isnan(got)) and got != ref:
            return False
    rng = np.random.default_rng(4)
    xs = (rng.standard_normal(500) * 10.0 ** rng.integers(-9, 6, 500)).astype(np.float32)
    ties = [np.float32((float(np.uint16(b).view(np.float16)) +
                        float(np.uint16(b + 1).view(np.float16))) / 2)
            for b in list(range(1, 0x400, 61)) + list(range(0x400, 0x7BFF, 1499))]
    with np.errstate(over="ignore"):
        return all(o.fp16_from_double(float(x)) == brute.fp16_bits_np(x)
                   for x in list(xs) + ties)


def check_quantizer_golden(o):
    for line in _golden_lines("quantizer_cases.txt"):
        qmax, vals, sb, codes = [p.strip() for p in line.split(";")]
        vals = [float(v) for v in vals.split()]
        codes = [int(c) for c in codes.split()]
        x = np.zeros(32, np.float32)
        x[:len(vals)] = vals
        c, s = o.quantize_group(x, int(qmax))
        if s != int(sb, 16) or list(c[:len(codes)]) != codes:
            return False
    return True


def check_quantizer_argmin(o):
    rng = np.random.default_rng(9)
    for qmax, n in ((127, 64), (7, 32)):
        for _ in range(10):
            x = rng.standard_normal(n).astype(np.float32)
            c, sb = o.quantize_group(x, qmax)
            if sb != brute.fp16_bits_np(np.float32(np.max(np.abs(x))) / np.float32(qmax)):
                return False
            s = brute.fp16_value_np(sb)
            for xi, ci in zip(x, c):
                q = float(xi) / s
                if abs(q - math.floor(q) - 0.5) < 1e-6 * max(1.0, abs(q)):
                    continue
                if int(ci) != brute.argmin_code(float(xi), s, qmax):
                    return False
    return True


def _check_format_file(o, name, vbits):
    for line in _golden_lines(name):
        lhs, rhs = line.split("->")
        what, P, D, s, idx = (int(x) for x in lhs.split())
        if o.format_offset(what, P, D, s, idx, vbits=vbits) != tuple(int(x) for x in rhs.split()):
            return False
    return True


def check_format_golden(o):
    return _check_format_file(o, "format_offsets.txt", 4)


def check_format_golden_v8(o):
    return _check_format_file(o, "format_offsets_v8.txt", 8)


def _fill(o, inp, vbits=4, kv_format=None):
    wl = inp.wl
    pool = o.new_pool(wl.pool_pages, wl.page_size, wl.num_kv_heads, wl.head_dim, vbits)
    k, v, slots = inp.all_tokens()
    o.append(pool, wl.pool_pages, wl.page_size, wl.num_kv_heads, wl.head_dim, k, v, slots,
             vbits=vbits, kv_format=kv_format)
    return pool


def _attend(o, inp, pool, scale=0.0, vbits=4, kv_format=None):
    wl = inp.wl
    return o.decode_attn(pool, wl.pool_pages, wl.page_size, wl.num_kv_heads, wl.head_dim,
                         inp.q_bits, inp.page_table, inp.seq_lens, wl.n_rows, wl.n_q_heads,
                         softmax_scale=scale, vbits=vbits, kv_format=kv_format)


def _brute_force(o, vbits, cases, kv_format=None):
    for i in cases:
        inp = _case(i)
        out, lse = _attend(o, inp, _fill(o, inp, vbits, kv_format), vbits=vbits,
                           kv_format=kv_format)
        out_b, lse_b = _brute_ref(i, "fp8" if kv_format == 2 else 127 if vbits == 8 else 7)
        if not (np.allclose(out, out_b, rtol=0, atol=1e-12) and
                np.allclose(lse, lse_b, rtol=0, atol=1e-11)):
            return False
    return True


def check_brute_force(o):
    return _brute_force(o, 4, range(len(BRUTE_CASES)))


def check_brute_force_v8(o):
    """K8/V8: the same brute force with 8-bit V codes (qmax 127)."""
    return _brute_force(o, 8, range(2))


def check_brute_force_f8(o):
    """fp8: the same brute force with E4M3 codes (PyTorch's conversion) for K and V."""
    return _brute_force(o, 8, range(2), kv_format=2)


def check_e4m3(o):
    """The E4M3 value of every code, and the encoding of a sweep holding every tie between
    neighbouring values (subnormal, normal, the top of the range), signed zeros and the range
    ends: against PyTorch's float8_e4m3fn and an argmin over all codes."""
    vals = brute.e4m3_values_torch()
    for c in range(256):
        got = o.e4m3_to_double(c)
        if not (np.isnan(vals[c]) and np.isnan(got)) and not (got == vals[c] and
                                                              math.copysign(1, got) == math.copysign(1, vals[c])):
            return False
    finite = np.unique(vals[~np.isnan(vals)])
    mids = (finite[:-1] + finite[1:]) / 2
    ys = np.concatenate([finite, mids, np.nextafter(mids, 0), np.nextafter(mids, 1e9),
                         [0.0, -0.0, 448.0, -448.0, 2.0 ** -12, -2.0 ** -12]]).astype(np.float32)
    ys = ys[np.abs(ys) <= 448]
    ref = brute.e4m3_codes_torch(ys)
    got = np.array([o.e4m3_from_float(float(y)) for y in ys], np.uint8)
    if not np.array_equal(got, ref):
        return False
    rng = np.random.default_rng(31)
    for y in list(rng.choice(ys, 60, replace=False)) + [float(np.float32(-0.0))]:
        if o.e4m3_from_float(float(y)) != brute.e4m3_argmin(float(y)):
            return False
    # the group quantizer: numpy scale and PyTorch codes, zeros and a zero group included
    for seed in range(4):
        x = np.random.default_rng(40 + seed).standard_normal(32).astype(np.float32) * 3
        x[seed] = -0.0
        codes, sb = o.quantize_group_f8(x)
        rc, rsb = brute.quantize_group_f8_np(x)
        if sb != rsb or not np.array_equal(codes, rc):
            return False
    codes, sb = o.quantize_group_f8(np.zeros(32, np.float32))
    return sb == 0 and not codes.any()


def check_closed_forms(o):
    # zero query -> uniform mean, lse = ln L
    inp = W.custom(n_seq=1, seq_lens=(40,), num_kv_heads=1, n_q_heads=2, head_dim=64,
                   page_size=16, n_rows=1, seed=23)
    inp.q_bits[:] = 0
    out, lse = _attend(o, inp, _fill(o, inp))
    if not abs(lse[0, 0, 0] - math.log(40)) < 1e-12:
        return False
    kc_vs = [brute.quantize_token_np(inp.k[0, t, 0], inp.v[0, t, 0]) for t in range(40)]
    mean = np.mean([c[2].astype(float) * np.repeat([brute.fp16_value_np(x) for x in c[3]], 32)
                    for c in kc_vs], 0)
    if not np.allclose(out[0, 0, 0], mean, rtol=0, atol=1e-13):
        return False
    # weights sum to 1 under the causal mask
    inp = W.custom(n_seq=1, seq_lens=(70,), num_kv_heads=2, n_q_heads=4, head_dim=64,
                   page_size=16, n_rows=4, seed=26)
    pool = _fill(o, inp)
    for i in range(4):
        w, n = o.attn_weights(pool, inp.wl.pool_pages, 16, 2, 64, inp.q_bits, inp.page_table,
                              inp.seq_lens, 4, 4, 0, i, 3)
        if n != 67 + i or abs(w.sum() - 1.0) > 1e-12:
            return False
    return True


def check_large_logits(o):
    """Two tokens with logits in the thousands: the blend is the sigmoid closed form and the
    log-sum-exp is max + log1p(exp(-gap)); a softmax without its max shift overflows."""
    inp = W.custom(n_seq=1, seq_lens=(2,), num_kv_heads=1, n_q_heads=1, head_dim=64,
                   page_size=16, n_rows=1, seed=24)
    scale = 900.0
    out, lse = _attend(o, inp, _fill(o, inp), scale=scale)
    kv = [brute.quantize_token_np(inp.k[0, t, 0], inp.v[0, t, 0]) for t in range(2)]
    q = inp.q_bits[0, 0, 0].view(np.float16).astype(float)
    z = [scale * (q @ (c[0].astype(float) * brute.fp16_value_np(c[1]))) for c in kv]
    v = [c[2].astype(float) * np.repeat([brute.fp16_value_np(x) for x in c[3]], 32) for c in kv]
    gap = z[1] - z[0]
    sig = 1.0 / (1.0 + math.exp(gap)) if gap < 700 else 0.0
    if not np.allclose(out[0, 0, 0], sig * v[0] + (1 - sig) * v[1], rtol=0, atol=1e-12):
        return False
    return abs(lse[0, 0, 0] - (max(z) + math.log1p(math.exp(-abs(gap))))) < 1e-9 * abs(max(z))


def check_window_ring(o):
    """Sliding window over ring pages: the oracle, reading a ring table that holds only each
    sequence's last ring_pages pages, against the pure-Python brute force of windowed
    attention over the logical tokens (MTP rows, ragged lengths, GQA 3); and a one-token window,
    whose output is the row's own V and whose log-sum-exp is its own logit."""
    wl_i, window, ring = 1, 10, 2
    inp = _case(wl_i)
    wl = inp.wl
    table, (k, v, slots) = inp.ring(ring)
    pool = o.new_pool(wl.pool_pages, wl.page_size, wl.num_kv_heads, wl.head_dim)
    o.append(pool, wl.pool_pages, wl.page_size, wl.num_kv_heads, wl.head_dim, k, v, slots)
    out, lse = o.decode_attn(pool, wl.pool_pages, wl.page_size, wl.num_kv_heads, wl.head_dim,
                             inp.q_bits, table, inp.seq_lens, wl.n_rows, wl.n_q_heads,
                             window=window, ring_pages=ring)
    out_b, lse_b = _brute_ref(wl_i, 7, window)
    if not (np.allclose(out, out_b, rtol=0, atol=1e-12) and
            np.allclose(lse, lse_b, rtol=0, atol=1e-11)):
        return False
    # window 1: row i of sequence b sees token L - R + i alone
    out, lse = o.decode_attn(pool, wl.pool_pages, wl.page_size, wl.num_kv_heads, wl.head_dim,
                             inp.q_bits, table, inp.seq_lens, wl.n_rows, wl.n_q_heads,
                             window=1, ring_pages=ring)
    G = wl.n_q_heads // wl.num_kv_heads
    scale = 1.0 / math.sqrt(wl.head_dim)
    for b in range(wl.n_seq):
        for i in range(wl.n_rows):
            t = int(inp.seq_lens[b]) - wl.n_rows + i
            for hq in range(wl.n_q_heads):
                kc, ks, vc, vs = brute.quantize_token_np(inp.k[b, t, hq // G], inp.v[b, t, hq // G])
                vd = vc.astype(float) * np.repeat([brute.fp16_value_np(x) for x in vs], 32)
                q = inp.q_bits[b, i, hq].view(np.float16).astype(float)
                z = scale * (q @ (kc.astype(float) * brute.fp16_value_np(ks)))
                if not (np.allclose(out[b, i, hq], vd, rtol=0, atol=1e-13) and
                        abs(lse[b, i, hq] - z) < 1e-12):
                    return False
    return True


def clamped_page_brute(inp, bad_table, vqmax=7):
    """Pure-Python attention of ``inp`` read through ``bad_table``, whose out-of-range entries
    name the nearest page in range (the library header's contract: an id below 0 reads page 0,
    one at or past num_pages reads the last page).  The pool was filled through the valid
    table, so each slot of a clamped page holds the token the valid table put there, or nothing
    (zero codes and scales) where no token was appended."""
    wl = inp.wl
    P, H, D = wl.page_size, wl.num_kv_heads, wl.head_dim
    owner = {}  # physical page -> (sequence, logical page) of the valid table
    for b in range(wl.n_seq):
        for n in range(-(-int(inp.seq_lens[b]) // P)):
            owner[int(inp.page_table[b, n])] = (b, n)
    n, L = wl.n_seq, wl.seq_len
    kc = np.zeros((n, L, H, D), np.int8)
    vc = np.zeros((n, L, H, D), np.int8)
    ks = np.zeros((n, L, H), np.uint16)
    vs = np.zeros((n, L, H, D // 32), np.uint16)
    for b in range(n):
        for t in range(int(inp.seq_lens[b])):
            phys = min(max(int(bad_table[b, t // P]), 0), wl.pool_pages - 1)
            if phys not in owner:
                continue
            b2, n2 = owner[phys]
            t2 = n2 * P + t % P
            if t2 >= int(inp.seq_lens[b2]):
                continue
            for h in range(H):
                kc[b, t, h], ks[b, t, h], vc[b, t, h], vs[b, t, h] = brute.quantize_token_np(
                    inp.k[b2, t2, h], inp.v[b2, t2, h], vqmax)
    return brute.attention_brute(inp.q_bits, kc, ks, vc, vs, inp.seq_lens, wl.n_rows,
                                 wl.n_q_heads, H, 1.0 / math.sqrt(D))


def clamp_case():
    """Two sequences whose valid table leaves page 0 and the last page holding different
    tokens, and a table with entries -1, -7, num_pages + 5 and 2^31 - 1 in place of valid ones."""
    inp = W.custom(n_seq=2, seq_lens=(45, 29), num_kv_heads=2, n_q_heads=6, head_dim=64,
                   page_size=16, n_rows=2, extra_pages=3, seed=4242)
    wl = inp.wl
    used = {int(inp.page_table[b, n]) for b in range(wl.n_seq)
            for n in range(-(-int(inp.seq_lens[b]) // wl.page_size))}
    assert 0 in used and wl.pool_pages - 1 in used, "case must put tokens in both end pages"
    bad = inp.page_table.copy()
    bad[0, 1] = -1
    bad[0, 2] = wl.pool_pages + 5
    bad[1, 0] = 2 ** 31 - 1
    bad[1, 1] = -7
    return inp, bad


def check_page_clamp(o):
    """Out-of-range page-table entries read the clamped page, against the brute force."""
    inp, bad = clamp_case()
    wl = inp.wl
    pool = _fill(o, inp)
    out, lse = o.decode_attn(pool, wl.pool_pages, wl.page_size, wl.num_kv_heads, wl.head_dim,
                             inp.q_bits, bad, inp.seq_lens, wl.n_rows, wl.n_q_heads)
    out_b, lse_b = clamped_page_brute(inp, bad)
    return (np.allclose(out, out_b, rtol=0, atol=1e-12) and
            np.allclose(lse, lse_b, rtol=0, atol=1e-11))


CHECKS = [check_page_clamp, check_window_ring, check_fp16, check_quantizer_golden, check_quantizer_argmin, check_format_golden,
          check_brute_force, check_closed_forms, check_large_logits, check_format_golden_v8,
          check_brute_force_v8, check_e4m3, check_brute_force_f8]


def run(o):
    failed = []
    for chk in CHECKS:
        try:
            ok = chk(o)
        except Exception:  # a crash inside a check counts as a caught mistake
            ok = False
        if not ok:
            failed.append(chk.__name__)
    return failed

"""Tiny-input brute force for pinning the CPU oracle.

Independent of ``oracle/kvq_oracle.c``: the quantizer here uses numpy's float32 arithmetic and
numpy's float16 conversion, the quantizer pins use an argmin over every code, and the attention
is a pure-Python loop in fp64 over codes held in plain arrays (never through the page format).
Only for small inputs (L <= a few hundred, D <= 256).
"""
from __future__ import annotations

import math

import numpy as np


def fp16_bits_np(x) -> int:
    """numpy's float32 -> float16 conversion (round to nearest even), as bits."""
    return int(np.float32(x).astype(np.float16).view(np.uint16))


def fp16_value_np(bits: int) -> float:
    return float(np.uint16(bits).view(np.float16))


def quantize_group_np(x, qmax: int):
    """Quantize one group with numpy float32 arithmetic: (codes int8, scale bits)."""
    x = np.asarray(x, np.float32)
    a = np.max(np.abs(x)) if x.size else np.float32(0)
    with np.errstate(over="ignore"):
        s16 = (np.float32(a) / np.float32(qmax)).astype(np.float16)
    if np.isinf(s16):
        s16 = np.float16(65504.0)
    s = np.float32(s16)
    if s == 0:
        return np.zeros(x.size, np.int8), int(s16.view(np.uint16))
    c = np.clip(np.rint(x / s), -qmax, qmax).astype(np.int8)
    return c, int(s16.view(np.uint16))


def e4m3_values_torch():
    """Value of each of the 256 OCP E4M3 codes, from PyTorch's float8_e4m3fn dtype."""
    import torch
    return torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).to(
        torch.float64).numpy()


def e4m3_codes_torch(y):
    """PyTorch's float32 -> float8_e4m3fn conversion (round to nearest even), as codes."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(y, np.float32))
    return t.to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def e4m3_argmin(y: float) -> int:
    """The finite E4M3 code nearest to y in exact arithmetic, ties to the even code, with the
    sign of y on zero."""
    vals = e4m3_values_torch()
    best, best_err = None, None
    for c in range(256):
        if np.isnan(vals[c]) or (vals[c] == 0 and (c >> 7) != int(np.signbit(y))):
            continue
        err = abs(float(y) - vals[c])
        if best is None or err < best_err or (err == best_err and c % 2 == 0):
            best, best_err = c, err
    return best


def quantize_group_f8_np(x):
    """fp8 group: scale as for the integer codes with qmax 448 (numpy float32 / float16), codes
    torch's E4M3 conversion of the fp32 quotients clamped to +-448."""
    x = np.asarray(x, np.float32)
    a = np.max(np.abs(x)) if x.size else np.float32(0)
    with np.errstate(over="ignore"):
        s16 = (np.float32(a) / np.float32(448)).astype(np.float16)
    if np.isinf(s16):
        s16 = np.float16(65504.0)
    s = np.float32(s16)
    if s == 0:
        return np.zeros(x.size, np.uint8), int(s16.view(np.uint16))
    y = np.clip((x / s).astype(np.float32), np.float32(-448), np.float32(448))
    return e4m3_codes_torch(y), int(s16.view(np.uint16))


def argmin_code(x: float, s: float, qmax: int) -> int:
    """The code c in [-qmax, qmax] minimizing |x - c*s| in exact arithmetic, ties to even.
    x, s are fp32 values; c*s and the differences are exact in fp64."""
    best, best_err = None, None
    for c in range(-qmax, qmax + 1):
        err = abs(float(x) - c * float(s))
        if best is None or err < best_err or (err == best_err and c % 2 == 0):
            best, best_err = c, err
    return best


def quantize_token_np(krow, vrow, vqmax=7):
    """K row -> (codes, scale bits); V row -> (codes, [scale bits per 32 dims]).  vqmax 7: 4-bit
    V codes (K8/V4), 127: 8-bit (K8/V8), "fp8": E4M3 codes (uint8) for K and V."""
    f8 = vqmax == "fp8"
    kc, ks = quantize_group_f8_np(krow) if f8 else quantize_group_np(krow, 127)
    D = len(vrow)
    vc = np.zeros(D, np.uint8 if f8 else np.int8)
    vs = []
    for j in range(D // 32):
        g = vrow[32 * j:32 * j + 32]
        c, sb = quantize_group_f8_np(g) if f8 else quantize_group_np(g, vqmax)
        vc[32 * j:32 * j + 32] = c
        vs.append(sb)
    return kc, ks, vc, vs


def attention_brute(q_bits, kc, ks, vc, vs, seq_lens, n_rows, n_q_heads, num_kv_heads, scale,
                    window=0, code_value=None):
    """Pure-Python fp64 attention (``window`` > 0: each row sees only its last ``window``
    tokens, its own position included; ``code_value`` maps a stored code to its value, the
    integer itself by default).

    q_bits: [n_seq][n_rows][Hq][D] fp16 bits; kc/vc: [n_seq][L][Hkv][D] codes;
    ks: [n_seq][L][Hkv] scale bits; vs: [n_seq][L][Hkv][D/32] scale bits.
    Returns out [n_seq][n_rows][Hq][D] and lse [n_seq][n_rows][Hq] as nested lists.
    """
    cv = code_value or int
    n_seq = len(seq_lens)
    D = len(q_bits[0][0][0])
    G = n_q_heads // num_kv_heads
    out, lse = [], []
    for b in range(n_seq):
        L = int(seq_lens[b])
        ob, lb = [], []
        for i in range(n_rows):
            oi, li = [], []
            for hq in range(n_q_heads):
                h = hq // G
                q = [fp16_value_np(int(x)) for x in q_bits[b][i][hq]]
                last = L - n_rows + i
                first = max(0, last - window + 1) if window > 0 else 0
                z = []
                for t in range(first, last + 1):
                    sk = fp16_value_np(int(ks[b][t][h]))
                    dot = 0.0
                    for d in range(D):
                        dot += q[d] * (cv(kc[b][t][h][d]) * sk)
                    z.append(scale * dot)
                if not z:
                    oi.append([0.0] * D)
                    li.append(-math.inf)
                    continue
                m = max(z)
                e = [math.exp(x - m) for x in z]
                tot = sum(e)
                o = [0.0] * D
                for t, et in zip(range(first, last + 1), e):
                    w = et / tot
                    for d in range(D):
                        sv = fp16_value_np(int(vs[b][t][h][d // 32]))
                        o[d] += w * (cv(vc[b][t][h][d]) * sv)
                oi.append(o)
                li.append(m + math.log(tot))
            ob.append(oi)
            lb.append(li)
        out.append(ob)
        lse.append(lb)
    return np.array(out), np.array(lse)

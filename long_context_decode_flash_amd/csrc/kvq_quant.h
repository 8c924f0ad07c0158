// kvq_quant.h — the K8/V4 (and K8/V8, fp8) quantizer of one (token, KV head) row, written into its
// cache slot by one 64-lane wave.  Shared by the append kernel and the decode kernel's fused
// append, so both write the same bytes.
//
// K8/V4 ("rk8v4" in the launch-flag table of the forum post "3090 单卡跑 Qwen3.8-27B：NInfer
// 上机实测（180K 上下文 / C2 并发 / 4bit KV）", 一、部署): K as int8 with one fp16 scale per token
// and KV head, V as 4-bit codes with one fp16 scale per 32 dims, the granularity and rounding
// the library header defines.  Each lane holds D/64 consecutive dims, the absmax reductions are
// wave shuffles, and every byte written belongs to this token alone.
#pragma once

#include "kvq_internal.h"

namespace kvq {

// Lanes of one wave hand data to each other through LDS (one lane writes bytes another lane
// reads): this ordering point keeps the compiler from moving the reads above the writes.  It
// emits no instruction; a wave's LDS operations complete in program order.
__device__ inline void wave_lds_order() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// max over each aligned group of W lanes (W a power of two <= 64) of a non-negative float
// given by its bits (for those, unsigned order of the bits is value order), with DPP moves
// inside rows of 16 lanes and the gfx950 row / half swaps across them: VALU only, no LDS round
// trips.  After the quad steps a lane holds its quad's max; the half-row mirror pairs the two
// quads of an 8-lane group, the row mirror the two halves of a row.
template <int W>
__device__ inline uint32_t group_max_bits(uint32_t u) {
  static_assert(W >= 1 && W <= 64 && (W & (W - 1)) == 0, "group width");
  auto mx = [](uint32_t a, int b) { return a > (uint32_t)b ? a : (uint32_t)b; };
  if constexpr (W >= 2) u = mx(u, __builtin_amdgcn_mov_dpp((int)u, 0xB1, 0xF, 0xF, true));   // quad_perm [1,0,3,2]
  if constexpr (W >= 4) u = mx(u, __builtin_amdgcn_mov_dpp((int)u, 0x4E, 0xF, 0xF, true));   // quad_perm [2,3,0,1]
  if constexpr (W >= 8) u = mx(u, __builtin_amdgcn_mov_dpp((int)u, 0x141, 0xF, 0xF, true));  // row_half_mirror
  if constexpr (W >= 16) u = mx(u, __builtin_amdgcn_mov_dpp((int)u, 0x140, 0xF, 0xF, true)); // row_mirror
  if constexpr (W >= 32) {  // rows (0, 1) and (2, 3) meet
    const auto a = __builtin_amdgcn_permlane16_swap(u, u, false, false);
    u = mx(a[0], (int)a[1]);
  }
  if constexpr (W >= 64) {  // the two halves meet
    const auto a = __builtin_amdgcn_permlane32_swap(u, u, false, false);
    u = mx(a[0], (int)a[1]);
  }
  return u;
}

// absolute-value bits of a float (non-finite inputs are undefined)
__device__ inline uint32_t abs_bits(float x) { return __builtin_bit_cast(uint32_t, x) & 0x7FFFFFFFu; }

// The IEEE fp32 quotient x / d (round to nearest even) from r = recip_for(d), so that every
// element of a group shares one reciprocal.  These are the steps of the correctly rounded
// divide this library is built with (reciprocal, one refinement, then two fused remainder
// corrections of the quotient) without its range scaling, which only acts when x or x / d is
// near the subnormal range or their exponents lie about 96 or more apart.  Every quotient the
// quantizer takes is outside those cases for finite inputs except two whose result does not
// depend on the last bit: a subnormal x (code 0) and a saturated scale (|x / d| far above the
// largest code, clamped).  Unlike the full divide it returns +0 for x = -0 (the corrections add
// +0); a caller that needs the sign of a zero quotient restores it.  Non-finite inputs are
// undefined.
__device__ inline float recip_for(float d) {
  const float r = __builtin_amdgcn_rcpf(d);
  return __builtin_fmaf(__builtin_fmaf(-d, r, 1.0f), r, r);
}
__device__ inline float div_rn(float x, float d, float r) {
  float y = x * r;
  y = __builtin_fmaf(__builtin_fmaf(-d, y, x), r, y);
  return __builtin_fmaf(__builtin_fmaf(-d, y, x), r, y);
}

// fp16 scale of one group: round-to-nearest-even of the fp32 quotient, saturated to the largest
// finite fp16.  Returns the fp16 bits; *s receives its value in fp32.
__device__ inline uint16_t group_scale(float absmax, float qmax, float* s) {
  float s32 = div_rn(absmax, qmax, recip_for(qmax));  // the IEEE fp32 quotient
  _Float16 h = (_Float16)s32;  // v_cvt_f16_f32: round to nearest even
  uint16_t bits = __builtin_bit_cast(uint16_t, h);
  if ((bits & 0x7FFF) == 0x7C00) bits = 0x7BFF;
  *s = (float)__builtin_bit_cast(_Float16, bits);
  return bits;
}

// code of x at scale s (r = recip_for(s)); a zero scale gives code 0 (the quotient is then
// computed and dropped: a select, not a branch per element)
__device__ inline int quantize_one(float x, float s, float r, float qmax) {
  const float c = __builtin_rintf(div_rn(x, s, r));  // IEEE quotient, round half to even
  const int code = (int)__builtin_amdgcn_fmed3f(c, -qmax, qmax);
  return s == 0.0f ? 0 : code;
}

// OCP FP8 E4M3 code of y, |y| <= 448, rounded to the nearest E4M3 value with ties to the even
// mantissa.  Below 2^-6 the values are the multiples of 2^-9 (code = y * 2^9, exact scaling,
// then rint); from 2^-6 on the code is the fp32 exponent and top three mantissa bits, rounded to
// nearest even on the 20 dropped bits (a carry moves into the exponent), rebased from bias 127 to
// bias 7.  The sign bit is y's.
__device__ inline uint32_t e4m3_rne(float y) {
  const uint32_t u = __builtin_bit_cast(uint32_t, y);
  const uint32_t sign = (u >> 24) & 0x80u;
  const uint32_t a = u & 0x7FFFFFFFu;
  uint32_t mag;
  if (a < 0x3C800000u)  // |y| < 2^-6: subnormal codes 0..7, and 8 (= 2^-6) when rounding up
    mag = (uint32_t)__builtin_rintf(__builtin_bit_cast(float, a) * 512.0f);
  else
    mag = ((a + 0x7FFFFu + ((a >> 20) & 1u)) >> 20) - (120u << 3);
  return sign | mag;
}

__device__ inline uint32_t quantize_one_f8(float x, float s, float r) {
  // IEEE quotient; the corrections turn -0 / s into +0, so the sign (s > 0) is x's: -0 keeps
  // its own code (0x80), as in the IEEE divide
  const float y = __builtin_copysignf(div_rn(x, s, r), x);
  const uint32_t code = e4m3_rne(__builtin_amdgcn_fmed3f(y, -448.0f, 448.0f));
  return s == 0.0f ? 0u : code;
}

// A wave's share of one token's K and V rows: lane l holds dims E*l .. E*l + E-1.
template <int D>
struct RowVals {
  static constexpr int E = D / kWave;  // dims per lane: 1, 2 or 4
  float k[E], v[E];
};

// The lane's E values of a token's K and V rows, loaded non-temporally (each input row is read
// once).
template <int D>
__device__ __attribute__((always_inline)) inline RowVals<D> load_row(const float* krow_base, const float* vrow_base, int lane) {
  RowVals<D> r;
  const int d0 = lane * RowVals<D>::E;
#pragma unroll
  for (int e = 0; e < RowVals<D>::E; ++e) {
    r.k[e] = __builtin_nontemporal_load(krow_base + d0 + e);
    r.v[e] = __builtin_nontemporal_load(vrow_base + d0 + e);
  }
  return r;
}

// Quantize one token's K and V rows (already in the wave's registers) into slot s of the
// (page, KV head) block at blk, with VB-bit V codes; F8 (with VB = 8): K and V as E4M3 codes
// at 448 in place of qmax.  Called by all 64 lanes of a wave.
template <int D, int VB = 4, bool F8 = false>
__device__ __attribute__((always_inline)) inline void store_row(uint8_t* blk, int P, int s, const RowVals<D>& r, int lane) {
  static_assert(!F8 || VB == 8, "fp8 codes use the 8-bit layout");
  constexpr int E = RowVals<D>::E;
  const int tile = s / kTile, t = s % kTile;
  const int d0 = lane * E;
  const float* kx = r.k;
  const float* vx = r.v;

  // ---- K: one scale per token and head (qmax 127) ----
  uint32_t kab = 0;
#pragma unroll
  for (int e = 0; e < E; ++e) kab = max(kab, abs_bits(kx[e]));
  const float ka = __builtin_bit_cast(float, group_max_bits<kWave>(kab));
  float ks;
  const uint16_t ks_bits = group_scale(ka, F8 ? 448.0f : 127.0f, &ks);
  const float kr = recip_for(ks);
  uint32_t kpacked = 0;
#pragma unroll
  for (int e = 0; e < E; ++e)
    kpacked |= (F8 ? quantize_one_f8(kx[e], ks, kr) : (uint32_t)(quantize_one(kx[e], ks, kr, 127.0f) & 0xFF)) << (8 * e);
  // K code (t, d) at 16*D*tile + 256*(d/16) + 16*t + d%16; E consecutive dims stay in one chunk
  uint8_t* kdst = blk + (size_t)16 * D * tile + 256 * (d0 / 16) + 16 * t + d0 % 16;
  if constexpr (E == 4) {
    *(uint32_t*)kdst = kpacked;
  } else if constexpr (E == 2) {
    *(uint16_t*)kdst = (uint16_t)kpacked;
  } else {
    *kdst = (uint8_t)kpacked;
  }
  if (lane == 0) *(uint16_t*)(blk + k_scales_at(P, D) + 2 * s) = ks_bits;

  // ---- V: one scale per 32 dims (qmax 7, or 127 for 8-bit codes), 32/E lanes per group ----
  constexpr float vqmax = F8 ? 448.0f : VB == 8 ? 127.0f : 7.0f;
  uint32_t vab = 0;
#pragma unroll
  for (int e = 0; e < E; ++e) vab = max(vab, abs_bits(vx[e]));
  const float va = __builtin_bit_cast(float, group_max_bits<32 / E>(vab));
  float vsc;
  const uint16_t vs_bits = group_scale(va, vqmax, &vsc);
  const float vr = recip_for(vsc);
  const int j = d0 / 32;
  if (d0 % 32 == 0) *(uint16_t*)(blk + v_scales_at(P, D, VB) + 2 * ((size_t)s * (D / 32) + j)) = vs_bits;
  if constexpr (VB == 8) {
    // V8 code (t, d) at 16*D*tile + 512*w*(j/w) + 8*w*lane + 8*(j%w) + 4*((d/16)%2) + t%4 within
    // the V section, lane = 16*(t/4) + d%16, w = min(D/32, 2): one byte per code
    constexpr int w = (D / 32) < 2 ? (D / 32) : 2;
    uint8_t* vbase = blk + v_codes_at(P, D) + (size_t)16 * D * tile + 512 * w * (j / w) + 8 * (j % w) +
                     4 * ((d0 / 16) & 1) + t % 4;
#pragma unroll
    for (int e = 0; e < E; ++e) {
      const int vlane = 16 * (t / 4) + (d0 + e) % 16;
      vbase[8 * w * vlane] = F8 ? (uint8_t)quantize_one_f8(vx[e], vsc, vr) : (uint8_t)(quantize_one(vx[e], vsc, vr, vqmax) & 0xFF);
    }
    return;
  }
  uint32_t vnib = 0;  // E nibbles, dim d0+e at bits 4e
#pragma unroll
  for (int e = 0; e < E; ++e) vnib |= (uint32_t)(quantize_one(vx[e], vsc, vr, 7.0f) & 0xF) << (4 * e);

  // Dims d (d/16 even) and d+16 share a byte (low / high nibble).  The lane holding d gets the
  // partner's nibbles from 16/E lanes up and writes the E bytes.  With E = 4 or 2 the partner is
  // in the same row of 16 lanes (DPP row shift left: lane i reads lane i + 16/E); with E = 1 it
  // is in the next row.
  uint32_t partner;
  if constexpr (E == 4)
    partner = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)vnib, 0x104, 0xF, 0xF, false);  // row_shl:4
  else if constexpr (E == 2)
    partner = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)vnib, 0x108, 0xF, 0xF, false);  // row_shl:8
  else
    partner = __shfl_down(vnib, 16, kWave);
  if (((d0 / 16) & 1) == 0) {
    constexpr int w = (D / 32) < 4 ? (D / 32) : 4;
    const int r = t % 4;
    uint8_t* vbase = blk + v_codes_at(P, D) + (size_t)8 * D * tile + 256 * w * (j / w) + 4 * (j % w) + r;
#pragma unroll
    for (int e = 0; e < E; ++e) {
      const int d = d0 + e;
      const int vlane = 16 * (t / 4) + d % 16;
      const uint8_t byte = (uint8_t)(((vnib >> (4 * e)) & 0xF) | (((partner >> (4 * e)) & 0xF) << 4));
      vbase[4 * w * vlane] = byte;
    }
  }
}

// Load and quantize one token's rows (krow/vrow point at the rows' first values) into slot s.
template <int D, int VB = 4, bool F8 = false>
__device__ inline void append_row(uint8_t* blk, int P, int s, const float* krow_base,
                                  const float* vrow_base, int lane) {
  store_row<D, VB, F8>(blk, P, s, load_row<D>(krow_base, vrow_base, lane), lane);
}

}  // namespace kvq

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

__device__ inline float wave_max(float x, int width) {
  // butterfly over groups of `width` lanes (width a power of two <= 64)
  for (int off = width / 2; off > 0; off >>= 1) x = fmaxf(x, __shfl_xor(x, off, kWave));
  return x;
}

// fp16 scale of one group: round-to-nearest-even of the fp32 quotient, saturated to the largest
// finite fp16.  Returns the fp16 bits; *s receives its value in fp32.
__device__ inline uint16_t group_scale(float absmax, float qmax, float* s) {
  float s32 = absmax / qmax;  // IEEE fp32 division (built with correctly rounded divide)
  _Float16 h = (_Float16)s32;  // v_cvt_f16_f32: round to nearest even
  uint16_t bits = __builtin_bit_cast(uint16_t, h);
  if ((bits & 0x7FFF) == 0x7C00) bits = 0x7BFF;
  *s = (float)__builtin_bit_cast(_Float16, bits);
  return bits;
}

__device__ inline int quantize_one(float x, float s, float qmax) {
  if (s == 0.0f) return 0;
  float c = __builtin_rintf(x / s);  // IEEE divide, round half to even
  c = fminf(fmaxf(c, -qmax), qmax);
  return (int)c;
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

__device__ inline uint32_t quantize_one_f8(float x, float s) {
  if (s == 0.0f) return 0u;
  const float y = x / s;  // IEEE divide
  return e4m3_rne(fminf(fmaxf(y, -448.0f), 448.0f));
}

// A wave's share of one token's K and V rows: lane l holds dims E*l .. E*l + E-1.
template <int D>
struct RowVals {
  static constexpr int E = D / kWave;  // dims per lane: 1, 2 or 4
  float k[E], v[E];
};

template <int D>
__device__ __attribute__((always_inline)) inline RowVals<D> load_row(const float* krow_base, const float* vrow_base, int lane) {
  RowVals<D> r;
  const int d0 = lane * RowVals<D>::E;
#pragma unroll
  for (int e = 0; e < RowVals<D>::E; ++e) {
    r.k[e] = krow_base[d0 + e];
    r.v[e] = vrow_base[d0 + e];
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
  float ka = 0.0f;
#pragma unroll
  for (int e = 0; e < E; ++e) ka = fmaxf(ka, fabsf(kx[e]));
  ka = wave_max(ka, kWave);
  float ks;
  const uint16_t ks_bits = group_scale(ka, F8 ? 448.0f : 127.0f, &ks);
  uint32_t kpacked = 0;
#pragma unroll
  for (int e = 0; e < E; ++e)
    kpacked |= (F8 ? quantize_one_f8(kx[e], ks) : (uint32_t)(quantize_one(kx[e], ks, 127.0f) & 0xFF)) << (8 * e);
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
  float va = 0.0f;
#pragma unroll
  for (int e = 0; e < E; ++e) va = fmaxf(va, fabsf(vx[e]));
  va = wave_max(va, 32 / E);
  float vsc;
  const uint16_t vs_bits = group_scale(va, vqmax, &vsc);
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
      vbase[8 * w * vlane] = F8 ? (uint8_t)quantize_one_f8(vx[e], vsc) : (uint8_t)(quantize_one(vx[e], vsc, vqmax) & 0xFF);
    }
    return;
  }
  uint32_t vnib = 0;  // E nibbles, dim d0+e at bits 4e
#pragma unroll
  for (int e = 0; e < E; ++e) vnib |= (uint32_t)(quantize_one(vx[e], vsc, 7.0f) & 0xF) << (4 * e);

  // Dims d (d/16 even) and d+16 share a byte (low / high nibble).  The lane holding d gets the
  // partner's nibbles from 16/E lanes up and writes the E bytes.
  const uint32_t partner = __shfl_down(vnib, 16 / E, kWave);
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

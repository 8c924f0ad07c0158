// kvq_attn_block.h — the attention building blocks the decode and prefill kernels share:
// staging of 32-token blocks of the paged cache in LDS with direct-to-LDS loads, the
// matrix-core step of one block for up to 32 query rows (Q K^T, online softmax, P V), and the
// log-sum-exp merge of context pieces.  Every definition is in an unnamed namespace, so each
// kernel file gets its own copy.
#pragma once

#include "kvq_quant.h"

namespace kvq {
namespace {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef _Float16 half2v __attribute__((ext_vector_type(2)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef int i32x4 __attribute__((ext_vector_type(4)));

constexpr float kNegInf = -__builtin_inff();
constexpr int cmax(int x, int y) { return x > y ? x : y; }

__device__ inline half2v as_h2(uint32_t u) { return __builtin_bit_cast(half2v, u); }
__device__ inline uint32_t as_u32(half2v h) { return __builtin_bit_cast(uint32_t, h); }

// One V dword holds, for four tokens r = 0..3 (byte r), the codes of two dims (low nibble: a
// dim of the even 16-dim block, high nibble: the same dim of the odd block), 4-bit two's
// complement.  Returns fp16 pairs (token 0, token 2) and (token 1, token 3) for both dims.
__device__ inline void i4x8_to_h2x4(uint32_t x, uint32_t& lo02, uint32_t& lo13, uint32_t& hi02,
                                    uint32_t& hi13) {
  // nibble n (two's complement code c) xor 8 = c + 8; 0x6400 | m is the fp16 value 1024 + m, so
  // (x & 0x000F000F) ^ 0x64086408 is 1024 + c + 8 per half (and the same with 16 (c + 8) for the
  // high nibbles), one and-xor each
  const uint32_t x8 = x >> 8;
  const half2v off_lo = {(_Float16)-1032.0f, (_Float16)-1032.0f};
  const half2v sixteenth = {(_Float16)0.0625f, (_Float16)0.0625f};
  const half2v off_hi = {(_Float16)-72.0f, (_Float16)-72.0f};
  lo02 = as_u32(as_h2((x & 0x000F000Fu) ^ 0x64086408u) + off_lo);
  lo13 = as_u32(as_h2((x8 & 0x000F000Fu) ^ 0x64086408u) + off_lo);
  hi02 = as_u32(__builtin_elementwise_fma(as_h2((x & 0x00F000F0u) ^ 0x64806480u), sixteenth, off_hi));
  hi13 = as_u32(__builtin_elementwise_fma(as_h2((x8 & 0x00F000F0u) ^ 0x64806480u), sixteenth, off_hi));
}

// The 8-bit form: lo_w holds, for four tokens r = 0..3 (byte r), the int8 codes of a dim of the
// even 16-dim block, hi_w the same dim of the odd block.  Same outputs as i4x8_to_h2x4: byte b
// (code c) xor 0x80 is c + 128, and 0x6400 | m is the fp16 value 1024 + m, so
// ((x & 0x00FF00FF) ^ 0x64806480) - 1152 per half is c, exactly.
__device__ inline void i8x8_to_h2x4(uint32_t lo_w, uint32_t hi_w, uint32_t& lo02, uint32_t& lo13,
                                    uint32_t& hi02, uint32_t& hi13) {
  const half2v off = {(_Float16)-1152.0f, (_Float16)-1152.0f};
  lo02 = as_u32(as_h2((lo_w & 0x00FF00FFu) ^ 0x64806480u) + off);
  lo13 = as_u32(as_h2(((lo_w >> 8) & 0x00FF00FFu) ^ 0x64806480u) + off);
  hi02 = as_u32(as_h2((hi_w & 0x00FF00FFu) ^ 0x64806480u) + off);
  hi13 = as_u32(as_h2(((hi_w >> 8) & 0x00FF00FFu) ^ 0x64806480u) + off);
}

// The E4M3 form: lo_w / hi_w as for i8x8_to_h2x4, each byte an OCP E4M3 code.  Every E4M3
// value (magnitudes 2^-9 .. 448) is an fp16 value, so the gfx950 converter (scale 1) is exact; a
// byte permute first pairs tokens (0, 2) and (1, 3).
template <bool HI_WORD>
__device__ inline uint32_t e4m3x2_to_h2(uint32_t x) {
  return as_u32(__builtin_amdgcn_cvt_scalef32_pk_f16_fp8(x, 1.0f, HI_WORD));
}
__device__ inline void f8x8_to_h2x4(uint32_t lo_w, uint32_t hi_w, uint32_t& lo02, uint32_t& lo13,
                                    uint32_t& hi02, uint32_t& hi13) {
  const uint32_t l = __builtin_amdgcn_perm(lo_w, lo_w, 0x03010200u);  // bytes (0, 2, 1, 3)
  const uint32_t h = __builtin_amdgcn_perm(hi_w, hi_w, 0x03010200u);
  lo02 = e4m3x2_to_h2<false>(l);
  lo13 = e4m3x2_to_h2<true>(l);
  hi02 = e4m3x2_to_h2<false>(h);
  hi13 = e4m3x2_to_h2<true>(h);
}

// p0 * s0 and p1 * s1 (p fp32, s the low fp16 half of sw0 / sw1) as fp16 hi + lo pairs:
// hi = rne(p * s) and lo = rne(p * s - hi) straight from the exact products (v_fma_mix*), so the
// two halves always belong together and hi + lo = p * s to about 2^-22.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ inline void mix_hi_lo(float p0, uint32_t sw0, float p1, uint32_t sw1, uint32_t& hi, uint32_t& lo) {
  uint32_t h, l;  // the lo-half writes declare the whole register as output; the hi-half writes keep it
  asm("v_fma_mixlo_f16 %0, %1, %2, 0 op_sel:[0,0,0] op_sel_hi:[0,1,0]" : "=v"(h) : "v"(p0), "v"(sw0));
  asm("v_fma_mixhi_f16 %0, %1, %2, 0 op_sel:[0,0,0] op_sel_hi:[0,1,0]" : "+v"(h) : "v"(p1), "v"(sw1));
  asm("v_fma_mixlo_f16 %0, %1, %2, -%3 op_sel:[0,0,0] op_sel_hi:[0,1,1]" : "=&v"(l) : "v"(p0), "v"(sw0), "v"(h));
  asm("v_fma_mixhi_f16 %0, %1, %2, -%3 op_sel:[0,0,1] op_sel_hi:[0,1,1]" : "+v"(l) : "v"(p1), "v"(sw1), "v"(h));
  hi = h;
  lo = l;
}
#pragma clang diagnostic pop

__device__ inline float h_at(const uint32_t* words, int idx) {
  const uint32_t w = words[idx >> 1];
  return (float)__builtin_bit_cast(_Float16, (uint16_t)((idx & 1) ? (w >> 16) : (w & 0xFFFF)));
}

typedef uint16_t u16x2 __attribute__((ext_vector_type(2)));

// max of x over the four lanes m16, m16 + 16, m16 + 32, m16 + 48 (the lanes of one query row in
// the 16x16 matrix-core layouts), with the gfx950 cross-row swaps instead of LDS permutes.
__device__ inline float max_over_rows(float x) {
  // (max of two lanes' floats that are never NaN: one plain v_max_f32, without the quieting the
  // compiler adds to fmaxf of values it cannot see)
  auto mx = [](uint32_t p, uint32_t q) {
    float r;
    asm("v_max_f32 %0, %1, %2" : "=v"(r) : "v"(p), "v"(q));
    return r;
  };
  const uint32_t u = __builtin_bit_cast(uint32_t, x);
  const auto a = __builtin_amdgcn_permlane16_swap(u, u, false, false);  // rows (0,1), (2,3) meet
  const uint32_t v = __builtin_bit_cast(uint32_t, mx(a[0], a[1]));
  const auto b = __builtin_amdgcn_permlane32_swap(v, v, false, false);  // halves meet
  return mx(b[0], b[1]);
}

// sum of x over the four lanes m16, m16 + 16, m16 + 32, m16 + 48
__device__ inline float sum_over_rows(float x) {
  const uint32_t u = __builtin_bit_cast(uint32_t, x);
  const auto a = __builtin_amdgcn_permlane16_swap(u, u, false, false);
  const uint32_t a0 = a[0], a1 = a[1];
  x = __builtin_bit_cast(float, a0) + __builtin_bit_cast(float, a1);
  const uint32_t v = __builtin_bit_cast(uint32_t, x);
  const auto b = __builtin_amdgcn_permlane32_swap(v, v, false, false);
  const uint32_t b0 = b[0], b1 = b[1];
  return __builtin_bit_cast(float, b0) + __builtin_bit_cast(float, b1);
}

// Wave-wide max / sum of a float (the same value in every lane for the max; the sum is taken
// from lane 0 and broadcast, so every lane agrees on it bit for bit).
template <bool kSum>
__device__ inline float wave_reduce(float x) {
  auto op = [](float p, float q) { return kSum ? p + q : fmaxf(p, q); };
#define KVQ_DPP(v, ctrl) \
  __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), ctrl, 0xF, 0xF, false))
  x = op(x, KVQ_DPP(x, 0xB1));   // quad_perm [1,0,3,2]
  x = op(x, KVQ_DPP(x, 0x4E));   // quad_perm [2,3,0,1]
  x = op(x, KVQ_DPP(x, 0x141));  // row_half_mirror
  x = op(x, KVQ_DPP(x, 0x140));  // row_mirror
#undef KVQ_DPP
  const uint32_t u = __builtin_bit_cast(uint32_t, x);
  const auto a = __builtin_amdgcn_permlane16_swap(u, u, false, false);
  const uint32_t a0 = a[0], a1 = a[1];
  x = op(__builtin_bit_cast(float, a0), __builtin_bit_cast(float, a1));
  const uint32_t v = __builtin_bit_cast(uint32_t, x);
  const auto b = __builtin_amdgcn_permlane32_swap(v, v, false, false);
  const uint32_t b0 = b[0], b1 = b[1];
  x = op(__builtin_bit_cast(float, b0), __builtin_bit_cast(float, b1));
  return kSum ? __builtin_bit_cast(float, __builtin_amdgcn_readfirstlane(__builtin_bit_cast(int, x))) : x;
}

// Largest of the 128 fp16 halves of x over the wave (as 16-bit patterns, in both halves).
__device__ inline uint32_t wave_max_u16x2(uint32_t x) {
  auto mx = [](uint32_t p, uint32_t q) {
    return __builtin_bit_cast(uint32_t, __builtin_elementwise_max(__builtin_bit_cast(u16x2, p),
                                                                  __builtin_bit_cast(u16x2, q)));
  };
  x = mx(x, __builtin_amdgcn_update_dpp(0u, x, 0xB1, 0xF, 0xF, false));   // quad_perm [1,0,3,2]
  x = mx(x, __builtin_amdgcn_update_dpp(0u, x, 0x4E, 0xF, 0xF, false));   // quad_perm [2,3,0,1]
  x = mx(x, __builtin_amdgcn_update_dpp(0u, x, 0x141, 0xF, 0xF, false));  // row_half_mirror
  x = mx(x, __builtin_amdgcn_update_dpp(0u, x, 0x140, 0xF, 0xF, false));  // row_mirror
  const auto a = __builtin_amdgcn_permlane16_swap(x, x, false, false);
  x = mx(a[0], a[1]);
  const auto b = __builtin_amdgcn_permlane32_swap(x, x, false, false);
  x = mx(b[0], b[1]);
  return mx(x, (x >> 16) | (x << 16));
}

template <int D, int VB>
struct TileRaw {
  static constexpr int kLoadsK = D / 64;                    // 16-byte loads of K codes per lane
  static constexpr int kVWords = D * VB / 128;              // V code dwords per lane
  static constexpr int kVsWords = D / 16;                   // V scale dwords per lane (4 tokens x D/32)
  u32x4 k[kLoadsK];
  uint32_t v[kVWords];
  uint32_t vs[kVsWords];
  uint32_t ks[2];                                           // K scales of tokens 4g..4g+3
};

// ---- staging of one block (two tiles) in LDS --------------------------------------------
// A staged tile is an exact copy of the tile's four sections, packed:
//   [K codes 16*D][V codes 16*D*VB/8][V scales D][K scales 32]  (25*D + 32 bytes for 4-bit V
// codes, 33*D + 32 for 8-bit ones).
template <int D, int VB>
struct Stage {
  static constexpr int kK = 0;
  static constexpr int kV = 16 * D;
  static constexpr int kVBytes = 2 * D * VB;  // V codes of a tile
  static constexpr int kVs = kV + kVBytes;
  static constexpr int kKs = kVs + D;
  static constexpr int kTileBytes = kKs + 32;
  static constexpr int kBlockBytes = 2 * kTileBytes;
  // direct-to-LDS loads per block (vmcnt units): K codes, V codes, then V and K scales in one
  // load (they sit back to back in the stage, D/16 lanes of V scales and 2 of K scales)
  static constexpr int kLoadsV = VB == 8 ? D / 64 : (D >= 128 ? D / 128 : 1);
  static constexpr int kLoads = 2 * (D / 64 + kLoadsV + 1);
  static constexpr int kScaleLanes = D / 16 + 2;
};

typedef __attribute__((address_space(3))) void lds_void;

// M0 is named as clobbered below: these kernels set it themselves before each group of
// direct-to-LDS loads and use it for nothing else, so the compiler's warning is moot.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
// N x 16 bytes per lane: load i moves sbase + voff + 1024 i to LDS lds + 1024 i + 16 lane (gfx950
// global_load_lds_dwordx4 with a scalar base; the immediate offset applies to both addresses, and
// the LDS side of a lane is always 16 * lane past M0).  Issued as inline asm: the waits for these
// loads are this file's explicit s_waitcnt vmcnt, which keep two blocks in flight (the compiler
// would otherwise drain every load before each LDS read).  The "memory" clobber keeps LDS reads
// of the buffer on their side of it.  M0 is written one instruction ahead of its first DMA use.
// The loads are non-temporal: every cache byte is read once per call, and keeping the stream
// out of the caches' normal replacement measured 9% faster on the 184K-token workload.
// With LANES < 64 only lanes 0 .. LANES-1 load (exec is narrowed and restored inside).
template <int N, int LANES = kWave>
__device__ inline void dma16(const uint8_t* sbase, uint32_t voff, uint32_t lds) {
  static_assert(N >= 1 && N <= 4 && (LANES == kWave || N == 1), "shape");
  if constexpr (LANES < kWave) {
    uint64_t saved;
    asm volatile("s_mov_b64 %0, exec\n\ts_bfm_b64 exec, %4, 0\n\ts_mov_b32 m0, %3\n\ts_nop 0\n\t"
                 "global_load_lds_dwordx4 %2, %1 nt\n\ts_mov_b64 exec, %0"
                 : "=&s"(saved) : "s"(sbase), "v"(voff), "s"(lds), "n"(LANES) : "memory", "m0");
  } else if constexpr (N == 1) {
    asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, %0 nt"
                 ::"s"(sbase), "v"(voff), "s"(lds) : "memory", "m0");
  } else if constexpr (N == 2) {
    asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, %0 nt\n\t"
                 "global_load_lds_dwordx4 %1, %0 offset:1024 nt"
                 ::"s"(sbase), "v"(voff), "s"(lds) : "memory", "m0");
  } else {
    asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, %0 nt\n\t"
                 "global_load_lds_dwordx4 %1, %0 offset:1024 nt\n\t"
                 "global_load_lds_dwordx4 %1, %0 offset:2048 nt\n\t"
                 "global_load_lds_dwordx4 %1, %0 offset:3072 nt"
                 ::"s"(sbase), "v"(voff), "s"(lds) : "memory", "m0");
  }
}
#pragma clang diagnostic pop

template <int N>
__device__ inline void wait_vmcnt() {
  // loads complete in order: at most N of this wave's loads may still be in flight
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// Per-lane byte offsets, within a (page, KV head) block, of the merged scale load of a tile
// starting at slot 0: lanes below D/16 take 16 bytes each of the V scales, the next two the K
// scales; a tile at slot0 adds slot0 * scale_step (2 * D/32 or 2 bytes per slot).
struct ScaleLane {
  uint32_t off0, step;
};

template <int D, int VB>
__device__ inline ScaleLane scale_lane(int P, int lane) {
  if (lane < D / 16) return {(uint32_t)v_scales_at(P, D, VB) + 16u * lane, (uint32_t)(D / 16)};
  const int kl = min(lane - D / 16, 1);  // lanes past the two K-scale lanes are masked off
  return {(uint32_t)k_scales_at(P, D) + 16u * kl, 2u};
}

// Issue the loads of one tile of the (page, KV head) block at pb (slot0 = the tile's first slot
// in the page) into LDS at byte address dst (wave-uniform).
template <int D, int VB>
__device__ inline void stage_tile(const uint8_t* pb, int P, int slot0, uint32_t dst, uint32_t lane16,
                                  ScaleLane sl) {
  static_assert(D == 64 || D == 128 || D == 256, "head_dim");
  using S = Stage<D, VB>;
  const uint32_t tip = (uint32_t)slot0 >> 4;  // offsets within one block are 32-bit
  dma16<D / 64>(pb + tip * (16u * D), lane16, dst + S::kK);
  const uint8_t* vb = pb + ((uint32_t)v_codes_at(P, D) + tip * (uint32_t)S::kVBytes);
  if constexpr (VB == 8)
    dma16<D / 64>(vb, lane16, dst + S::kV);
  else if constexpr (D >= 128)
    dma16<D / 128>(vb, lane16, dst + S::kV);
  else
    dma16<1, 32>(vb, lane16, dst + S::kV);
  dma16<1, S::kScaleLanes>(pb, sl.off0 + (uint32_t)slot0 * sl.step, dst + S::kVs);
}

// Read one staged tile into this lane's registers (the lane's share of every section).
template <int D, int VB>
__device__ inline void read_tile(TileRaw<D, VB>& r, const uint8_t* src, int lane) {
  using S = Stage<D, VB>;
  const int g = lane >> 4;
#pragma unroll
  for (int jj = 0; jj < TileRaw<D, VB>::kLoadsK; ++jj)
    r.k[jj] = *(const u32x4*)(src + S::kK + 1024 * jj + 16 * lane);
  const u32x2 ks = *(const u32x2*)(src + S::kKs + 8 * g);
  r.ks[0] = ks[0];
  r.ks[1] = ks[1];
  if constexpr (VB == 8) {
    // 16 bytes per lane per 1 KB: two scale groups' (even-block dim, odd-block dim) dwords
#pragma unroll
    for (int c = 0; c < D / 64; ++c) {
      const u32x4 w = *(const u32x4*)(src + S::kV + 1024 * c + 16 * lane);
#pragma unroll
      for (int e = 0; e < 4; ++e) r.v[4 * c + e] = w[e];
    }
  } else if constexpr (D == 64) {
    const u32x2 w = *(const u32x2*)(src + S::kV + 8 * lane);
    r.v[0] = w[0];
    r.v[1] = w[1];
  } else {
#pragma unroll
    for (int c = 0; c < D / 128; ++c) {
      const u32x4 w = *(const u32x4*)(src + S::kV + 1024 * c + 16 * lane);
#pragma unroll
      for (int e = 0; e < 4; ++e) r.v[4 * c + e] = w[e];
    }
  }
#pragma unroll
  for (int c = 0; c < TileRaw<D, VB>::kVsWords / 4; ++c) {
    const u32x4 w = *(const u32x4*)(src + S::kVs + g * (D / 4) + 16 * c);
#pragma unroll
    for (int e = 0; e < 4; ++e) r.vs[4 * c + e] = w[e];
  }
}

// E4M3 codes: a slot no row sees may never have been written, and a NaN code times a zero
// scale is no zero.  Clears the lane's V code bytes of the tile's slots outside [lo, hi): byte r
// of every V word of lane group g is slot 4g + r of the tile starting at token tok0.
template <int D, int VB>
__device__ inline void clear_unseen_v(TileRaw<D, VB>& r, int tok0, int g, int lo, int hi) {
  uint32_t keep = 0;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const int t = tok0 + 4 * g + e;
    keep |= (t >= lo && t < hi) ? 0xFFu << (8 * e) : 0u;
  }
#pragma unroll
  for (int i = 0; i < TileRaw<D, VB>::kVWords; ++i) r.v[i] &= keep;
}

// One 32-token block of one wave: S^T = K Q^T, online softmax, O^T += V^T P^T.
// Running state of one wave, per query row (the lane's row in each 16-row block nb):
//   base   integer exponent offset (or -inf before any unmasked token): l_run and acc hold
//          sums of 2^(z - base) * (1, v);  it only moves up, in whole powers of two, when a block's
//          largest logit and V scale would push p * v_scale past 2^15 (fp16 headroom), so most
//          blocks rescale nothing and every rescale is exact.
// Q K^T of one block: sc[tau][nb][e] is the dot product of the lane's query row with token
// 4g + e of tile tau, in units of the query scale (before the K scale and cz).
template <int D, int NB, int VB, bool F8>
__device__ __attribute__((always_inline)) inline void block_scores(TileRaw<D, VB> (&raw)[2],
                                                                   const i32x4 (&qd)[NB][3][D / 64],
                                                                   const u32x4 (&qw)[NB][D / 64][2],
                                                                   float (&sc)[2][NB][4]) {
  // ---- S^T = K Q^T: int8 codes on the int8 matrix cores with three digit planes of Q; E4M3
  // codes widened to fp16 (exactly) on the f16 matrix cores with Q's own fp16 values ----
  i32x4 sd[2][NB][3];
  floatx4 sf[2][NB];
#pragma unroll
  for (int tau = 0; tau < 2; ++tau)
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      sf[tau][nb] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int pc = 0; pc < 3; ++pc) sd[tau][nb][pc] = i32x4{0, 0, 0, 0};
    }
  // tile by tile: the first tile's scores are complete after half of the products, so their
  // conversion and logits can go on beside the second tile's
#pragma unroll
  for (int tau = 0; tau < 2; ++tau)
#pragma unroll
    for (int jj = 0; jj < D / 64; ++jj) {
      if constexpr (F8) {
        // dword i of the lane's 16 codes holds dims 4i .. 4i+3: halves 0..7 and 8..15 pair with
        // the query's two fp16 words of the same 16 dims
        const u32x4 kc = raw[tau].k[jj];
        uint32_t kh[8];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          kh[2 * i] = e4m3x2_to_h2<false>(kc[i]);
          kh[2 * i + 1] = e4m3x2_to_h2<true>(kc[i]);
        }
        const half8 k0 = __builtin_bit_cast(half8, u32x4{kh[0], kh[1], kh[2], kh[3]});
        const half8 k1 = __builtin_bit_cast(half8, u32x4{kh[4], kh[5], kh[6], kh[7]});
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
          sf[tau][nb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(k0, __builtin_bit_cast(half8, qw[nb][jj][0]),
                                                               sf[tau][nb], 0, 0, 0);
          sf[tau][nb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(k1, __builtin_bit_cast(half8, qw[nb][jj][1]),
                                                               sf[tau][nb], 0, 0, 0);
        }
      } else {
        const i32x4 ka = __builtin_bit_cast(i32x4, raw[tau].k[jj]);
#pragma unroll
        for (int nb = 0; nb < NB; ++nb)
#pragma unroll
          for (int pc = 0; pc < 3; ++pc)
            sd[tau][nb][pc] = __builtin_amdgcn_mfma_i32_16x16x64_i8(ka, qd[nb][pc][jj], sd[tau][nb][pc], 0, 0, 0);
      }
    }
#pragma unroll
  for (int nb = 0; nb < NB; ++nb)
#pragma unroll
    for (int tau = 0; tau < 2; ++tau)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        if constexpr (F8) {
          sc[tau][nb][e] = sf[tau][nb][e];
        } else {
          const int hm = (sd[tau][nb][0][e] << 8) + sd[tau][nb][1][e];  // |.| < 2^30: exact
          sc[tau][nb][e] = __builtin_fmaf((float)hm, 256.0f, (float)sd[tau][nb][2][e]);
        }
      }
}

// The online softmax of one block from its scores: z = sc * k_scale * cz in log2 units, the
// masks, and the block's p = 2^(z - base) per row and token in pexp (the acc rescale included).
// ks_words: the K-scale words of the two tiles (fp16 scales of tokens 4g .. 4g + 3).
template <int D, int NB, bool WIN>
__device__ __attribute__((always_inline)) inline void block_softmax_scores(
    const float (&sc)[2][NB][4], const uint32_t (&ks_words)[2][2], int blk, bool masked, float e5,
    const float (&cz)[NB], const int (&first_tok)[NB], const int (&last_tok)[NB], int g,
    floatx4 (&acc)[NB][D / 16], float (&base)[NB], float (&l_run)[NB], float (&pexp)[NB][2][4]) {
  constexpr int DB = D / 16;
  float ks[2][4];
#pragma unroll
  for (int tau = 0; tau < 2; ++tau)
#pragma unroll
    for (int e = 0; e < 4; ++e) ks[tau][e] = h_at(ks_words[tau], e);

  // ---- logits and the online softmax (log2 units) ----
  float z[NB][2][4], lm[NB];
  bool over = false;  // some row needs a larger exponent offset than it has
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
#pragma unroll
    for (int tau = 0; tau < 2; ++tau)
#pragma unroll
      for (int e = 0; e < 4; ++e) z[nb][tau][e] = sc[tau][nb][e] * (ks[tau][e] * cz[nb]);
    if (masked) {  // wave-uniform: only the blocks at the end of a context
#pragma unroll
      for (int tau = 0; tau < 2; ++tau)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int t = blk * kBlock + kTile * tau + 4 * g + e;
          const bool seen = WIN ? (t <= last_tok[nb] && t >= first_tok[nb]) : t <= last_tok[nb];
          z[nb][tau][e] = seen ? z[nb][tau][e] : kNegInf;
        }
    }
    lm[nb] = kNegInf;
#pragma unroll
    for (int tau = 0; tau < 2; ++tau)
#pragma unroll
      for (int e = 0; e < 4; ++e) lm[nb] = fmaxf(lm[nb], z[nb][tau][e]);
    // p * v_scale < 2^(bm - base + e5 - 14) must stay below 2^15, bm the row's largest logit.
    // Rounding is monotone, so a row's fl(bm + (e5 - 29)) exceeds its base exactly when one of
    // its four lanes' fl(lm + (e5 - 29)) does: the lanes test their own maxima, and the row
    // maximum (a cross-lane reduction) is formed only on the rare blocks that move a base.
    over |= lm[nb] + (e5 - 29.0f) > base[nb];
  }
  float alpha[NB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) alpha[nb] = 1.0f;
  if (__builtin_expect(__any(over), 0)) {  // a wave's first block, or a larger logit or V scale
    bool rescale = false;
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      const float need = max_over_rows(lm[nb]) + (e5 - 29.0f);
      if (need > base[nb]) {
        const float b_new = __builtin_ceilf(need) + 2.0f;  // two powers of two of headroom for later blocks
        if (base[nb] != kNegInf) {
          alpha[nb] = __builtin_ldexpf(1.0f, (int)(base[nb] - b_new));
          rescale = true;
        }
        base[nb] = b_new;
      }
    }
    if (__any(rescale)) {
#pragma unroll
      for (int nb = 0; nb < NB; ++nb)
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
          for (int e = 0; e < 4; ++e) acc[nb][db][e] *= alpha[nb];
    }
  }
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    const float b_use = (base[nb] == kNegInf) ? 0.0f : base[nb];
    float lsum = 0.0f;
#pragma unroll
    for (int tau = 0; tau < 2; ++tau)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        pexp[nb][tau][e] = __builtin_amdgcn_exp2f(z[nb][tau][e] - b_use);
        lsum += pexp[nb][tau][e];
      }
    l_run[nb] = l_run[nb] * alpha[nb] + lsum;
  }
}

// The first half of the block step: Q K^T and the online softmax, leaving the block's
// p = 2^(z - base) per row and token in pexp (the acc rescale included).
template <int D, int NB, int VB, bool WIN, bool F8>
__device__ __attribute__((always_inline)) inline void block_softmax(
    TileRaw<D, VB> (&raw)[2], int blk, bool masked, float e5, const i32x4 (&qd)[NB][3][D / 64],
    const u32x4 (&qw)[NB][D / 64][2], const float (&cz)[NB],
    const int (&first_tok)[NB], const int (&last_tok)[NB], int g, floatx4 (&acc)[NB][D / 16], float (&base)[NB],
    float (&l_run)[NB], float (&pexp)[NB][2][4]) {
  float sc[2][NB][4];
  block_scores<D, NB, VB, F8>(raw, qd, qw, sc);
  const uint32_t ksw[2][2] = {{raw[0].ks[0], raw[0].ks[1]}, {raw[1].ks[0], raw[1].ks[1]}};
  block_softmax_scores<D, NB, WIN>(sc, ksw, blk, masked, e5, cz, first_tok, last_tok, g, acc, base, l_run, pexp);
}

// The second half of the block step: O^T += V^T P^T with the V scale on the V side.  A code
// times its fp16 scale has at most 18 significant bits (an 8-bit integer code; 14 for 4-bit
// codes, 15 for E4M3), so v = code * s_v splits exactly into fp16 hi = rne(v) (one packed
// multiply) and lo = v - hi (one packed fma, exact).  P splits once per row into fp16 hi + lo,
// and each operand pair takes three products (hi*hi, hi*lo, lo*hi; lo*lo is below 2^-22 of the
// product).  Folding the scale into P instead (hi and lo of p * s_v per 32-dim group and row)
// needs two matrix-core products per pair but 128 more VALU instructions per row block, and its
// P halves, written per group right before their products, put a wait in front of every
// group's matrix-core instructions; on the 184K step this form measured 0.7 us faster in the
// first milliseconds, and 10% faster on the two-row-block MTP step.  p stays below 2^13 under
// the offsets (the caller passes e5 = 14: no V-scale exponent enters them).
template <int D, int NB, int VB, bool F8>
__device__ __attribute__((always_inline)) inline void block_pv_vhat_regs(TileRaw<D, VB> (&raw)[2],
                                                                         const float (&pexp)[NB][2][4],
                                                                         floatx4 (&acc)[NB][D / 16]) {
  constexpr int NG = D / 32;
  constexpr uint32_t kOne = 0x3C003C00u;  // fp16 1.0 in both halves
  uint32_t hw[NB][4], lw[NB][4];  // token order of the operand: (tau0: 0,2,1,3), (tau1: 0,2,1,3)
#pragma unroll
  for (int nb = 0; nb < NB; ++nb)
#pragma unroll
    for (int tau = 0; tau < 2; ++tau) {
      mix_hi_lo(pexp[nb][tau][0], kOne, pexp[nb][tau][2], kOne, hw[nb][2 * tau], lw[nb][2 * tau]);
      mix_hi_lo(pexp[nb][tau][1], kOne, pexp[nb][tau][3], kOne, hw[nb][2 * tau + 1], lw[nb][2 * tau + 1]);
    }
  // two wait states between the inline-asm writes of P and the matrix-core reads (the
  // compiler's hazard tracking does not see inline-asm results)
#pragma unroll
  for (int nb = 0; nb < NB; ++nb)
    asm("s_nop 1" : "+v"(hw[nb][0]), "+v"(hw[nb][1]), "+v"(hw[nb][2]), "+v"(hw[nb][3]), "+v"(lw[nb][0]),
        "+v"(lw[nb][1]), "+v"(lw[nb][2]), "+v"(lw[nb][3]));
#pragma unroll
  for (int j = 0; j < NG; ++j) {
    uint32_t l02[2], l13[2], h02[2], h13[2], s02[2], s13[2];
#pragma unroll
    for (int tau = 0; tau < 2; ++tau) {
      if constexpr (F8)
        f8x8_to_h2x4(raw[tau].v[2 * j], raw[tau].v[2 * j + 1], l02[tau], l13[tau], h02[tau], h13[tau]);
      else if constexpr (VB == 8)
        i8x8_to_h2x4(raw[tau].v[2 * j], raw[tau].v[2 * j + 1], l02[tau], l13[tau], h02[tau], h13[tau]);
      else
        i4x8_to_h2x4(raw[tau].v[j], l02[tau], l13[tau], h02[tau], h13[tau]);
      // the scales of tokens (0, 2) and (1, 3) for group j: fp16 half (j & 1) of word (e NG + j) / 2
      const uint32_t* vs = raw[tau].vs;
      constexpr uint32_t kSel[2] = {0x05040100u, 0x07060302u};
      s02[tau] = __builtin_amdgcn_perm(vs[(2 * NG + j) / 2], vs[(0 * NG + j) / 2], kSel[j & 1]);
      s13[tau] = __builtin_amdgcn_perm(vs[(3 * NG + j) / 2], vs[(1 * NG + j) / 2], kSel[j & 1]);
    }
    uint32_t vh[2][2][4];  // [dim half][hi, lo][word]
#pragma unroll
    for (int tau = 0; tau < 2; ++tau) {
      const uint32_t c[2][2] = {{l02[tau], l13[tau]}, {h02[tau], h13[tau]}};
      const uint32_t sc[2] = {s02[tau], s13[tau]};
#pragma unroll
      for (int dh = 0; dh < 2; ++dh)
#pragma unroll
        for (int k = 0; k < 2; ++k) {
          const half2v cv = as_h2(c[dh][k]), sv = as_h2(sc[k]);
          const half2v hi = cv * sv;
          const half2v lo = __builtin_elementwise_fma(cv, sv, -hi);
          vh[dh][0][2 * tau + k] = as_u32(hi);
          vh[dh][1][2 * tau + k] = as_u32(lo);
        }
    }
#pragma unroll
    for (int dh = 0; dh < 2; ++dh) {
      const half8 vhi = __builtin_bit_cast(half8, u32x4{vh[dh][0][0], vh[dh][0][1], vh[dh][0][2], vh[dh][0][3]});
      const half8 vlo = __builtin_bit_cast(half8, u32x4{vh[dh][1][0], vh[dh][1][1], vh[dh][1][2], vh[dh][1][3]});
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        const half8 phi = __builtin_bit_cast(half8, u32x4{hw[nb][0], hw[nb][1], hw[nb][2], hw[nb][3]});
        const half8 plo = __builtin_bit_cast(half8, u32x4{lw[nb][0], lw[nb][1], lw[nb][2], lw[nb][3]});
        floatx4& c = acc[nb][2 * j + dh];
        c = __builtin_amdgcn_mfma_f32_16x16x32_f16(vhi, phi, c, 0, 0, 0);
        c = __builtin_amdgcn_mfma_f32_16x16x32_f16(vhi, plo, c, 0, 0, 0);
        c = __builtin_amdgcn_mfma_f32_16x16x32_f16(vlo, phi, c, 0, 0, 0);
      }
    }
  }
}

template <int D, int NB, int VB, bool WIN, bool F8>
__device__ __attribute__((always_inline)) inline void process_block(
    TileRaw<D, VB> (&raw)[2], int blk, bool masked, float e5, const i32x4 (&qd)[NB][3][D / 64],
    const u32x4 (&qw)[NB][D / 64][2], const float (&cz)[NB],
    const int (&first_tok)[NB], const int (&last_tok)[NB], int g, floatx4 (&acc)[NB][D / 16], float (&base)[NB],
    float (&l_run)[NB]) {
  float pexp[NB][2][4];
  block_softmax<D, NB, VB, WIN, F8>(raw, blk, masked, e5, qd, qw, cz, first_tok, last_tok, g, acc, base, l_run,
                                    pexp);
  block_pv_vhat_regs<D, NB, VB, F8>(raw, pexp, acc);
}

// The query rows' B operands of Q K^T, from the raw fp16 words qw (lane: query row 16*nb + m16
// and the 16 dims 16*(4*jj + g) .. +15 of each 64-dim step jj).  cz[nb] receives the factor
// that turns a row's dot products into log2-unit logits (before the K scale).
template <int D, int NB, bool F8>
__device__ __attribute__((always_inline)) inline void prepare_queries(
    const u32x4 (&qw)[NB][D / 64][2], float scale_log2, i32x4 (&qd)[NB][3][D / 64], float (&cz)[NB]) {
  // Q^T as three int8 digit planes (B of QK^T).  Per row, q * 2^F = h*2^16 + m*2^8 + l with
  // balanced digits in [-128, 127] and |q * 2^F| < 2^22 for the row's largest |q|; exact for every
  // element within 2^12 of it, the rest rounded to the 2^-F grid.  E4M3 keys
  // use the fp16 words as they are (cz = softmax_scale * log2(e)); qd is then left unset.
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    if constexpr (F8) {  // the fp16 query words are the B operands as they are
      cz[nb] = scale_log2;
      continue;
    }
    float amax = 0.0f;
#pragma unroll
    for (int jj = 0; jj < D / 64; ++jj)
#pragma unroll
      for (int hf = 0; hf < 2; ++hf) {
        const half8 h8 = __builtin_bit_cast(half8, qw[nb][jj][hf]);
#pragma unroll
        for (int e = 0; e < 8; ++e) amax = fmaxf(amax, fabsf((float)h8[e]));
      }
    amax = max_over_rows(amax);
    int E = 0;
    if (amax > 0.0f) (void)__builtin_frexpf(amax, &E);  // amax < 2^E
    const int F = amax > 0.0f ? 22 - E : 0;
    const float scale_f = __builtin_ldexpf(1.0f, F);
    cz[nb] = __builtin_ldexpf(scale_log2, -F);
#pragma unroll
    for (int jj = 0; jj < D / 64; ++jj) {
      uint32_t wd[3][4];
#pragma unroll
      for (int w4 = 0; w4 < 4; ++w4) {
        // x + 1.5 * 2^23 rounds x to an integer (ties to even) in the low mantissa bits; adding
        // 128 * (1 + 2^8 + 2^16) then makes byte k of the word digit k + 128, so xor 0x80 per byte
        // leaves the balanced digits as int8
        uint32_t wq[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int el = 4 * w4 + e;
          const half8 h8 = __builtin_bit_cast(half8, qw[nb][jj][el >> 3]);
          const float x = (float)h8[el & 7];
          const uint32_t y = __builtin_bit_cast(uint32_t, __builtin_fmaf(x, scale_f, 12582912.0f));
          wq[e] = (y - (0x4B400000u - 0x808080u)) ^ 0x808080u;
        }
        // 4x3 byte transpose: plane k gets byte k of the four words
        const uint32_t t01 = __builtin_amdgcn_perm(wq[1], wq[0], 0x05010400u);
        const uint32_t t23 = __builtin_amdgcn_perm(wq[3], wq[2], 0x05010400u);
        const uint32_t u01 = __builtin_amdgcn_perm(wq[1], wq[0], 0x0C0C0602u);
        const uint32_t u23 = __builtin_amdgcn_perm(wq[3], wq[2], 0x0C0C0602u);
        wd[2][w4] = __builtin_amdgcn_perm(t23, t01, 0x05040100u);  // low digits
        wd[1][w4] = __builtin_amdgcn_perm(t23, t01, 0x07060302u);
        wd[0][w4] = __builtin_amdgcn_perm(u23, u01, 0x05040100u);  // high digits
      }
#pragma unroll
      for (int pc = 0; pc < 3; ++pc)
        qd[nb][pc][jj] = __builtin_bit_cast(i32x4, u32x4{wd[pc][0], wd[pc][1], wd[pc][2], wd[pc][3]});
    }
  }
}

// The log-sum-exp merge of the splits.  Eight lanes per (unit, query row, 4 dims) item, 8 items
// per wave: lane p of an item takes the splits p, p + 8, p + 16, ... with an online max (all of
// a batch's loads in flight at once), and the eight lanes combine through DPP moves within each
// row of 16 lanes, so the merge needs no LDS and no barrier.  The partials come from the
// previous launch on the stream.  On the 184K-token step (32 splits) one lane per item took
// about 1 us longer per step than 4 lanes, and 8 and 16 lanes measured 0.3-0.6 us below 4.

// The partials' addresses and shape come as separate leading kernel arguments (preloaded into
// SGPRs, like the decode's), so the partial loads issue without a kernel-argument load first.
template <int D>
__global__ __launch_bounds__(64) void merge_kernel(const float* ws_acc, const float2* ws_ml, float* out,
                                                   float* lse, int splits, int rows, int num_kv_heads,
                                                   int group, int n_rows, int n_q_heads, DecodeArgs args) {
  DecodeArgs a = args;
  a.ws_acc = (float*)ws_acc;
  a.ws_ml = (float2*)ws_ml;
  a.out = out;
  a.lse = lse;
  a.splits = splits;
  a.rows = rows;
  a.num_kv_heads = num_kv_heads;
  a.group = group;
  a.n_rows = n_rows;
  a.n_q_heads = n_q_heads;
  constexpr int NQ = D / 4;
  constexpr int U = 32 / kMergeLanes;  // splits per lane per batch
  const int S = a.splits, R = a.rows;
  const int items = R * NQ;
  const int per_unit = (int)merge_groups(R, D);
  const int unit = blockIdx.x / per_unit;
  const int part = threadIdx.x & (kMergeLanes - 1);
  const int it0 = (blockIdx.x % per_unit) * kMergeItems + (int)(threadIdx.x / kMergeLanes);
  const bool live = it0 < items;  // the same for every lane of an item
  const int it = live ? it0 : items - 1;
  const int n = it / NQ, q = it % NQ;
  const int b = unit / a.num_kv_heads, h = unit % a.num_kv_heads;
  const float2* ml = a.ws_ml + (size_t)unit * ml_stride(S, R) + n;
  const float* prt = a.ws_acc + ((size_t)unit * S * R + n) * D + 4 * q;
  float mx = kNegInf, den = 0.0f;
  floatx4 num = {0.f, 0.f, 0.f, 0.f};
  for (int s0 = part; s0 < S; s0 += kMergeLanes * U) {
    float2 mv[U];
    floatx4 v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {  // indices clamped into range: all loads issued at once
      const int sp = min(s0 + kMergeLanes * u, S - 1);
      mv[u] = ml[(size_t)sp * R];
      v[u] = *(const floatx4*)(prt + (size_t)sp * R * D);
    }
    // the batch's largest max; the running sums move to it (once per batch, exactly)
    float bm = kNegInf;
#pragma unroll
    for (int u = 0; u < U; ++u) bm = s0 + kMergeLanes * u < S ? fmaxf(bm, mv[u].x) : bm;
    if (bm > mx) {
      const float f = __builtin_amdgcn_exp2f(mx - bm);  // 0 while mx is -inf
      num *= f;
      den *= f;
      mx = bm;
    }
    const float m_use = mx == kNegInf ? 0.0f : mx;  // no split has seen a token yet
#pragma unroll
    for (int u = 0; u < U; ++u) {
      // a split that saw nothing has max -inf and weight 0
      const float wgt = s0 + kMergeLanes * u < S ? __builtin_amdgcn_exp2f(mv[u].x - m_use) : 0.0f;
      num += wgt * v[u];
      den += wgt * mv[u].y;
    }
  }
  // the lanes of the item: common max, then sums (quad_perm [1,0,3,2] and [2,3,0,1], then
  // row_half_mirror and row_mirror for groups of 8 and 16)
#define KVQ_QUAD(v, ctrl) \
  __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), ctrl, 0xF, 0xF, false))
  float M = fmaxf(mx, KVQ_QUAD(mx, 0xB1));
  M = fmaxf(M, KVQ_QUAD(M, 0x4E));
  if constexpr (kMergeLanes >= 8) M = fmaxf(M, KVQ_QUAD(M, 0x141));
  if constexpr (kMergeLanes >= 16) M = fmaxf(M, KVQ_QUAD(M, 0x140));
  const float f = mx == kNegInf ? 0.0f : __builtin_amdgcn_exp2f(mx - M);
  den *= f;
  num *= f;
  den += KVQ_QUAD(den, 0xB1);
  den += KVQ_QUAD(den, 0x4E);
  if constexpr (kMergeLanes >= 8) den += KVQ_QUAD(den, 0x141);
  if constexpr (kMergeLanes >= 16) den += KVQ_QUAD(den, 0x140);
  // (elements are copied to scalars first: a bit cast of a vector element reads element 0 with
  // this compiler)
  float nv[4] = {num[0], num[1], num[2], num[3]};
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    nv[e] += KVQ_QUAD(nv[e], 0xB1);
    nv[e] += KVQ_QUAD(nv[e], 0x4E);
    if constexpr (kMergeLanes >= 8) nv[e] += KVQ_QUAD(nv[e], 0x141);
    if constexpr (kMergeLanes >= 16) nv[e] += KVQ_QUAD(nv[e], 0x140);
  }
  num = floatx4{nv[0], nv[1], nv[2], nv[3]};
#undef KVQ_QUAD
  if (!live || part != 0) return;
  const int i = n / a.group, hq = h * a.group + n % a.group;
  const size_t o = ((size_t)b * a.n_rows + i) * a.n_q_heads + hq;
  *(floatx4*)(a.out + o * D + 4 * q) = num * (den > 0.0f ? 1.0f / den : 0.0f);
  if (q == 0 && a.lse) a.lse[o] = den > 0.0f ? (M + log2f(den)) * 0.69314718055994530942f : kNegInf;
}

template <int D>
void launch_merge(const DecodeArgs& a, unsigned groups, hipStream_t stream) {
  hipLaunchKernelGGL((merge_kernel<D>), dim3(groups), dim3(kWave), 0, stream, a.ws_acc, a.ws_ml, a.out, a.lse,
                     a.splits, a.rows, a.num_kv_heads, a.group, a.n_rows, a.n_q_heads, a);
}

}  // namespace
}  // namespace kvq

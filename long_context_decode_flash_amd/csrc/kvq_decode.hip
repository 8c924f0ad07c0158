// kvq_decode.hip — split-KV decode attention over the paged K8/V4 cache and the log-sum-exp
// merge of the pieces.
//
// The pages describe a decode kernel tuned for one long request over a KV cache handled in
// pieces of the context, loading only the current piece on chip (blog page "標籤: vLLM",
// 重點說明 part 2), and decode whose speed is bound by the bytes read per token (forum post
// "3090 单卡跑 Qwen3.8-27B：NInfer 上机实测（180K 上下文 / C2 并发 / 4bit KV）", 二、测评 and the
// replies on 4-bit vs fp16 KV).  The split-KV scheme here is this library's MI355X design:
//
//   * one workgroup of 4 waves per piece of a (sequence, KV head) context; each wave streams
//     32-token blocks through three LDS stage buffers with direct-to-LDS 16-byte loads, so two
//     blocks are in flight while it computes one;
//   * Q K^T runs on the int8 matrix cores: the K codes of one 16-byte load per lane are the A
//     operand of v_mfma_i32_16x16x64_i8 as they sit in the page, and each query row is split
//     exactly into three int8 digits at a per-row power-of-two scale (B operands, query rows of
//     the GQA group x MTP rows on N), so the dot products are exact integers;
//   * the 16x16 logit tile comes out with each lane holding one query row and four tokens, the
//     B-operand layout of the P V product (tokens on K), so P never leaves the registers; V codes
//     arrive pre-arranged as the A operand of v_mfma_f32_16x16x32_f16 and are widened with
//     exact bit tricks; the V scale (per token and 32 dims) is folded into P, split into fp16
//     high and low parts from one single-rounding multiply so the product keeps fp32 accuracy;
//   * online softmax in log2 units whose exponent offset only moves in powers of two when a
//     block needs it, so most blocks rescale nothing;
//   * the waves merge through LDS into one partial per workgroup (or straight into the output
//     when a context is one piece); a second, wide launch merges the pieces' partials, one
//     lane per (sequence, KV head, query row, 4 dims).
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

// p0 * s0 and p1 * s1 (p fp32, s an fp16 half of sw0 / sw1 selected by SH) as fp16 hi + lo pairs:
// hi = rne(p * s) and lo = rne(p * s - hi) straight from the exact products (v_fma_mix*), so the
// two halves always belong together and hi + lo = p * s to about 2^-22.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
template <int SH>
__device__ inline void mix_hi_lo(float p0, uint32_t sw0, float p1, uint32_t sw1, uint32_t& hi,
                                 uint32_t& lo) {
  uint32_t h, l;  // the lo-half writes declare the whole register as output; the hi-half writes keep it
  if constexpr (SH == 0) {
    asm("v_fma_mixlo_f16 %0, %1, %2, 0 op_sel:[0,0,0] op_sel_hi:[0,1,0]" : "=v"(h) : "v"(p0), "v"(sw0));
    asm("v_fma_mixhi_f16 %0, %1, %2, 0 op_sel:[0,0,0] op_sel_hi:[0,1,0]" : "+v"(h) : "v"(p1), "v"(sw1));
    asm("v_fma_mixlo_f16 %0, %1, %2, -%3 op_sel:[0,0,0] op_sel_hi:[0,1,1]" : "=&v"(l) : "v"(p0), "v"(sw0), "v"(h));
    asm("v_fma_mixhi_f16 %0, %1, %2, -%3 op_sel:[0,0,1] op_sel_hi:[0,1,1]" : "+v"(l) : "v"(p1), "v"(sw1), "v"(h));
  } else {
    asm("v_fma_mixlo_f16 %0, %1, %2, 0 op_sel:[0,1,0] op_sel_hi:[0,1,0]" : "=v"(h) : "v"(p0), "v"(sw0));
    asm("v_fma_mixhi_f16 %0, %1, %2, 0 op_sel:[0,1,0] op_sel_hi:[0,1,0]" : "+v"(h) : "v"(p1), "v"(sw1));
    asm("v_fma_mixlo_f16 %0, %1, %2, -%3 op_sel:[0,1,0] op_sel_hi:[0,1,1]" : "=&v"(l) : "v"(p0), "v"(sw0), "v"(h));
    asm("v_fma_mixhi_f16 %0, %1, %2, -%3 op_sel:[0,1,1] op_sel_hi:[0,1,1]" : "+v"(l) : "v"(p1), "v"(sw1), "v"(h));
  }
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

// One 32-token block of one wave: S^T = K Q^T, online softmax, O^T += V^T P^T.
// Running state of one wave, per query row (the lane's row in each 16-row block nb):
//   base   integer exponent offset (or -inf before any unmasked token): l_run and acc hold
//          sums of 2^(z - base) * (1, v);  it only moves up, in whole powers of two, when a block's
//          largest logit and V scale would push p * v_scale past 2^15 (fp16 headroom), so most
//          blocks rescale nothing and every rescale is exact.
template <int D, int NB, int VB, bool WIN, bool F8>
__device__ __attribute__((always_inline)) inline void process_block(
    TileRaw<D, VB> (&raw)[2], int blk, bool masked, float e5, const i32x4 (&qd)[NB][3][D / 64],
    const u32x4 (&qw)[NB][D / 64][2], const float (&cz)[NB],
    const int (&first_tok)[NB], const int (&last_tok)[NB], int g, floatx4 (&acc)[NB][D / 16], float (&base)[NB],
    float (&l_run)[NB]) {
  constexpr int DB = D / 16;
  constexpr int NG = D / 32;
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
#pragma unroll
  for (int jj = 0; jj < D / 64; ++jj)
#pragma unroll
    for (int tau = 0; tau < 2; ++tau) {
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
  float ks[2][4];
#pragma unroll
  for (int tau = 0; tau < 2; ++tau)
#pragma unroll
    for (int e = 0; e < 4; ++e) ks[tau][e] = h_at(raw[tau].ks, e);

  // ---- logits and the online softmax (log2 units) ----
  float pexp[NB][2][4];
  bool rescale = false;
  float alpha[NB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    float z[2][4];
    float bm = kNegInf;
#pragma unroll
    for (int tau = 0; tau < 2; ++tau)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        float sc;
        if constexpr (F8) {
          sc = sf[tau][nb][e];
        } else {
          const int hm = (sd[tau][nb][0][e] << 8) + sd[tau][nb][1][e];  // |.| < 2^30: exact
          sc = __builtin_fmaf((float)hm, 256.0f, (float)sd[tau][nb][2][e]);
        }
        z[tau][e] = sc * (ks[tau][e] * cz[nb]);
      }
    if (masked) {  // wave-uniform: only the blocks at the end of a context
#pragma unroll
      for (int tau = 0; tau < 2; ++tau)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int t = blk * kBlock + kTile * tau + 4 * g + e;
          const bool seen = WIN ? (t <= last_tok[nb] && t >= first_tok[nb]) : t <= last_tok[nb];
          z[tau][e] = seen ? z[tau][e] : kNegInf;
        }
    }
#pragma unroll
    for (int tau = 0; tau < 2; ++tau)
#pragma unroll
      for (int e = 0; e < 4; ++e) bm = fmaxf(bm, z[tau][e]);
    bm = max_over_rows(bm);
    // p * v_scale < 2^(bm - base + e5 - 14) must stay below 2^15
    const float need = bm + (e5 - 29.0f);
    float b_new = base[nb];
    alpha[nb] = 1.0f;
    if (need > b_new) {
      b_new = __builtin_ceilf(need) + 2.0f;  // two powers of two of headroom for later blocks
      if (base[nb] != kNegInf) {
        alpha[nb] = __builtin_ldexpf(1.0f, (int)(base[nb] - b_new));
        rescale = true;
      }
      base[nb] = b_new;
    }
    const float b_use = (b_new == kNegInf) ? 0.0f : b_new;
    float lsum = 0.0f;
#pragma unroll
    for (int tau = 0; tau < 2; ++tau)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        pexp[nb][tau][e] = __builtin_amdgcn_exp2f(z[tau][e] - b_use);
        lsum += pexp[nb][tau][e];
      }
    l_run[nb] = l_run[nb] * alpha[nb] + lsum;
  }
  if (__builtin_expect(__any(rescale), 0)) {  // rare: a larger logit or V scale than this wave has seen
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int e = 0; e < 4; ++e) acc[nb][db][e] *= alpha[nb];
  }

  // ---- O^T += V^T P^T, one 32-dim scale group at a time ----
#pragma unroll
  for (int j = 0; j < NG; ++j) {
    uint32_t l02[2], l13[2], h02[2], h13[2];
#pragma unroll
    for (int tau = 0; tau < 2; ++tau) {
      if constexpr (F8)
        f8x8_to_h2x4(raw[tau].v[2 * j], raw[tau].v[2 * j + 1], l02[tau], l13[tau], h02[tau], h13[tau]);
      else if constexpr (VB == 8)
        i8x8_to_h2x4(raw[tau].v[2 * j], raw[tau].v[2 * j + 1], l02[tau], l13[tau], h02[tau], h13[tau]);
      else
        i4x8_to_h2x4(raw[tau].v[j], l02[tau], l13[tau], h02[tau], h13[tau]);
    }
    const half8 vlo = __builtin_bit_cast(half8, u32x4{l02[0], l13[0], l02[1], l13[1]});
    const half8 vhi = __builtin_bit_cast(half8, u32x4{h02[0], h13[0], h02[1], h13[1]});
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      // token order of the operand: (tau0: 0,2,1,3), (tau1: 0,2,1,3); the scale of token e, group
      // j is fp16 half (j & 1) of word (e * NG + j) / 2
      uint32_t hw[4], lw[4];
#pragma unroll
      for (int tau = 0; tau < 2; ++tau) {
        const uint32_t* vs = raw[tau].vs;
        if (j & 1) {  // resolved at compile time once the group loop is unrolled
          mix_hi_lo<1>(pexp[nb][tau][0], vs[(0 * NG + j) / 2], pexp[nb][tau][2], vs[(2 * NG + j) / 2],
                       hw[2 * tau], lw[2 * tau]);
          mix_hi_lo<1>(pexp[nb][tau][1], vs[(1 * NG + j) / 2], pexp[nb][tau][3], vs[(3 * NG + j) / 2],
                       hw[2 * tau + 1], lw[2 * tau + 1]);
        } else {
          mix_hi_lo<0>(pexp[nb][tau][0], vs[(0 * NG + j) / 2], pexp[nb][tau][2], vs[(2 * NG + j) / 2],
                       hw[2 * tau], lw[2 * tau]);
          mix_hi_lo<0>(pexp[nb][tau][1], vs[(1 * NG + j) / 2], pexp[nb][tau][3], vs[(3 * NG + j) / 2],
                       hw[2 * tau + 1], lw[2 * tau + 1]);
        }
      }
      // The halves come from inline asm, which the compiler's hazard tracking does not see, so
      // it may issue an MFMA reading them one instruction after the last write (that read stale
      // data).  This nop, ordered after every write and before every read of the eight
      // registers, gives the matrix core the two wait states a VALU result needs before an MFMA
      // reads it.  (The same values from plain fp16 code, which the compiler tracks, measured
      // slower: it builds the upper-half products with two more instructions.)
      asm("s_nop 1" : "+v"(hw[0]), "+v"(hw[1]), "+v"(hw[2]), "+v"(hw[3]), "+v"(lw[0]), "+v"(lw[1]),
          "+v"(lw[2]), "+v"(lw[3]));
      const half8 phi = __builtin_bit_cast(half8, u32x4{hw[0], hw[1], hw[2], hw[3]});
      const half8 plo = __builtin_bit_cast(half8, u32x4{lw[0], lw[1], lw[2], lw[3]});
      acc[nb][2 * j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(vlo, phi, acc[nb][2 * j], 0, 0, 0);
      acc[nb][2 * j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(vlo, plo, acc[nb][2 * j], 0, 0, 0);
      acc[nb][2 * j + 1] = __builtin_amdgcn_mfma_f32_16x16x32_f16(vhi, phi, acc[nb][2 * j + 1], 0, 0, 0);
      acc[nb][2 * j + 1] = __builtin_amdgcn_mfma_f32_16x16x32_f16(vhi, plo, acc[nb][2 * j + 1], 0, 0, 0);
    }
  }
}

// One workgroup (4 waves) per (unit, split); wave w takes the split's blocks w, w+4, w+8, ...
// Each wave streams its blocks through NSTAGE LDS stage buffers with direct-to-LDS loads, so
// NSTAGE - 1 blocks are in flight while it computes one.  The waves merge through LDS into one
// partial (the output itself when the context is a single piece).  WIN: a sliding window (the
// pieces start at the first row's window start; pages may be a ring).
template <int D, int NB, int VB, bool WIN, bool F8>
__global__ __launch_bounds__(256) void decode_kernel(DecodeArgs a) {
  constexpr int DB = D / 16;
  constexpr int ROWS = 16 * NB;
  constexpr int LDS_STRIDE = D + 4;  // floats; padding spreads the 16 rows over banks
  // stage buffers per wave: two at D = 256 (one block in flight while one is processed: for
  // 4-bit V codes this measured 1 us faster per 184K-token step than three, and 8-bit ones
  // leave no room for a third), three for the smaller head dims
  constexpr int NSTAGE = D == 256 ? 2 : 3;
  constexpr int BS = Stage<D, VB>::kBlockBytes;
  constexpr int NL = Stage<D, VB>::kLoads;
  constexpr int CHUNK = kWavesPerGroup * 32;  // blocks per chunk: 32 per wave, page ids in lanes
  static_assert(2 * NL <= 63, "vmcnt range");
  // After the main loop the same LDS holds the wave merge (4 waves x ROWS x LDS_STRIDE floats).
  constexpr int WAVE_MERGE_BYTES = kWavesPerGroup * ROWS * LDS_STRIDE * 4;
  constexpr int STAGE_BYTES = kWavesPerGroup * NSTAGE * BS;
  constexpr int LDS_BYTES = cmax(STAGE_BYTES, WAVE_MERGE_BYTES);
  static_assert(LDS_BYTES <= 160 * 1024 - 1024, "LDS");
  __shared__ __attribute__((aligned(16))) uint8_t s_lds[LDS_BYTES];
  typedef uint8_t StageBuf[NSTAGE][BS];
  StageBuf* s_stage = (StageBuf*)s_lds;
  __shared__ float s_m[kWavesPerGroup][ROWS];
  __shared__ float s_l[kWavesPerGroup][ROWS];

  const int lane = threadIdx.x & (kWave - 1);
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int unit = blockIdx.x / a.splits, split = blockIdx.x % a.splits;
  const int b = unit / a.num_kv_heads, h = unit % a.num_kv_heads;
  const int P = a.page_size;
  const int L = a.seq_lens[b];
  const int Lc = min(L, a.max_seq_len);  // tokens past max_seq_len are not attended
  const int nblk = (max(Lc, 0) + kBlock - 1) / kBlock;
  // first token any row sees: the first row's window start (WIN: a sliding window; without
  // one the first page ids load without waiting for the sequence length)
  const int t_lo = WIN ? max(L - a.n_rows - a.window + 1, 0) : 0;
  const int g_blk0 = (t_lo >> 5) + split * a.blocks_per_split;
  const int g_blk1 = min(g_blk0 + a.blocks_per_split, nblk);
  const int m16 = lane & 15, g = lane >> 4;
  const size_t bb = block_bytes(P, D, VB);
  const size_t page_stride = (size_t)a.num_kv_heads * bb;
  const uint8_t* pool_h = a.pool + (size_t)h * bb;
  const int32_t* pt = a.page_table + (size_t)b * a.max_pages;
  const int nblk_max = (a.max_seq_len + kBlock - 1) / kBlock;
  const int lgP = a.log2_page;
  const int ring = WIN ? a.ring : 0;
  // page-table entry of logical page n (a ring reuses its entries cyclically)
  auto entry = [&](int n) { return WIN && ring > 0 ? n % ring : n; };
  int c0 = g_blk0, first = 0, n_my = 0, my_pid = 0;
  // Lane kk < 32 holds the physical page of tile 0 of this wave's kk-th block of the chunk, lane
  // 32 + kk that of tile 1.  The ids are loaded for the blocks below max_seq_len, so the load
  // does not wait for the sequence length; blocks and tiles past the context are not staged.
  auto chunk_pages = [&]() {
    const int c1 = min(c0 + CHUNK, min(g_blk0 + a.blocks_per_split, nblk_max));
    first = c0 + w;
    const int n_ids = first < c1 ? (c1 - first + kWavesPerGroup - 1) / kWavesPerGroup : 0;
    const int kk = lane & 31;
    const int blk = first + kWavesPerGroup * kk;
    int tok0 = blk * kBlock + kTile * (lane >> 5);
    if (tok0 >= a.max_seq_len) tok0 = blk * kBlock;
    my_pid = pt[kk < n_ids ? entry(tok0 >> lgP) : 0];  // every lane loads (entry 0 always exists)
  };
  chunk_pages();  // the first chunk's ids load alongside the sequence length and the queries


  // ---- raw query words: lane holds query row 16*nb + m16 and the 16 dims 16*(4*jj + g) .. +15
  // of each 64-dim step jj (the B-operand layout of QK^T) ----
  u32x4 qw[NB][D / 64][2];
  int last_tok[NB], first_tok[NB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    const int n = 16 * nb + m16;
    const bool real = n < a.rows;
    const int i = real ? n / a.group : 0;
    const int hq = h * a.group + (real ? n % a.group : 0);
    last_tok[nb] = min(real ? L - a.n_rows + i : L - 1, Lc - 1);  // padding rows: q = 0
    first_tok[nb] = WIN ? (real ? L - a.n_rows + i : L - 1) - a.window + 1 : 0;
    const uint16_t* qrow = a.q + (((size_t)b * a.n_rows + i) * a.n_q_heads + hq) * D;
#pragma unroll
    for (int jj = 0; jj < D / 64; ++jj)
#pragma unroll
      for (int hf = 0; hf < 2; ++hf)
        qw[nb][jj][hf] = real ? *(const u32x4*)(qrow + 16 * (4 * jj + g) + 8 * hf) : u32x4{0, 0, 0, 0};
  }
  // first token that some row may mask (causal MTP rows, the ragged end, max_seq_len), and the
  // token below which some row may mask (the last row's window start)
  const int mask_from = min(L - a.n_rows + 1, Lc);
  const int mask_below = WIN ? L - a.window : 0;

  // ---- chunks of the split: page ids in lanes, blocks staged through the LDS buffers ----
  // LDS byte address of this wave's stage buffers (wave-uniform, computed once)
  const uint32_t my_stage_lds =
      __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(lds_void*)&s_stage[w][0][0]);
  const uint8_t* my_stage = &s_stage[w][0][0];
  const uint32_t lane16 = 16u * lane;
  const uint32_t page_stride32 = (uint32_t)page_stride;  // < 2^32, checked on the host
  const ScaleLane sl = scale_lane<D, VB>(P, lane);
  uint32_t st_issue = my_stage_lds;
  auto issue = [&](int k, uint32_t dst) {
#pragma unroll
    for (int tau = 0; tau < 2; ++tau) {
      const int blk = first + kWavesPerGroup * k;
      int tok0 = blk * kBlock + kTile * tau;
      const bool past = tok0 >= Lc;  // a tile past the end stages tile 0 again, all of it masked
      if (past) tok0 = blk * kBlock;
      const int phys = __builtin_amdgcn_readlane(my_pid, (tau == 1 && !past) ? 32 + k : k);
      stage_tile<D, VB>(pool_h + (uint64_t)(uint32_t)phys * page_stride32, P, tok0 & (P - 1),
                    dst + (uint32_t)(tau * Stage<D, VB>::kTileBytes), lane16, sl);
    }
  };
  // stage buffer of block k: k % NSTAGE, tracked incrementally
  auto next_stage = [&](uint32_t x) { return x == my_stage_lds + (NSTAGE - 1) * BS ? my_stage_lds : x + BS; };
  // chunk set-up: this wave's page ids into lanes, then the loads of its first NSTAGE - 1 blocks
  auto chunk_count = [&]() {
    const int c1 = min(c0 + CHUNK, g_blk1);
    n_my = first < c1 ? (c1 - first + kWavesPerGroup - 1) / kWavesPerGroup : 0;
    my_pid = min(max(my_pid, 0), a.num_pages - 1);  // out-of-range ids are clamped, never followed
  };
  auto chunk_start = [&]() {
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // page ids in; the DMA counting starts here
    st_issue = my_stage_lds;
#pragma unroll
    for (int i = 0; i < NSTAGE - 1; ++i) {
      if (n_my > i) issue(i, st_issue);
      st_issue = next_stage(st_issue);
    }
  };
  // The first chunk's first blocks are in flight while the queries are prepared (an empty split
  // gets n_my = 0).  The query words are used here on every path, so the compiler's own wait for
  // them (loaded with the page ids, one round trip for both) sits here and not after the DMAs.
  // Fused append: the wave that will stage the block of a new token quantizes the token's K/V
  // rows (this KV head) into its slot first; chunk_start's wait covers the stores, so the
  // block's loads see them.
  for (int j = 0; j < a.n_new; ++j) {
    const int t = L - a.n_new + j;
    const int blk = t >> 5;
    if (t < 0 || blk < g_blk0 || blk >= g_blk1 || ((blk - g_blk0) & (kWavesPerGroup - 1)) != w) continue;
    const int page = min(max(pt[entry(t >> lgP)], 0), a.num_pages - 1);
    const size_t row = (((size_t)b * a.n_new + j) * a.num_kv_heads + h) * D;
    append_row<D, VB, F8>(a.pool_rw + ((size_t)page * a.num_kv_heads + h) * bb, P, t & (P - 1), a.k_new + row,
                  a.v_new + row, lane);
  }
  chunk_count();
  asm volatile("" ::"v"(my_pid));
#pragma unroll
  for (int nb = 0; nb < NB; ++nb)
#pragma unroll
    for (int jj = 0; jj < D / 64; ++jj) asm volatile("" ::"v"(qw[nb][jj][0]), "v"(qw[nb][jj][1]));
  chunk_start();

  // ---- Q^T as three int8 digit planes (B of QK^T).  Per row, q * 2^F = h*2^16 + m*2^8 + l with
  // balanced digits in [-128, 127] and |q * 2^F| < 2^22 for the row's largest |q|; exact for every
  // element within 2^12 of it, the rest rounded to the 2^-F grid. ----
  i32x4 qd[NB][3][D / 64];
  float cz[NB];  // 2^-F * softmax_scale * log2(e); E4M3 keys: softmax_scale * log2(e)
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    if constexpr (F8) {  // the fp16 query words are the B operands as they are
      cz[nb] = a.scale_log2;
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
    cz[nb] = __builtin_ldexpf(a.scale_log2, -F);
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

  floatx4 acc[NB][DB];
  float base[NB], l_run[NB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
#pragma unroll
    for (int db = 0; db < DB; ++db) acc[nb][db] = floatx4{0.f, 0.f, 0.f, 0.f};
    base[nb] = kNegInf;
    l_run[nb] = 0.0f;
  }

  while (c0 < g_blk1) {
    int st_read = 0;
    for (int k = 0; k < n_my; ++k) {
      if constexpr (NSTAGE == 3) {
        if (k + 2 < n_my) {
          asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // reads of the buffer being refilled are done
          issue(k + 2, st_issue);
          st_issue = next_stage(st_issue);
          wait_vmcnt<2 * NL>();
        } else if (k + 1 < n_my) {
          wait_vmcnt<NL>();
        } else {
          wait_vmcnt<0>();
        }
      } else {
        if (k + 1 < n_my) {
          asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // reads of the buffer being refilled are done
          issue(k + 1, st_issue);
          st_issue = next_stage(st_issue);
          wait_vmcnt<NL>();
        } else {
          wait_vmcnt<0>();
        }
      }
      const uint8_t* src = my_stage + st_read * BS;
      st_read = st_read == NSTAGE - 1 ? 0 : st_read + 1;
      const int blk = first + kWavesPerGroup * k;
      const bool masked = blk * kBlock + kBlock - 1 >= mask_from || (WIN && blk * kBlock < mask_below);
      if (masked && lane < kBlock) {
        // a slot no row sees (past the context, or before every window) may hold junk scale
        // bits, and 0 * Inf is no zero: clear the V scales of those slots in the staged copy
        // (the same wave reads them below, in order)
        if (blk * kBlock + lane >= Lc || (WIN && blk * kBlock + lane < t_lo)) {
          uint8_t* vs = (uint8_t*)src + (lane >> 4) * Stage<D, VB>::kTileBytes + Stage<D, VB>::kVs + (lane & 15) * (D / 16);
          if constexpr (D == 256) *(u32x4*)vs = u32x4{0, 0, 0, 0};
          else if constexpr (D == 128) *(u32x2*)vs = u32x2{0, 0};
          else *(uint32_t*)vs = 0u;
        }
      }
      TileRaw<D, VB> raw[2];
      read_tile<D, VB>(raw[0], src, lane);
      read_tile<D, VB>(raw[1], src + Stage<D, VB>::kTileBytes, lane);
      // binary exponent of the block's largest V scale (positive fp16: bit order is value order);
      // every scale is below 2^(e5 - 14)
      float e5;
      {
        const uint32_t* vsw = (const uint32_t*)(src + Stage<D, VB>::kVs) + (lane & (D / 4 - 1));
        const uint32_t m = wave_max_u16x2(__builtin_bit_cast(uint32_t, __builtin_elementwise_max(
            __builtin_bit_cast(u16x2, vsw[0]), __builtin_bit_cast(u16x2, vsw[Stage<D, VB>::kTileBytes / 4]))));
        e5 = (float)((m >> 10) & 31);
      }
      process_block<D, NB, VB, WIN, F8>(raw, blk, masked, e5, qd, qw, cz, first_tok, last_tok, g, acc, base,
                                        l_run);
    }
    c0 += CHUNK;
    if (c0 < g_blk1) {
      chunk_pages();
      chunk_count();
      chunk_start();
    }
  }
  __syncthreads();  // every wave is done with its stage buffers (reused below for the merge)

  // ---- merge the 4 waves through LDS: every wave parks its state, then all 256 threads
  // combine the four copies of each (row, 4 dims): the output itself when the context is one
  // split, else this workgroup's partial for the merge kernel ----
  constexpr int NQ = D / 4;  // float4 columns of a row
  float* s_accw = (float*)s_lds;  // [wave][ROWS][LDS_STRIDE]
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    const float l = sum_over_rows(l_run[nb]);
    if (g == 0) {
      s_m[w][16 * nb + m16] = base[nb];
      s_l[w][16 * nb + m16] = l;
    }
#pragma unroll
    for (int db = 0; db < DB; ++db)
      *(floatx4*)(s_accw + (w * ROWS + 16 * nb + m16) * LDS_STRIDE + 16 * db + 4 * g) = acc[nb][db];
  }
  __syncthreads();
  const size_t prow0 = ((size_t)unit * a.splits + split) * a.rows;
  for (int it = threadIdx.x; it < a.rows * NQ; it += kWave * kWavesPerGroup) {
    const int n = it / NQ, q = it % NQ;
    float mw[kWavesPerGroup];
    float mm = kNegInf;
#pragma unroll
    for (int v = 0; v < kWavesPerGroup; ++v) {
      mw[v] = s_m[v][n];
      mm = fmaxf(mm, mw[v]);
    }
    const float m_use = (mm == kNegInf) ? 0.0f : mm;
    floatx4 t = {0.f, 0.f, 0.f, 0.f};
    float lt = 0.0f;
#pragma unroll
    for (int v = 0; v < kWavesPerGroup; ++v) {
      const float f = __builtin_amdgcn_exp2f(mw[v] - m_use);  // 0 for a wave that saw nothing
      t += f * *(const floatx4*)(s_accw + (v * ROWS + n) * LDS_STRIDE + 4 * q);
      lt += f * s_l[v][n];
    }
    if (a.splits == 1) {
      const int i = n / a.group, hq = h * a.group + n % a.group;
      const size_t o = ((size_t)b * a.n_rows + i) * a.n_q_heads + hq;
      *(floatx4*)(a.out + o * D + 4 * q) = t * (lt > 0.0f ? 1.0f / lt : 0.0f);
      if (q == 0 && a.lse) a.lse[o] = lt > 0.0f ? (mm + log2f(lt)) * 0.69314718055994530942f : kNegInf;
    } else {
      *(floatx4*)(a.ws_acc + (prow0 + n) * D + 4 * q) = t;
      if (q == 0) a.ws_ml[(size_t)unit * ml_stride(a.splits, a.rows) + split * a.rows + n] = float2{mm, lt};
    }
  }
}

// The log-sum-exp merge of the splits.  One wave per 64 (unit, query row, 4 dims) items: each
// lane takes one item over every split, with an online max, so the merge needs no LDS and no
// barrier and all of a lane's loads of a batch are in flight at once.  The partials come from
// the previous launch on the stream.
template <int D>
__global__ __launch_bounds__(64) void merge_kernel(DecodeArgs a) {
  constexpr int NQ = D / 4;
  constexpr int U = 32;  // splits per batch
  const int S = a.splits, R = a.rows;
  const int items = R * NQ;
  const int per_unit = (items + kWave - 1) / kWave;
  const int unit = blockIdx.x / per_unit;
  const int it = (blockIdx.x % per_unit) * kWave + (int)threadIdx.x;
  if (it >= items) return;
  const int n = it / NQ, q = it % NQ;
  const int b = unit / a.num_kv_heads, h = unit % a.num_kv_heads;
  const float2* ml = a.ws_ml + (size_t)unit * ml_stride(S, R) + n;
  const float* part = a.ws_acc + ((size_t)unit * S * R + n) * D + 4 * q;
  float mx = kNegInf, den = 0.0f;
  floatx4 num = {0.f, 0.f, 0.f, 0.f};
  for (int s0 = 0; s0 < S; s0 += U) {
    float2 mv[U];
    floatx4 v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {  // indices clamped into range: all loads issued at once
      const int sp = min(s0 + u, S - 1);
      mv[u] = ml[(size_t)sp * R];
      v[u] = *(const floatx4*)(part + (size_t)sp * R * D);
    }
    // the batch's largest max; the running sums move to it (once per batch, exactly)
    float bm = kNegInf;
#pragma unroll
    for (int u = 0; u < U; ++u) bm = s0 + u < S ? fmaxf(bm, mv[u].x) : bm;
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
      const float wgt = s0 + u < S ? __builtin_amdgcn_exp2f(mv[u].x - m_use) : 0.0f;
      num += wgt * v[u];
      den += wgt * mv[u].y;
    }
  }
  const int i = n / a.group, hq = h * a.group + n % a.group;
  const size_t o = ((size_t)b * a.n_rows + i) * a.n_q_heads + hq;
  *(floatx4*)(a.out + o * D + 4 * q) = num * (den > 0.0f ? 1.0f / den : 0.0f);
  if (q == 0 && a.lse) a.lse[o] = den > 0.0f ? (mx + log2f(den)) * 0.69314718055994530942f : kNegInf;
}

template <int D, bool WIN, int VB, bool F8>
void launch_attn_f(const DecodeArgs& a, dim3 grid, dim3 block, hipStream_t stream) {
  if (a.rows <= 16)
    hipLaunchKernelGGL((decode_kernel<D, 1, VB, WIN, F8>), grid, block, 0, stream, a);
  else
    hipLaunchKernelGGL((decode_kernel<D, 2, VB, WIN, F8>), grid, block, 0, stream, a);
}

template <int D, bool WIN>
void launch_attn(const DecodeArgs& a, dim3 grid, dim3 block, hipStream_t stream) {
  if (a.fp8)
    launch_attn_f<D, WIN, 8, true>(a, grid, block, stream);
  else if (a.vbits == 8)
    launch_attn_f<D, WIN, 8, false>(a, grid, block, stream);
  else
    launch_attn_f<D, WIN, 4, false>(a, grid, block, stream);
}

template <int D>
hipError_t launch_decode_d(const DecodeArgs& a, hipStream_t stream) {
  const unsigned units = (unsigned)((long long)a.n_seq * a.num_kv_heads);
  const unsigned grid = units * (unsigned)a.splits;
  const dim3 block(kWave * kWavesPerGroup);
  if (a.window > 0)
    launch_attn<D, true>(a, dim3(grid), block, stream);
  else
    launch_attn<D, false>(a, dim3(grid), block, stream);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || a.splits == 1) return e;
  const unsigned per_unit = (unsigned)((a.rows * (D / 4) + kWave - 1) / kWave);
  hipLaunchKernelGGL((merge_kernel<D>), dim3(units * per_unit), dim3(kWave), 0, stream, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_decode(int head_dim, const DecodeArgs& a, hipStream_t stream) {
  switch (head_dim) {
    case 64: return launch_decode_d<64>(a, stream);
    case 128: return launch_decode_d<128>(a, stream);
    case 256: return launch_decode_d<256>(a, stream);
  }
  return hipErrorInvalidValue;
}

}  // namespace kvq

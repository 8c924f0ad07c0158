// kvq_decode.hip — split-KV decode attention over the paged K8/V4 cache, and the merge of the
// splits by log-sum-exp.
//
// The pages describe a decode kernel tuned for one long request over a KV cache handled in
// pieces of the context, loading only the current piece on chip (blog page "標籤: vLLM",
// 重點說明 part 2), and decode whose speed is bound by the bytes read per token (forum post
// "3090 单卡跑 Qwen3.8-27B：NInfer 上机实测（180K 上下文 / C2 并发 / 4bit KV）", 二、测评 and the
// replies on 4-bit vs fp16 KV).  The split-KV scheme here is this library's MI355X design:
//
//   * one 64-lane wave owns one split (a run of 32-token blocks) of one (sequence, KV head);
//     the grid has units * splits waves so that a single long sequence fills the 256 CUs;
//   * K codes arrive with one 16-byte load per lane in exactly the layout of the A operand of
//     v_mfma_f32_16x16x32_f16 (tokens on M, dims on K), Q^T is the B operand (query rows of
//     the GQA group x MTP rows on N), so QK^T is 8 MFMAs per 16 tokens for D = 256;
//   * the 16x16 logit tile comes out with each lane holding one query row and four tokens,
//     which is the B-operand layout of the PV product (tokens on K), so P never leaves the
//     registers; V codes arrive pre-arranged as the A operand (dims on M, tokens on K);
//   * int8 and int4 codes are widened to fp16 with exact integer bit tricks; the V scale
//     (per token and 32 dims) is folded into P, split into an fp16 high and low part so the
//     PV product keeps fp32 accuracy;
//   * online softmax in log2 units with wave shuffles for the row max, one partial
//     (acc, max, sum) per split in the workspace, then a second kernel merges them.
#include "kvq_internal.h"

namespace kvq {
namespace {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef _Float16 half2v __attribute__((ext_vector_type(2)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr float kNegInf = -__builtin_inff();

__device__ inline half2v as_h2(uint32_t u) { return __builtin_bit_cast(half2v, u); }
__device__ inline uint32_t as_u32(half2v h) { return __builtin_bit_cast(uint32_t, h); }

// Four int8 codes (bytes b0..b3 of x) -> fp16 pairs (c0, c2) and (c1, c3), exact:
// 0x6400 | u is the fp16 value 1024 + u for u < 1024, and u = c + 128 after flipping the sign bit.
__device__ inline void i8x4_to_h2x2(uint32_t x, uint32_t& c02, uint32_t& c13) {
  const uint32_t u = x ^ 0x80808080u;
  const half2v off = {(_Float16)1152.0f, (_Float16)1152.0f};
  c02 = as_u32(as_h2((u & 0x00FF00FFu) | 0x64006400u) - off);
  c13 = as_u32(as_h2(((u >> 8) & 0x00FF00FFu) | 0x64006400u) - off);
}

// 16 int8 codes of one token (one 16-byte load) -> the two 8-wide MFMA operands.  Element order
// within each operand is dims [0,2,1,3,4,6,5,7] (+8 for the second); Q is permuted to match.
__device__ inline void k_operands(const u32x4 raw, half8& lo, half8& hi) {
  uint32_t a0, a1, b0, b1, c0, c1, d0, d1;
  i8x4_to_h2x2(raw[0], a0, a1);
  i8x4_to_h2x2(raw[1], b0, b1);
  i8x4_to_h2x2(raw[2], c0, c1);
  i8x4_to_h2x2(raw[3], d0, d1);
  lo = __builtin_bit_cast(half8, u32x4{a0, a1, b0, b1});
  hi = __builtin_bit_cast(half8, u32x4{c0, c1, d0, d1});
}

// One V dword holds, for four tokens r = 0..3 (byte r), the codes of two dims (low nibble: a
// dim of the even 16-dim block, high nibble: the same dim of the odd block), 4-bit two's
// complement.  Returns fp16 pairs (token 0, token 2) and (token 1, token 3) for both dims.
__device__ inline void i4x8_to_h2x4(uint32_t x, uint32_t& lo02, uint32_t& lo13, uint32_t& hi02,
                                    uint32_t& hi13) {
  const uint32_t u = x ^ 0x88888888u;  // nibble n' = code + 8 in [0, 15]
  const uint32_t u8 = u >> 8;
  const half2v off_lo = {(_Float16)1032.0f, (_Float16)1032.0f};
  const half2v sixteenth = {(_Float16)0.0625f, (_Float16)0.0625f};
  const half2v off_hi = {(_Float16)72.0f, (_Float16)72.0f};
  lo02 = as_u32(as_h2((u & 0x000F000Fu) | 0x64006400u) - off_lo);           // 1024 + n' - 1032
  lo13 = as_u32(as_h2((u8 & 0x000F000Fu) | 0x64006400u) - off_lo);
  hi02 = as_u32(as_h2((u & 0x00F000F0u) | 0x64006400u) * sixteenth - off_hi);  // (1024+16n')/16 - 72
  hi13 = as_u32(as_h2((u8 & 0x00F000F0u) | 0x64006400u) * sixteenth - off_hi);
}

// Two fp32 values as fp16 pairs hi + lo with hi + lo = x to about 2^-21 relative.  hi comes from
// one truncating conversion whose bits feed both the operand and the residual; with an ordinary
// (half) cast the compiler may compute hi twice in different ways (e.g. once as a fused
// multiply-convert from the exact product, once from the rounded fp32 product), and near an fp16
// rounding boundary the two differ by an ulp, which the residual then no longer corrects.
__device__ inline void split_hi_lo(float x0, float x1, uint32_t& hi, uint32_t& lo) {
  const auto h = __builtin_amdgcn_cvt_pkrtz(x0, x1);
  hi = __builtin_bit_cast(uint32_t, h);
  const float r0 = x0 - (float)h[0];
  const float r1 = x1 - (float)h[1];
  lo = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(r0, r1));
}

__device__ inline float h_at(const uint32_t* words, int idx) {
  const uint32_t w = words[idx >> 1];
  return (float)__builtin_bit_cast(_Float16, (uint16_t)((idx & 1) ? (w >> 16) : (w & 0xFFFF)));
}

template <int D>
struct TileRaw {
  static constexpr int kLoadsK = D / 64;                    // 16-byte loads of K codes per lane
  static constexpr int kVWords = D / 32;                    // V code dwords per lane
  static constexpr int kVsWords = D / 16;                   // V scale dwords per lane (4 tokens x D/32)
  u32x4 k[kLoadsK];
  uint32_t v[kVWords];
  uint32_t vs[kVsWords];
  uint32_t ks[2];                                           // K scales of tokens 4g..4g+3
};

// ---- staging of one block (two tiles) in LDS --------------------------------------------
// A staged tile is an exact copy of the tile's four sections, packed:
//   [K codes 16*D][V codes 8*D][V scales D][K scales 32]  = 25*D + 32 bytes.
template <int D>
struct Stage {
  static constexpr int kK = 0;
  static constexpr int kV = 16 * D;
  static constexpr int kVs = 24 * D;
  static constexpr int kKs = 25 * D;
  static constexpr int kTileBytes = 25 * D + 32;
  static constexpr int kBlockBytes = 2 * kTileBytes;
  // direct-to-LDS loads per block (vmcnt units)
  static constexpr int kLoads = 2 * (D / 64 + (D >= 128 ? D / 128 : 1) + 2);
};

typedef __attribute__((address_space(3))) void lds_void;

// M0 is named as clobbered below: these kernels set it themselves before each direct-to-LDS
// load and use it for nothing else, so the compiler's warning about reserved registers is moot.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ inline void dma16(const uint8_t* src, uint8_t* lds_dst) {
  // 16 bytes per active lane from src to lds_dst + 16 * lane_id (gfx950 global_load_lds_dwordx4).
  // Issued as inline asm: the waits for these loads are this file's explicit s_waitcnt vmcnt,
  // which keep two blocks in flight (the compiler would otherwise drain every load before each
  // LDS read).  The "memory" clobber keeps LDS reads of the buffer on their side of it.
  const uint32_t lds = (uint32_t)(uintptr_t)(lds_void*)lds_dst;
  asm volatile(
      "s_mov_b32 m0, %1\n\t"
      "global_load_lds_dwordx4 %0, off"
      :
      : "v"(src), "s"(__builtin_amdgcn_readfirstlane(lds))
      : "memory", "m0");
}
#pragma clang diagnostic pop

template <int N>
__device__ inline void wait_vmcnt() {
  // loads complete in order: at most N of this wave's loads may still be in flight
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// Issue the loads of one tile (slot0 = first slot of the tile in its page) into LDS.
template <int D>
__device__ inline void stage_tile(const uint8_t* base, int P, int slot0, uint8_t* dst, int lane) {
  const int tip = slot0 / kTile;
#pragma unroll
  for (int jj = 0; jj < D / 64; ++jj)
    dma16(base + (size_t)16 * D * tip + 1024 * jj + 16 * lane, dst + Stage<D>::kK + 1024 * jj);
  const uint8_t* vb = base + v_codes_at(P, D) + (size_t)8 * D * tip;
  if constexpr (D >= 128) {
#pragma unroll
    for (int c = 0; c < D / 128; ++c) dma16(vb + 1024 * c + 16 * lane, dst + Stage<D>::kV + 1024 * c);
  } else {
    if (lane < 32) dma16(vb + 16 * lane, dst + Stage<D>::kV);
  }
  if (lane < D / 16)
    dma16(base + v_scales_at(P, D) + (size_t)2 * slot0 * (D / 32) + 16 * lane, dst + Stage<D>::kVs);
  if (lane < 2) dma16(base + k_scales_at(P, D) + 2 * slot0 + 16 * lane, dst + Stage<D>::kKs);
}

// Read one staged tile into this lane's registers (the lane's share of every section).
template <int D>
__device__ inline void read_tile(TileRaw<D>& r, const uint8_t* src, int lane) {
  const int g = lane >> 4;
#pragma unroll
  for (int jj = 0; jj < TileRaw<D>::kLoadsK; ++jj)
    r.k[jj] = *(const u32x4*)(src + Stage<D>::kK + 1024 * jj + 16 * lane);
  const u32x2 ks = *(const u32x2*)(src + Stage<D>::kKs + 8 * g);
  r.ks[0] = ks[0];
  r.ks[1] = ks[1];
  if constexpr (D == 64) {
    const u32x2 w = *(const u32x2*)(src + Stage<D>::kV + 8 * lane);
    r.v[0] = w[0];
    r.v[1] = w[1];
  } else {
#pragma unroll
    for (int c = 0; c < D / 128; ++c) {
      const u32x4 w = *(const u32x4*)(src + Stage<D>::kV + 1024 * c + 16 * lane);
#pragma unroll
      for (int e = 0; e < 4; ++e) r.v[4 * c + e] = w[e];
    }
  }
#pragma unroll
  for (int c = 0; c < TileRaw<D>::kVsWords / 4; ++c) {
    const u32x4 w = *(const u32x4*)(src + Stage<D>::kVs + g * (D / 4) + 16 * c);
#pragma unroll
    for (int e = 0; e < 4; ++e) r.vs[4 * c + e] = w[e];
  }
}

// One 32-token block of one wave: S^T = K Q^T, online softmax, O^T += V^T P^T.
// Running state of one wave, per query row (lane's row in each 16-row block nb):
//   m_run  the largest logit seen (log2 units), -inf before any unmasked token;
//   base   the exponent offset of l_run and acc: they hold sums of 2^(z - base) * (...);
//   base = m_run - k, where 2^k is a per-block power of two that keeps p * v_scale near the top of
//   the fp16 range, so the fp16 high and low parts of P both stay normal numbers.
template <int D, int NB, bool MASK>
__device__ __attribute__((always_inline)) inline void process_block(
    const TileRaw<D> (&raw)[2], int blk, const half8 (&qop)[NB][D / 32], const int (&last_tok)[NB],
    float scale_log2, int g, floatx4 (&acc)[NB][D / 16], float (&m_run)[NB], float (&base)[NB],
    float (&l_run)[NB]) {
  constexpr int DB = D / 16;
  constexpr int NG = D / 32;
  // ---- logits: lane gets row (16nb + m16) and tokens 4g..4g+3 of each tile ----
  floatx4 s[2][NB];
#pragma unroll
  for (int tau = 0; tau < 2; ++tau) {
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) s[tau][nb] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int jj = 0; jj < D / 64; ++jj) {
      half8 klo, khi;
      k_operands(raw[tau].k[jj], klo, khi);
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        s[tau][nb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(klo, qop[nb][2 * jj], s[tau][nb], 0, 0, 0);
        s[tau][nb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(khi, qop[nb][2 * jj + 1], s[tau][nb], 0, 0, 0);
      }
    }
  }
  float ks[2][4];
#pragma unroll
  for (int tau = 0; tau < 2; ++tau)
#pragma unroll
    for (int e = 0; e < 4; ++e) ks[tau][e] = h_at(raw[tau].ks, e) * scale_log2;

  // ---- exponent of the block's largest V scale: k = 29 - e5 keeps p' * scale < 2^15 ----
  typedef uint16_t u16x2 __attribute__((ext_vector_type(2)));
  u16x2 vmax = {0, 0};
#pragma unroll
  for (int tau = 0; tau < 2; ++tau)
#pragma unroll
    for (int c = 0; c < TileRaw<D>::kVsWords; ++c)
      vmax = __builtin_elementwise_max(vmax, __builtin_bit_cast(u16x2, raw[tau].vs[c]));
  int smax = max((int)vmax[0], (int)vmax[1]);  // positive fp16: bit order is value order
  smax = max(smax, __shfl_xor(smax, 16, kWave));
  smax = max(smax, __shfl_xor(smax, 32, kWave));
  const float kshift = (float)(29 - ((smax >> 10) & 31));

  // ---- online softmax in log2 units ----
  float pexp[NB][2][4];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    float z[2][4];
    float bm = kNegInf;
#pragma unroll
    for (int tau = 0; tau < 2; ++tau)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        float zz = s[tau][nb][e] * ks[tau][e];
        if (MASK) {
          const int t = blk * kBlock + kTile * tau + 4 * g + e;
          zz = (t <= last_tok[nb]) ? zz : kNegInf;
        }
        z[tau][e] = zz;
        bm = fmaxf(bm, zz);
      }
    bm = fmaxf(bm, __shfl_xor(bm, 16, kWave));
    bm = fmaxf(bm, __shfl_xor(bm, 32, kWave));
    const float m_new = fmaxf(m_run[nb], bm);
    // empty so far: keep the state at zero (alpha = 0 scales nothing, every p is 0)
    const float b_new = (m_new == kNegInf) ? 0.0f : m_new - kshift;
    const float alpha = __builtin_amdgcn_exp2f(base[nb] - b_new);
    m_run[nb] = m_new;
    base[nb] = (m_new == kNegInf) ? kNegInf : b_new;
    float lsum = 0.0f;
#pragma unroll
    for (int tau = 0; tau < 2; ++tau)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        pexp[nb][tau][e] = __builtin_amdgcn_exp2f(z[tau][e] - b_new);
        lsum += pexp[nb][tau][e];
      }
    l_run[nb] = l_run[nb] * alpha + lsum;
#pragma unroll
    for (int db = 0; db < DB; ++db) acc[nb][db] *= alpha;
  }

  // ---- O^T += V^T P^T, one 32-dim scale group at a time ----
#pragma unroll
  for (int j = 0; j < NG; ++j) {
    uint32_t l02[2], l13[2], h02[2], h13[2];
#pragma unroll
    for (int tau = 0; tau < 2; ++tau) i4x8_to_h2x4(raw[tau].v[j], l02[tau], l13[tau], h02[tau], h13[tau]);
    const half8 vlo = __builtin_bit_cast(half8, u32x4{l02[0], l13[0], l02[1], l13[1]});
    const half8 vhi = __builtin_bit_cast(half8, u32x4{h02[0], h13[0], h02[1], h13[1]});
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      // token order of the operand: (tau0: 0,2,1,3), (tau1: 0,2,1,3)
      float px[2][4];
#pragma unroll
      for (int tau = 0; tau < 2; ++tau)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          px[tau][e] = pexp[nb][tau][e] * h_at(raw[tau].vs, e * NG + j);
          if (MASK) px[tau][e] = (pexp[nb][tau][e] == 0.0f) ? 0.0f : px[tau][e];  // junk scale of a masked slot
        }
      uint32_t hw[4], lw[4];
#pragma unroll
      for (int tau = 0; tau < 2; ++tau) {
        split_hi_lo(px[tau][0], px[tau][2], hw[2 * tau], lw[2 * tau]);
        split_hi_lo(px[tau][1], px[tau][3], hw[2 * tau + 1], lw[2 * tau + 1]);
      }
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
// Each wave streams its blocks through three LDS stage buffers with direct-to-LDS loads, so two
// blocks are in flight while it computes the third.  The waves merge through LDS into one
// partial; the last workgroup of a unit to finish merges the unit's partials into the output.
template <int D, int NB>
__global__ __launch_bounds__(256) void decode_kernel(DecodeArgs a) {
  constexpr int KK = D / 32;
  constexpr int DB = D / 16;
  constexpr int ROWS = 16 * NB;
  constexpr int LDS_STRIDE = D + 4;  // floats; padding spreads the 16 rows over banks
  constexpr int NSTAGE = 3;
  constexpr int BS = Stage<D>::kBlockBytes;
  constexpr int NL = Stage<D>::kLoads;
  constexpr int CHUNK = 128;            // blocks whose page ids sit in LDS at once
  constexpr int PT_CAP = 2 * CHUNK + 2;
  static_assert(2 * NL <= 63, "vmcnt range");
  // After the main loop the stage buffers hold the wave merge (ROWS x LDS_STRIDE floats) and then
  // the final merge: (max, sum) of kMaxSplits x ROWS, ROWS floats, PARTS x 4 rows x D floats.
  constexpr int MERGE_BYTES = kMaxSplits * ROWS * 8 + ROWS * 4 + 16 + 16 * D * (1024 / D);
  constexpr int STAGE_BYTES = kWavesPerGroup * NSTAGE * BS;
  constexpr int LDS_BYTES = STAGE_BYTES > MERGE_BYTES ? STAGE_BYTES : MERGE_BYTES;
  static_assert(ROWS * LDS_STRIDE * 4 <= LDS_BYTES, "wave merge buffer fits");
  __shared__ __attribute__((aligned(16))) uint8_t s_lds[LDS_BYTES];
  typedef uint8_t StageBuf[NSTAGE][BS];
  StageBuf* s_stage = (StageBuf*)s_lds;
  __shared__ int s_pt[PT_CAP];
  __shared__ float s_m[kWavesPerGroup][ROWS];
  __shared__ float s_l[kWavesPerGroup][ROWS];
  __shared__ int s_last;

  const int lane = threadIdx.x & (kWave - 1);
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int unit = blockIdx.x / a.splits, split = blockIdx.x % a.splits;
  const int b = unit / a.num_kv_heads, h = unit % a.num_kv_heads;
  const int P = a.page_size;
  const int L = a.seq_lens[b];
  const int Lc = min(L, a.max_seq_len);  // tokens past max_seq_len are not attended
  const int nblk = (max(Lc, 0) + kBlock - 1) / kBlock;
  const int g_blk0 = split * a.blocks_per_split;
  const int g_blk1 = min(g_blk0 + a.blocks_per_split, nblk);
  const int m16 = lane & 15, g = lane >> 4;
  const size_t bb = block_bytes(P, D);
  const size_t page_stride = (size_t)a.num_kv_heads * bb;
  const uint8_t* pool_h = a.pool + (size_t)h * bb;
  const int32_t* pt = a.page_table + (size_t)b * a.max_pages;

  // ---- Q^T operands (B of QK^T): lane holds query row 16*nb + m16, dims of lane group g ----
  half8 qop[NB][KK];
  int last_tok[NB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    const int n = 16 * nb + m16;
    const bool real = n < a.rows;
    const int i = real ? n / a.group : 0;
    const int hq = h * a.group + (real ? n % a.group : 0);
    last_tok[nb] = min(real ? L - a.n_rows + i : L - 1, Lc - 1);  // padding rows: q = 0
    const uint16_t* qrow = a.q + (((size_t)b * a.n_rows + i) * a.n_q_heads + hq) * D;
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) {
      const int dim0 = 16 * (4 * (kk / 2) + g) + 8 * (kk % 2);
      u32x4 q8 = real ? *(const u32x4*)(qrow + dim0) : u32x4{0, 0, 0, 0};
      // dims [0..7] -> operand order [0,2,1,3,4,6,5,7]: swap halves 1<->2 and 5<->6
      const uint32_t p0 = (q8[0] & 0xFFFFu) | (q8[1] << 16);
      const uint32_t p1 = (q8[0] >> 16) | (q8[1] & 0xFFFF0000u);
      const uint32_t p2 = (q8[2] & 0xFFFFu) | (q8[3] << 16);
      const uint32_t p3 = (q8[2] >> 16) | (q8[3] & 0xFFFF0000u);
      qop[nb][kk] = __builtin_bit_cast(half8, u32x4{p0, p1, p2, p3});
    }
  }
  // first token that some row may mask (causal MTP rows, the ragged end, max_seq_len)
  const int mask_from = min(L - a.n_rows + 1, Lc);

  floatx4 acc[NB][DB];
  float m_run[NB], base[NB], l_run[NB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
#pragma unroll
    for (int db = 0; db < DB; ++db) acc[nb][db] = floatx4{0.f, 0.f, 0.f, 0.f};
    m_run[nb] = kNegInf;
    base[nb] = kNegInf;
    l_run[nb] = 0.0f;
  }

  uint8_t* my_stage = &s_stage[w][0][0];
  for (int c0 = g_blk0; c0 < g_blk1; c0 += CHUNK) {
    const int c1 = min(c0 + CHUNK, g_blk1);
    const int lp0 = (c0 * kBlock) / P;
    const int lp1 = (c1 * kBlock - 1) / P + 1;
    __syncthreads();  // the previous chunk's page ids are no longer read
    for (int e = threadIdx.x; e < lp1 - lp0; e += blockDim.x)
      s_pt[e] = min(max(pt[lp0 + e], 0), a.num_pages - 1);
    __syncthreads();

    const int first = c0 + w;
    const int n_my = first < c1 ? (c1 - first + kWavesPerGroup - 1) / kWavesPerGroup : 0;
    auto issue = [&](int k) {
      const int blk = first + kWavesPerGroup * k;
      uint8_t* dst = my_stage + (k % NSTAGE) * BS;
#pragma unroll
      for (int tau = 0; tau < 2; ++tau) {
        int tok0 = blk * kBlock + kTile * tau;
        if (tok0 >= Lc) tok0 = blk * kBlock;  // tile past the end: stage tile 0 again, all masked
        const int phys = s_pt[tok0 / P - lp0];
        stage_tile<D>(pool_h + (size_t)phys * page_stride, P, tok0 % P, dst + tau * Stage<D>::kTileBytes, lane);
      }
    };
    if (n_my > 0) issue(0);
    if (n_my > 1) issue(1);
    for (int k = 0; k < n_my; ++k) {
      if (k + 2 < n_my) {
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // reads of the buffer being refilled are done
        issue(k + 2);
      }
      const int ahead = min(n_my - 1 - k, 2);  // blocks issued after this one
      if (ahead == 2)
        wait_vmcnt<2 * NL>();
      else if (ahead == 1)
        wait_vmcnt<NL>();
      else
        wait_vmcnt<0>();
      const uint8_t* src = my_stage + (k % NSTAGE) * BS;
      TileRaw<D> raw[2];
      read_tile<D>(raw[0], src, lane);
      read_tile<D>(raw[1], src + Stage<D>::kTileBytes, lane);
      const int blk = first + kWavesPerGroup * k;
      if (blk * kBlock + kBlock - 1 >= mask_from)
        process_block<D, NB, true>(raw, blk, qop, last_tok, a.scale_log2, g, acc, m_run, base, l_run);
      else
        process_block<D, NB, false>(raw, blk, qop, last_tok, a.scale_log2, g, acc, m_run, base, l_run);
    }
  }
  __syncthreads();  // every wave is done with its stage buffers (reused below for the merge)

  // ---- merge the 4 waves through LDS ----
  float* s_acc = (float*)&s_stage[0][0][0];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    l_run[nb] += __shfl_xor(l_run[nb], 16, kWave);
    l_run[nb] += __shfl_xor(l_run[nb], 32, kWave);
    if (g == 0) {
      s_m[w][16 * nb + m16] = base[nb];
      s_l[w][16 * nb + m16] = l_run[nb];
    }
  }
  __syncthreads();
  float M[NB], l_tot[NB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    const int row = 16 * nb + m16;
    float mm = kNegInf;
#pragma unroll
    for (int v = 0; v < kWavesPerGroup; ++v) mm = fmaxf(mm, s_m[v][row]);
    const float m_use = (mm == kNegInf) ? 0.0f : mm;
    float lt = 0.0f;
#pragma unroll
    for (int v = 0; v < kWavesPerGroup; ++v) lt += s_l[v][row] * __builtin_amdgcn_exp2f(s_m[v][row] - m_use);
    M[nb] = mm;
    l_tot[nb] = lt;
    const float f = __builtin_amdgcn_exp2f(base[nb] - m_use);
#pragma unroll
    for (int db = 0; db < DB; ++db) acc[nb][db] *= f;
  }
  for (int src = 1; src < kWavesPerGroup; ++src) {
    if (w == src) {
#pragma unroll
      for (int nb = 0; nb < NB; ++nb)
#pragma unroll
        for (int db = 0; db < DB; ++db)
          *(floatx4*)(s_acc + (16 * nb + m16) * LDS_STRIDE + 16 * db + 4 * g) = acc[nb][db];
    }
    __syncthreads();
    if (w == 0) {
#pragma unroll
      for (int nb = 0; nb < NB; ++nb)
#pragma unroll
        for (int db = 0; db < DB; ++db)
          acc[nb][db] += *(const floatx4*)(s_acc + (16 * nb + m16) * LDS_STRIDE + 16 * db + 4 * g);
    }
    __syncthreads();
  }
  if (w == 0) {
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      const int n = 16 * nb + m16;
      if (n < a.rows) {
        const size_t prow = ((size_t)unit * a.splits + split) * a.rows + n;
        float* dst = a.ws_acc + prow * D + 4 * g;
#pragma unroll
        for (int db = 0; db < DB; ++db) *(floatx4*)(dst + 16 * db) = acc[nb][db];
        if (g == 0) a.ws_ml[prow] = make_float2(M[nb], l_tot[nb]);
      }
    }
  }

  // ---- the last workgroup of this unit merges every split ----
  __threadfence();  // release: this workgroup's partial is visible to all XCDs
  __syncthreads();
  if (threadIdx.x == 0) s_last = (atomicAdd(&a.ws_count[unit], 1u) == (unsigned)(a.splits - 1));
  __syncthreads();
  if (!s_last) return;
  __threadfence();  // acquire: every other workgroup's partial
  {
    // (max, sum) of every (split, row) into LDS, then per-row max M, weights 2^(m - M) and the
    // denominator; then the numerators in batches of independent loads.
    constexpr int NQ = D / 4;                  // float4 columns of a row
    constexpr int PARTS = (kWave * kWavesPerGroup) / NQ;
    const int S = a.splits, R = a.rows;
    const size_t p0 = (size_t)unit * S * R;
    float2* s_ml = (float2*)&s_stage[0][0][0];  // [S][R]
    float* s_M = (float*)(s_ml + S * R);          // [R]: 1/den
    floatx4* s_red = (floatx4*)(s_lds + ((S * R * 8 + R * 4 + 15) & ~15));  // [PARTS][4][NQ]
    for (int e = threadIdx.x; e < S * R; e += blockDim.x) s_ml[e] = a.ws_ml[p0 + e];
    __syncthreads();
    for (int n = w; n < R; n += kWavesPerGroup) {
      float mx = kNegInf;
      for (int sp = lane; sp < S; sp += kWave) mx = fmaxf(mx, s_ml[sp * R + n].x);
#pragma unroll
      for (int off = 32; off > 0; off >>= 1) mx = fmaxf(mx, __shfl_xor(mx, off, kWave));
      float den = 0.0f;
      for (int sp = lane; sp < S; sp += kWave) {
        const float2 ml = s_ml[sp * R + n];
        const float wgt = (ml.x == kNegInf) ? 0.0f : __builtin_amdgcn_exp2f(ml.x - mx);
        s_ml[sp * R + n].x = wgt;  // the weight replaces the max
        den += wgt * ml.y;
      }
#pragma unroll
      for (int off = 32; off > 0; off >>= 1) den += __shfl_xor(den, off, kWave);
      if (lane == 0) {
        s_M[n] = den > 0.0f ? 1.0f / den : 0.0f;
        if (a.lse) {
          const int i = n / a.group, hq = h * a.group + n % a.group;
          const size_t o = ((size_t)b * a.n_rows + i) * a.n_q_heads + hq;
          a.lse[o] = den > 0.0f ? (mx + log2f(den)) * 0.69314718055994530942f : kNegInf;
        }
      }
    }
    __syncthreads();
    const int q = threadIdx.x % NQ, part = threadIdx.x / NQ;
    for (int n0 = 0; n0 < R; n0 += 4) {
      floatx4 num[4] = {};
      for (int sp0 = part; sp0 < S; sp0 += 8 * PARTS) {
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          const int sp = sp0 + u * PARTS;
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int n = n0 + r;
            if (sp < S && n < R) {
              const float wgt = s_ml[sp * R + n].x;
              num[r] += wgt * *(const floatx4*)(a.ws_acc + (p0 + (size_t)sp * R + n) * D + 4 * q);
            }
          }
        }
      }
#pragma unroll
      for (int r = 0; r < 4; ++r) s_red[(part * 4 + r) * NQ + q] = num[r];
      __syncthreads();
      for (int e = threadIdx.x; e < 4 * NQ; e += blockDim.x) {
        const int r = e / NQ, qq = e % NQ, n = n0 + r;
        if (n < R) {
          floatx4 t = s_red[r * NQ + qq];
          for (int pp = 1; pp < PARTS; ++pp) t += s_red[(pp * 4 + r) * NQ + qq];
          const int i = n / a.group, hq = h * a.group + n % a.group;
          const size_t o = ((size_t)b * a.n_rows + i) * a.n_q_heads + hq;
          *(floatx4*)(a.out + o * D + 4 * qq) = t * s_M[n];
        }
      }
      __syncthreads();
    }
  }
  if (threadIdx.x == 0) atomicExch(&a.ws_count[unit], 0u);  // leave the counter zeroed
}

template <int D>
hipError_t launch_decode_d(const DecodeArgs& a, hipStream_t stream) {
  const unsigned grid = (unsigned)((long long)a.n_seq * a.num_kv_heads * a.splits);
  if (a.rows <= 16)
    hipLaunchKernelGGL((decode_kernel<D, 1>), dim3(grid), dim3(kWave * kWavesPerGroup), 0, stream, a);
  else
    hipLaunchKernelGGL((decode_kernel<D, 2>), dim3(grid), dim3(kWave * kWavesPerGroup), 0, stream, a);
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

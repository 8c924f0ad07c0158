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

template <int D>
__device__ inline void load_tile(TileRaw<D>& r, const uint8_t* base, int P, int slot0, int lane) {
  const int g = lane >> 4;
  const int tip = slot0 / kTile;
#pragma unroll
  for (int jj = 0; jj < TileRaw<D>::kLoadsK; ++jj)
    r.k[jj] = *(const u32x4*)(base + (size_t)16 * D * tip + 1024 * jj + 16 * lane);
  const u32x2 ks = *(const u32x2*)(base + k_scales_at(P, D) + 2 * (slot0 + 4 * g));
  r.ks[0] = ks[0];
  r.ks[1] = ks[1];
  const uint8_t* vb = base + v_codes_at(P, D) + (size_t)8 * D * tip;
  if constexpr (D == 64) {
    const u32x2 w = *(const u32x2*)(vb + 8 * lane);
    r.v[0] = w[0];
    r.v[1] = w[1];
  } else {
#pragma unroll
    for (int c = 0; c < D / 128; ++c) {
      const u32x4 w = *(const u32x4*)(vb + 1024 * c + 16 * lane);
#pragma unroll
      for (int e = 0; e < 4; ++e) r.v[4 * c + e] = w[e];
    }
  }
  const uint8_t* sb = base + v_scales_at(P, D) + (size_t)2 * (slot0 + 4 * g) * (D / 32);
#pragma unroll
  for (int c = 0; c < TileRaw<D>::kVsWords / 4; ++c) {
    const u32x4 w = *(const u32x4*)(sb + 16 * c);
#pragma unroll
    for (int e = 0; e < 4; ++e) r.vs[4 * c + e] = w[e];
  }
}

template <int D, int NB>
__global__ __launch_bounds__(256) void decode_split_kernel(DecodeArgs a) {
  constexpr int KK = D / 32;       // QK MFMAs per tile (K = 32 dims each)
  constexpr int DB = D / 16;       // 16-dim blocks of the output
  constexpr int NG = D / 32;       // V scale groups
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int units = a.n_seq * a.num_kv_heads;
  if (wave >= units * a.splits) return;
  const int unit = wave / a.splits, split = wave % a.splits;
  const int b = unit / a.num_kv_heads, h = unit % a.num_kv_heads;
  const int P = a.page_size;
  const int L = a.seq_lens[b];
  // tokens past max_seq_len are not attended (the grid and the page table stop there)
  const int nblk = (min(L, a.max_seq_len) + kBlock - 1) / kBlock;
  const int blk0 = split * a.blocks_per_split;
  const int blk1 = min(blk0 + a.blocks_per_split, nblk);
  const int m16 = lane & 15, g = lane >> 4;
  const size_t bb = block_bytes(P, D);
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
    last_tok[nb] = real ? L - a.n_rows + i : L - 1;  // padding rows: q = 0, never stored
    const uint16_t* qrow = a.q + (((size_t)b * a.n_rows + i) * a.n_q_heads + hq) * D;
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) {
      const int dim0 = 16 * (4 * (kk / 2) + g) + 8 * (kk % 2);
      u32x4 w = real ? *(const u32x4*)(qrow + dim0) : u32x4{0, 0, 0, 0};
      // dims [0..7] -> operand order [0,2,1,3,4,6,5,7]: swap halves 1<->2 and 5<->6
      const uint32_t p0 = (w[0] & 0xFFFFu) | (w[1] << 16);
      const uint32_t p1 = (w[0] >> 16) | (w[1] & 0xFFFF0000u);
      const uint32_t p2 = (w[2] & 0xFFFFu) | (w[3] << 16);
      const uint32_t p3 = (w[2] >> 16) | (w[3] & 0xFFFF0000u);
      qop[nb][kk] = __builtin_bit_cast(half8, u32x4{p0, p1, p2, p3});
    }
  }

  floatx4 acc[NB][DB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb)
#pragma unroll
    for (int db = 0; db < DB; ++db) acc[nb][db] = floatx4{0.f, 0.f, 0.f, 0.f};
  float m_run[NB], l_run[NB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    m_run[nb] = kNegInf;
    l_run[nb] = 0.0f;
  }

  for (int blk = blk0; blk < blk1; ++blk) {
    TileRaw<D> raw[2];
#pragma unroll
    for (int tau = 0; tau < 2; ++tau) {
      int tok0 = blk * kBlock + kTile * tau;
      if (tok0 >= min(L, a.max_seq_len)) tok0 = blk * kBlock;  // tile past the end: read tile 0 again, all masked
      int phys = pt[tok0 / P];
      phys = min(max(phys, 0), a.num_pages - 1);
      load_tile<D>(raw[tau], pool_h + (size_t)phys * a.num_kv_heads * bb, P, tok0 % P, lane);
    }

    // ---- S^T = K Q^T per tile: lane gets row (16nb + m16), tokens 4g..4g+3 ----
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

    // ---- online softmax (log2 units) ----
    float pexp[NB][2][4];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      float z[2][4];
      float bm = kNegInf;
#pragma unroll
      for (int tau = 0; tau < 2; ++tau)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int t = blk * kBlock + kTile * tau + 4 * g + e;
          const float zz = s[tau][nb][e] * h_at(raw[tau].ks, e) * a.scale_log2;
          z[tau][e] = (t <= last_tok[nb]) ? zz : kNegInf;
          bm = fmaxf(bm, z[tau][e]);
        }
      bm = fmaxf(bm, __shfl_xor(bm, 16, kWave));
      bm = fmaxf(bm, __shfl_xor(bm, 32, kWave));
      const float m_new = fmaxf(m_run[nb], bm);
      const float m_use = (m_new == kNegInf) ? 0.0f : m_new;
      const float alpha = exp2f(m_run[nb] - m_use);
      m_run[nb] = m_new;
      float lsum = 0.0f;
#pragma unroll
      for (int tau = 0; tau < 2; ++tau)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          pexp[nb][tau][e] = exp2f(z[tau][e] - m_use);
          lsum += pexp[nb][tau][e];
        }
      l_run[nb] = l_run[nb] * alpha + lsum;
#pragma unroll
      for (int db = 0; db < DB; ++db) acc[nb][db] *= alpha;
    }

    // ---- O^T += V^T P^T per 32-dim scale group ----
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
        half8 phi, plo;
#pragma unroll
        for (int tau = 0; tau < 2; ++tau)
#pragma unroll
          for (int k = 0; k < 4; ++k) {
            const int e = (k == 1) ? 2 : (k == 2) ? 1 : k;
            const float x = pexp[nb][tau][e] * h_at(raw[tau].vs, e * NG + j);
            const float px = (pexp[nb][tau][e] == 0.0f) ? 0.0f : x;  // masked: ignore the scale
            const _Float16 hi = (_Float16)px;
            phi[4 * tau + k] = hi;
            plo[4 * tau + k] = (_Float16)(px - (float)hi);
          }
        acc[nb][2 * j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(vlo, phi, acc[nb][2 * j], 0, 0, 0);
        acc[nb][2 * j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(vlo, plo, acc[nb][2 * j], 0, 0, 0);
        acc[nb][2 * j + 1] = __builtin_amdgcn_mfma_f32_16x16x32_f16(vhi, phi, acc[nb][2 * j + 1], 0, 0, 0);
        acc[nb][2 * j + 1] = __builtin_amdgcn_mfma_f32_16x16x32_f16(vhi, plo, acc[nb][2 * j + 1], 0, 0, 0);
      }
    }
  }

  // ---- partial of this split ----
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    float l = l_run[nb];
    l += __shfl_xor(l, 16, kWave);
    l += __shfl_xor(l, 32, kWave);
    const int n = 16 * nb + m16;
    if (n < a.rows) {
      const size_t prow = ((size_t)unit * a.splits + split) * a.rows + n;
      float* dst = a.ws_acc + prow * D + 4 * g;
#pragma unroll
      for (int db = 0; db < DB; ++db) *(floatx4*)(dst + 16 * db) = acc[nb][db];
      if (g == 0) a.ws_ml[prow] = make_float2(m_run[nb], l);
    }
  }
}

// One workgroup of D threads per (unit, row): weights 2^(m_j - M) over the splits.
template <int D>
__global__ __launch_bounds__(256) void merge_kernel(DecodeArgs a) {
  const int idx = blockIdx.x;
  const int unit = idx / a.rows, n = idx % a.rows;
  const int b = unit / a.num_kv_heads, h = unit % a.num_kv_heads;
  const int i = n / a.group, hq = h * a.group + n % a.group;
  const int d = threadIdx.x;
  const size_t row0 = (size_t)unit * a.splits * a.rows + n;
  float M = kNegInf;
  for (int sp = 0; sp < a.splits; ++sp) M = fmaxf(M, a.ws_ml[row0 + (size_t)sp * a.rows].x);
  float num = 0.0f, den = 0.0f;
  if (M != kNegInf) {
    for (int sp = 0; sp < a.splits; ++sp) {
      const float2 ml = a.ws_ml[row0 + (size_t)sp * a.rows];
      if (ml.x == kNegInf) continue;
      const float w = exp2f(ml.x - M);
      num += w * a.ws_acc[(row0 + (size_t)sp * a.rows) * D + d];
      den += w * ml.y;
    }
  }
  const size_t o = ((size_t)b * a.n_rows + i) * a.n_q_heads + hq;
  a.out[o * D + d] = den > 0.0f ? num / den : 0.0f;
  if (d == 0 && a.lse) a.lse[o] = den > 0.0f ? (M + log2f(den)) * 0.69314718055994530942f : kNegInf;
}

template <int D>
hipError_t launch_decode_d(const DecodeArgs& a, hipStream_t stream) {
  const long long waves = (long long)a.n_seq * a.num_kv_heads * a.splits;
  const unsigned grid = (unsigned)((waves + 3) / 4);
  if (a.rows <= 16)
    hipLaunchKernelGGL((decode_split_kernel<D, 1>), dim3(grid), dim3(256), 0, stream, a);
  else
    hipLaunchKernelGGL((decode_split_kernel<D, 2>), dim3(grid), dim3(256), 0, stream, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const unsigned mgrid = (unsigned)(a.n_seq * a.num_kv_heads * a.rows);
  hipLaunchKernelGGL(merge_kernel<D>, dim3(mgrid), dim3(D), 0, stream, a);
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

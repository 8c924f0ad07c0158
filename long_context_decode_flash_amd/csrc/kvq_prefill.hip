// kvq_prefill.hip — chunked-prefill attention over the paged cache.
//
// The forum post "3090 单卡跑 Qwen3.8-27B：NInfer 上机实测（180K 上下文 / C2 并发 / 4bit KV）"
// (一、部署, launch-flag table) prefills prompts in chunks of 1,024 tokens and names prefill as
// the cost behind the time to first token (二、测评).  Once a chunk's tokens are appended to the
// cache, each position of the chunk attends causally to the cache up to itself: position i of a
// chunk of C at the end of a context of L tokens sees tokens 0 .. L - C + i.  That is the
// decode's multi-row attention with C rows; what changes is the shape.  Every cached byte now
// meets thousands of query rows, so the work is dense matrix-core work, not a byte stream:
//
//   * one workgroup of 8 waves per (sequence, KV head, tile of 256 query rows, piece of the
//     context); the rows of a KV head are (chunk position, query head of its group) pairs in
//     position-major order, and wave w owns rows 32w .. 32w + 31 of the tile as two 16-row
//     blocks, with the decode's online softmax;
//   * both products take their K and V operands from LDS, built once per block for all eight
//     waves: K codes widened to fp16 (exact; the K scale multiplies the logit) against the
//     rows' own fp16 query words, and V codes times V scale as exact fp16 hi + lo pairs (the
//     decode instead folds the scale into each row's P, which costs per row what this costs
//     once); every operand read serves both row blocks of a wave;
//   * waves 0 and 1 stage tiles 0 and 1 of each 32-token block into one of three LDS buffers
//     shared by all eight waves, so two blocks are in flight while the workgroup computes one;
//     one barrier per block publishes the staged block, a second its V operands;
//   * blocks past the tile's last position are never loaded; a wave skips blocks past its last
//     row's position and masks the blocks that cross its rows' positions;
//   * each wave writes its rows: the output itself (one piece per context) or a partial that the
//     decode's log-sum-exp merge launch combines.
#include "kvq_attn_block.h"

namespace kvq {
namespace {

constexpr int kIdsPerChunk = kWave;  // blocks whose page ids a staging wave keeps in its lanes

// ---- V of a staged block as scaled fp16 operands, built once per workgroup ----
// For 32-dim group j and half dh (dims 32j + 16dh .. + 15), lane l holds the A operand of the
// P V product for dim 32j + 16dh + l%16 and the eight tokens of its lane group in the order the
// P operand uses (tokens 0, 2, 1, 3 of the group's four in tile 0, then in tile 1), as an fp16
// hi and lo pair: v = code * v_scale * 2^(15 - e5) is exact in fp32, hi = rne16(v) and
// lo = rne16(v - hi).  e5 is the block's largest V-scale exponent field, so |v| < 2^9 and
// nothing overflows; the P operand carries the 2^(e5 - 15).  One copy serves every wave, in
// place of each wave widening the codes and folding the scale into its own rows' P.
template <int NG>
struct VHat {
  u32x4 w[NG][2][2][kWave];  // [group][dim half][hi, lo][lane]
};

#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
// hi = rne16(c * s), lo = rne16(c * s - hi) for both fp16 halves of c and s (v_fma_mix forms
// the exact product in fp32 and rounds once).
__device__ inline void mul16_hi_lo(uint32_t c, uint32_t s, uint32_t& hi, uint32_t& lo) {
  uint32_t h, l;
  asm("v_fma_mixlo_f16 %0, %1, %2, 0 op_sel:[0,0,0] op_sel_hi:[1,1,0]" : "=v"(h) : "v"(c), "v"(s));
  asm("v_fma_mixhi_f16 %0, %1, %2, 0 op_sel:[1,1,0] op_sel_hi:[1,1,0]" : "+v"(h) : "v"(c), "v"(s));
  asm("v_fma_mixlo_f16 %0, %1, %2, -%3 op_sel:[0,0,0] op_sel_hi:[1,1,1]" : "=&v"(l) : "v"(c), "v"(s), "v"(h));
  asm("v_fma_mixhi_f16 %0, %1, %2, -%3 op_sel:[1,1,1] op_sel_hi:[1,1,1]" : "+v"(l) : "v"(c), "v"(s), "v"(h));
  hi = h;
  lo = l;
}
#pragma clang diagnostic pop

// The code dword of V word index x of a staged tile, for this lane (the read_tile layout).
template <int D, int VB>
__device__ inline uint32_t v_word(const uint8_t* tile, int x, int lane) {
  using S = Stage<D, VB>;
  if constexpr (VB == 4 && D == 64) return *(const uint32_t*)(tile + S::kV + 8 * lane + 4 * x);
  return *(const uint32_t*)(tile + S::kV + 1024 * (x / 4) + 16 * lane + 4 * (x % 4));
}

// Item it = (group j, dim half dh) of the block staged at src: codes of slots at or past lc are
// taken as 0 (never-written slots may hold NaN codes), scales times vfac = 2^(15 - e5).
template <int D, int VB, bool F8>
__device__ inline void build_vhat(const uint8_t* src, VHat<D / 32>& vh, int it, int lane, int tok0, int lc,
                                  half2v vfac) {
  constexpr int NG = D / 32;
  using S = Stage<D, VB>;
  const int j = it >> 1, dh = it & 1, g = lane >> 4;
  uint32_t hi[4], lo[4];
#pragma unroll
  for (int tau = 0; tau < 2; ++tau) {
    const uint8_t* tile = src + tau * S::kTileBytes;
    uint32_t keep = 0;  // byte r of a code word is slot 4g + r of the tile
#pragma unroll
    for (int e = 0; e < 4; ++e) keep |= (tok0 + kTile * tau + 4 * g + e < lc) ? 0xFFu << (8 * e) : 0u;
    uint32_t l02, l13, h02, h13;
    if constexpr (VB == 4) {
      i4x8_to_h2x4(v_word<D, VB>(tile, j, lane) & keep, l02, l13, h02, h13);
    } else {
      const uint32_t lw = v_word<D, VB>(tile, 2 * j, lane) & keep, hw = v_word<D, VB>(tile, 2 * j + 1, lane) & keep;
      if constexpr (F8)
        f8x8_to_h2x4(lw, hw, l02, l13, h02, h13);
      else
        i8x8_to_h2x4(lw, hw, l02, l13, h02, h13);
    }
    // scales of the lane group's tokens e = 0, 2 and 1, 3 for group j, times vfac
    const uint16_t* vs = (const uint16_t*)(tile + S::kVs + g * (D / 4)) + j;
    const half2v s02 = __builtin_bit_cast(half2v, (uint32_t)vs[0] | ((uint32_t)vs[2 * NG] << 16)) * vfac;
    const half2v s13 = __builtin_bit_cast(half2v, (uint32_t)vs[NG] | ((uint32_t)vs[3 * NG] << 16)) * vfac;
    mul16_hi_lo(dh ? h02 : l02, as_u32(s02), hi[2 * tau], lo[2 * tau]);
    mul16_hi_lo(dh ? h13 : l13, as_u32(s13), hi[2 * tau + 1], lo[2 * tau + 1]);
  }
  vh.w[j][dh][0][lane] = u32x4{hi[0], hi[1], hi[2], hi[3]};
  vh.w[j][dh][1][lane] = u32x4{lo[0], lo[1], lo[2], lo[3]};
}

// ---- K of a staged block as fp16 operands, built once per workgroup ----
// For tile tau and 64-dim step jj, lane l holds the A operand of Q K^T for token l%16 of the tile
// and the 16 dims 16(4jj + l/16) .. + 15, as two half8 words (dims + 0..7, + 8..15): the codes
// widened to fp16, exact for int8 and E4M3 alike; the K scale multiplies the logit.
template <int D>
struct KHat {
  u32x4 w[2][D / 64][2][kWave];  // [tile][64-dim step][half][lane]
};

template <int D, int VB, bool F8>
__device__ inline void build_khat(const uint8_t* src, KHat<D>& kh, int it, int lane) {
  using S = Stage<D, VB>;
  const int tau = it / (D / 64), jj = it % (D / 64);
  const u32x4 x = *(const u32x4*)(src + tau * S::kTileBytes + S::kK + 1024 * jj + 16 * lane);
  const half2v off = {(_Float16)-1152.0f, (_Float16)-1152.0f};
  const uint32_t xw[4] = {x[0], x[1], x[2], x[3]};
  uint32_t o[8];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    if constexpr (F8) {
      o[2 * i] = e4m3x2_to_h2<false>(xw[i]);
      o[2 * i + 1] = e4m3x2_to_h2<true>(xw[i]);
    } else {
      // bytes (0, 1) and (2, 3) into the low bytes of the halves; byte ^ 0x80 is code + 128 and
      // 0x6400 | m is the fp16 value 1024 + m, so the half minus 1152 is the code, exactly
      o[2 * i] = as_u32(as_h2(__builtin_amdgcn_perm(xw[i], xw[i], 0x0C010C00u) ^ 0x64806480u) + off);
      o[2 * i + 1] = as_u32(as_h2(__builtin_amdgcn_perm(xw[i], xw[i], 0x0C030C02u) ^ 0x64806480u) + off);
    }
  }
  kh.w[tau][jj][0][lane] = u32x4{o[0], o[1], o[2], o[3]};
  kh.w[tau][jj][1][lane] = u32x4{o[4], o[5], o[6], o[7]};
}

// Q K^T from the shared K operands and the rows' own fp16 query words: sc[tau][nb][e] is the
// dot product of the lane's query row (block nb) with token 4g + e of tile tau.
template <int D, int NB>
__device__ __attribute__((always_inline)) inline void block_scores_khat(const KHat<D>& kh, int lane,
                                                                        const u32x4 (&qw)[NB][D / 64][2],
                                                                        float (&sc)[2][NB][4]) {
  floatx4 sf[2][NB];
#pragma unroll
  for (int tau = 0; tau < 2; ++tau)
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) sf[tau][nb] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int jj = 0; jj < D / 64; ++jj)
#pragma unroll
    for (int hf = 0; hf < 2; ++hf)
#pragma unroll
      for (int tau = 0; tau < 2; ++tau) {
        const half8 k8 = __builtin_bit_cast(half8, kh.w[tau][jj][hf][lane]);
#pragma unroll
        for (int nb = 0; nb < NB; ++nb)
          sf[tau][nb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(k8, __builtin_bit_cast(half8, qw[nb][jj][hf]),
                                                               sf[tau][nb], 0, 0, 0);
      }
#pragma unroll
  for (int tau = 0; tau < 2; ++tau)
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      const floatx4 v = sf[tau][nb];
      sc[tau][nb][0] = v[0];
      sc[tau][nb][1] = v[1];
      sc[tau][nb][2] = v[2];
      sc[tau][nb][3] = v[3];
    }
}

// O^T += V^T P^T from the shared operands: P as fp16 hi + lo with 2^(e5 - 15) applied, three
// products per operand pair (hi*hi, hi*lo, lo*hi; lo*lo is below 2^-22 of the product); each V
// operand read from LDS serves every row block of the wave.
template <int D, int NB>
__device__ __attribute__((always_inline)) inline void block_pv_vhat(const VHat<D / 32>& vh, int lane,
                                                                    const float (&pexp)[NB][2][4], float pf,
                                                                    floatx4 (&acc)[NB][D / 16]) {
  constexpr int NG = D / 32;
  constexpr uint32_t kOne = 0x3C003C00u;  // fp16 1.0 in both halves
  uint32_t hw[NB][4], lw[NB][4];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
#pragma unroll
    for (int tau = 0; tau < 2; ++tau) {
      mix_hi_lo(pexp[nb][tau][0] * pf, kOne, pexp[nb][tau][2] * pf, kOne, hw[nb][2 * tau], lw[nb][2 * tau]);
      mix_hi_lo(pexp[nb][tau][1] * pf, kOne, pexp[nb][tau][3] * pf, kOne, hw[nb][2 * tau + 1],
                   lw[nb][2 * tau + 1]);
    }
    // two wait states between the inline-asm writes of P and the matrix-core reads (the
    // compiler's hazard tracking does not see inline-asm results)
    asm("s_nop 1" : "+v"(hw[nb][0]), "+v"(hw[nb][1]), "+v"(hw[nb][2]), "+v"(hw[nb][3]), "+v"(lw[nb][0]),
        "+v"(lw[nb][1]), "+v"(lw[nb][2]), "+v"(lw[nb][3]));
  }
#pragma unroll
  for (int j = 0; j < NG; ++j)
#pragma unroll
    for (int dh = 0; dh < 2; ++dh) {
      const half8 vhi = __builtin_bit_cast(half8, vh.w[j][dh][0][lane]);
      const half8 vlo = __builtin_bit_cast(half8, vh.w[j][dh][1][lane]);
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

// NB: 16-row blocks per wave; the rows of a tile take kPrefillRowsPerTile / (16 NB) waves.
template <int D, int VB, bool F8, int NB>
__global__ __launch_bounds__(kPrefillRowsPerTile / 16 / NB * kWave) void prefill_kernel(DecodeArgs a) {
  constexpr int kRowsPerWave = 16 * NB;
  constexpr int DB = D / 16;
  constexpr int NSTAGE = 3;
  constexpr int BS = Stage<D, VB>::kBlockBytes;
  constexpr int TB = Stage<D, VB>::kTileBytes;
  constexpr int NLT = Stage<D, VB>::kLoads / 2;  // direct-to-LDS loads of one tile
  static_assert(NLT <= 63, "vmcnt range");
  constexpr int NWAVES = kPrefillRowsPerTile / kRowsPerWave;
  __shared__ __attribute__((aligned(16))) uint8_t s_stage[NSTAGE][BS];
  __shared__ VHat<D / 32> s_vh;
  __shared__ KHat<D> s_kh;

  const int lane = threadIdx.x & (kWave - 1);
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int split = blockIdx.x % a.splits;
  const int ut = blockIdx.x / a.splits;
  const int tile = ut % a.row_tiles, unit = ut / a.row_tiles;
  const int b = unit / a.num_kv_heads, h = unit % a.num_kv_heads;
  const int P = a.page_size;
  const int L = a.seq_lens[b];
  const int Lc = min(L, a.max_seq_len);  // tokens past max_seq_len are not attended
  const int m16 = lane & 15, g = lane >> 4;
  const int C = a.n_rows;  // chunk positions

  // ---- the tile's and the wave's rows (position i = n / group of row n) ----
  const int n_tile0 = tile * kPrefillRowsPerTile;
  const int n_tile1 = min(n_tile0 + kPrefillRowsPerTile, a.rows) - 1;
  const int t_hi = min(L - C + n_tile1 / a.group, Lc - 1);  // last token a row of the tile sees
  const int nblk = t_hi >= 0 ? t_hi / kBlock + 1 : 0;
  const int g_blk0 = split * a.blocks_per_split;
  const int n_blocks = max(min(g_blk0 + a.blocks_per_split, nblk) - g_blk0, 0);
  const int nw0 = n_tile0 + kRowsPerWave * w;
  const int nw1 = min(nw0 + kRowsPerWave, a.rows) - 1;  // below nw0: the wave holds only padding
  // last token every row of the wave sees, and last token some row of it sees
  const int w_all = nw1 >= nw0 ? min(L - C + nw0 / a.group, Lc - 1) : -1;
  const int w_any = nw1 >= nw0 ? min(L - C + nw1 / a.group, Lc - 1) : -1;

  const size_t bb = block_bytes(P, D, VB);
  const uint32_t page_stride32 = (uint32_t)(a.num_kv_heads * bb);  // < 2^32, checked on the host
  const uint8_t* pool_h = a.pool + (size_t)h * bb;
  const int32_t* pt = a.page_table + (size_t)b * a.max_pages;
  const int lgP = a.log2_page;

  // ---- raw query words (the decode's B-operand layout); padding rows: q = 0, see nothing ----
  u32x4 qw[NB][D / 64][2];
  int last_tok[NB], first_tok[NB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    const int n = nw0 + 16 * nb + m16;
    const bool real = n < a.rows;
    const int i = real ? n / a.group : 0;
    const int hq = h * a.group + (real ? n % a.group : 0);
    last_tok[nb] = real ? min(L - C + i, Lc - 1) : -1;
    first_tok[nb] = 0;
    const uint16_t* qrow = a.q + (((size_t)b * C + i) * a.n_q_heads + hq) * D;
#pragma unroll
    for (int jj = 0; jj < D / 64; ++jj)
#pragma unroll
      for (int hf = 0; hf < 2; ++hf)
        qw[nb][jj][hf] = real ? *(const u32x4*)(qrow + 16 * (4 * jj + g) + 8 * hf) : u32x4{0, 0, 0, 0};
  }

  // ---- staging: wave tau (0 or 1) loads tile tau of every block; lane k holds the physical page
  // of that tile for block k of the current group of kIdsPerChunk blocks ----
  const uint32_t stage0 = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(lds_void*)&s_stage[0][0]);
  const uint32_t lane16 = 16u * lane;
  const ScaleLane sl = scale_lane<D, VB>(P, lane);
  const bool stager = w < 2;
  int my_pid = 0;
  auto load_ids = [&](int k0) {
    const int blk = g_blk0 + k0 + lane;
    int tok0 = blk * kBlock + kTile * w;
    if (tok0 >= Lc) tok0 = blk * kBlock;  // a tile past the end stages tile 0 again, all masked
    const int id = pt[k0 + lane < n_blocks ? (tok0 >> lgP) : 0];  // entry 0 always exists
    debug_report(a.dbg, k0 + lane < n_blocks && (id < 0 || id >= a.num_pages), kDbgPageId);
    my_pid = min(max(id, 0), a.num_pages - 1);  // out-of-range ids are clamped, never followed
  };
  auto issue = [&](int k) {
    const int blk = g_blk0 + k;
    int tok0 = blk * kBlock + kTile * w;
    if (tok0 >= Lc) tok0 = blk * kBlock;
    const int phys = __builtin_amdgcn_readlane(my_pid, k % kIdsPerChunk);
    stage_tile<D, VB>(pool_h + (uint64_t)(uint32_t)phys * page_stride32, P, tok0 & (P - 1),
                      stage0 + (uint32_t)((k % NSTAGE) * BS + w * TB), lane16, sl);
  };
  if (stager) {
    load_ids(0);
    // the query words are used here, so the compiler's wait for them (one round trip with the
    // page ids) is not placed after the block loads
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
      for (int jj = 0; jj < D / 64; ++jj) asm volatile("" ::"v"(qw[nb][jj][0]), "v"(qw[nb][jj][1]));
    asm volatile("" ::"v"(my_pid));
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // the DMA counting starts here
    if (n_blocks > 0) issue(0);
    if (n_blocks > 1) issue(1);
  }

  float cz[NB];  // the query's fp16 words are the B operands as they are
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) cz[nb] = a.scale_log2;

  floatx4 acc[NB][DB];
  float base[NB], l_run[NB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
#pragma unroll
    for (int db = 0; db < DB; ++db) acc[nb][db] = floatx4{0.f, 0.f, 0.f, 0.f};
    base[nb] = kNegInf;
    l_run[nb] = 0.0f;
  }

  for (int k = 0; k < n_blocks; ++k) {
    const int blk = g_blk0 + k;
    const uint8_t* src = &s_stage[k % NSTAGE][0];
    if (stager) {
      if (k + 1 < n_blocks)
        wait_vmcnt<NLT>();  // this tile of block k is in; block k + 1's may still be in flight
      else
        wait_vmcnt<0>();
      // slots at or past the context end may hold junk scale bits, and 0 * Inf is no zero:
      // clear their V scales in the staged copy before any wave reads it
      const int t = blk * kBlock + kTile * w + lane;
      if (lane < kTile && t >= Lc) {
        uint8_t* vs = (uint8_t*)src + w * TB + Stage<D, VB>::kVs + lane * (D / 16);
        if constexpr (D == 256) *(u32x4*)vs = u32x4{0, 0, 0, 0};
        else if constexpr (D == 128) *(u32x2*)vs = u32x2{0, 0};
        else *(uint32_t*)vs = 0u;
      }
    }
    // block k staged for every wave (the stagers waited for their loads above), and every
    // wave's reads of block k - 1's buffer are complete, so it may be refilled; the loads of
    // block k + 1 stay in flight across the barrier
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    if (stager && k + 2 < n_blocks) {
      if ((k + 2) % kIdsPerChunk == 0) load_ids(k + 2);  // the compiler waits for the ids (and all loads)
      issue(k + 2);
    }
    // the block's largest V-scale exponent field (every wave reads the same staged scales)
    float e5;
    {
      const uint32_t* vsw = (const uint32_t*)(src + Stage<D, VB>::kVs) + (lane & (D / 4 - 1));
      const uint32_t m = wave_max_u16x2(__builtin_bit_cast(uint32_t, __builtin_elementwise_max(
          __builtin_bit_cast(u16x2, vsw[0]), __builtin_bit_cast(u16x2, vsw[TB / 4]))));
      e5 = (float)((m >> 10) & 31);
    }
    // the block's scaled V operands, each wave building its share of the (group, half) items
    {
      const _Float16 f = (_Float16)__builtin_ldexpf(1.0f, 15 - (int)e5);  // a power of two, exact
      const half2v vfac = {f, f};
#pragma unroll
      for (int it = w; it < 2 * (D / 32); it += NWAVES) build_vhat<D, VB, F8>(src, s_vh, it, lane, blk * kBlock, Lc, vfac);
#pragma unroll
      for (int it = w; it < 2 * (D / 64); it += NWAVES) build_khat<D, VB, F8>(src, s_kh, it, lane);
    }
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    __builtin_amdgcn_s_barrier();  // the operands are complete
    asm volatile("" ::: "memory");
    if (blk * kBlock > w_any) continue;  // no row of this wave sees the block (wave-uniform)
    const bool masked = blk * kBlock + kBlock - 1 > w_all;
    float sc[2][NB][4];
    block_scores_khat<D, NB>(s_kh, lane, qw, sc);
    uint32_t ksw[2][2];
#pragma unroll
    for (int tau = 0; tau < 2; ++tau) {
      const u32x2 kw = *(const u32x2*)(src + tau * TB + Stage<D, VB>::kKs + 8 * g);
      ksw[tau][0] = kw[0];
      ksw[tau][1] = kw[1];
    }
    float pexp[NB][2][4];
    block_softmax_scores<D, NB, false>(sc, ksw, blk, masked, e5, cz, first_tok, last_tok, g, acc, base, l_run,
                                       pexp);
    block_pv_vhat<D, NB>(s_vh, lane, pexp, __builtin_ldexpf(1.0f, (int)e5 - 15), acc);
  }

  // ---- each wave writes its own rows: the output (one piece) or this piece's partial ----
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    const float l = sum_over_rows(l_run[nb]);
    const int n = nw0 + 16 * nb + m16;
    if (n >= a.rows) continue;
    if (a.splits == 1) {
      const int i = n / a.group, hq = h * a.group + n % a.group;
      const size_t o = ((size_t)b * C + i) * a.n_q_heads + hq;
      const float inv = l > 0.0f ? 1.0f / l : 0.0f;
#pragma unroll
      for (int db = 0; db < DB; ++db) *(floatx4*)(a.out + o * D + 16 * db + 4 * g) = acc[nb][db] * inv;
      if (g == 0 && a.lse) a.lse[o] = l > 0.0f ? (base[nb] + log2f(l)) * 0.69314718055994530942f : kNegInf;
    } else {
      const size_t prow = ((size_t)unit * a.splits + split) * a.rows + n;
#pragma unroll
      for (int db = 0; db < DB; ++db) *(floatx4*)(a.ws_acc + prow * D + 16 * db + 4 * g) = acc[nb][db];
      if (g == 0) a.ws_ml[(size_t)unit * ml_stride(a.splits, a.rows) + (size_t)split * a.rows + n] = float2{base[nb], l};
    }
  }
}

// Two 16-row blocks per wave, eight waves per tile (two waves per SIMD).  The query's fp16 words
// (64 VGPRs at head dim 256, against 96 for three int8 digit planes) leave room for the second
// row block; at head dim 256 the kernel still spills about 20 dwords per lane.  On the
// 1,024-position chunk of the 184K-token pool this took 10.3 ms, against 11.6 ms for one 16-row
// block per wave with int8 digit planes (128-row tiles), and 14.0 ms for four waves of two.
constexpr int kPrefillNB = 2;

template <int D>
hipError_t launch_prefill_d(const DecodeArgs& a, hipStream_t stream) {
  const unsigned units = (unsigned)((long long)a.n_seq * a.num_kv_heads);
  static_assert(kPrefillRowsPerTile / 16 / kPrefillNB * kWave == kPrefillThreads, "prefill block");
  const dim3 grid(units * (unsigned)a.row_tiles * (unsigned)a.splits), block(kPrefillThreads);
  if (a.fp8)
    hipLaunchKernelGGL((prefill_kernel<D, 8, true, kPrefillNB>), grid, block, 0, stream, a);
  else if (a.vbits == 8)
    hipLaunchKernelGGL((prefill_kernel<D, 8, false, kPrefillNB>), grid, block, 0, stream, a);
  else
    hipLaunchKernelGGL((prefill_kernel<D, 4, false, kPrefillNB>), grid, block, 0, stream, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || a.splits == 1) return e;
  const unsigned per_unit = (unsigned)merge_groups(a.rows, D);  // grid size checked on the host
  launch_merge<D>(a, units * per_unit, stream);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_prefill(int head_dim, const DecodeArgs& a, hipStream_t stream) {
  switch (head_dim) {
    case 64: return launch_prefill_d<64>(a, stream);
    case 128: return launch_prefill_d<128>(a, stream);
    case 256: return launch_prefill_d<256>(a, stream);
  }
  return hipErrorInvalidValue;
}

}  // namespace kvq

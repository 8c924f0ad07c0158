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
//     32-token blocks through LDS stage buffers with direct-to-LDS 16-byte loads (two buffers
//     at head dim 256, one block in flight while it computes one; three below);
//   * Q K^T runs on the int8 matrix cores: the K codes of one 16-byte load per lane are the A
//     operand of v_mfma_i32_16x16x64_i8 as they sit in the page, and each query row is split
//     exactly into three int8 digits at a per-row power-of-two scale (B operands, query rows of
//     the GQA group x MTP rows on N), so the dot products are exact integers;
//   * the 16x16 logit tile comes out with each lane holding one query row and four tokens, the
//     B-operand layout of the P V product (tokens on K), so P never leaves the registers; V codes
//     arrive pre-arranged as the A operand of v_mfma_f32_16x16x32_f16 and are widened with
//     exact bit tricks; the V scale (per token and 32 dims) multiplies the codes, and both that
//     exact product and P split into fp16 high and low parts, so the product keeps fp32 accuracy;
//   * online softmax in log2 units whose exponent offset only moves in powers of two when a
//     block needs it, so most blocks rescale nothing and form no cross-lane row maximum;
//   * the waves merge through LDS into one partial per workgroup (or straight into the output
//     when a context is one piece); a second, wide launch merges the pieces' partials, eight
//     lanes per (sequence, KV head, query row, 4 dims).
#include "kvq_attn_block.h"

namespace kvq {
namespace {

// One workgroup (4 waves) per (unit, split); wave w takes the split's blocks w, w+4, w+8, ...
// Each wave streams its blocks through NSTAGE LDS stage buffers with direct-to-LDS loads, so
// NSTAGE - 1 blocks are in flight while it computes one.  The waves merge through LDS into one
// partial (the output itself when the context is a single piece).  WIN: a sliding window (the
// pieces start at the first row's window start; pages may be a ring).
//
// The scalars of the first memory accesses (the sequence length, the page ids, the queries)
// come as separate leading kernel arguments: with kernel-argument preloading the first 14
// argument dwords (all that gfx950's user SGPRs hold besides the argument pointer) are in SGPRs
// when the wave starts, so those loads need no kernel-argument load before them.  n_q_heads and
// rows follow from them; the rest comes from the argument struct.
template <int D, int NB, int VB, bool WIN, bool F8>
__global__ __launch_bounds__(256) void decode_kernel(const int32_t* page_table, const int32_t* seq_lens,
                                                      const uint16_t* q, int splits, int num_kv_heads,
                                                      int max_pages, int blocks_per_split, int log2_page,
                                                      int max_seq_len, int n_rows, int group, DecodeArgs args) {
  DecodeArgs a = args;
  a.page_table = page_table;
  a.seq_lens = seq_lens;
  a.q = q;
  a.splits = splits;
  a.num_kv_heads = num_kv_heads;
  a.max_pages = max_pages;
  a.blocks_per_split = blocks_per_split;
  a.log2_page = log2_page;
  a.max_seq_len = max_seq_len;
  a.n_rows = n_rows;
  a.group = group;
  a.n_q_heads = group * num_kv_heads;
  a.rows = group * n_rows;
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
  bool my_id_real = false;  // this lane's id is a real entry of the chunk (not the entry-0 filler)
  int my_tok0 = 0;          // first token of the tile this lane's id is for
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
    my_id_real = kk < n_ids;
    my_tok0 = tok0;
    my_pid = pt[my_id_real ? entry(tok0 >> lgP) : 0];  // every lane loads (entry 0 always exists)
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
    // (only ids of tiles inside the context are followed; past it an entry may be padding)
    debug_report(a.dbg, my_id_real && my_tok0 < Lc && (my_pid < 0 || my_pid >= a.num_pages), kDbgPageId);
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
  //
  // Fused append: the wave that will stage the block of a new token quantizes the token's K/V
  // rows (this KV head) into its slot, and the block's loads must see those bytes.  The new
  // tokens L - n_new .. L - 1 fall in at most three consecutive blocks, so a wave owns at most
  // one run [ta, tb) of them, in one block at place kb of its list (blocks w, w + 4, ... of the
  // split).
  //   * Usual case (the block at place kb >= 2 NSTAGE - 2, at most kFastTokens tokens): the rows
  //     and page ids load with the queries and page ids (one round trip for all), and the
  //     quantized bytes are stored once the first stage loads are out, so the work overlaps the
  //     first block's flight.  Vector memory operations complete in issue order; the stores go
  //     out between the loads of places NSTAGE - 2 and NSTAGE - 1, the loop's wait at iteration
  //     NSTAGE - 2 retires everything issued before the loads of place NSTAGE - 1, and the
  //     block at place kb >= 2 NSTAGE - 2 is issued after that wait (a block of a later chunk:
  //     that chunk's chunk_start waits for everything).  On the 184K-token step the token is its
  //     wave's last block; written before the first loads, it held its workgroup ~2 us behind
  //     the others.
  //   * Otherwise (a block whose loads may leave before that wait, or a longer run) the tokens
  //     are written before the first loads, and chunk_start's wait covers their stores.
  constexpr int kEarlyPlaces = 2 * NSTAGE - 2;
  constexpr int kFastTokens = 4;
  int ta = 0, tb = 0, kb_app = -1;
  if (a.n_new > 0) {
    const int t_first = max(L - a.n_new, 0);
    for (int blk = t_first >> 5; blk <= (L - 1) >> 5; ++blk)
      if (blk >= g_blk0 && blk < g_blk1 && ((blk - g_blk0) & (kWavesPerGroup - 1)) == w) {
        ta = max(t_first, blk * kBlock);
        tb = min(L, blk * kBlock + kBlock);
        kb_app = (blk - g_blk0) / kWavesPerGroup;
      }
  }
  const bool app_fast = kb_app >= kEarlyPlaces && tb - ta <= kFastTokens;
  auto new_row = [&](int t) { return (((size_t)b * a.n_new + (t - (L - a.n_new))) * a.num_kv_heads + h) * D; };
  auto slot_block = [&](int pid) {
    debug_report(a.dbg, pid < 0 || pid >= a.num_pages, kDbgPageId);
    return a.pool_rw + ((size_t)min(max(pid, 0), a.num_pages - 1) * a.num_kv_heads + h) * bb;
  };
  if (kb_app >= 0 && !app_fast)
    for (int t = ta; t < tb; ++t)
      append_row<D, VB, F8>(slot_block(pt[entry(t >> lgP)]), P, t & (P - 1), a.k_new + new_row(t), a.v_new + new_row(t),
                            lane);
  RowVals<D> app_rows[kFastTokens];
  int app_pid[kFastTokens];
#pragma unroll
  for (int i = 0; i < kFastTokens; ++i) {
    const bool on = app_fast && ta + i < tb;
    const int t = on ? ta + i : 0;
    app_pid[i] = on ? pt[entry(t >> lgP)] : 0;
    app_rows[i] = RowVals<D>{};
    if (on) app_rows[i] = load_row<D>(a.k_new + new_row(t), a.v_new + new_row(t), lane);
  }
  chunk_count();
  asm volatile("" ::"v"(my_pid));
#pragma unroll
  for (int nb = 0; nb < NB; ++nb)
#pragma unroll
    for (int jj = 0; jj < D / 64; ++jj) asm volatile("" ::"v"(qw[nb][jj][0]), "v"(qw[nb][jj][1]));
#pragma unroll
  for (int i = 0; i < kFastTokens; ++i) {
    asm volatile("" ::"v"(app_pid[i]));
#pragma unroll
    for (int e = 0; e < RowVals<D>::E; ++e) asm volatile("" ::"v"(app_rows[i].k[e]), "v"(app_rows[i].v[e]));
  }
  chunk_start();
#pragma unroll
  for (int i = 0; i < kFastTokens; ++i) {
    const int t = ta + i;
    if (app_fast && t < tb) store_row<D, VB, F8>(slot_block(app_pid[i]), P, t & (P - 1), app_rows[i], lane);
  }

  i32x4 qd[NB][3][D / 64];
  float cz[NB];
  prepare_queries<D, NB, F8>(qw, a.scale_log2, qd, cz);

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
      if (masked) wave_lds_order();  // every lane reads the scales lanes < 32 cleared
      TileRaw<D, VB> raw[2];
      read_tile<D, VB>(raw[0], src, lane);
      read_tile<D, VB>(raw[1], src + Stage<D, VB>::kTileBytes, lane);
      if constexpr (F8) {
        if (masked) {
          clear_unseen_v<D, VB>(raw[0], blk * kBlock, g, t_lo, Lc);
          clear_unseen_v<D, VB>(raw[1], blk * kBlock + kTile, g, t_lo, Lc);
        }
      }
      // p stays below 2^13 (the V scale is applied on the V side: no V-scale exponent)
      process_block<D, NB, VB, WIN, F8>(raw, blk, masked, 14.0f, qd, qw, cz, first_tok, last_tok, g, acc, base,
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

template <int D, bool WIN, int VB, bool F8>
void launch_attn_f(const DecodeArgs& a, dim3 grid, dim3 block, hipStream_t stream) {
#define KVQ_DECODE_ARGS                                                                                    \
  a.page_table, a.seq_lens, a.q, a.splits, a.num_kv_heads, a.max_pages, a.blocks_per_split, a.log2_page, \
      a.max_seq_len, a.n_rows, a.group, a
  if (a.rows <= 16)
    hipLaunchKernelGGL((decode_kernel<D, 1, VB, WIN, F8>), grid, block, 0, stream, KVQ_DECODE_ARGS);
  else
    hipLaunchKernelGGL((decode_kernel<D, 2, VB, WIN, F8>), grid, block, 0, stream, KVQ_DECODE_ARGS);
#undef KVQ_DECODE_ARGS
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
  const unsigned per_unit = (unsigned)merge_groups(a.rows, D);  // grid size checked on the host
  launch_merge<D>(a, units * per_unit, stream);
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

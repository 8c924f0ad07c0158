// kvq_append.hip — quantize new tokens' K/V rows and write them into their cache slots: one
// 64-lane wave per row of one token and KV head, four rows per wave, with the row quantizer of
// kvq_quant.h.  Every byte written belongs to its token alone, so concurrent tokens never
// touch the same byte.
#include "kvq_quant.h"

namespace kvq {
namespace {

// One workgroup (4 waves) per 16 consecutive tokens of one KV head; wave w quantizes tokens
// 4w .. 4w + 3 of the group.  When the 16 tokens go to the 16 slots of one tile, in order (a
// prefill, or a chunk of one), the waves quantize them into an LDS copy of that tile and then
// all 256 threads write the tile's four sections with 16-byte stores that fill whole cache
// lines; the copy is laid out as a page of one tile (P = 16), which has the tile's byte layout,
// so the same row quantizer produces the same bytes.  Otherwise each token is written into its
// own slot.  A wave's four rows are loaded before any is quantized, so its loads are in flight
// together; four rows per wave keep the registers low enough for eight waves per SIMD, and a
// 1024-token chunk of four KV heads is 1024 waves.
constexpr int kGroupTokens = kTile;
constexpr int kRowsPerWave = kGroupTokens / 4;

template <int D>
__device__ inline void copy16(uint8_t* dst, const uint8_t* src, int bytes, int tid) {
  typedef uint32_t u32x4v __attribute__((ext_vector_type(4)));
  for (int o = 16 * tid; o < bytes; o += 16 * 256)
    __builtin_nontemporal_store(*(const u32x4v*)(src + o), (u32x4v*)(dst + o));  // written once, not re-read here
}

template <int D, int VB, bool F8>
__global__ __launch_bounds__(256) void append_kernel(AppendArgs a) {
  constexpr int TB = (int)block_bytes(kTile, D, VB);  // one tile as a one-tile page
  __shared__ __attribute__((aligned(16))) uint8_t s_tile[TB];
  const int lane = threadIdx.x & (kWave - 1);
  const int wv = threadIdx.x >> 6;
  const long long item = blockIdx.x;  // (group of 16 tokens, KV head): uniform over the workgroup
  const long long groups = ((long long)a.n_tok + kGroupTokens - 1) / kGroupTokens;
  if (item >= groups * a.num_kv_heads) return;
  const int h = (int)(item % a.num_kv_heads);
  const int n0 = (int)(item / a.num_kv_heads) * kGroupTokens;
  const int cnt = min(kGroupTokens, a.n_tok - n0);
  const int P = a.page_size;
  const long long pool_slots = (long long)a.num_pages * P;
  // slots of the group: lane i < cnt holds token n0 + i's (every wave loads all 16, so each
  // takes the same tile-or-rows decision on its own)
  const long long my_slot = lane < cnt ? (long long)a.slots[n0 + lane] : -1;
  debug_report(a.dbg, my_slot >= pool_slots, kDbgSlot);  // (negative slots mark padding)
  RowVals<D> rv[kRowsPerWave];
#pragma unroll
  for (int i = 0; i < kRowsPerWave; ++i) {
    const int n = n0 + min(kRowsPerWave * wv + i, cnt - 1);  // (past a short group: its last row again)
    const size_t row = ((size_t)n * a.num_kv_heads + h) * D;
    rv[i] = load_row<D>(a.k + row, a.v + row, lane);
  }
  const long long s0 = __builtin_amdgcn_readfirstlane((int)my_slot);  // slots fit in int32
  const bool in_tile = lane >= kTile || my_slot == s0 + lane;
  const bool whole = cnt == kTile && s0 >= 0 && (s0 & (kTile - 1)) == 0 && s0 + kTile <= pool_slots &&
                     __ballot(!in_tile) == 0;
  if (whole) {  // the same in every wave of the workgroup
#pragma unroll
    for (int i = 0; i < kRowsPerWave; ++i) store_row<D, VB, F8>(s_tile, kTile, kRowsPerWave * wv + i, rv[i], lane);
    __syncthreads();  // the copies below read bytes every wave wrote
    const int tid = threadIdx.x;
    const int page = (int)(s0 / P), tile = (int)(s0 % P) / kTile;
    uint8_t* blk = a.pool + ((size_t)page * a.num_kv_heads + h) * block_bytes(P, D, VB);
    copy16<D>(blk + (size_t)kTile * D * tile, s_tile, kTile * D, tid);                                 // K codes
    copy16<D>(blk + k_scales_at(P, D) + 2 * kTile * tile, s_tile + k_scales_at(kTile, D), 2 * kTile, tid);
    constexpr int VT = kTile * D * VB / 8;  // V code bytes of one tile
    copy16<D>(blk + v_codes_at(P, D) + (size_t)VT * tile, s_tile + v_codes_at(kTile, D), VT, tid);
    copy16<D>(blk + v_scales_at(P, D, VB) + (size_t)2 * kTile * (D / 32) * tile, s_tile + v_scales_at(kTile, D, VB),
              2 * kTile * (D / 32), tid);
    return;
  }
#pragma unroll
  for (int i = 0; i < kRowsPerWave; ++i) {  // (a constant trip count: rv stays in registers)
    const int t = kRowsPerWave * wv + i;
    const long long slot = __builtin_amdgcn_readlane((int)my_slot, t);
    if (t < cnt && slot >= 0 && slot < pool_slots) {  // padding / out of pool: skip
      const int page = (int)(slot / P), s = (int)(slot % P);
      store_row<D, VB, F8>(a.pool + ((size_t)page * a.num_kv_heads + h) * block_bytes(P, D, VB), P, s, rv[i], lane);
    }
  }
}

}  // namespace

hipError_t launch_append(int head_dim, const AppendArgs& a, hipStream_t stream) {
  const long long groups = ((long long)a.n_tok + kGroupTokens - 1) / kGroupTokens;
  const long long items = groups * a.num_kv_heads;  // one workgroup each (grid size checked on the host)
  const dim3 grid((unsigned)items), block(256);
  const int kind = a.fp8 ? 2 : a.vbits == 8 ? 1 : 0;  // fp8 / 8-bit / 4-bit V codes
  switch (head_dim * 4 + kind) {
#define KVQ_APPEND_CASE(D)                                                                      \
  case 4 * D + 0: hipLaunchKernelGGL((append_kernel<D, 4, false>), grid, block, 0, stream, a); break; \
  case 4 * D + 1: hipLaunchKernelGGL((append_kernel<D, 8, false>), grid, block, 0, stream, a); break; \
  case 4 * D + 2: hipLaunchKernelGGL((append_kernel<D, 8, true>), grid, block, 0, stream, a); break;
    KVQ_APPEND_CASE(64)
    KVQ_APPEND_CASE(128)
    KVQ_APPEND_CASE(256)
#undef KVQ_APPEND_CASE
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace kvq

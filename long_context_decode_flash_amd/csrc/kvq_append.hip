// kvq_append.hip — quantize new tokens' K/V rows and write them into their cache slots: one
// 64-lane wave per group of consecutive tokens of one KV head, the row quantizer of
// kvq_quant.h.  Every byte written belongs to its token alone, so concurrent tokens never
// touch the same byte.
#include "kvq_quant.h"

namespace kvq {
namespace {

// One wave per 16 consecutive tokens of one KV head.  When the 16 tokens go to the 16 slots of
// one tile, in order (a prefill, or a chunk of one), the wave quantizes them into an LDS copy of
// that tile and writes the tile's four sections with 16-byte stores that fill whole cache lines;
// the copy is laid out as a page of one tile (P = 16), which has the tile's byte layout, so the
// same row quantizer produces the same bytes.  Otherwise each token is written into its own slot.
// All of a wave's rows are loaded before any is quantized, so its loads are in flight together.
constexpr int kTokensPerWave = kTile;

template <int D>
__device__ inline void copy16(uint8_t* dst, const uint8_t* src, int bytes, int lane) {
  for (int o = 16 * lane; o < bytes; o += 16 * kWave) *(uint4*)(dst + o) = *(const uint4*)(src + o);
}

template <int D, int VB, bool F8>
__global__ __launch_bounds__(256) void append_kernel(AppendArgs a) {
  constexpr int TB = (int)block_bytes(kTile, D, VB);  // one tile as a one-tile page
  __shared__ __attribute__((aligned(16))) uint8_t s_tile[4][TB];
  const int lane = threadIdx.x & (kWave - 1);
  const int wv = threadIdx.x >> 6;
  const long long item = (long long)blockIdx.x * 4 + wv;
  const long long groups = ((long long)a.n_tok + kTokensPerWave - 1) / kTokensPerWave;
  if (item >= groups * a.num_kv_heads) return;
  const int h = (int)(item % a.num_kv_heads);
  const int n0 = (int)(item / a.num_kv_heads) * kTokensPerWave;
  const int cnt = min(kTokensPerWave, a.n_tok - n0);
  const int P = a.page_size;
  const long long pool_slots = (long long)a.num_pages * P;
  // slots of the group: lane i < cnt holds token n0 + i's
  const long long my_slot = lane < cnt ? (long long)a.slots[n0 + lane] : -1;
  RowVals<D> rv[kTokensPerWave];
#pragma unroll
  for (int i = 0; i < kTokensPerWave; ++i) {
    const int n = n0 + min(i, cnt - 1);  // (a short last group reloads its last row)
    const size_t row = ((size_t)n * a.num_kv_heads + h) * D;
    rv[i] = load_row<D>(a.k + row, a.v + row, lane);
  }
  const long long s0 = __builtin_amdgcn_readfirstlane((int)my_slot);  // slots fit in int32
  const bool in_tile = lane >= kTile || my_slot == s0 + lane;
  const bool whole = cnt == kTile && s0 >= 0 && (s0 & (kTile - 1)) == 0 && s0 + kTile <= pool_slots &&
                     __ballot(!in_tile) == 0;
  if (whole) {
    uint8_t* st = s_tile[wv];
#pragma unroll
    for (int i = 0; i < kTokensPerWave; ++i) store_row<D, VB, F8>(st, kTile, i, rv[i], lane);
    wave_lds_order();  // the copies below read bytes other lanes wrote
    const int page = (int)(s0 / P), tile = (int)(s0 % P) / kTile;
    uint8_t* blk = a.pool + ((size_t)page * a.num_kv_heads + h) * block_bytes(P, D, VB);
    copy16<D>(blk + (size_t)kTile * D * tile, st, kTile * D, lane);                                 // K codes
    copy16<D>(blk + k_scales_at(P, D) + 2 * kTile * tile, st + k_scales_at(kTile, D), 2 * kTile, lane);
    constexpr int VT = kTile * D * VB / 8;  // V code bytes of one tile
    copy16<D>(blk + v_codes_at(P, D) + (size_t)VT * tile, st + v_codes_at(kTile, D), VT, lane);
    copy16<D>(blk + v_scales_at(P, D, VB) + (size_t)2 * kTile * (D / 32) * tile, st + v_scales_at(kTile, D, VB),
              2 * kTile * (D / 32), lane);
    return;
  }
#pragma unroll
  for (int i = 0; i < kTokensPerWave; ++i) {  // (a constant trip count: rv stays in registers)
    const long long slot = __builtin_amdgcn_readlane((int)my_slot, i);
    if (i < cnt && slot >= 0 && slot < pool_slots) {  // padding / out of pool: skip
      const int page = (int)(slot / P), s = (int)(slot % P);
      store_row<D, VB, F8>(a.pool + ((size_t)page * a.num_kv_heads + h) * block_bytes(P, D, VB), P, s, rv[i], lane);
    }
  }
}

}  // namespace

hipError_t launch_append(int head_dim, const AppendArgs& a, hipStream_t stream) {
  const long long groups = ((long long)a.n_tok + kTokensPerWave - 1) / kTokensPerWave;
  const long long items = groups * a.num_kv_heads;
  const dim3 grid((unsigned)((items + 3) / 4)), block(256);
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

// kvq_internal.h — shared declarations of the HIP library (device code for gfx950 only).
//
// The page format is the one stated in include/kvq.h; the helpers here are the library's own
// implementation of it (the CPU oracle has a separate one).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "kvq.h"

namespace kvq {

constexpr int kTile = 16;        // tokens per tile
constexpr int kBlock = 32;       // tokens per decode step of one wave (two tiles)
constexpr int kWave = 64;
constexpr int kWavesPerGroup = 4;  // waves of one decode workgroup
constexpr int kMaxSplits = 128;    // workgroups per (sequence, KV head) at most

// VB: bits per V code, 4 (K8/V4: two codes per byte) or 8 (K8/V8: one per byte).
__host__ __device__ constexpr size_t block_bytes(int P, int D, int VB = 4) {
  return (size_t)P * (size_t)(D + 2 + D * VB / 8 + D / 16);
}
__host__ __device__ constexpr size_t k_scales_at(int P, int D) { return (size_t)P * D; }
__host__ __device__ constexpr size_t v_codes_at(int P, int D) { return (size_t)P * D + 2 * (size_t)P; }
__host__ __device__ constexpr size_t v_scales_at(int P, int D, int VB = 4) {
  return (size_t)P * D + 2 * (size_t)P + (size_t)P * D * VB / 8;
}

// (max, sum) entries per unit in the decode workspace: splits x rows, rounded up to an even
// count so each unit's entries start 16-byte aligned.
__host__ __device__ constexpr int ml_stride(int splits, int rows) { return (splits * rows + 1) & ~1; }

struct AppendArgs {
  uint8_t* pool;
  int num_pages, page_size, num_kv_heads;
  int vbits;  // 4 or 8
  int fp8;    // 1: K and V as OCP e4m3 codes (8-bit V layout)
  const float* k;
  const float* v;
  const int32_t* slots;
  int n_tok;
  unsigned* dbg;  // KVQ_DEBUG builds: the word range reports are ORed into (null otherwise)
};

struct DecodeArgs {
  const uint8_t* pool;
  int num_pages, page_size, num_kv_heads;
  int vbits;  // 4 or 8
  int fp8;    // 1: K and V as OCP e4m3 codes (8-bit V layout)
  int log2_page;  // page_size = 1 << log2_page
  const uint16_t* q;
  const int32_t* page_table;
  const int32_t* seq_lens;
  int n_seq, n_rows, n_q_heads, group, rows;  // rows = group * n_rows (query rows per KV head)
  int max_pages, max_seq_len;
  // window > 0: row i sees only tokens L - n_rows + i - window + 1 ..; the splits then cover the
  // blocks from the first row's window start on.  ring > 0: logical page n of a sequence is in
  // page-table entry n % ring.  0 and 0: the whole context through a linear page table.
  int window, ring;
  int splits, blocks_per_split;  // workgroups per (sequence, KV head), 32-token blocks each
  int row_tiles;  // prefill: tiles of 128 query rows per (sequence, KV head)
  float scale_log2;  // softmax_scale * log2(e)
  float* ws_acc;     // [units][splits][rows][D] partial numerators
  float2* ws_ml;     // [units][ml_stride(splits, rows)] (max in log2 units, sum of exp2)
  float* out;
  float* lse;
  // fused append (kvq_decode_step): the last n_new tokens of each sequence, fp32
  // [n_seq][n_new][num_kv_heads][D], quantized into their slots before they are attended
  uint8_t* pool_rw;
  const float* k_new;
  const float* v_new;
  int n_new;
  unsigned* dbg;  // KVQ_DEBUG builds: the word range reports are ORed into (null otherwise)
};

// ---- KVQ_DEBUG builds: device-side range reports ----
// Bits of the report word (KVQ_DBG_PAGE_ID and KVQ_DBG_SLOT of kvq_debug_errors).  The kernels still clamp an
// out-of-range page id and skip an out-of-pool slot; a debug build also records that it saw one.
constexpr unsigned kDbgPageId = KVQ_DBG_PAGE_ID;  // a page-table entry outside [0, num_pages)
constexpr unsigned kDbgSlot = KVQ_DBG_SLOT;       // an append slot at or past num_pages * page_size

__device__ inline void debug_report(unsigned* dbg, bool bad, unsigned bit) {
#ifdef KVQ_DEBUG
  if (bad) atomicOr(dbg, bit);
#else
  (void)dbg;
  (void)bad;
  (void)bit;
#endif
}

hipError_t launch_append(int head_dim, const AppendArgs& a, hipStream_t stream);
hipError_t launch_decode(int head_dim, const DecodeArgs& a, hipStream_t stream);
hipError_t launch_prefill(int head_dim, const DecodeArgs& a, hipStream_t stream);
hipError_t launch_stream_probe(const void* buf, size_t bytes, int mode, int workgroups, uint32_t* sink,
                               hipStream_t stream);
hipError_t launch_clock_probe(unsigned long long* out, int workgroups, unsigned ticks, hipStream_t stream);

constexpr int kPrefillRowsPerTile = 256;  // query rows of one prefill workgroup (32 per wave)
constexpr int kPrefillThreads = 512;      // 8 waves per prefill workgroup

// The split merge launch: kMergeLanes lanes per (unit, query row, 4 dims) item, kMergeItems
// items per 64-lane workgroup, merge_groups(rows, D) workgroups per unit.
constexpr int kMergeLanes = 8;                       // lanes per output item (4, 8 or 16)
constexpr int kMergeItems = kWave / kMergeLanes;     // items per wave
__host__ __device__ constexpr unsigned long long merge_groups(int rows, int head_dim) {
  return ((unsigned long long)rows * (head_dim / 4) + kMergeItems - 1) / kMergeItems;
}

}  // namespace kvq

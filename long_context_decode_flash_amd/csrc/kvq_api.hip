// kvq_api.hip — the C ABI of include/kvq.h: argument validation (all on the host, before any
// HIP call), split planning, workspace sizing and the launches.
#include "kvq.h"

#include <math.h>

#include <algorithm>
#include <mutex>

#include "kvq_internal.h"

namespace {

bool pow2_in(int x, int lo, int hi) { return x >= lo && x <= hi && (x & (x - 1)) == 0; }
bool head_dim_ok(int d) { return d == 64 || d == 128 || d == 256; }
// bits per V code of a KV format (the fp8 format uses the 8-bit V layout), or 0 for an unknown
// format
int vbits_of(int32_t kv_format) {
  return kv_format == KVQ_FORMAT_K8V4 ? 4
         : (kv_format == KVQ_FORMAT_K8V8 || kv_format == KVQ_FORMAT_FP8) ? 8
                                                                          : 0;
}

// Workgroups (4 waves each) the decode grid aims for: one per CU of the 256.
constexpr long long kTargetGroups = 256;
// A split covers at least one 32-token block per wave of its workgroup.
constexpr long long kMinBlocksPerSplit = kvq::kWavesPerGroup;
// Workgroups that keep HBM saturated (90% of the CUs): with at least this many streaming, a
// bandwidth-bound decode gains nothing from more.
constexpr long long kSaturatingGroups = 230;

long long ceil_div(long long a, long long b) { return (a + b - 1) / b; }

struct Plan {
  int splits;
  int blocks_per_split;
};

// wave_bound: the format's block step is bound by the issue of its own wave (4-bit V: the V
// widening and the split of P * s_v); otherwise by HBM bandwidth (8-bit V: 32% more bytes per
// token for about the same instructions).
int plan_splits(int n_seq, int num_kv_heads, int max_seq_len, int request, Plan* plan,
                bool wave_bound) {
  if (n_seq <= 0 || num_kv_heads <= 0 || max_seq_len <= 0 || request < 0) return KVQ_ERR_ARG;
  const long long nblk = ceil_div(max_seq_len, kvq::kBlock);
  const long long units = (long long)n_seq * num_kv_heads;
  long long s;
  if (request > 0) {
    s = request;
  } else {
    // At most one workgroup per CU, about (a grid past the CU count runs in rounds).  A split's
    // blocks go to its 4 waves in turn.  Wave-bound: one wave per SIMD cannot hide its own block
    // step, so the time follows the blocks of the busiest wave: (blocks of the busiest wave) x
    // (rounds of workgroups), the fewest splits on ties (less partial traffic and merge work).
    // Bandwidth-bound: a wave with one block more than the others idles part of its CU's
    // bandwidth at the end, and fewer workgroups than the saturating count each stream
    // proportionally faster: (blocks of the busiest wave) x max(workgroups, saturating count),
    // the most splits on ties.
    long long s_max = ceil_div(kTargetGroups, units);
    const long long cap = ceil_div(nblk, kMinBlocksPerSplit);
    s_max = s_max < cap ? s_max : cap;
    s = 1;
    long long best = -1;
    for (long long c = 1; c <= s_max; ++c) {
      const long long bps = ceil_div(nblk, c);
      const long long used = ceil_div(nblk, bps);  // splits that start inside the context
      const long long groups = units * used;
      const long long per_wave = ceil_div(bps, kvq::kWavesPerGroup);
      const long long t = wave_bound ? per_wave * ceil_div(groups, kTargetGroups)
                                     : per_wave * (groups > kSaturatingGroups ? groups : kSaturatingGroups);
      if (best < 0 || (wave_bound ? t < best : t <= best)) {
        best = t;
        s = c;
      }
    }
  }
  if (s < 1) s = 1;
  if (s > nblk) s = nblk;
  if (s > kvq::kMaxSplits) s = kvq::kMaxSplits;
  const long long bps = ceil_div(nblk, s);
  s = ceil_div(nblk, bps);  // drop splits that would start past the last block
  if (units * s > (1LL << 30)) return KVQ_ERR_ARG;
  plan->splits = (int)s;
  plan->blocks_per_split = (int)bps;
  return KVQ_OK;
}

// Workspace: [partial numerators units x splits x rows x D fp32][partial (max, sum)
// units x ml_stride(splits, rows) x 2 fp32].  Nothing in it needs initializing.
size_t workspace_for(long long units, int splits, int rows, int head_dim) {
  if (splits == 1) return 16;  // one split writes the output directly
  const size_t acc = (size_t)units * splits * rows * head_dim * sizeof(float);
  const size_t ml = (size_t)units * kvq::ml_stride(splits, rows) * 2 * sizeof(float);
  return acc + ml;
}

// Every launch of a call counts fewer than 2^32 work-items (HIP's grid limit): the attention
// grid (units x row tiles x splits workgroups of `threads`) and, with more than one split, the
// merge grid (units x merge_groups(rows, D) workgroups of one wave).
bool grids_fit(long long units, int row_tiles, int splits, int threads, int rows, int head_dim) {
  const unsigned long long lim = 1ULL << 32;
  const unsigned long long attn = (unsigned long long)units * row_tiles * splits * threads;
  const unsigned long long merge =
      splits > 1 ? (unsigned long long)units * kvq::merge_groups(rows, head_dim) * kvq::kWave : 0;
  return attn < lim && merge < lim;
}

int pool_args_ok(const void* pool, int32_t num_pages, int32_t page_size, int32_t num_kv_heads,
                 int32_t head_dim, int vb) {
  if (!pool || num_pages <= 0 || num_kv_heads <= 0 || page_size <= 0) return KVQ_ERR_ARG;
  if (vb == 0 || !head_dim_ok(head_dim) || !pow2_in(page_size, 16, 256)) return KVQ_ERR_UNSUPPORTED;
  if (((uintptr_t)pool & 15) != 0) return KVQ_ERR_ARG;
  // one page of all KV heads stays below 4 GiB (the kernels address within it in 32 bits)
  if ((unsigned long long)num_kv_heads * kvq::block_bytes(page_size, head_dim, vb) >= (1ULL << 32))
    return KVQ_ERR_UNSUPPORTED;
  return KVQ_OK;
}

#ifdef KVQ_DEBUG
// The range-report word of KVQ_DEBUG builds: one per GPU; host code reaches it only through the
// address hipGetSymbolAddress returns for the current device, looked up once per device.
static __device__ __align__(256) unsigned debug_word;
std::mutex g_dbg_mu;
unsigned* g_dbg_at[64];  // per device (up to 64): the device address of `debug_word`
#endif

// Device address of the current device's report word (KVQ_DEBUG builds), or nullptr in other
// builds; KVQ_ERR_HIP if the lookup fails.
int debug_address(unsigned** at) {
  *at = nullptr;
#ifdef KVQ_DEBUG
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return KVQ_ERR_HIP;
  std::lock_guard<std::mutex> lock(g_dbg_mu);
  if (g_dbg_at[dev] == nullptr) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(debug_word)) != hipSuccess || p == nullptr) return KVQ_ERR_HIP;
    g_dbg_at[dev] = (unsigned*)p;
  }
  *at = g_dbg_at[dev];
#endif
  return KVQ_OK;
}

}  // namespace

extern "C" {

size_t kvq_block_bytes_fmt(int32_t kv_format, int32_t page_size, int32_t head_dim) {
  const int vb = vbits_of(kv_format);
  if (vb == 0 || !head_dim_ok(head_dim) || !pow2_in(page_size, 16, 256)) return 0;
  return kvq::block_bytes(page_size, head_dim, vb);
}

size_t kvq_block_bytes(int32_t page_size, int32_t head_dim) {
  return kvq_block_bytes_fmt(KVQ_FORMAT_K8V4, page_size, head_dim);
}

const char* kvq_strerror(int code) {
  switch (code) {
    case KVQ_OK: return "ok";
    case KVQ_ERR_ARG: return "invalid argument (NULL pointer, non-positive or inconsistent size)";
    case KVQ_ERR_UNSUPPORTED: return "unsupported shape (head_dim, page_size or rows per KV head)";
    case KVQ_ERR_WORKSPACE: return "workspace missing or smaller than kvq_decode_workspace_bytes()";
    case KVQ_ERR_HIP: return "HIP launch error";
    case KVQ_ERR_SCRATCH:
      return "the call needs more split scratch than the library's static array holds (KVQ_NOALLOC_SCRATCH_BYTES)";
  }
  return "unknown kvq error code";
}

int32_t kvq_decode_num_splits(int32_t n_seq, int32_t num_kv_heads, int32_t max_seq_len,
                              int32_t num_splits_request) {
  Plan p;
  const int rc = plan_splits(n_seq, num_kv_heads, max_seq_len, num_splits_request, &p, true);
  return rc == KVQ_OK ? p.splits : rc;
}

size_t kvq_decode_workspace_bytes(int32_t n_seq, int32_t n_rows, int32_t n_q_heads,
                                  int32_t num_kv_heads, int32_t head_dim, int32_t max_seq_len,
                                  int32_t num_splits_request) {
  if (n_rows <= 0 || n_q_heads <= 0 || num_kv_heads <= 0 || n_q_heads % num_kv_heads != 0 ||
      !head_dim_ok(head_dim))
    return 0;
  // the larger of the two formats' plans (the workspace grows with the splits)
  Plan p, p8;
  if (plan_splits(n_seq, num_kv_heads, max_seq_len, num_splits_request, &p, true) != KVQ_OK ||
      plan_splits(n_seq, num_kv_heads, max_seq_len, num_splits_request, &p8, false) != KVQ_OK)
    return 0;
  const int rows = (n_q_heads / num_kv_heads) * n_rows;
  const int splits = p.splits > p8.splits ? p.splits : p8.splits;
  return workspace_for((long long)n_seq * num_kv_heads, splits, rows, head_dim);
}

int kvq_append_fmt(int32_t kv_format, void* pool, int32_t num_pages, int32_t page_size,
                   int32_t num_kv_heads, int32_t head_dim, const float* k, const float* v,
                   const int32_t* slot_mapping, int32_t n_tok, void* stream) {
  const int vb = vbits_of(kv_format);
  int rc = pool_args_ok(pool, num_pages, page_size, num_kv_heads, head_dim, vb);
  if (rc != KVQ_OK) return rc;
  if (n_tok < 0) return KVQ_ERR_ARG;
  if (n_tok == 0) return KVQ_OK;
  if (!k || !v || !slot_mapping) return KVQ_ERR_ARG;
  // one 256-thread workgroup per 16 tokens and KV head: fewer than 2^32 work-items
  if ((unsigned long long)((n_tok + 15) / 16) * num_kv_heads * 256 >= (1ULL << 32)) return KVQ_ERR_UNSUPPORTED;
  kvq::AppendArgs a{(uint8_t*)pool, num_pages,    page_size, num_kv_heads, vb,
                    kv_format == KVQ_FORMAT_FP8, k, v,         slot_mapping, n_tok, nullptr};
  rc = debug_address(&a.dbg);
  if (rc != KVQ_OK) return rc;
  (void)hipGetLastError();  // start from a clean error state
  return kvq::launch_append(head_dim, a, (hipStream_t)stream) == hipSuccess ? KVQ_OK : KVQ_ERR_HIP;
}

int kvq_append(void* pool, int32_t num_pages, int32_t page_size, int32_t num_kv_heads,
               int32_t head_dim, const float* k, const float* v, const int32_t* slot_mapping,
               int32_t n_tok, void* stream) {
  return kvq_append_fmt(KVQ_FORMAT_K8V4, pool, num_pages, page_size, num_kv_heads, head_dim, k, v,
                        slot_mapping, n_tok, stream);
}

}  // extern "C"

namespace {

// Tokens whose blocks one context piece plan covers: the whole context, or with a window the
// W + n_rows - 1 positions the rows see plus up to 31 tokens of the first block before them.
long long span_tokens(int32_t max_seq_len, int32_t n_rows, int32_t window) {
  if (window <= 0) return max_seq_len;
  const long long w = (long long)window + n_rows - 1 + (kvq::kBlock - 1);
  return w < max_seq_len ? w : max_seq_len;
}

// Ring pages every call must hold so that no token a row sees has been overwritten: W + n_rows
// - 1 consecutive tokens at any offset within a page span at most this many pages.
long long ring_pages_needed(int32_t page_size, int32_t n_rows, int32_t window) {
  return ((long long)window + n_rows - 1 + page_size - 2) / page_size + 1;
}

// The split partials of kvq_decode_step_noalloc (nothing in them needs clearing: every entry
// a launch reads, the same launch wrote first).  Each GPU the library runs on holds its own
// copy until the process ends; host code reaches it only through the address that
// hipGetSymbolAddress returns for the current device, never through the array's name.
static __device__ __align__(256) uint8_t scratch[KVQ_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_at[kMaxDevices];  // per device: the device address of `scratch`, once looked up

// Device address of the current device's copy of `scratch`, looked up on the first call on
// that device (with it current) and kept.
int scratch_address(void** at) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return KVQ_ERR_HIP;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_at[dev] == nullptr) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) return KVQ_ERR_HIP;
    g_scratch_at[dev] = p;
  }
  *at = g_scratch_at[dev];
  return KVQ_OK;
}

int decode_impl(int32_t kv_format, const void* pool, int32_t num_pages, int32_t page_size,
                int32_t num_kv_heads, int32_t head_dim, const float* k_new, const float* v_new, int32_t n_new,
                const uint16_t* q, const int32_t* page_table, const int32_t* seq_lens, int32_t n_seq,
                int32_t n_rows, int32_t n_q_heads, int32_t max_pages_per_seq, int32_t max_seq_len,
                int32_t window, int32_t ring_pages, float softmax_scale, int32_t num_splits,
                float* out, float* lse, void* workspace, size_t workspace_bytes, void* stream,
                bool noalloc = false) {
  const int vb = vbits_of(kv_format);
  int rc = pool_args_ok(pool, num_pages, page_size, num_kv_heads, head_dim, vb);
  if (rc != KVQ_OK) return rc;
  if (!q || !page_table || !seq_lens || !out) return KVQ_ERR_ARG;
  if (n_seq <= 0 || n_q_heads <= 0 || max_pages_per_seq <= 0 || max_seq_len <= 0 ||
      num_splits < 0)
    return KVQ_ERR_ARG;
  if (n_rows < 1 || n_rows > KVQ_MAX_N_ROWS) return KVQ_ERR_UNSUPPORTED;
  if (n_q_heads % num_kv_heads != 0) return KVQ_ERR_ARG;
  const int group = n_q_heads / num_kv_heads;
  if ((long long)group * n_rows > KVQ_MAX_ROWS_PER_KV) return KVQ_ERR_UNSUPPORTED;
  if (window < 0 || ring_pages < 0 || (ring_pages > 0 && window == 0)) return KVQ_ERR_ARG;
  if (ring_pages > 0) {
    if (ring_pages > max_pages_per_seq || ring_pages < ring_pages_needed(page_size, n_rows, window))
      return KVQ_ERR_ARG;
  } else if ((long long)max_seq_len > (long long)max_pages_per_seq * page_size) {
    return KVQ_ERR_ARG;
  }
  // a fused step appends only tokens some row sees (the pieces that attend them write them)
  if (window > 0 && (long long)n_new > (long long)window + n_rows - 1) return KVQ_ERR_ARG;
  if (!(softmax_scale == softmax_scale) || isinf(softmax_scale)) return KVQ_ERR_ARG;
  if (((uintptr_t)q & 15) != 0 || ((uintptr_t)out & 15) != 0) return KVQ_ERR_ARG;
  Plan plan;
  rc = plan_splits(n_seq, num_kv_heads, (int)span_tokens(max_seq_len, n_rows, window), num_splits,
                   &plan, vb == 4);
  if (rc != KVQ_OK) return rc;
  const int rows = group * n_rows;
  const long long units = (long long)n_seq * num_kv_heads;
  if (!grids_fit(units, 1, plan.splits, kvq::kWave * kvq::kWavesPerGroup, rows, head_dim))
    return KVQ_ERR_UNSUPPORTED;
  const size_t need = workspace_for(units, plan.splits, rows, head_dim);
  if (noalloc) {
    // the partials go to this device's copy of the library's static array instead
    if (need > (size_t)KVQ_NOALLOC_SCRATCH_BYTES) return KVQ_ERR_SCRATCH;
    rc = scratch_address(&workspace);
    if (rc != KVQ_OK) return rc;
    workspace_bytes = KVQ_NOALLOC_SCRATCH_BYTES;
  }
  if (!workspace || workspace_bytes < need || ((uintptr_t)workspace & 15) != 0)
    return KVQ_ERR_WORKSPACE;
  const double scale = softmax_scale > 0.0f ? (double)softmax_scale : 1.0 / sqrt((double)head_dim);

  kvq::DecodeArgs a{};
  a.pool = (const uint8_t*)pool;
  a.num_pages = num_pages;
  a.page_size = page_size;
  a.num_kv_heads = num_kv_heads;
  a.vbits = vb;
  a.fp8 = kv_format == KVQ_FORMAT_FP8;
  a.log2_page = __builtin_ctz((unsigned)page_size);
  a.q = q;
  a.page_table = page_table;
  a.seq_lens = seq_lens;
  a.n_seq = n_seq;
  a.n_rows = n_rows;
  a.n_q_heads = n_q_heads;
  a.group = group;
  a.rows = rows;
  a.max_pages = max_pages_per_seq;
  a.max_seq_len = max_seq_len;
  a.window = window;
  a.ring = ring_pages;
  a.splits = plan.splits;
  a.blocks_per_split = plan.blocks_per_split;
  a.scale_log2 = (float)(scale * 1.4426950408889634074);
  a.ws_acc = (float*)workspace;
  a.ws_ml = (float2*)((char*)a.ws_acc + (size_t)units * plan.splits * rows * head_dim * sizeof(float));
  a.out = out;
  a.lse = lse;
  a.pool_rw = (uint8_t*)pool;
  a.k_new = k_new;
  a.v_new = v_new;
  a.n_new = n_new;
  rc = debug_address(&a.dbg);
  if (rc != KVQ_OK) return rc;
  (void)hipGetLastError();
  return kvq::launch_decode(head_dim, a, (hipStream_t)stream) == hipSuccess ? KVQ_OK : KVQ_ERR_HIP;
}

}  // namespace

extern "C" {

int kvq_decode_attn_fmt(int32_t kv_format, const void* pool, int32_t num_pages, int32_t page_size,
                        int32_t num_kv_heads, int32_t head_dim, const uint16_t* q,
                        const int32_t* page_table, const int32_t* seq_lens, int32_t n_seq,
                        int32_t n_rows, int32_t n_q_heads, int32_t max_pages_per_seq,
                        int32_t max_seq_len, float softmax_scale, int32_t num_splits, float* out,
                        float* lse, void* workspace, size_t workspace_bytes, void* stream) {
  return decode_impl(kv_format, pool, num_pages, page_size, num_kv_heads, head_dim, nullptr, nullptr, 0,
                     q, page_table, seq_lens, n_seq, n_rows, n_q_heads, max_pages_per_seq,
                     max_seq_len, 0, 0, softmax_scale, num_splits, out, lse, workspace,
                     workspace_bytes, stream);
}

int kvq_decode_attn(const void* pool, int32_t num_pages, int32_t page_size,
                    int32_t num_kv_heads, int32_t head_dim, const uint16_t* q,
                    const int32_t* page_table, const int32_t* seq_lens, int32_t n_seq,
                    int32_t n_rows, int32_t n_q_heads, int32_t max_pages_per_seq,
                    int32_t max_seq_len, float softmax_scale, int32_t num_splits, float* out,
                    float* lse, void* workspace, size_t workspace_bytes, void* stream) {
  return kvq_decode_attn_fmt(KVQ_FORMAT_K8V4, pool, num_pages, page_size, num_kv_heads, head_dim, q,
                             page_table, seq_lens, n_seq, n_rows, n_q_heads, max_pages_per_seq,
                             max_seq_len, softmax_scale, num_splits, out, lse, workspace,
                             workspace_bytes, stream);
}

int kvq_decode_step_fmt(int32_t kv_format, void* pool, int32_t num_pages, int32_t page_size,
                        int32_t num_kv_heads, int32_t head_dim, const float* k_new,
                        const float* v_new, int32_t n_new, const uint16_t* q,
                        const int32_t* page_table, const int32_t* seq_lens, int32_t n_seq,
                        int32_t n_rows, int32_t n_q_heads, int32_t max_pages_per_seq,
                        int32_t max_seq_len, float softmax_scale, int32_t num_splits, float* out,
                        float* lse, void* workspace, size_t workspace_bytes, void* stream) {
  if (n_new < 0 || n_new > KVQ_MAX_STEP_TOKENS) return KVQ_ERR_ARG;
  if (n_new > 0 && (!k_new || !v_new)) return KVQ_ERR_ARG;
  return decode_impl(kv_format, pool, num_pages, page_size, num_kv_heads, head_dim, k_new, v_new, n_new,
                     q, page_table, seq_lens, n_seq, n_rows, n_q_heads, max_pages_per_seq,
                     max_seq_len, 0, 0, softmax_scale, num_splits, out, lse, workspace,
                     workspace_bytes, stream);
}

int kvq_decode_step(void* pool, int32_t num_pages, int32_t page_size, int32_t num_kv_heads,
                    int32_t head_dim, const float* k_new, const float* v_new, int32_t n_new,
                    const uint16_t* q, const int32_t* page_table, const int32_t* seq_lens,
                    int32_t n_seq, int32_t n_rows, int32_t n_q_heads, int32_t max_pages_per_seq,
                    int32_t max_seq_len, float softmax_scale, int32_t num_splits, float* out,
                    float* lse, void* workspace, size_t workspace_bytes, void* stream) {
  return kvq_decode_step_fmt(KVQ_FORMAT_K8V4, pool, num_pages, page_size, num_kv_heads, head_dim, k_new,
                             v_new, n_new, q, page_table, seq_lens, n_seq, n_rows, n_q_heads,
                             max_pages_per_seq, max_seq_len, softmax_scale, num_splits, out, lse,
                             workspace, workspace_bytes, stream);
}

int kvq_decode_step_noalloc(int32_t kv_format, void* pool, int32_t num_pages, int32_t page_size,
                            int32_t num_kv_heads, int32_t head_dim, const float* k_new,
                            const float* v_new, int32_t n_new, const uint16_t* q,
                            const int32_t* page_table, const int32_t* seq_lens, int32_t n_seq,
                            int32_t n_rows, int32_t n_q_heads, int32_t max_pages_per_seq,
                            int32_t max_seq_len, float softmax_scale, int32_t num_splits,
                            float* out, float* lse, void* stream) {
  if (n_new < 0 || n_new > KVQ_MAX_STEP_TOKENS) return KVQ_ERR_ARG;
  if (n_new > 0 && (!k_new || !v_new)) return KVQ_ERR_ARG;
  return decode_impl(kv_format, pool, num_pages, page_size, num_kv_heads, head_dim, k_new, v_new, n_new,
                     q, page_table, seq_lens, n_seq, n_rows, n_q_heads, max_pages_per_seq,
                     max_seq_len, 0, 0, softmax_scale, num_splits, out, lse, nullptr, 0, stream,
                     /*noalloc=*/true);
}

int32_t kvq_decode_num_splits_win(int32_t n_seq, int32_t num_kv_heads, int32_t max_seq_len,
                                  int32_t n_rows, int32_t window, int32_t num_splits_request) {
  return kvq_decode_num_splits_fmt(KVQ_FORMAT_K8V4, n_seq, num_kv_heads, max_seq_len, n_rows, window,
                                   num_splits_request);
}

int32_t kvq_decode_num_splits_fmt(int32_t kv_format, int32_t n_seq, int32_t num_kv_heads,
                                  int32_t max_seq_len, int32_t n_rows, int32_t window,
                                  int32_t num_splits_request) {
  const int vb = vbits_of(kv_format);
  if (vb == 0) return KVQ_ERR_UNSUPPORTED;
  if (n_rows < 1 || window < 0) return KVQ_ERR_ARG;
  Plan p;
  const int rc = plan_splits(n_seq, num_kv_heads, (int)span_tokens(max_seq_len, n_rows, window),
                             num_splits_request, &p, vb == 4);
  return rc == KVQ_OK ? p.splits : rc;
}

size_t kvq_decode_workspace_bytes_win(int32_t n_seq, int32_t n_rows, int32_t n_q_heads,
                                      int32_t num_kv_heads, int32_t head_dim, int32_t max_seq_len,
                                      int32_t window, int32_t num_splits_request) {
  if (n_rows <= 0 || window < 0) return 0;
  return kvq_decode_workspace_bytes(n_seq, n_rows, n_q_heads, num_kv_heads, head_dim,
                                    (int32_t)span_tokens(max_seq_len, n_rows, window),
                                    num_splits_request);
}

int kvq_decode_attn_win(int32_t kv_format, const void* pool, int32_t num_pages, int32_t page_size,
                        int32_t num_kv_heads, int32_t head_dim, const uint16_t* q,
                        const int32_t* page_table, const int32_t* seq_lens, int32_t n_seq,
                        int32_t n_rows, int32_t n_q_heads, int32_t max_pages_per_seq,
                        int32_t max_seq_len, int32_t window, int32_t ring_pages,
                        float softmax_scale, int32_t num_splits, float* out, float* lse,
                        void* workspace, size_t workspace_bytes, void* stream) {
  return decode_impl(kv_format, pool, num_pages, page_size, num_kv_heads, head_dim, nullptr, nullptr, 0,
                     q, page_table, seq_lens, n_seq, n_rows, n_q_heads, max_pages_per_seq,
                     max_seq_len, window, ring_pages, softmax_scale, num_splits, out, lse,
                     workspace, workspace_bytes, stream);
}

int kvq_decode_step_win(int32_t kv_format, void* pool, int32_t num_pages, int32_t page_size,
                        int32_t num_kv_heads, int32_t head_dim, const float* k_new,
                        const float* v_new, int32_t n_new, const uint16_t* q,
                        const int32_t* page_table, const int32_t* seq_lens, int32_t n_seq,
                        int32_t n_rows, int32_t n_q_heads, int32_t max_pages_per_seq,
                        int32_t max_seq_len, int32_t window, int32_t ring_pages,
                        float softmax_scale, int32_t num_splits, float* out, float* lse,
                        void* workspace, size_t workspace_bytes, void* stream) {
  if (n_new < 0 || n_new > KVQ_MAX_STEP_TOKENS) return KVQ_ERR_ARG;
  if (n_new > 0 && (!k_new || !v_new)) return KVQ_ERR_ARG;
  return decode_impl(kv_format, pool, num_pages, page_size, num_kv_heads, head_dim, k_new, v_new, n_new,
                     q, page_table, seq_lens, n_seq, n_rows, n_q_heads, max_pages_per_seq,
                     max_seq_len, window, ring_pages, softmax_scale, num_splits, out, lse,
                     workspace, workspace_bytes, stream);
}

}  // extern "C"

// ---- chunked prefill ------------------------------------------------------------------------

namespace {

// Pieces per (sequence, KV head, row tile) for the prefill: the count whose grid fills the 256
// CUs in the fewest rounds per unit of work (one workgroup per CU), each piece keeping at least
// 8 blocks, the smallest such count on ties (fewer partials to merge).
int plan_prefill(int n_seq, int num_kv_heads, int rows, int max_seq_len, int request, Plan* plan,
                 int* row_tiles) {
  if (n_seq <= 0 || num_kv_heads <= 0 || rows <= 0 || max_seq_len <= 0 || request < 0)
    return KVQ_ERR_ARG;
  const long long nblk = ceil_div(max_seq_len, kvq::kBlock);
  const long long tiles = ceil_div(rows, kvq::kPrefillRowsPerTile);
  const long long work = (long long)n_seq * num_kv_heads * tiles;
  long long s = 1;
  if (request > 0) {
    s = request;
  } else {
    const long long s_max = std::max(1LL, std::min(16LL, nblk / 8));
    double best = 0.0;
    for (long long c = 1; c <= s_max; ++c) {
      const double eff = (double)(work * c) / (double)(kTargetGroups * ceil_div(work * c, kTargetGroups));
      if (eff > best + 0.02) {
        best = eff;
        s = c;
      }
    }
  }
  if (s > nblk) s = nblk;
  if (s > kvq::kMaxSplits) s = kvq::kMaxSplits;
  const long long bps = ceil_div(nblk, s);
  s = ceil_div(nblk, bps);
  if (work * s >= (1LL << 31)) return KVQ_ERR_ARG;
  plan->splits = (int)s;
  plan->blocks_per_split = (int)bps;
  *row_tiles = (int)tiles;
  return KVQ_OK;
}

}  // namespace

extern "C" {

int32_t kvq_prefill_num_splits(int32_t n_seq, int32_t chunk, int32_t n_q_heads,
                               int32_t num_kv_heads, int32_t max_seq_len,
                               int32_t num_splits_request) {
  if (chunk < 1 || chunk > KVQ_MAX_CHUNK || num_kv_heads <= 0 || n_q_heads <= 0 ||
      n_q_heads % num_kv_heads != 0)
    return KVQ_ERR_ARG;
  Plan p;
  int tiles;
  const int rc = plan_prefill(n_seq, num_kv_heads, chunk * (n_q_heads / num_kv_heads), max_seq_len,
                              num_splits_request, &p, &tiles);
  return rc == KVQ_OK ? p.splits : rc;
}

size_t kvq_prefill_workspace_bytes(int32_t n_seq, int32_t chunk, int32_t n_q_heads,
                                   int32_t num_kv_heads, int32_t head_dim, int32_t max_seq_len,
                                   int32_t num_splits_request) {
  if (chunk < 1 || chunk > KVQ_MAX_CHUNK || num_kv_heads <= 0 || n_q_heads <= 0 ||
      n_q_heads % num_kv_heads != 0 || !head_dim_ok(head_dim))
    return 0;
  const int rows = chunk * (n_q_heads / num_kv_heads);
  Plan p;
  int tiles;
  if (plan_prefill(n_seq, num_kv_heads, rows, max_seq_len, num_splits_request, &p, &tiles) != KVQ_OK)
    return 0;
  return workspace_for((long long)n_seq * num_kv_heads, p.splits, rows, head_dim);
}

int kvq_prefill_attn(int32_t kv_format, const void* pool, int32_t num_pages, int32_t page_size,
                     int32_t num_kv_heads, int32_t head_dim, const uint16_t* q,
                     const int32_t* page_table, const int32_t* seq_lens, int32_t n_seq,
                     int32_t chunk, int32_t n_q_heads, int32_t max_pages_per_seq,
                     int32_t max_seq_len, float softmax_scale, int32_t num_splits, float* out,
                     float* lse, void* workspace, size_t workspace_bytes, void* stream) {
  const int vb = vbits_of(kv_format);
  int rc = pool_args_ok(pool, num_pages, page_size, num_kv_heads, head_dim, vb);
  if (rc != KVQ_OK) return rc;
  if (!q || !page_table || !seq_lens || !out) return KVQ_ERR_ARG;
  if (n_seq <= 0 || n_q_heads <= 0 || max_pages_per_seq <= 0 || max_seq_len <= 0 ||
      num_splits < 0 || chunk < 1)
    return KVQ_ERR_ARG;
  if (chunk > KVQ_MAX_CHUNK) return KVQ_ERR_UNSUPPORTED;
  if (n_q_heads % num_kv_heads != 0) return KVQ_ERR_ARG;
  const int group = n_q_heads / num_kv_heads;
  if ((long long)group * chunk > KVQ_MAX_PREFILL_ROWS) return KVQ_ERR_UNSUPPORTED;
  if ((long long)max_seq_len > (long long)max_pages_per_seq * page_size) return KVQ_ERR_ARG;
  if (!(softmax_scale == softmax_scale) || isinf(softmax_scale)) return KVQ_ERR_ARG;
  if (((uintptr_t)q & 15) != 0 || ((uintptr_t)out & 15) != 0) return KVQ_ERR_ARG;
  const int rows = group * chunk;
  Plan plan;
  int tiles;
  rc = plan_prefill(n_seq, num_kv_heads, rows, max_seq_len, num_splits, &plan, &tiles);
  if (rc != KVQ_OK) return rc;
  const long long units = (long long)n_seq * num_kv_heads;
  if (!grids_fit(units, tiles, plan.splits, kvq::kPrefillThreads, rows, head_dim))
    return KVQ_ERR_UNSUPPORTED;
  const size_t need = workspace_for(units, plan.splits, rows, head_dim);
  if (!workspace || workspace_bytes < need || ((uintptr_t)workspace & 15) != 0)
    return KVQ_ERR_WORKSPACE;
  const double scale = softmax_scale > 0.0f ? (double)softmax_scale : 1.0 / sqrt((double)head_dim);

  kvq::DecodeArgs a{};
  a.pool = (const uint8_t*)pool;
  a.num_pages = num_pages;
  a.page_size = page_size;
  a.num_kv_heads = num_kv_heads;
  a.vbits = vb;
  a.fp8 = kv_format == KVQ_FORMAT_FP8;
  a.log2_page = __builtin_ctz((unsigned)page_size);
  a.q = q;
  a.page_table = page_table;
  a.seq_lens = seq_lens;
  a.n_seq = n_seq;
  a.n_rows = chunk;
  a.n_q_heads = n_q_heads;
  a.group = group;
  a.rows = rows;
  a.max_pages = max_pages_per_seq;
  a.max_seq_len = max_seq_len;
  a.splits = plan.splits;
  a.blocks_per_split = plan.blocks_per_split;
  a.row_tiles = tiles;
  a.scale_log2 = (float)(scale * 1.4426950408889634074);
  a.ws_acc = (float*)workspace;
  a.ws_ml = plan.splits > 1
                ? (float2*)((char*)a.ws_acc + (size_t)units * plan.splits * rows * head_dim * sizeof(float))
                : nullptr;
  a.out = out;
  a.lse = lse;
  const int drc = debug_address(&a.dbg);
  if (drc != KVQ_OK) return drc;
  (void)hipGetLastError();
  return kvq::launch_prefill(head_dim, a, (hipStream_t)stream) == hipSuccess ? KVQ_OK : KVQ_ERR_HIP;
}

}  // extern "C"

// ---- measurement helper ----------------------------------------------------------------------

extern "C" int kvq_probe_stream_read(const void* buf, size_t bytes, int32_t mode, int32_t workgroups,
                                     uint32_t* sink, void* stream) {
  if (!buf || !sink || bytes == 0 || (bytes & 4095) != 0 || ((uintptr_t)buf & 4095) != 0) return KVQ_ERR_ARG;
  if (mode < 0 || mode > 2 || workgroups < 1 || workgroups > (1 << 20)) return KVQ_ERR_ARG;
  (void)hipGetLastError();
  return kvq::launch_stream_probe(buf, bytes, mode, workgroups, sink, (hipStream_t)stream) == hipSuccess
             ? KVQ_OK
             : KVQ_ERR_HIP;
}

extern "C" int kvq_probe_clock(uint64_t* out, int32_t workgroups, uint32_t spin_ticks, int32_t* const_rate_khz,
                               void* stream) {
  const bool query_only = !out && workgroups == 0;  // only the constant counter's rate
  if (query_only ? !const_rate_khz : (!out || ((uintptr_t)out & 7) != 0 || workgroups < 1 || workgroups > 4096))
    return KVQ_ERR_ARG;
  if (!query_only && (spin_ticks < 1 || spin_ticks > 10000000u)) return KVQ_ERR_ARG;
  (void)hipGetLastError();
  if (const_rate_khz) {
    int dev = 0, khz = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&khz, hipDeviceAttributeWallClockRate, dev) != hipSuccess)
      return KVQ_ERR_HIP;
    *const_rate_khz = khz;
  }
  if (query_only) return KVQ_OK;
  return kvq::launch_clock_probe((unsigned long long*)out, workgroups, spin_ticks, (hipStream_t)stream) ==
                 hipSuccess
             ? KVQ_OK
             : KVQ_ERR_HIP;
}

// ---- KVQ_DEBUG builds: the range-report word ----

extern "C" int kvq_debug_errors(uint32_t* errors, int32_t clear, void* stream) {
#ifdef KVQ_DEBUG
  if (!errors) return KVQ_ERR_ARG;
  unsigned* at = nullptr;
  int rc = debug_address(&at);
  if (rc != KVQ_OK) return rc;
  (void)hipGetLastError();
  if (hipStreamSynchronize((hipStream_t)stream) != hipSuccess) return KVQ_ERR_HIP;
  unsigned v = 0;
  if (hipMemcpy(&v, at, sizeof(v), hipMemcpyDeviceToHost) != hipSuccess) return KVQ_ERR_HIP;
  *errors = v;
  if (clear) {
    const unsigned zero = 0;
    if (hipMemcpy(at, &zero, sizeof(zero), hipMemcpyHostToDevice) != hipSuccess) return KVQ_ERR_HIP;
  }
  return KVQ_OK;
#else
  (void)errors;
  (void)clear;
  (void)stream;
  return KVQ_ERR_UNSUPPORTED;
#endif
}

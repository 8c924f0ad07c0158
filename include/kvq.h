/*
 * kvq.h — paged K8/V4 KV cache and long-context decode attention on MI355X (gfx950).
 *
 * Two calls make up the library: kvq_append (quantize new tokens' K/V into cache pages)
 * and kvq_decode_attn (softmax(Q K^T * scale) V over the paged cache through a page table).
 * The rest of this header is the byte format those calls share and small host-side helpers.
 *
 * Sources.  The KV dtype "rk8v4" (K stored in 8 bits, V in 4 bits) is the engine's
 * --kv-dtype flag in the forum post "3090 单卡跑 Qwen3.8-27B：NInfer 上机实测（180K 上下文 /
 * C2 并发 / 4bit KV）", section 一、部署, launch-flag table: it lets a 184,320-token pool serve
 * two concurrent requests.  The same post and the blog page "標籤: vLLM" (section 重點說明,
 * part 2 "C++/CUDA 層的 kernel fusion 與 KV cache 策略") describe a KV cache managed in
 * segments of the context rather than one buffer, and a decode kernel tuned for one long
 * request.  None of the pages fixes the scale granularity or rounding of rk8v4; this library
 * defines it (below) and does not claim byte compatibility with any other engine.
 *
 * Conventions for every call:
 *   - All array arguments are device pointers to memory the caller owns (e.g. torch tensors).
 *     The library allocates nothing, keeps no state between calls, never synchronizes, and
 *     enqueues its kernels on `stream` (a hipStream_t passed as void*; NULL = default stream).
 *     The one exception is kvq_decode_step_noalloc, whose scratch is a static device array of
 *     the library (stated with that call).
 *   - Calls are asynchronous and stream-ordered: kvq_append followed by kvq_decode_attn on
 *     the same stream makes the appended tokens visible to the attention.
 *   - Every scalar argument is validated on the host before any HIP call; a bad argument
 *     returns a negative KVQ_ERR_* code and enqueues nothing.  Contents of device arrays
 *     (slot numbers, page ids, sequence lengths) cannot be checked on the host; how the
 *     kernels treat out-of-range values is stated per call.
 */
#ifndef KVQ_H
#define KVQ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ---- return codes ---------------------------------------------------------------------- */
#define KVQ_OK               0
#define KVQ_ERR_ARG         (-1)  /* NULL pointer where one is required, or a size <= 0 / inconsistent */
#define KVQ_ERR_UNSUPPORTED (-2)  /* head_dim, page_size, rows-per-KV-head or KV format not built     */
#define KVQ_ERR_WORKSPACE   (-3)  /* workspace NULL or smaller than kvq_decode_workspace_bytes()      */
#define KVQ_ERR_HIP         (-4)  /* a HIP launch reported an error (hipGetLastError)                 */
#define KVQ_ERR_SCRATCH     (-5)  /* kvq_decode_step_noalloc: needs more than its static scratch      */

/* ---- supported shapes ------------------------------------------------------------------ */
/* head_dim D in {64, 128, 256}; page_size P a power of two in [16, 256];
 * rows per KV head (GQA group size G = n_q_heads / num_kv_heads, times n_rows) <= 32;
 * n_rows (query rows per sequence: 1 for plain decode, 1 + drafts for an MTP verify step) in [1, 4]. */
#define KVQ_TILE_TOKENS     16
#define KVQ_MAX_ROWS_PER_KV 32
#define KVQ_MAX_N_ROWS      4
#define KVQ_MAX_STEP_TOKENS 64
/* chunked prefill (kvq_prefill_attn): chunk positions per sequence, and chunk * G rows per KV head */
#define KVQ_MAX_CHUNK        8192
#define KVQ_MAX_PREFILL_ROWS 65536

/* ---- quantization (defined by this library; the pages give only "K8/V4") ---------------
 * Per token and KV head, with inputs in fp32:
 *   K row (D values):  a = max_d |k_d|;  s = fp16_rne(a / 127.0f)   (IEEE fp32 divide, then
 *                      round-to-nearest-even to fp16, saturating at 65504);
 *                      code_d = clamp(rint_half_even(k_d / (float)s), -127, 127) as int8
 *                      (fp32 IEEE divide); if s == 0 every code is 0.
 *   V row: the same per group of 32 contiguous dims with 7 in place of 127, codes in [-7, 7]
 *          stored as 4-bit two's complement; one fp16 scale per group (D/32 per token).
 *   Dequantized values are code * scale (exact in fp32).  Non-finite inputs are undefined.
 *
 * ---- page format ----------------------------------------------------------------------
 * The pool is num_pages pages; page p holds num_kv_heads blocks.  The block of (page p,
 * KV head h) starts at byte (p * num_kv_heads + h) * kvq_block_bytes(P, D) and holds the
 * P token slots of that page for that head in four sections:
 *
 *   K codes   P*D bytes     at 0
 *   K scales  P fp16        at P*D
 *   V codes   P*D/2 bytes   at P*D + 2*P
 *   V scales  P*D/32 fp16   at P*D + 2*P + P*D/2
 *
 * so block_bytes = P * (D + 2 + D/2 + D/16): 25,728 B for P=64, D=256.
 * Slots are grouped in tiles of 16 (slot s -> tile s/16, t = s%16).  Within a tile the codes
 * are laid out so that one 16-byte load per lane of a 64-lane wave delivers matrix-core
 * operands directly (see kvq_decode_attn):
 *
 *   K code (t, d):  byte  16*D*tile + 256*(d/16) + 16*t + d%16            (int8)
 *   K scale (s):    fp16 index s
 *   V code (t, d):  with j = d/32 (scale group), lane = 16*(t/4) + d%16, r = t%4,
 *                   w = min(D/32, 4):
 *                   byte  8*D*tile + 256*w*(j/w) + 4*w*lane + 4*(j%w) + r,
 *                   low nibble if (d/16) is even, high nibble if odd  (4-bit two's complement)
 *   V scale (s, j): fp16 index s*(D/32) + j
 *
 * Every byte of a token's codes belongs to that token alone, so appends of different
 * tokens never write the same byte.
 */
size_t kvq_block_bytes(int32_t page_size, int32_t head_dim);

/* ---- KV formats ------------------------------------------------------------------------
 * The calls above and below use K8/V4.  The _fmt variants take the format first:
 *   KVQ_FORMAT_K8V4  4-bit V codes, the format above.
 *   KVQ_FORMAT_K8V8  8-bit V codes: the int8 KV the same forum post sets against rk8v4 (一、部署
 *                    and its replies: the same decode speed, a 160K- instead of a 180K-token
 *                    pool).  K, its scales and the V scales are as above, and V is quantized as
 *                    above with 127 in place of 7, codes in [-127, 127] stored as int8.  The
 *                    block is [K codes P*D][K scales 2P][V codes P*D][V scales P*D/16], so
 *                    block_bytes = P * (2D + 2 + D/16) (33,920 B for P=64, D=256).  In a tile,
 *                    with j = d/32, lane = 16*(t/4) + d%16, w = min(D/32, 2):
 *                      V code (t, d):  byte  16*D*tile + 512*w*(j/w) + 8*w*lane + 8*(j%w)
 *                                            + 4*((d/16)%2) + t%4   (int8)
 *                    (the two nibbles of a 4-bit byte become two bytes, 4 apart).
 *   KVQ_FORMAT_FP8   K and V as 8-bit floating-point codes: the fp8 KV the replies to the same
 *                    forum post find missing on their card.  Codes are OCP FP8 E4M3 (sign bit 7,
 *                    exponent bits 6..3 with bias 7, mantissa bits 2..0; exponent 0 is
 *                    subnormal, m * 2^-9; largest finite value 448; 0x7F and 0xFF are NaN and
 *                    never produced).  The scale granularity is that of K8/V8 (one fp16 scale per
 *                    token and KV head for K, one per 32 dims for V), with 448 in place of qmax:
 *                    s = fp16_rne(absmax / 448.0f) (fp32 IEEE divide, saturated at 65504), and
 *                    code = e4m3_rne(clamp(x / s, -448, 448)) with the divide in fp32 and the
 *                    stored scale, rounded to the nearest E4M3 value, ties to the even
 *                    mantissa; the sign bit is the quotient's (a negative value that rounds to
 *                    zero is 0x80).  s == 0 gives code 0 for every element.  Dequantized:
 *                    value(code) * s.  The byte layout and block_bytes are those of K8/V8.
 * kvq_decode_workspace_bytes does not depend on the format (it covers the plan of every format);
 * the automatic split count does (kvq_decode_num_splits_fmt). */
#define KVQ_FORMAT_K8V4 0
#define KVQ_FORMAT_K8V8 1
#define KVQ_FORMAT_FP8 2

/* Block bytes of a format (0 for an unknown format or unsupported shape).  Host only. */
size_t kvq_block_bytes_fmt(int32_t kv_format, int32_t page_size, int32_t head_dim);

/* ---- kvq_append ------------------------------------------------------------------------
 * Quantizes n_tok new tokens and writes each into its cache slot.
 *   pool          device, num_pages * num_kv_heads * kvq_block_bytes(page_size, head_dim) bytes,
 *                 16-byte aligned; written in place (only the bytes of the target slots).
 *   k, v          device fp32 [n_tok][num_kv_heads][head_dim], contiguous.
 *   slot_mapping  device int32 [n_tok]; slot = page * page_size + offset.  A slot < 0 or
 *                 >= num_pages * page_size is skipped (no write), so -1 can mark padding.
 *                 Two tokens with the same slot in one call race; the result is undefined.
 *   n_tok         >= 0 (0 enqueues nothing and returns KVQ_OK).
 * Tokens are taken in groups of 16 (token indices 16i .. 16i+15).  A group whose slots are the
 * 16 slots of one tile in order (a prefill or a chunk of one, starting at a tile boundary) is
 * written as whole tiles, which is the fast case; any other group token by token.  The bytes
 * are the same either way.  Each group and KV head is one workgroup of 256 threads, so a call
 * with ceil(n_tok / 16) * num_kv_heads * 256 >= 2^32 (HIP's grid limit) is refused with
 * KVQ_ERR_UNSUPPORTED.
 * Returns KVQ_OK, KVQ_ERR_ARG, KVQ_ERR_UNSUPPORTED or KVQ_ERR_HIP.
 */
int kvq_append(void* pool, int32_t num_pages, int32_t page_size, int32_t num_kv_heads,
               int32_t head_dim, const float* k, const float* v, const int32_t* slot_mapping,
               int32_t n_tok, void* stream);

/* ---- kvq_decode_attn -------------------------------------------------------------------
 * For each sequence b, query row i (0..n_rows-1) and query head hq, with KV head
 * h = hq / (n_q_heads / num_kv_heads) (contiguous GQA groups) and L = seq_lens[b]:
 *   z_t = softmax_scale * sum_d q[b][i][hq][d] * K^[t][d]         for t = 0 .. L - n_rows + i
 *   out[b][i][hq][:] = sum_t softmax(z)_t * V^[t][:],   lse[b][i][hq] = ln sum_t exp(z_t)
 * where K^, V^ are the dequantized cache entries of logical token t of sequence b, found at
 * page page_table[b][t / page_size], slot t % page_size.  n_rows > 1 is an MTP verify step:
 * row i sees the cache up to and including the i-th of the last n_rows tokens (causal mask),
 * so the last row sees all L tokens.  (Multi-token-prediction with 3 draft tokens is the
 * engine's --spec mtp --draft-tokens 3 in the forum post's launch-flag table.)
 *
 *   pool, num_pages, page_size, num_kv_heads, head_dim   as for kvq_append (read only).
 *   q             device fp16 bits [n_seq][n_rows][n_q_heads][head_dim], 16-byte aligned.
 *   page_table    device int32 [n_seq][max_pages_per_seq], logical -> physical page.  Entries
 *                 up to ceil(max_seq_len / page_size) of a row may be read, but only the first
 *                 ceil(L / page_size) are used; an entry outside [0, num_pages) is clamped into
 *                 range (wrong values, never a fault).
 *   seq_lens      device int32 [n_seq]: tokens seen by the last row.  Must satisfy
 *                 n_rows <= L <= max_seq_len; tokens beyond max_seq_len are not attended, and a
 *                 row that sees no token gets out = 0 and lse = -inf.
 *   max_seq_len   host-side upper bound on seq_lens; sizes the grid and the workspace.
 *   softmax_scale <= 0 selects 1/sqrt(head_dim).
 *   num_splits    0 = choose automatically (kvq_decode_num_splits); otherwise the number of
 *                 pieces each (sequence, KV head) context is cut into (one workgroup each),
 *                 clamped to the number of 32-token blocks and to 128.  The result does not depend on it
 *                 beyond fp32 rounding.
 *   out           device fp32 [n_seq][n_rows][n_q_heads][head_dim], 16-byte aligned.
 *   lse           device fp32 [n_seq][n_rows][n_q_heads], or NULL.
 *   workspace     device scratch of at least kvq_decode_workspace_bytes(...) bytes, 16-byte
 *                 aligned, for the pieces' partial results (numerators, running max and sum).
 *                 It needs no initialization and carries nothing from one call to the next;
 *                 two calls in flight at once must not share it.
 * With more than one piece per context the call is two launches on `stream`: the split-KV
 * attention, then the log-sum-exp merge of the pieces.
 * Returns KVQ_OK, KVQ_ERR_ARG, KVQ_ERR_UNSUPPORTED, KVQ_ERR_WORKSPACE or KVQ_ERR_HIP.
 * KVQ_ERR_UNSUPPORTED also covers a call whose attention or merge grid would count 2^32
 * work-items or more (HIP's grid limit): such a call is refused, never launched truncated.
 */
int kvq_decode_attn(const void* pool, int32_t num_pages, int32_t page_size,
                    int32_t num_kv_heads, int32_t head_dim, const uint16_t* q,
                    const int32_t* page_table, const int32_t* seq_lens, int32_t n_seq,
                    int32_t n_rows, int32_t n_q_heads, int32_t max_pages_per_seq,
                    int32_t max_seq_len, float softmax_scale, int32_t num_splits, float* out,
                    float* lse, void* workspace, size_t workspace_bytes, void* stream);

/* ---- kvq_decode_step ---------------------------------------------------------------------
 * One decode step in one call: kvq_append of each sequence's newest n_new tokens, then
 * kvq_decode_attn over the cache that now holds them.  The result (pool bytes, out, lse) is the
 * same as those two calls with slot_mapping taken from the page table, so the appended tokens
 * must be the last n_new of each sequence: token L - n_new + j of sequence b (L = seq_lens[b])
 * gets k_new[b][j], v_new[b][j] and is written to page page_table[b][t / page_size], slot
 * t % page_size.  (An MTP verify step appends its 1 + 3 rows' tokens this way, forum post
 * "3090 单卡跑 Qwen3.8-27B：NInfer 上机实测（180K 上下文 / C2 并发 / 4bit KV）", 一、部署,
 * launch-flag table.)  Each new token is quantized by the workgroup that attends its block, before
 * that block is read, so the step needs no separate append launch.
 *   pool          as for kvq_decode_attn, but written (the new tokens' slots only).
 *   k_new, v_new  device fp32 [n_seq][n_new][num_kv_heads][head_dim], contiguous; may be NULL
 *                 when n_new = 0.
 *   n_new         0 .. KVQ_MAX_STEP_TOKENS, and n_new <= L for every sequence (tokens at
 *                 negative positions are skipped).
 *   other arguments as for kvq_decode_attn (the workspace need is the same).
 * Returns KVQ_OK, KVQ_ERR_ARG, KVQ_ERR_UNSUPPORTED, KVQ_ERR_WORKSPACE or KVQ_ERR_HIP.
 */
int kvq_decode_step(void* pool, int32_t num_pages, int32_t page_size, int32_t num_kv_heads,
                    int32_t head_dim, const float* k_new, const float* v_new, int32_t n_new,
                    const uint16_t* q, const int32_t* page_table, const int32_t* seq_lens,
                    int32_t n_seq, int32_t n_rows, int32_t n_q_heads, int32_t max_pages_per_seq,
                    int32_t max_seq_len, float softmax_scale, int32_t num_splits, float* out,
                    float* lse, void* workspace, size_t workspace_bytes, void* stream);

/* Number of context pieces kvq_decode_attn uses per (sequence, KV head) for these shapes in the
 * K8/V4 format (num_splits_request as in kvq_decode_attn), or a negative KVQ_ERR_* code.
 * Host only.  kvq_decode_num_splits_fmt gives the count for any format. */
int32_t kvq_decode_num_splits(int32_t n_seq, int32_t num_kv_heads, int32_t max_seq_len,
                              int32_t num_splits_request);

/* Workspace bytes kvq_decode_attn needs for these shapes, in any format (0 on invalid shapes).
 * Host only. */
size_t kvq_decode_workspace_bytes(int32_t n_seq, int32_t n_rows, int32_t n_q_heads,
                                  int32_t num_kv_heads, int32_t head_dim, int32_t max_seq_len,
                                  int32_t num_splits_request);

/* The calls above in a given KV format (pool laid out as that format defines; an unknown
 * format returns KVQ_ERR_UNSUPPORTED).  Arguments otherwise as documented above. */
int kvq_append_fmt(int32_t kv_format, void* pool, int32_t num_pages, int32_t page_size,
                   int32_t num_kv_heads, int32_t head_dim, const float* k, const float* v,
                   const int32_t* slot_mapping, int32_t n_tok, void* stream);
int kvq_decode_attn_fmt(int32_t kv_format, const void* pool, int32_t num_pages, int32_t page_size,
                        int32_t num_kv_heads, int32_t head_dim, const uint16_t* q,
                        const int32_t* page_table, const int32_t* seq_lens, int32_t n_seq,
                        int32_t n_rows, int32_t n_q_heads, int32_t max_pages_per_seq,
                        int32_t max_seq_len, float softmax_scale, int32_t num_splits, float* out,
                        float* lse, void* workspace, size_t workspace_bytes, void* stream);
int kvq_decode_step_fmt(int32_t kv_format, void* pool, int32_t num_pages, int32_t page_size,
                        int32_t num_kv_heads, int32_t head_dim, const float* k_new,
                        const float* v_new, int32_t n_new, const uint16_t* q,
                        const int32_t* page_table, const int32_t* seq_lens, int32_t n_seq,
                        int32_t n_rows, int32_t n_q_heads, int32_t max_pages_per_seq,
                        int32_t max_seq_len, float softmax_scale, int32_t num_splits, float* out,
                        float* lse, void* workspace, size_t workspace_bytes, void* stream);

/* ---- sliding window over ring pages ---------------------------------------------------
 * kvq_decode_attn / kvq_decode_step (in format kv_format) where each row sees only the last
 * `window` tokens up to its own position, and the pages of a sequence may be a ring: the
 * ring-buffer / sliding-window KV that blog page "標籤: vLLM" (section 重點說明, part 2) names
 * for steady latency at long context.  With L = seq_lens[b], row i is at position
 * p = L - n_rows + i and
 *   z_t = softmax_scale * q . K^[t]   for t = max(0, p - window + 1) .. p
 * (window = 0: from token 0, as kvq_decode_attn).  The pieces cover only the blocks from the
 * first row's window start on, so the work per call is bounded by the window, not by L.
 *   window        0, or the number of tokens each row sees (its own included).
 *   ring_pages    0: token t is at page page_table[b][t / page_size], slot t % page_size, and
 *                 max_seq_len <= max_pages_per_seq * page_size as before.  > 0 (needs
 *                 window > 0): logical page n of a sequence is entry n % ring_pages of its row,
 *                 so a sequence needs only ring_pages pages however long it grows; L may exceed
 *                 max_pages_per_seq * page_size (max_seq_len still bounds it).  Requires
 *                 ring_pages <= max_pages_per_seq and
 *                 ring_pages >= (window + n_rows - 1 + page_size - 2) / page_size + 1, the most
 *                 pages window + n_rows - 1 consecutive tokens can touch; then no token a row
 *                 sees has been overwritten by a later one.  The caller's slot_mapping for
 *                 kvq_append follows the same map.
 *   n_new         (step) at most window + n_rows - 1: every appended token is one some row sees.
 * The workspace need is kvq_decode_workspace_bytes_win; kvq_decode_num_splits_win gives the
 * pieces per context.  Returns as kvq_decode_attn; an inconsistent window / ring gives
 * KVQ_ERR_ARG. */
int kvq_decode_attn_win(int32_t kv_format, const void* pool, int32_t num_pages, int32_t page_size,
                        int32_t num_kv_heads, int32_t head_dim, const uint16_t* q,
                        const int32_t* page_table, const int32_t* seq_lens, int32_t n_seq,
                        int32_t n_rows, int32_t n_q_heads, int32_t max_pages_per_seq,
                        int32_t max_seq_len, int32_t window, int32_t ring_pages,
                        float softmax_scale, int32_t num_splits, float* out, float* lse,
                        void* workspace, size_t workspace_bytes, void* stream);
int kvq_decode_step_win(int32_t kv_format, void* pool, int32_t num_pages, int32_t page_size,
                        int32_t num_kv_heads, int32_t head_dim, const float* k_new,
                        const float* v_new, int32_t n_new, const uint16_t* q,
                        const int32_t* page_table, const int32_t* seq_lens, int32_t n_seq,
                        int32_t n_rows, int32_t n_q_heads, int32_t max_pages_per_seq,
                        int32_t max_seq_len, int32_t window, int32_t ring_pages,
                        float softmax_scale, int32_t num_splits, float* out, float* lse,
                        void* workspace, size_t workspace_bytes, void* stream);
/* ---- kvq_decode_step_noalloc: the decode step without a workspace ------------------------
 * For callers that cannot allocate device memory (code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc): kvq_decode_step_fmt with the same arguments minus
 * (workspace, workspace_bytes).  The split partials (the workspace of kvq_decode_step_fmt) go to
 * a static device array of KVQ_NOALLOC_SCRATCH_BYTES inside the library instead: one copy per
 * GPU, on the device current on the calling thread (`stream` must belong to it), held until
 * the process ends.  The call allocates nothing and clears nothing (no entry of the array is
 * read before the same launch writes it), and gives bit-identical results to
 * kvq_decode_step_fmt with the same split plan.
 *   - A call whose partials would exceed the array (its format's split plan needs more than
 *     KVQ_NOALLOC_SCRATCH_BYTES; kvq_decode_workspace_bytes() bounds that need for every format)
 *     returns KVQ_ERR_SCRATCH and enqueues nothing.  Every automatic plan of the supported
 *     shapes fits (at most about 8.5 MB at 32 rows per KV head, D = 256).
 *   - All calls on one GPU share its array: calls that may overlap in time on one GPU (different
 *     streams without ordering between them) race on it and give undefined results.  Order them
 *     on one stream, or use kvq_decode_step_fmt with a workspace per stream.
 *   - The first call on a device looks the array's address up (hipGetSymbolAddress) and keeps
 *     it; KVQ_ERR_HIP if that fails. */
#define KVQ_NOALLOC_SCRATCH_BYTES (16u << 20)
int kvq_decode_step_noalloc(int32_t kv_format, void* pool, int32_t num_pages, int32_t page_size,
                            int32_t num_kv_heads, int32_t head_dim, const float* k_new,
                            const float* v_new, int32_t n_new, const uint16_t* q,
                            const int32_t* page_table, const int32_t* seq_lens, int32_t n_seq,
                            int32_t n_rows, int32_t n_q_heads, int32_t max_pages_per_seq,
                            int32_t max_seq_len, float softmax_scale, int32_t num_splits,
                            float* out, float* lse, void* stream);

int32_t kvq_decode_num_splits_win(int32_t n_seq, int32_t num_kv_heads, int32_t max_seq_len,
                                  int32_t n_rows, int32_t window, int32_t num_splits_request);
size_t kvq_decode_workspace_bytes_win(int32_t n_seq, int32_t n_rows, int32_t n_q_heads,
                                      int32_t num_kv_heads, int32_t head_dim, int32_t max_seq_len,
                                      int32_t window, int32_t num_splits_request);

/* The number of context pieces per (sequence, KV head) every decode call of this format uses
 * for these shapes (window 0 = none; num_splits_request as in kvq_decode_attn), or a negative
 * KVQ_ERR_* code (KVQ_ERR_UNSUPPORTED for an unknown format).  With a request of 0 the plan
 * depends on the format: the 4-bit-V format's block step is bound by the issue of its own wave
 * and gets the plan whose busiest wave has the fewest blocks; the 8-bit-V formats, 32% more
 * bytes per token, are bandwidth-bound and may use fewer splits.  Host only. */
int32_t kvq_decode_num_splits_fmt(int32_t kv_format, int32_t n_seq, int32_t num_kv_heads,
                                  int32_t max_seq_len, int32_t n_rows, int32_t window,
                                  int32_t num_splits_request);

/* ---- kvq_prefill_attn: chunked-prefill attention -------------------------------------------
 * The forum post's engine prefills prompts in chunks of 1,024 tokens (一、部署, launch-flag table,
 * --prefill-chunk 1024) and names prefill as the cost behind the time to first token (二、测评).
 * After a chunk's tokens are appended (kvq_append), every position of the chunk attends
 * causally to the cache up to itself.  For sequence b with L = seq_lens[b] tokens, the last
 * `chunk` of them being the chunk, position i (0 <= i < chunk) sees tokens 0 .. L - chunk + i:
 * the definition of kvq_decode_attn with n_rows = chunk, for any chunk up to KVQ_MAX_CHUNK.
 *   q             fp16 bits [n_seq][chunk][n_q_heads][head_dim], 16-byte aligned.
 *   out           fp32 [n_seq][chunk][n_q_heads][head_dim], 16-byte aligned; lse (nullable) fp32
 *                 [n_seq][chunk][n_q_heads], natural log, of the scaled logits.  A position that
 *                 sees no token (L - chunk + i < 0) gets out = 0 and lse = -inf.
 *   chunk         1 .. KVQ_MAX_CHUNK, and chunk * n_q_heads / num_kv_heads <= KVQ_MAX_PREFILL_ROWS.
 *   num_splits    0 = automatic; otherwise pieces per (sequence, KV head, 256-row tile).
 *   workspace     device memory of at least kvq_prefill_workspace_bytes(...) bytes, 16-byte
 *                 aligned, never initialized by the caller; its contents after the call are
 *                 unspecified.
 * Other arguments, the KV formats, the page table and the device-data contract are those of
 * kvq_decode_attn_fmt.  Stream-ordered, allocates nothing, never synchronizes.  Returns KVQ_OK,
 * KVQ_ERR_ARG, KVQ_ERR_UNSUPPORTED, KVQ_ERR_WORKSPACE or KVQ_ERR_HIP; every argument error is
 * found on the host before any launch (KVQ_ERR_UNSUPPORTED for a grid of 2^32 work-items or more,
 * as for kvq_decode_attn). */
int kvq_prefill_attn(int32_t kv_format, const void* pool, int32_t num_pages, int32_t page_size,
                     int32_t num_kv_heads, int32_t head_dim, const uint16_t* q,
                     const int32_t* page_table, const int32_t* seq_lens, int32_t n_seq,
                     int32_t chunk, int32_t n_q_heads, int32_t max_pages_per_seq,
                     int32_t max_seq_len, float softmax_scale, int32_t num_splits, float* out,
                     float* lse, void* workspace, size_t workspace_bytes, void* stream);
/* Pieces per (sequence, KV head, row tile) the call above would use (negative: an error code). */
int32_t kvq_prefill_num_splits(int32_t n_seq, int32_t chunk, int32_t n_q_heads,
                               int32_t num_kv_heads, int32_t max_seq_len,
                               int32_t num_splits_request);
/* Workspace bytes kvq_prefill_attn needs (0 for invalid arguments).  Host only. */
size_t kvq_prefill_workspace_bytes(int32_t n_seq, int32_t chunk, int32_t n_q_heads,
                                   int32_t num_kv_heads, int32_t head_dim, int32_t max_seq_len,
                                   int32_t num_splits_request);

/* Static description of a return code. */
const char* kvq_strerror(int code);

/* ---- KVQ_DEBUG builds: device-side range reports -------------------------------------------
 * The library built with -DKVQ_DEBUG (libkvq_debug.so) computes exactly what the normal build
 * does, and its kernels also record, in one word per GPU, any input they had to correct: bit
 * KVQ_DBG_PAGE_ID when a page-table entry the call reads lies outside [0, num_pages) (decode,
 * fused append, prefill; the id is still clamped, never followed), bit KVQ_DBG_SLOT when an
 * append slot lies at or past num_pages * page_size (still skipped; negative slots mark padding
 * and are not reported).  This is the device-side counterpart of the host's argument checks:
 * ids and slots live in device memory, so only the kernels see them.
 * kvq_debug_errors: waits for `stream`, writes the word to *errors (host), and clears it when
 * `clear` is non-zero.  Host-synchronous; not for use under graph capture.  Every call on a GPU
 * reports into the same word.  Returns KVQ_OK, KVQ_ERR_ARG (errors NULL) or KVQ_ERR_HIP in a
 * KVQ_DEBUG build, and KVQ_ERR_UNSUPPORTED in any other build. */
#define KVQ_DBG_PAGE_ID 1u
#define KVQ_DBG_SLOT 2u
int kvq_debug_errors(uint32_t* errors, int32_t clear, void* stream);

/* ---- measurement helper (not part of the method) -------------------------------------------
 * kvq_probe_stream_read: read `bytes` of device memory at `buf` once, as a plain stream, so that
 * a benchmark can set the decode's achieved bandwidth against what this GPU attains for a pure
 * read (the forum post, 二、测评, weighs decode speed as bytes per token against the card's
 * bandwidth).  mode 0: 16-byte non-temporal loads into registers; 1: the same with normal
 * caching; 2: gfx950 direct-to-LDS 16-byte non-temporal loads, the decode kernel's own form.
 * `workgroups` of 256 threads share the buffer (grid-stride).  `sink` (one device uint32) is
 * written only for data that xors to a fixed improbable value; it exists so the loads cannot be
 * dropped.  buf 4096-byte aligned, bytes a non-zero multiple of 4096, workgroups 1 .. 2^20.
 * Returns KVQ_OK, KVQ_ERR_ARG or KVQ_ERR_HIP. */
int kvq_probe_stream_read(const void* buf, size_t bytes, int32_t mode, int32_t workgroups,
                          uint32_t* sink, void* stream);

/* kvq_probe_clock: the shader clock the GPU runs at right now, read from its own counters (the
 * forum post, 二、测评, reports core clock and power cap beside its decode speeds, since both move
 * them).  Each of `workgroups` one-wave workgroups spins until the GPU's constant-rate counter
 * has advanced `spin_ticks` ticks and writes three uint64 to out[3 i .. 3 i + 2]: the
 * shader-clock cycles counted over the spin, the constant-rate ticks, and the XCD (accelerator
 * complex die) the wave ran on.  cycles / ticks * *const_rate_khz is the clock in kHz.
 * out: device memory, 8-byte aligned, 3 * workgroups entries, written by the kernel;
 * const_rate_khz: host, may be NULL, receives the constant counter's rate when not NULL.
 * workgroups 1 .. 4096, spin_ticks 1 .. 10,000,000.  With out NULL and workgroups 0 nothing is
 * launched and only *const_rate_khz is written (it must then be given).  Returns KVQ_OK,
 * KVQ_ERR_ARG or KVQ_ERR_HIP. */
int kvq_probe_clock(uint64_t* out, int32_t workgroups, uint32_t spin_ticks, int32_t* const_rate_khz,
                    void* stream);

#ifdef __cplusplus
}
#endif

#endif /* KVQ_H */

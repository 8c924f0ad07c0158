/*
 * kvq_oracle.c — the plain CPU oracle for the paged K8/V4 cache and its decode attention.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the benchmark's CPU-baseline
 * leg may load this library.  It shares no code with the HIP library: the byte format, the
 * quantizer, the fp16 conversion and the attention are written here again from their
 * definitions, slowly and in the order the definitions state them.
 *
 * What it computes (the definition; the GPU's split-KV flash-decoding reaches the same value
 * up to fp32 rounding):
 *   - quantization of each new token's K row to int8 with one fp16 scale, and of its V row to
 *     int4 (vb = 4) or int8 (vb = 8) with one fp16 scale per 32 dims (the engine's "rk8v4"
 *     K8-V4 KV dtype, and the int8 KV it is compared with; or K and V both as OCP fp8 e4m3
 *     codes at the same scale granularity, the fp8 KV the same post finds missing on its card:
 *     forum post
 *     "3090 单卡跑 Qwen3.8-27B：NInfer 上机实测（180K 上下文 / C2 并发 / 4bit KV）", section
 *     一、部署, launch-flag table; the pages leave the scale granularity open, the library
 *     header fixes it and this file follows that definition);
 *   - the page format of that header (the KV cache kept in fixed-size pieces of the context,
 *     blog page "標籤: vLLM", section 重點說明 part 2 on segmented KV);
 *   - exact attention in fp64 over the dequantized entries, token by token in logical order
 *     through the page table, with the causal mask of an MTP verify step (same forum post,
 *     --spec mtp --draft-tokens 3);
 *   - optionally a sliding window over ring pages (blog page "標籤: vLLM", section 重點說明
 *     part 2, which names the ring-buffer / sliding-window approach without details): row i
 *     sees only the last `window` tokens up to its own position, and logical page n of a
 *     sequence lives in page-table entry n mod ring_pages.
 *
 * Build: gcc -O2 -std=c11 -fopenmp -ffp-contract=off -shared -fPIC (no fast-math: the quantizer
 * relies on IEEE fp32 division and round-half-to-even).
 */
#include <math.h>
#include <stddef.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* ---------------------------------------------------------------- IEEE binary16 ---------- */

/* Value of an IEEE 754 binary16 bit pattern: subnormals are f * 2^-24, normals are
 * (1024 + f) * 2^(e - 25) for biased exponent e in 1..30. */
double kvq_oracle_fp16_to_double(uint16_t h) {
  int sign = (h >> 15) & 1;
  int e = (h >> 10) & 31;
  int f = h & 1023;
  double v;
  if (e == 0)
    v = ldexp((double)f, -24);
  else if (e == 31)
    v = f ? NAN : INFINITY;
  else
    v = ldexp(1024.0 + (double)f, e - 25);
  return sign ? -v : v;
}

/* Round x to the nearest binary16 value, ties to even (IEEE default rounding).  The spacing
 * of binary16 values near |x| is 2^(E-10) with E = max(floor(log2|x|), -14); rounding |x| to a
 * multiple of that spacing is the definition of round-to-nearest.  Magnitudes that round to
 * 65520 or above overflow to infinity. */
uint16_t kvq_oracle_fp16_from_double(double x) {
  if (isnan(x)) return 0x7E00;
  uint16_t sign = signbit(x) ? 0x8000 : 0;
  double a = fabs(x);
  if (a == 0.0) return sign;
  int E;
  frexp(a, &E);           /* a = m * 2^E, m in [0.5, 1)  ->  floor(log2 a) = E - 1 */
  int e = E - 1;
  if (e < -14) e = -14;   /* below the normal range the spacing stays 2^-24 */
  double quantum = ldexp(1.0, e - 10);
  double n = nearbyint(a / quantum); /* exact quotient (power-of-two scaling); ties to even */
  double r = n * quantum;
  if (r >= 65520.0) return sign | 0x7C00;
  if (r < ldexp(1.0, -14)) return sign | (uint16_t)n; /* subnormal: field = r / 2^-24 */
  int Er;
  frexp(r, &Er);
  int ebits = (Er - 1) + 15;
  int mbits = (int)(ldexp(r, -(Er - 1)) * 1024.0 - 1024.0);
  return sign | (uint16_t)(ebits << 10) | (uint16_t)mbits;
}

/* ---------------------------------------------------------------- quantizer -------------- */

/* One scale group: absmax -> scale = fp16_rne(absmax / qmax) (fp32 IEEE divide, saturated to
 * the largest finite fp16) -> code = clamp(rint_half_even(x / scale), -qmax, qmax) with the
 * divide in fp32 and the stored fp16 scale, all codes 0 when the scale is 0. */
static float group_scale(const float* x, int n, int qmax, uint16_t* scale_bits) {
  float a = 0.0f;
  for (int i = 0; i < n; ++i) {
    float m = fabsf(x[i]);
    if (m > a) a = m;
  }
  float s32 = a / (float)qmax;
  uint16_t sb = kvq_oracle_fp16_from_double((double)s32);
  if ((sb & 0x7FFF) == 0x7C00) sb = (uint16_t)((sb & 0x8000) | 0x7BFF);
  *scale_bits = sb;
  return (float)kvq_oracle_fp16_to_double(sb); /* codes divide by the stored scale */
}

void kvq_oracle_quantize_group(const float* x, int n, int qmax, int8_t* codes,
                               uint16_t* scale_bits) {
  float s = group_scale(x, n, qmax, scale_bits);
  for (int i = 0; i < n; ++i) {
    if (s == 0.0f) {
      codes[i] = 0;
      continue;
    }
    float y = x[i] / s;
    float c = nearbyintf(y);
    if (c > (float)qmax) c = (float)qmax;
    if (c < (float)-qmax) c = (float)-qmax;
    codes[i] = (int8_t)c;
  }
}

/* ---------------------------------------------------------------- OCP fp8 e4m3 ---------- */

/* Value of an OCP 8-bit E4M3 code: sign bit 7, exponent bits 6..3 (bias 7), mantissa bits
 * 2..0.  Exponent field 0 is subnormal, m * 2^-9; otherwise (8 + m) * 2^(e - 10).  The two
 * codes with every exponent and mantissa bit set are NaN; there is no infinity. */
double kvq_oracle_e4m3_to_double(uint8_t c) {
  int sign = c >> 7, e = (c >> 3) & 15, m = c & 7;
  if (e == 15 && m == 7) return NAN;
  double mag = e == 0 ? ldexp((double)m, -9) : ldexp((double)(8 + m), e - 10);
  return sign ? -mag : mag;
}

/* Round y (|y| <= 448) to the nearest E4M3 value, ties to the even mantissa.  Near |y| the
 * spacing of E4M3 values is 2^(E-3), E = max(floor(log2|y|), -6); rounding |y| to a multiple
 * of it is the definition of round-to-nearest (a result of 2^(E+1) is the next binade's
 * first value).  The sign bit is y's, zeros included. */
uint8_t kvq_oracle_e4m3_from_float(float y) {
  uint8_t sign = signbit(y) ? 0x80 : 0;
  double a = fabs((double)y);
  if (a > 448.0) a = 448.0;
  if (a == 0.0) return sign;
  int E = (int)floor(log2(a));
  if (E < -6) E = -6;
  double quantum = ldexp(1.0, E - 3);
  double r = nearbyint(a / quantum) * quantum; /* the current rounding mode: to nearest even */
  if (r == 0.0) return sign;
  if (r < ldexp(1.0, -6)) return sign | (uint8_t)(r / ldexp(1.0, -9)); /* subnormal */
  int Er = (int)floor(log2(r));
  int mbits = (int)(ldexp(r, -Er) * 8.0 - 8.0);
  return sign | (uint8_t)((Er + 7) << 3) | (uint8_t)mbits;
}

/* One fp8 scale group: scale = fp16_rne(absmax / 448) as for the integer codes; then
 * code = e4m3_rne(clamp(x / scale, -448, 448)) with the divide in fp32 and the stored fp16
 * scale, all codes 0 when the scale is 0. */
void kvq_oracle_quantize_group_f8(const float* x, int n, uint8_t* codes, uint16_t* scale_bits) {
  float s = group_scale(x, n, 448, scale_bits);
  for (int i = 0; i < n; ++i) {
    if (s == 0.0f) {
      codes[i] = 0;
      continue;
    }
    float y = x[i] / s;
    if (y > 448.0f) y = 448.0f;
    if (y < -448.0f) y = -448.0f;
    codes[i] = kvq_oracle_e4m3_from_float(y);
  }
}

/* ---------------------------------------------------------------- page format ------------ */

/* KV formats, as the library header numbers them: 0 K8/V4, 1 K8/V8, 2 fp8 (K and V e4m3, the
 * K8/V8 byte layout).  vb is the bits per V code the layout uses. */
static int vb_of(int kf) { return kf == 0 ? 4 : 8; }

/* vb = bits per V code: 4 (K8/V4, two codes per byte) or 8 (K8/V8, one per byte). */
size_t kvq_oracle_block_bytes_fmt(int P, int D, int vb) {
  return (size_t)P * (size_t)(D + 2 + D * vb / 8 + D / 16);
}
size_t kvq_oracle_block_bytes(int P, int D) { return kvq_oracle_block_bytes_fmt(P, D, 4); }

static size_t k_code_offset(int D, int s, int d) {
  int tile = s / 16, t = s % 16;
  return (size_t)16 * D * tile + (size_t)256 * (d / 16) + (size_t)16 * t + (size_t)(d % 16);
}
static size_t k_scale_offset(int P, int D, int s) { return (size_t)P * D + (size_t)2 * s; }
static size_t v_code_offset(int P, int D, int s, int d, int* high_nibble) {
  int tile = s / 16, t = s % 16;
  int j = d / 32;
  int lane = 16 * (t / 4) + d % 16;
  int r = t % 4;
  int w = D / 32 < 4 ? D / 32 : 4;
  *high_nibble = (d / 16) % 2;
  return (size_t)P * D + (size_t)2 * P + (size_t)8 * D * tile + (size_t)256 * w * (j / w) +
         (size_t)4 * w * lane + (size_t)4 * (j % w) + (size_t)r;
}
/* K8/V8: the two nibbles of a V4 byte become two bytes, 4 apart (dim of the even 16-dim block
 * first), in 8-byte units; up to two scale groups' units side by side per lane. */
static size_t v8_code_offset(int P, int D, int s, int d) {
  int tile = s / 16, t = s % 16, j = d / 32;
  int v8lane = 16 * (t / 4) + d % 16; /* as for 4-bit codes: four tokens, one dim pair per lane */
  int w = D / 32 < 2 ? D / 32 : 2;
  return (size_t)P * D + (size_t)2 * P + (size_t)16 * D * tile + (size_t)512 * w * (j / w) +
         (size_t)8 * w * v8lane + (size_t)8 * (j % w) + (size_t)4 * ((d / 16) % 2) + (size_t)(t % 4);
}
static size_t v_scale_offset_fmt(int P, int D, int vb, int s, int j) {
  return (size_t)P * D + (size_t)2 * P + (size_t)P * D * vb / 8 + (size_t)2 * ((size_t)s * (D / 32) + j);
}

/* Byte offset of a quantity within its block, exposed so tests can check the format's
 * bijectivity: what = 0 K code, 1 K scale, 2 V code (returns nibble in *aux; always 0 for
 * vb = 8), 3 V scale. */
long long kvq_oracle_format_offset_fmt(int what, int P, int D, int vb, int s, int d, int* aux) {
  *aux = 0;
  switch (what) {
    case 0: return (long long)k_code_offset(D, s, d);
    case 1: return (long long)k_scale_offset(P, D, s);
    case 2: return vb == 8 ? (long long)v8_code_offset(P, D, s, d) : (long long)v_code_offset(P, D, s, d, aux);
    case 3: return (long long)v_scale_offset_fmt(P, D, vb, s, d);
  }
  return -1;
}
long long kvq_oracle_format_offset(int what, int P, int D, int s, int d, int* aux) {
  return kvq_oracle_format_offset_fmt(what, P, D, 4, s, d, aux);
}

static uint8_t* block_of(uint8_t* pool, int Hkv, int P, int D, int vb, int page, int h) {
  return pool + ((size_t)page * Hkv + h) * kvq_oracle_block_bytes_fmt(P, D, vb);
}

/* Quantize n_tok tokens and write them into their slots (slot < 0 or beyond the pool: skip),
 * in KV format kf. */
void kvq_oracle_append_kf(uint8_t* pool, int num_pages, int P, int Hkv, int D, int kf,
                          const float* k, const float* v, const int32_t* slots, int n_tok) {
  const int vb = vb_of(kf);
  const int f8 = kf == 2;
  const int vqmax = vb == 8 ? 127 : 7;
  int8_t* codes = (int8_t*)malloc((size_t)D);
  for (int n = 0; n < n_tok; ++n) {
    long long slot = slots[n];
    if (slot < 0 || slot >= (long long)num_pages * P) continue;
    int page = (int)(slot / P), s = (int)(slot % P);
    for (int h = 0; h < Hkv; ++h) {
      uint8_t* blk = block_of(pool, Hkv, P, D, vb, page, h);
      const float* krow = k + ((size_t)n * Hkv + h) * D;
      const float* vrow = v + ((size_t)n * Hkv + h) * D;
      uint16_t sb;
      if (f8)
        kvq_oracle_quantize_group_f8(krow, D, (uint8_t*)codes, &sb);
      else
        kvq_oracle_quantize_group(krow, D, 127, codes, &sb);
      for (int d = 0; d < D; ++d) blk[k_code_offset(D, s, d)] = (uint8_t)codes[d];
      size_t so = k_scale_offset(P, D, s);
      blk[so] = (uint8_t)(sb & 0xFF);
      blk[so + 1] = (uint8_t)(sb >> 8);
      for (int j = 0; j < D / 32; ++j) {
        const float* vg = vrow + 32 * j; /* scale group j: 32 contiguous dims */
        if (f8)
          kvq_oracle_quantize_group_f8(vg, 32, (uint8_t*)codes + 32 * j, &sb);
        else
          kvq_oracle_quantize_group(vg, 32, vqmax, codes + 32 * j, &sb);
        size_t vo = v_scale_offset_fmt(P, D, vb, s, j);
        blk[vo] = (uint8_t)(sb & 0xFF);
        blk[vo + 1] = (uint8_t)(sb >> 8);
      }
      for (int d = 0; d < D; ++d) {
        if (vb == 8) {
          blk[v8_code_offset(P, D, s, d)] = (uint8_t)codes[d];
          continue;
        }
        int hi;
        size_t o = v_code_offset(P, D, s, d, &hi);
        uint8_t nib = (uint8_t)(codes[d] & 0x0F);
        blk[o] = hi ? (uint8_t)((blk[o] & 0x0F) | (nib << 4)) : (uint8_t)((blk[o] & 0xF0) | nib);
      }
    }
  }
  free(codes);
}
void kvq_oracle_append_fmt(uint8_t* pool, int num_pages, int P, int Hkv, int D, int vb,
                           const float* k, const float* v, const int32_t* slots, int n_tok) {
  kvq_oracle_append_kf(pool, num_pages, P, Hkv, D, vb == 8 ? 1 : 0, k, v, slots, n_tok);
}
void kvq_oracle_append(uint8_t* pool, int num_pages, int P, int Hkv, int D, const float* k,
                       const float* v, const int32_t* slots, int n_tok) {
  kvq_oracle_append_fmt(pool, num_pages, P, Hkv, D, 4, k, v, slots, n_tok);
}

/* Read back one slot of one head: codes and fp16 scale bits (kc[D], ks[1], vc[D], vs[D/32]). */
void kvq_oracle_read_slot_fmt(const uint8_t* pool, int P, int Hkv, int D, int vb, int page, int s,
                              int h, int8_t* kc, uint16_t* ks, int8_t* vc, uint16_t* vs) {
  const uint8_t* blk = pool + ((size_t)page * Hkv + h) * kvq_oracle_block_bytes_fmt(P, D, vb);
  for (int d = 0; d < D; ++d) kc[d] = (int8_t)blk[k_code_offset(D, s, d)];
  size_t so = k_scale_offset(P, D, s);
  *ks = (uint16_t)(blk[so] | (blk[so + 1] << 8));
  for (int d = 0; d < D; ++d) {
    if (vb == 8) {
      vc[d] = (int8_t)blk[v8_code_offset(P, D, s, d)];
      continue;
    }
    int hi;
    size_t o = v_code_offset(P, D, s, d, &hi);
    int nib = hi ? (blk[o] >> 4) & 0xF : blk[o] & 0xF;
    vc[d] = (int8_t)(nib >= 8 ? nib - 16 : nib); /* 4-bit two's complement */
  }
  for (int j = 0; j < D / 32; ++j) {
    size_t vo = v_scale_offset_fmt(P, D, vb, s, j);
    vs[j] = (uint16_t)(blk[vo] | (blk[vo + 1] << 8));
  }
}
void kvq_oracle_read_slot(const uint8_t* pool, int P, int Hkv, int D, int page, int s, int h,
                          int8_t* kc, uint16_t* ks, int8_t* vc, uint16_t* vs) {
  kvq_oracle_read_slot_fmt(pool, P, Hkv, D, 4, page, s, h, kc, ks, vc, vs);
}

/* ---------------------------------------------------------------- attention -------------- */

/* Dequantized K and V of logical token t of sequence b, head h (page-table entries clamped
 * into [0, num_pages) as the library header specifies).  ring > 0: logical page t / P sits in
 * entry (t / P) mod ring of the sequence's page-table row; ring = 0: in entry t / P. */
static void token_kv(const uint8_t* pool, int num_pages, int P, int Hkv, int D, int kf, int ring,
                     const int32_t* pt_row, int t, int h, double* kd, double* vd, int8_t* kc,
                     int8_t* vc, uint16_t* vs) {
  const int vb = vb_of(kf);
  int page = pt_row[ring > 0 ? (t / P) % ring : t / P];
  if (page < 0) page = 0;
  if (page >= num_pages) page = num_pages - 1;
  uint16_t ks;
  kvq_oracle_read_slot_fmt(pool, P, Hkv, D, vb, page, t % P, h, kc, &ks, vc, vs);
  double sk = kvq_oracle_fp16_to_double(ks);
  /* fp8 (kf 2): the code bytes are E4M3 values; otherwise two's complement integers */
  for (int d = 0; d < D; ++d) {
    double kcode = kf == 2 ? kvq_oracle_e4m3_to_double((uint8_t)kc[d]) : (double)kc[d];
    kd[d] = kcode * sk;
  }
  for (int d = 0; d < D; ++d) {
    double vcode = kf == 2 ? kvq_oracle_e4m3_to_double((uint8_t)vc[d]) : (double)vc[d];
    vd[d] = vcode * kvq_oracle_fp16_to_double(vs[d / 32]);
  }
}

/* First and last token row i of a sequence of L tokens sees: the causal mask of an MTP verify
 * step ends row i at L - R + i; a window of W > 0 tokens starts it W - 1 tokens earlier (never
 * before token 0). */
static void row_range(int L, int R, int i, int window, int* first, int* last) {
  *last = L - R + i;
  *first = window > 0 ? *last - window + 1 : 0;
  if (*first < 0) *first = 0;
}

/* Softmax weights of one output row (sequence b, query row i, query head hq): w[t] for
 * t < L (0 where masked).  Returns the number of attended tokens; *m_out and *sum_out get the
 * max logit and sum of exp(z - max) for the log-sum-exp. */
static int row_weights(const uint8_t* pool, int num_pages, int P, int Hkv, int D, int kf,
                       int window, int ring, const uint16_t* q, const int32_t* page_table,
                       const int32_t* seq_lens, int R, int Hq, int max_pages, double scale, int b,
                       int i, int hq, double* w, double* m_out, double* sum_out) {
  int G = Hq / Hkv;
  int h = hq / G;
  int L = seq_lens[b];
  int first, last;
  row_range(L, R, i, window, &first, &last);
  int n = last - first + 1;
  if (last < 0 || n <= 0) {
    *m_out = -INFINITY;
    *sum_out = 0.0;
    return 0;
  }
  double* qd = (double*)malloc(sizeof(double) * D);
  double* kd = (double*)malloc(sizeof(double) * D);
  double* vd = (double*)malloc(sizeof(double) * D);
  int8_t* kc = (int8_t*)malloc((size_t)D);
  int8_t* vc = (int8_t*)malloc((size_t)D);
  uint16_t* vs = (uint16_t*)malloc(sizeof(uint16_t) * (D / 32));
  const uint16_t* qrow = q + (((size_t)b * R + i) * Hq + hq) * D;
  for (int d = 0; d < D; ++d) qd[d] = kvq_oracle_fp16_to_double(qrow[d]);
  const int32_t* pt_row = page_table + (size_t)b * max_pages;
  double m = -INFINITY;
  for (int t = first; t <= last; ++t) {
    token_kv(pool, num_pages, P, Hkv, D, kf, ring, pt_row, t, h, kd, vd, kc, vc, vs);
    double dot = 0.0;
    for (int d = 0; d < D; ++d) dot += qd[d] * kd[d];
    w[t] = scale * dot; /* logit z_t, replaced by its weight below */
    if (w[t] > m) m = w[t];
  }
  double sum = 0.0;
  for (int t = first; t <= last; ++t) {
    w[t] = exp(w[t] - m);
    sum += w[t];
  }
  for (int t = first; t <= last; ++t) w[t] /= sum;
  *m_out = m;
  *sum_out = sum;
  free(qd); free(kd); free(vd); free(kc); free(vc); free(vs);
  return n;
}

/* Attention outputs for a list of (b, i, hq) triples (sel, n_sel of them), or for every
 * output in [b][i][hq] order when sel is NULL.  out: [count][D] fp64, lse: [count] fp64. */
void kvq_oracle_decode_attn_kf(const uint8_t* pool, int num_pages, int P, int Hkv, int D, int kf,
                               int window, int ring, const uint16_t* q, const int32_t* page_table,
                                const int32_t* seq_lens, int n_seq, int R, int Hq, int max_pages,
                                double scale, const int32_t* sel, int n_sel, double* out,
                                double* lse) {
  if (scale <= 0.0) scale = 1.0 / sqrt((double)D);
  int count = sel ? n_sel : n_seq * R * Hq;
#pragma omp parallel for schedule(dynamic, 1)
  for (int o = 0; o < count; ++o) {
    int b, i, hq;
    if (sel) {
      b = sel[3 * o];
      i = sel[3 * o + 1];
      hq = sel[3 * o + 2];
    } else {
      b = o / (R * Hq);
      i = (o / Hq) % R;
      hq = o % Hq;
    }
    int L = seq_lens[b];
    double* w = (double*)malloc(sizeof(double) * (L > 0 ? (size_t)L : 1));
    double m, sum;
    int n = row_weights(pool, num_pages, P, Hkv, D, kf, window, ring, q, page_table, seq_lens, R,
                        Hq, max_pages, scale, b, i, hq, w, &m, &sum);
    double* o_row = out + (size_t)o * D;
    for (int d = 0; d < D; ++d) o_row[d] = 0.0;
    if (n > 0) {
      double* kd = (double*)malloc(sizeof(double) * D);
      double* vd = (double*)malloc(sizeof(double) * D);
      int8_t* kc = (int8_t*)malloc((size_t)D);
      int8_t* vc = (int8_t*)malloc((size_t)D);
      uint16_t* vs = (uint16_t*)malloc(sizeof(uint16_t) * (D / 32));
      const int32_t* pt_row = page_table + (size_t)b * max_pages;
      int h = hq / (Hq / Hkv);
      int first, last;
      row_range(L, R, i, window, &first, &last);
      for (int t = first; t <= last; ++t) {
        token_kv(pool, num_pages, P, Hkv, D, kf, ring, pt_row, t, h, kd, vd, kc, vc, vs);
        for (int d = 0; d < D; ++d) o_row[d] += w[t] * vd[d];
      }
      free(kd); free(vd); free(kc); free(vc); free(vs);
      lse[o] = m + log(sum);
    } else {
      lse[o] = -INFINITY;
    }
    free(w);
  }
}

void kvq_oracle_decode_attn_fmt(const uint8_t* pool, int num_pages, int P, int Hkv, int D, int vb,
                                const uint16_t* q, const int32_t* page_table,
                                const int32_t* seq_lens, int n_seq, int R, int Hq, int max_pages,
                                double scale, const int32_t* sel, int n_sel, double* out,
                                double* lse) {
  kvq_oracle_decode_attn_kf(pool, num_pages, P, Hkv, D, vb == 8 ? 1 : 0, 0, 0, q, page_table,
                            seq_lens, n_seq, R, Hq, max_pages, scale, sel, n_sel, out, lse);
}

void kvq_oracle_decode_attn(const uint8_t* pool, int num_pages, int P, int Hkv, int D,
                            const uint16_t* q, const int32_t* page_table,
                            const int32_t* seq_lens, int n_seq, int R, int Hq, int max_pages,
                            double scale, const int32_t* sel, int n_sel, double* out,
                            double* lse) {
  kvq_oracle_decode_attn_fmt(pool, num_pages, P, Hkv, D, 4, q, page_table, seq_lens, n_seq, R, Hq,
                             max_pages, scale, sel, n_sel, out, lse);
}

/* Softmax weights of one output row, w[0..L-1] (0 where masked). Returns attended count. */
int kvq_oracle_attn_weights_kf(const uint8_t* pool, int num_pages, int P, int Hkv, int D, int kf,
                               int window, int ring, const uint16_t* q,
                                const int32_t* page_table, const int32_t* seq_lens, int R, int Hq,
                                int max_pages, double scale, int b, int i, int hq, double* w) {
  if (scale <= 0.0) scale = 1.0 / sqrt((double)D);
  int L = seq_lens[b];
  for (int t = 0; t < L; ++t) w[t] = 0.0;
  double m, sum;
  return row_weights(pool, num_pages, P, Hkv, D, kf, window, ring, q, page_table, seq_lens, R, Hq,
                     max_pages, scale, b, i, hq, w, &m, &sum);
}
int kvq_oracle_attn_weights_fmt(const uint8_t* pool, int num_pages, int P, int Hkv, int D, int vb,
                                const uint16_t* q, const int32_t* page_table,
                                const int32_t* seq_lens, int R, int Hq, int max_pages, double scale,
                                int b, int i, int hq, double* w) {
  return kvq_oracle_attn_weights_kf(pool, num_pages, P, Hkv, D, vb == 8 ? 1 : 0, 0, 0, q,
                                    page_table, seq_lens, R, Hq, max_pages, scale, b, i, hq, w);
}
int kvq_oracle_attn_weights(const uint8_t* pool, int num_pages, int P, int Hkv, int D,
                            const uint16_t* q, const int32_t* page_table,
                            const int32_t* seq_lens, int R, int Hq, int max_pages, double scale,
                            int b, int i, int hq, double* w) {
  return kvq_oracle_attn_weights_fmt(pool, num_pages, P, Hkv, D, 4, q, page_table, seq_lens, R, Hq,
                                     max_pages, scale, b, i, hq, w);
}

int kvq_oracle_num_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}

/* Threads the attention loops use from now on (the benchmark's 1-thread baseline). */
void kvq_oracle_set_num_threads(int n) {
#ifdef _OPENMP
  if (n > 0) omp_set_num_threads(n);
#else
  (void)n;
#endif
}

/*
 * oracle.c -- plain, slow, single-threaded CPU oracle for paged FP8 decode attention.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may call, link or load this file:
 * only the tests, the smoke check and the CPU-baseline leg of the benchmark use it.  It shares
 * no code, header, table or constant generator with the HIP library.
 *
 * Sources (the web pages this project is built from):
 *   [CF §Quantize]  Cloudflare, "Smaller, faster, safer: running Kimi and GLM at scale", Chinese
 *                   translation on feinterview.poetries.top, section "量化 KV cache" (quantize the
 *                   KV cache): K and V of every processed token are kept as 8-bit floating point
 *                   (FP8, e4m3) instead of BF16, and the FP8 attention kernel converts the values
 *                   when it reads them.
 *   [CF §Protect]   same page, section "保护共享 KV cache" (protect the shared KV cache): every
 *                   physical cache page carries a tag that changes when the page is reallocated;
 *                   the server records which pages and tags each request expects; before a
 *                   supported decode operation reads the cache the mapping is checked and, on any
 *                   mismatch, the affected request is aborted.  The check runs as its own batched
 *                   pass, not fused into attention.
 *   [Siami §KVQ]    siami.tw digest, section "KV 快取量化" and its BF16-vs-FP8 table.
 *   [remio §Safety] remio.ai analysis "Cloudflare 小型模型服务降低内存占用，但安全性成为考验",
 *                   the passages on shared-cache safety: pages are allocated, read, freed and
 *                   reallocated continuously; the tag works like a generation counter.
 *
 * What the pages leave open (format variant, rounding, scales, layout, softmax form) is fixed
 * by the readings listed in the project's design notes; each function below states the reading
 * it uses.  Every floating-point result here is computed in fp64 except where the definition
 * itself is an fp32 operation (the fp32 division in quantisation, the fp32 scale).
 *
 * Layouts (the library boundary defines the same ones, independently):
 *   K pool : [num_pages][Hkv][Dk/C][page_size][C]   C = 64 / bytes-per-element dimensions per
 *            chunk (64 for FP8 codes, 32 for bf16): inside one (page, head) block the row of a
 *            token is cut into 64-byte chunks, stored chunk by chunk (all tokens' chunk 0, then
 *            all tokens' chunk 1, ...).  Dk is a multiple of 64.
 *   V pool : [num_pages][Hkv][Dv][page_size]   (inside one page-head block, one dimension's
 *                                               values for the page's tokens are contiguous)
 *   shared-KV mode (no V pool): V of a token is the first Dv dimensions of its K row.
 *   Token t of sequence b lives in physical page page_table[b*pt_stride + t/page_size],
 *   slot t % page_size.
 */
#include <fenv.h>
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORACLE_KV_FP8 0
#define ORACLE_KV_BF16 1
#define ORACLE_ACT_F32 0
#define ORACLE_ACT_BF16 1

/* ---------------------------------------------------------------------------------------------
 * FP8 e4m3 (OCP "E4M3FN": 1 sign bit, 4 exponent bits with bias 7, 3 mantissa bits, no
 * infinities, NaN = S.1111.111, largest finite magnitude 448).  [CF §Quantize] names "FP8,
 * e4m3"; the variant, round-to-nearest-even and saturation at +-448 are the readings adopted.
 * ------------------------------------------------------------------------------------------- */

/* Exact value of an e4m3 code, as a double (NaN for 0x7F / 0xFF). */
double oracle_e4m3_decode(uint8_t c) {
  int sign = (c >> 7) & 1;
  int e = (c >> 3) & 15;
  int m = c & 7;
  double mag;
  if (e == 15 && m == 7) {
    mag = NAN;
  } else if (e == 0) {
    mag = ldexp((double)m, -9); /* subnormal: m * 2^-6 / 8 */
  } else {
    mag = ldexp((double)(8 + m), e - 10); /* (1 + m/8) * 2^(e-7) */
  }
  return sign ? -mag : mag;
}

/* Round-to-nearest, ties to even, of a double that is exactly representable in fp64 to an
 * integer.  The default rounding mode of the C runtime is to-nearest-even. */
static double rne_integer(double v) { return nearbyint(v); }

/* Nearest e4m3 code to the fp32 value t, ties to even mantissa, saturating at +-448. */
uint8_t oracle_e4m3_encode(float t) {
  uint8_t sign = signbit(t) ? 0x80 : 0x00;
  if (isnan(t)) return (uint8_t)(sign | 0x7F);
  double a = fabs((double)t);
  if (a >= 448.0) return (uint8_t)(sign | 0x7E); /* saturate (includes infinity) */
  if (a < ldexp(1.0, -6)) {
    /* subnormal range: spacing 2^-9; m = 8 is the smallest normal 2^-6 (code 0x08) */
    double m = rne_integer(a * 512.0);
    return (uint8_t)(sign | (uint8_t)m);
  }
  int e;
  (void)frexp(a, &e); /* a = f * 2^e with f in [0.5, 1) */
  e -= 1;             /* now a = (1 + frac) * 2^e, e in [-6, 8] */
  double m = rne_integer((ldexp(a, -e) - 1.0) * 8.0); /* exact in fp64 */
  if (m == 8.0) {                                     /* rounded up into the next binade */
    e += 1;
    m = 0.0;
  }
  /* a < 448 implies m <= 6 when e == 8, so the NaN pattern is never produced here */
  return (uint8_t)(sign | (uint8_t)(((e + 7) << 3) | (int)m));
}

/* Quantise one value with a per-head scale: t = fp32(x / s) (IEEE division in single
 * precision, the reading adopted for "quantize on append"), then the nearest e4m3 code. */
uint8_t oracle_quantize_fp8(float x, float s) {
  volatile float t = x / s; /* single-precision division; volatile keeps it a float op */
  return oracle_e4m3_encode(t);
}

/* ---------------------------------------------------------------------------------------------
 * bf16 (1 sign, 8 exponent, 7 mantissa bits).  Conversion from fp32 picks the nearer of the two
 * bf16 neighbours of x; an exact tie goes to the one with an even last mantissa bit.
 * ------------------------------------------------------------------------------------------- */

float oracle_bf16_to_f32(uint16_t h) {
  uint32_t u = (uint32_t)h << 16;
  float f;
  memcpy(&f, &u, 4);
  return f;
}

uint16_t oracle_bf16_from_f32(float x) {
  uint16_t sign = signbit(x) ? 0x8000 : 0x0000;
  if (isnan(x)) return (uint16_t)(sign | 0x7FC0);
  uint32_t u;
  memcpy(&u, &x, 4);
  uint16_t lo = (uint16_t)(u >> 16); /* neighbour toward zero (same sign) */
  double ax = fabs((double)x);
  double alo = fabs((double)oracle_bf16_to_f32(lo));
  if (ax == alo) return lo; /* exactly representable, including +-inf and +-0 */
  uint16_t hi = (uint16_t)(lo + 1); /* neighbour away from zero */
  double ahi;
  if ((hi & 0x7FFF) == 0x7F80)
    ahi = ldexp(1.0, 128); /* overflow: round as if the exponent range were unbounded */
  else
    ahi = fabs((double)oracle_bf16_to_f32(hi));
  double dlo = ax - alo, dhi = ahi - ax;
  if (dlo < dhi) return lo;
  if (dhi < dlo) return hi;
  return (lo & 1) ? hi : lo;
}

/* Value of one activation element (fp32 or bf16 storage) as a float. */
static float act_load(const void* p, int dt, size_t i) {
  if (dt == ORACLE_ACT_BF16) return oracle_bf16_to_f32(((const uint16_t*)p)[i]);
  return ((const float*)p)[i];
}

/* Element offset of K[page][head h][token slot][dim d] in the dimension-chunked K pool. */
static size_t k_offset(int32_t page, int32_t h, int32_t slot, int32_t d, int32_t Hkv, int32_t P, int32_t Dk,
                       int kv_dt) {
  const int32_t C = (kv_dt == ORACLE_KV_FP8) ? 64 : 32;
  return ((size_t)page * Hkv + h) * (size_t)P * Dk + (size_t)(d / C) * P * C + (size_t)slot * C + (d % C);
}

/* Exact value of one stored KV element (FP8 code times its scale, or the bf16 value). */
static double kv_value(const void* pool, int kv_dt, size_t i, double scale) {
  if (kv_dt == ORACLE_KV_BF16) return (double)oracle_bf16_to_f32(((const uint16_t*)pool)[i]);
  return oracle_e4m3_decode(((const uint8_t*)pool)[i]) * scale; /* exact: 4-bit x 24-bit */
}

/* ---------------------------------------------------------------------------------------------
 * Scale setup.  Reading: per (layer, KV head) scale s = fp32(amax / 448), amax = largest |x|
 * over every token and dimension of that head in the initial fill; amax == 0 gives s = 1.
 * x : [T][H][D], fp32 or bf16.  scale_out : [H].
 * ------------------------------------------------------------------------------------------- */
/* amax[h] = max(amax[h], largest |x| of head h); lets a fill be processed in chunks.
 * NaN inputs never win a comparison and so are ignored. */
void oracle_kv_absmax_update(const void* x, int x_dt, int64_t T, int H, int D, float* amax) {
  for (int h = 0; h < H; ++h) {
    float m = amax[h];
    for (int64_t t = 0; t < T; ++t)
      for (int d = 0; d < D; ++d) {
        float v = fabsf(act_load(x, x_dt, ((size_t)t * H + h) * D + d));
        if (v > m) m = v;
      }
    amax[h] = m;
  }
}

/* s = fp32(amax / 448) (single-precision division); amax == 0 gives s = 1. */
float oracle_scale_from_absmax(float amax) {
  volatile float s = amax / 448.0f;
  return (amax == 0.0f) ? 1.0f : s;
}

void oracle_kv_scales(const void* x, int x_dt, int64_t T, int H, int D, float* scale_out) {
  for (int h = 0; h < H; ++h) scale_out[h] = 0.0f;
  oracle_kv_absmax_update(x, x_dt, T, H, D, scale_out);
  for (int h = 0; h < H; ++h) scale_out[h] = oracle_scale_from_absmax(scale_out[h]);
}

/* ---------------------------------------------------------------------------------------------
 * Quantize-on-append.  Token i belongs to sequence seq_ids[i] at position positions[i]; its
 * K row (Dk values per head) and V row (Dv values per head) are stored into the page slot the
 * page table names.  FP8: code = e4m3(fp32(x / s_head)).  BF16: the nearest bf16.
 * Rows of aborted sequences (abort_mask non-NULL and set) are not written.  A sequence id outside
 * [0, B), a position outside the page table or a page id outside [0, num_pages) names no slot, and
 * the token is skipped.
 * v_pool == NULL selects shared-KV mode: only K is stored, V is read from K's first Dv dims.
 * ------------------------------------------------------------------------------------------- */
void oracle_kv_append(const void* k_new, const void* v_new, int in_dt, void* k_pool, void* v_pool,
                      int kv_dt, const int32_t* page_table, int32_t pt_stride, const int32_t* seq_ids,
                      const int32_t* positions, int32_t T, const float* k_scale, const float* v_scale,
                      const uint8_t* abort_mask, int32_t B, int32_t Hkv, int32_t Dk, int32_t Dv,
                      int32_t page_size, int32_t num_pages) {
  for (int32_t i = 0; i < T; ++i) {
    int32_t b = seq_ids[i];
    int32_t pos = positions[i];
    if (b < 0 || b >= B) continue;
    if (abort_mask && abort_mask[b]) continue;
    if (pos < 0 || pos >= pt_stride * page_size) continue;
    int32_t page = page_table[(size_t)b * pt_stride + pos / page_size];
    int32_t slot = pos % page_size;
    if (page < 0 || page >= num_pages) continue;
    for (int32_t h = 0; h < Hkv; ++h) {
      for (int32_t d = 0; d < Dk; ++d) {
        float x = act_load(k_new, in_dt, ((size_t)i * Hkv + h) * Dk + d);
        size_t dst = k_offset(page, h, slot, d, Hkv, page_size, Dk, kv_dt);
        if (kv_dt == ORACLE_KV_FP8)
          ((uint8_t*)k_pool)[dst] = oracle_quantize_fp8(x, k_scale[h]);
        else
          ((uint16_t*)k_pool)[dst] = oracle_bf16_from_f32(x);
      }
      if (v_pool == NULL) continue;
      for (int32_t d = 0; d < Dv; ++d) {
        float x = act_load(v_new, in_dt, ((size_t)i * Hkv + h) * Dv + d);
        size_t dst = (((size_t)page * Hkv + h) * Dv + d) * page_size + slot;
        if (kv_dt == ORACLE_KV_FP8)
          ((uint8_t*)v_pool)[dst] = oracle_quantize_fp8(x, v_scale[h]);
        else
          ((uint16_t*)v_pool)[dst] = oracle_bf16_from_f32(x);
      }
    }
  }
}

/* ---------------------------------------------------------------------------------------------
 * Page transcode, BF16 cache -> FP8 cache: the pages keep BF16 for the compute-bound prefill pool
 * and FP8 for the memory-bound decode pool, so a request's cache changes format when it moves
 * from one to the other.  Reading: every stored value is quantised exactly as on append,
 * code = e4m3(fp32(x / s_head)) with x the bf16 value, and the token keeps its slot.  Page
 * src_pages[i] of the BF16 pools goes to page dst_pages[i] of the FP8 pools; a pair with an id out
 * of range is skipped.  v_src == NULL selects shared-KV pools (K only).
 * ------------------------------------------------------------------------------------------- */
void oracle_kv_transcode_pages(const void* k_src, const void* v_src, void* k_dst, void* v_dst,
                               const int32_t* src_pages, const int32_t* dst_pages, int32_t n_pages,
                               const float* k_scale, const float* v_scale, int32_t Hkv, int32_t Dk, int32_t Dv,
                               int32_t page_size, int32_t num_src_pages, int32_t num_dst_pages) {
  for (int32_t i = 0; i < n_pages; ++i) {
    int32_t sp = src_pages[i], dp = dst_pages[i];
    if (sp < 0 || sp >= num_src_pages || dp < 0 || dp >= num_dst_pages) continue;
    for (int32_t h = 0; h < Hkv; ++h)
      for (int32_t t = 0; t < page_size; ++t) {
        for (int32_t d = 0; d < Dk; ++d) {
          float x = oracle_bf16_to_f32(((const uint16_t*)k_src)[k_offset(sp, h, t, d, Hkv, page_size, Dk,
                                                                          ORACLE_KV_BF16)]);
          ((uint8_t*)k_dst)[k_offset(dp, h, t, d, Hkv, page_size, Dk, ORACLE_KV_FP8)] =
              oracle_quantize_fp8(x, k_scale[h]);
        }
        if (v_src == NULL) continue;
        for (int32_t d = 0; d < Dv; ++d) {
          float x = oracle_bf16_to_f32(((const uint16_t*)v_src)[(((size_t)sp * Hkv + h) * Dv + d) * page_size + t]);
          ((uint8_t*)v_dst)[(((size_t)dp * Hkv + h) * Dv + d) * page_size + t] = oracle_quantize_fp8(x, v_scale[h]);
        }
      }
  }
}

/* ---------------------------------------------------------------------------------------------
 * Page allocator and tag tracker.  Every physical page carries a tag that changes when the page is
 * reallocated, and each request records the (page, tag) pairs it expects, so a request still
 * holding a page that was given to someone else fails the tag check.  Readings: the free pages
 * form a stack (entries [0, *free_count) of free_list, the top last); a page's tag is incremented
 * (wrapping) each time it is handed out, and a request expects the tag the page had when it got
 * it; freeing changes no tag.  live_tags == NULL is the no-op tracker: pages only.
 * ------------------------------------------------------------------------------------------- */
void oracle_pages_init(int32_t* free_list, int32_t* free_count, uint32_t* live_tags, int32_t num_pages) {
  for (int32_t i = 0; i < num_pages; ++i) {
    free_list[i] = num_pages - 1 - i; /* page 0 ends up on top */
    if (live_tags) live_tags[i] = 0;
  }
  *free_count = num_pages;
}

/* Requests in order; request b wants counts[b] pages in slots first_slot[b] .. + counts[b] - 1 of
 * its page-table row.  An invalid request (negative count or slot, or a range past the row) is
 * refused and asks for nothing.  Pages are popped one at a time from the top; as soon as a valid
 * request does not fit, it and every later request are refused. */
void oracle_pages_alloc(int32_t* free_list, int32_t* free_count, uint32_t* live_tags, int32_t num_pages,
                        const int32_t* counts, const int32_t* first_slot, int32_t B, int32_t* page_table,
                        uint32_t* expected_tags, int32_t pt_stride, uint8_t* granted) {
  int32_t top = *free_count;
  if (top < 0) top = 0;
  if (top > num_pages) top = num_pages;
  int out_of_pages = 0;
  for (int32_t b = 0; b < B; ++b) {
    int32_t n = counts[b], f = first_slot[b];
    int valid = n >= 0 && f >= 0 && (int64_t)f + n <= pt_stride;
    granted[b] = 0;
    if (!valid) continue;
    if (out_of_pages || n > top) {
      out_of_pages = 1;
      continue;
    }
    granted[b] = 1;
    for (int32_t j = 0; j < n; ++j) {
      int32_t page = free_list[--top];
      size_t at = (size_t)b * pt_stride + f + j;
      page_table[at] = page;
      if (live_tags) {
        uint32_t tag = 0;
        if (page >= 0 && page < num_pages) tag = ++live_tags[page];
        if (expected_tags) expected_tags[at] = tag;
      }
    }
  }
  *free_count = top;
}

/* Push pages[0..n) in order; ids outside [0, num_pages) and ids that find the stack full are
 * rejected.  status[0] = pushed, status[1] = rejected. */
void oracle_pages_free(int32_t* free_list, int32_t* free_count, const int32_t* pages, int32_t n, int32_t num_pages,
                       int32_t* status) {
  int32_t top = *free_count;
  if (top < 0) top = 0;
  if (top > num_pages) top = num_pages;
  int32_t kept = 0;
  for (int32_t i = 0; i < n; ++i) {
    int32_t id = pages[i];
    if (id < 0 || id >= num_pages || top >= num_pages) continue;
    free_list[top++] = id;
    ++kept;
  }
  *free_count = top;
  status[0] = kept;
  status[1] = n - kept;
}

/* ---------------------------------------------------------------------------------------------
 * INT4 weight-only GEMV (decode with 4-bit integer weights).  Reading: symmetric integers
 * q in [-8, 7], one fp32 scale per output column and group of 128 consecutive k, bf16 activations:
 *   y[m][n] = sum_k x[m][k] * q[n][k] * s[n][k / 128]     (fp64, straight sum over k)
 * x : [M][K] bf16 bits;  q : [N][K] int8;  s : [N][K/128];  y : [M][N] double.
 * ------------------------------------------------------------------------------------------- */
void oracle_w4a16_gemv(const uint16_t* x, const int8_t* q, const float* s, int32_t M, int32_t N, int32_t K,
                       double* y) {
  int32_t G = K / 128;
  for (int32_t m = 0; m < M; ++m)
    for (int32_t n = 0; n < N; ++n) {
      double acc = 0.0;
      for (int32_t k = 0; k < K; ++k)
        acc += (double)oracle_bf16_to_f32(x[(size_t)m * K + k]) * (double)q[(size_t)n * K + k] *
               (double)s[(size_t)n * G + k / 128];
      y[(size_t)m * N + n] = acc;
    }
}

/* ---------------------------------------------------------------------------------------------
 * Batched page-tag check [CF §Protect].  For request b with n_b = ceil(L_b / page_size) pages,
 *   abort[b] = OR over j < n_b of ( page_table[b][j] not in [0, num_pages)
 *                                   or live_tags[page_table[b][j]] != expected_tags[b][j] ).
 * Entries j >= n_b are not part of the request and are ignored.  A length that is negative or
 * needs more than pt_stride pages cannot be checked and aborts the request.
 * ------------------------------------------------------------------------------------------- */
void oracle_kv_tag_verify(const int32_t* page_table, int32_t pt_stride, const uint32_t* expected_tags,
                          const int32_t* seq_lens, const uint32_t* live_tags, int32_t num_pages,
                          uint8_t* abort_mask, int32_t B, int32_t page_size) {
  for (int32_t b = 0; b < B; ++b) {
    int32_t L = seq_lens[b];
    uint8_t bad = 0;
    if (L < 0 || (int64_t)L > (int64_t)pt_stride * page_size) {
      bad = 1;
    } else {
      int32_t n = (L + page_size - 1) / page_size;
      for (int32_t j = 0; j < n; ++j) {
        int32_t p = page_table[(size_t)b * pt_stride + j];
        if (p < 0 || p >= num_pages || live_tags[p] != expected_tags[(size_t)b * pt_stride + j]) bad = 1;
      }
    }
    abort_mask[b] = bad;
  }
}

/* ---------------------------------------------------------------------------------------------
 * Attention for one (sequence b, query head h), fp64 throughout:
 *   g = h / G (contiguous query-head groups share KV head g), G = Hq / Hkv
 *   s_t = sm_scale * sum_d q[d] * K_t[d],  t in [t0, t1)
 *   m = max_t s_t,  w_t = exp(s_t - m),  l = sum_t w_t,  o[d] = sum_t w_t V_t[d]
 * K_t[d] and V_t[d] are the exact dequantised values (code times per-head scale, or bf16).
 * Writes m, l and the unnormalised o[Dv]; an empty range gives m = -inf, l = 0, o = 0.
 * ------------------------------------------------------------------------------------------- */
static void attn_partial(const void* q, int q_dt, const void* k_pool, const void* v_pool, int kv_dt,
                         const int32_t* page_table, int32_t pt_stride, const float* k_scale,
                         const float* v_scale, double sm_scale, int32_t b, int32_t h, int32_t Hq,
                         int32_t Hkv, int32_t Dk, int32_t Dv, int32_t page_size, int32_t t0, int32_t t1,
                         double* m_out, double* l_out, double* o) {
  int32_t G = Hq / Hkv;
  int32_t g = h / G;
  double sk = (kv_dt == ORACLE_KV_FP8) ? (double)k_scale[g] : 1.0;
  double sv = (kv_dt == ORACLE_KV_FP8) ? (double)(v_pool ? v_scale[g] : k_scale[g]) : 1.0;
  int32_t n = t1 - t0;
  for (int32_t d = 0; d < Dv; ++d) o[d] = 0.0;
  if (n <= 0) {
    *m_out = -INFINITY;
    *l_out = 0.0;
    return;
  }
  double* s = (double*)malloc(sizeof(double) * (size_t)n);
  /* pass 1: scores */
  for (int32_t t = t0; t < t1; ++t) {
    int32_t page = page_table[(size_t)b * pt_stride + t / page_size];
    int32_t slot = t % page_size;
    double acc = 0.0;
    for (int32_t d = 0; d < Dk; ++d) {
      double qd = (double)act_load(q, q_dt, ((size_t)b * Hq + h) * Dk + d);
      acc += qd * kv_value(k_pool, kv_dt, k_offset(page, g, slot, d, Hkv, page_size, Dk, kv_dt), sk);
    }
    s[t - t0] = sm_scale * acc;
  }
  double m = s[0];
  for (int32_t i = 1; i < n; ++i)
    if (s[i] > m) m = s[i];
  /* pass 2: weights and weighted sum of V */
  double l = 0.0;
  for (int32_t t = t0; t < t1; ++t) {
    double w = exp(s[t - t0] - m);
    l += w;
    int32_t page = page_table[(size_t)b * pt_stride + t / page_size];
    int32_t slot = t % page_size;
    for (int32_t d = 0; d < Dv; ++d) {
      double v;
      if (v_pool)
        v = kv_value(v_pool, kv_dt, (((size_t)page * Hkv + g) * Dv + d) * page_size + slot, sv);
      else
        v = kv_value(k_pool, kv_dt, k_offset(page, g, slot, d, Hkv, page_size, Dk, kv_dt), sv);
      o[d] += w * v;
    }
  }
  free(s);
  *m_out = m;
  *l_out = l;
}

/* Full decode attention for the listed (b, h) rows; out_rows : [nrows][Dv] fp64.
 * Rows of aborted requests and rows with L_b <= 0 are all zeros. */
void oracle_paged_decode_attn_rows(const void* q, int q_dt, const void* k_pool, const void* v_pool, int kv_dt,
                                   const int32_t* page_table, int32_t pt_stride, const int32_t* seq_lens,
                                   const float* k_scale, const float* v_scale, const uint8_t* abort_mask,
                                   double sm_scale, int32_t Hq, int32_t Hkv, int32_t Dk, int32_t Dv,
                                   int32_t page_size, const int32_t* rows_b, const int32_t* rows_h,
                                   int32_t nrows, double* out_rows) {
  double* o = (double*)malloc(sizeof(double) * (size_t)Dv);
  for (int32_t r = 0; r < nrows; ++r) {
    int32_t b = rows_b[r], h = rows_h[r];
    double* dst = out_rows + (size_t)r * Dv;
    int32_t L = seq_lens[b];
    if ((abort_mask && abort_mask[b]) || L <= 0) {
      for (int32_t d = 0; d < Dv; ++d) dst[d] = 0.0;
      continue;
    }
    double m, l;
    attn_partial(q, q_dt, k_pool, v_pool, kv_dt, page_table, pt_stride, k_scale, v_scale, sm_scale, b, h, Hq,
                 Hkv, Dk, Dv, page_size, 0, L, &m, &l, o);
    for (int32_t d = 0; d < Dv; ++d) dst[d] = o[d] / l;
  }
  free(o);
}

/* All rows: out : [B][Hq][Dv] fp64. */
void oracle_paged_decode_attn(const void* q, int q_dt, const void* k_pool, const void* v_pool, int kv_dt,
                              const int32_t* page_table, int32_t pt_stride, const int32_t* seq_lens,
                              const float* k_scale, const float* v_scale, const uint8_t* abort_mask,
                              double sm_scale, int32_t B, int32_t Hq, int32_t Hkv, int32_t Dk, int32_t Dv,
                              int32_t page_size, double* out) {
  int32_t rb, rh;
  for (int32_t b = 0; b < B; ++b)
    for (int32_t h = 0; h < Hq; ++h) {
      rb = b;
      rh = h;
      oracle_paged_decode_attn_rows(q, q_dt, k_pool, v_pool, kv_dt, page_table, pt_stride, seq_lens, k_scale,
                                    v_scale, abort_mask, sm_scale, Hq, Hkv, Dk, Dv, page_size, &rb, &rh, 1,
                                    out + ((size_t)b * Hq + h) * Dv);
    }
}

/* ---------------------------------------------------------------------------------------------
 * Split-KV form of the same attention (the reading adopted for long contexts): partition i
 * covers tokens [i*split, (i+1)*split) of the sequence and yields (m_i, l_i, o_i) as above; the
 * partitions are combined by the log-sum-exp rule
 *   M = max_i m_i,  out = sum_i exp(m_i - M) o_i / sum_i exp(m_i - M) l_i.
 * Exactly equal to the single pass up to rounding.  out_rows : [nrows][Dv].
 * ------------------------------------------------------------------------------------------- */
void oracle_paged_decode_attn_split_rows(const void* q, int q_dt, const void* k_pool, const void* v_pool,
                                         int kv_dt, const int32_t* page_table, int32_t pt_stride,
                                         const int32_t* seq_lens, const float* k_scale, const float* v_scale,
                                         double sm_scale, int32_t Hq, int32_t Hkv, int32_t Dk, int32_t Dv,
                                         int32_t page_size, int32_t split, const int32_t* rows_b,
                                         const int32_t* rows_h, int32_t nrows, double* out_rows) {
  double* o = (double*)malloc(sizeof(double) * (size_t)Dv);
  for (int32_t r = 0; r < nrows; ++r) {
    int32_t b = rows_b[r], h = rows_h[r];
    int32_t L = seq_lens[b];
    double* dst = out_rows + (size_t)r * Dv;
    for (int32_t d = 0; d < Dv; ++d) dst[d] = 0.0;
    if (L <= 0) continue;
    int32_t np = (L + split - 1) / split;
    double* ms = (double*)malloc(sizeof(double) * (size_t)np);
    double* ls = (double*)malloc(sizeof(double) * (size_t)np);
    double* os = (double*)malloc(sizeof(double) * (size_t)np * Dv);
    double M = -INFINITY;
    for (int32_t i = 0; i < np; ++i) {
      int32_t t0 = i * split, t1 = (i + 1) * split < L ? (i + 1) * split : L;
      attn_partial(q, q_dt, k_pool, v_pool, kv_dt, page_table, pt_stride, k_scale, v_scale, sm_scale, b, h, Hq,
                   Hkv, Dk, Dv, page_size, t0, t1, &ms[i], &ls[i], os + (size_t)i * Dv);
      if (ms[i] > M) M = ms[i];
    }
    double den = 0.0;
    for (int32_t i = 0; i < np; ++i) den += exp(ms[i] - M) * ls[i];
    for (int32_t d = 0; d < Dv; ++d) {
      double num = 0.0;
      for (int32_t i = 0; i < np; ++i) num += exp(ms[i] - M) * os[(size_t)i * Dv + d];
      dst[d] = num / den;
    }
    free(ms);
    free(ls);
    free(os);
  }
  free(o);
}

/* Array helpers for tests (element-wise application of the scalar definitions above). */
void oracle_e4m3_encode_array(const float* t, int64_t n, uint8_t* out) {
  for (int64_t i = 0; i < n; ++i) out[i] = oracle_e4m3_encode(t[i]);
}
void oracle_e4m3_decode_array(const uint8_t* c, int64_t n, double* out) {
  for (int64_t i = 0; i < n; ++i) out[i] = oracle_e4m3_decode(c[i]);
}
void oracle_quantize_fp8_array(const float* x, float s, int64_t n, uint8_t* out) {
  for (int64_t i = 0; i < n; ++i) out[i] = oracle_quantize_fp8(x[i], s);
}
void oracle_bf16_from_f32_array(const float* x, int64_t n, uint16_t* out) {
  for (int64_t i = 0; i < n; ++i) out[i] = oracle_bf16_from_f32(x[i]);
}

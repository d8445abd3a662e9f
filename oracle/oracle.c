/*
 * oracle.c -- plain fp64 CPU reference for the long-KV-cache decode path.
 *
 * TEST INFRASTRUCTURE ONLY: loaded by the tests, the smoke check and the
 * benchmark's CPU-baseline leg; never by the product library.  Shares no code
 * with the GPU path.  Each routine cites the passage it follows.
 *
 * Build: gcc -O2 -fopenmp -shared -fPIC oracle.c -o liboracle.so -lm
 */
#include "oracle.h"

#include <math.h>
#include <pthread.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* ------------------------------------------------------------------------- */
/* Exact widening of 16-bit floats.                                           */
/* ------------------------------------------------------------------------- */

/* IEEE binary16: 1 sign, 5 exponent (bias 15), 10 fraction bits. */
static double widen_f16(uint16_t h) {
  int sign = h >> 15;
  int e = (h >> 10) & 0x1f;
  int f = h & 0x3ff;
  double mag;
  if (e == 0)
    mag = ldexp((double)f, -24);           /* subnormal: f * 2^-24 */
  else if (e == 31)
    mag = f ? NAN : INFINITY;
  else
    mag = ldexp((double)(1024 + f), e - 25); /* (1 + f/1024) * 2^(e-15) */
  return sign ? -mag : mag;
}

/* bfloat16 is the upper half of an IEEE binary32. */
static double widen_bf16(uint16_t h) {
  uint32_t u = (uint32_t)h << 16;
  float f;
  memcpy(&f, &u, sizeof f);
  return (double)f;
}

double orc_widen(uint16_t bits, int kind) {
  return kind == 0 ? widen_f16(bits) : widen_bf16(bits);
}

/* OCP 8-bit e4m3 (the "fn" variant: no infinities): 1 sign, 4 exponent
 * (bias 7) and 3 fraction bits; exponent 0 is subnormal (f * 2^-9); the one
 * pattern with every exponent and fraction bit set is NaN; the largest
 * magnitude is 448.  A KV element stored this way means code * scale, one
 * scale per tensor (the CLO page's open question on FP8 KV caches). */
static double widen_e4m3(uint8_t c) {
  int sign = c >> 7;
  int e = (c >> 3) & 0xf;
  int f = c & 0x7;
  double mag;
  if (e == 0xf && f == 0x7)
    mag = NAN;
  else if (e == 0)
    mag = ldexp((double)f, -9);
  else
    mag = ldexp((double)(8 + f), e - 10); /* (1 + f/8) * 2^(e-7) */
  return sign ? -mag : mag;
}

double orc_widen_e4m3(uint8_t code) { return widen_e4m3(code); }

/* Lookup table of the two widenings: 2 x 65536 doubles, filled once. */
static double g_lut[2][65536];
static pthread_once_t g_lut_once = PTHREAD_ONCE_INIT;
static void fill_lut(void) {
  for (int i = 0; i < 65536; ++i) {
    g_lut[0][i] = widen_f16((uint16_t)i);
    g_lut[1][i] = widen_bf16((uint16_t)i);
  }
}
static const double* lut(int kind) {
  pthread_once(&g_lut_once, fill_lut);
  return g_lut[kind ? 1 : 0];
}

void orc_widen_array(const uint16_t* src, double* dst, size_t n, int kind) {
  const double* L = lut(kind);
  for (size_t i = 0; i < n; ++i) dst[i] = L[src[i]];
}

void orc_widen_e4m3_array(const uint8_t* src, double* dst, size_t n) {
  for (size_t i = 0; i < n; ++i) dst[i] = widen_e4m3(src[i]);
}

/* A K or V tensor as the attention reads it: 16-bit elements of the query's
 * kind, or e4m3 codes times the tensor's scale. */
typedef struct {
  const void* base;
  int fp8;
  double scale;
  const double* lut;
} kv_view;

static inline double kv_elem(const kv_view* t, int64_t i) {
  return t->fp8 ? t->scale * widen_e4m3(((const uint8_t*)t->base)[i])
                : t->lut[((const uint16_t*)t->base)[i]];
}

static kv_view kv16(const uint16_t* base, int kind) {
  kv_view t = {base, 0, 1.0, lut(kind)};
  return t;
}

int orc_max_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}

static void set_threads(int nthreads) {
#ifdef _OPENMP
  if (nthreads > 0) omp_set_num_threads(nthreads);
#else
  (void)nthreads;
#endif
}

/* ------------------------------------------------------------------------- */
/* Attention of one query over a list of rows.                                */
/* KVPR page, section A3 (MHA equation): z = softmax(q K^T / sqrt(d)) V.      */
/* The softmax is evaluated as exp(s - max) / sum exp(s - max), which is the  */
/* same number as exp(s) / sum exp(s).                                         */
/* ------------------------------------------------------------------------- */

/* Scores s_t = scale * q . K_t for every listed row. */
static void scores(const double* L, int D, double scale, const uint16_t* q,
                   const kv_view* k, const int64_t* rows, int n, double* s) {
  for (int t = 0; t < n; ++t) {
    double acc = 0.0;
    for (int d = 0; d < D; ++d) acc += L[q[d]] * kv_elem(k, rows[t] + d);
    s[t] = scale * acc;
  }
}

static void attend_rows_view(int D, double scale, int kind, const uint16_t* q,
                             const kv_view* k, const kv_view* v, const int64_t* rows, int n,
                             double* o_unnorm, double* m_out, double* l_out) {
  const double* L = lut(kind);
  for (int d = 0; d < D; ++d) o_unnorm[d] = 0.0;
  if (n <= 0) {
    *m_out = -INFINITY;
    *l_out = 0.0;
    return;
  }
  double* s = (double*)malloc(sizeof(double) * (size_t)n);
  scores(L, D, scale, q, k, rows, n, s);
  double m = -INFINITY;
  for (int t = 0; t < n; ++t)
    if (s[t] > m) m = s[t];
  double l = 0.0;
  for (int t = 0; t < n; ++t) {
    double p = exp(s[t] - m);
    l += p;
    for (int d = 0; d < D; ++d) o_unnorm[d] += p * kv_elem(v, rows[t] + d);
  }
  free(s);
  *m_out = m;
  *l_out = l;
}

void orc_attend_rows(int D, double scale, int kind, const uint16_t* q,
                     const uint16_t* k, const uint16_t* v, const int64_t* rows, int n,
                     double* o_unnorm, double* m_out, double* l_out) {
  const kv_view kk = kv16(k, kind), vv = kv16(v, kind);
  attend_rows_view(D, scale, kind, q, &kk, &vv, rows, n, o_unnorm, m_out, l_out);
}

/* Normalised output and natural-log lse for one query. */
static void attend(int D, double scale, int kind, const uint16_t* q, const kv_view* k,
                   const kv_view* v, const int64_t* rows, int n, double* out,
                   double* lse) {
  double m, l;
  attend_rows_view(D, scale, kind, q, k, v, rows, n, out, &m, &l);
  if (n <= 0) {
    if (lse) *lse = -INFINITY;
    return;
  }
  for (int d = 0; d < D; ++d) out[d] /= l;
  if (lse) *lse = m + log(l);
}

/* ------------------------------------------------------------------------- */
/* Decode attention over dense, ragged or paged KV.                           */
/* Paged storage follows the vLLM-style page pool + per-sequence block table  */
/* that the Neo page names (background section and PACPU in the method       */
/* details): token t of sequence b lives in page block_table[b][t / page],   */
/* slot t % page.                                                             */
/* ------------------------------------------------------------------------- */

static int decode_attn_view(int B, int Hq, int Hkv, int D, double scale, int kind, int layout,
                            int S, int page, int max_pages, const uint16_t* q,
                            const kv_view* k, const kv_view* v, const int32_t* seqlens,
                            const int32_t* cu_seqlens, const int32_t* block_table, double* out,
                            double* lse, int nthreads) {
  if (B < 0 || Hq <= 0 || Hkv <= 0 || D <= 0 || Hq % Hkv != 0) return -1;
  if (layout == 1 && !cu_seqlens) return -1;
  if (layout == 2 && (!seqlens || !block_table || page <= 0)) return -1;
  if (layout < 0 || layout > 2) return -1;
  const int G = Hq / Hkv;
  set_threads(nthreads);
  int bad = 0;
#pragma omp parallel for schedule(dynamic) reduction(| : bad)
  for (long pair = 0; pair < (long)B * Hq; ++pair) {
    const int b = (int)(pair / Hq), j = (int)(pair % Hq);
    const int g = j / G;
    int n;
    if (layout == 0) n = seqlens ? seqlens[b] : S;
    else if (layout == 1) n = cu_seqlens[b + 1] - cu_seqlens[b];
    else n = seqlens[b];
    if (n < 0 || (layout == 0 && n > S) || (layout == 2 && n > max_pages * page)) {
      bad = 1;
      continue;
    }
    int64_t* rows = (int64_t*)malloc(sizeof(int64_t) * (size_t)(n > 0 ? n : 1));
    for (int t = 0; t < n; ++t) {
      int64_t token_row; /* index of the [D] row of KV head g for token t */
      if (layout == 0)
        token_row = ((int64_t)b * S + t) * Hkv + g;
      else if (layout == 1)
        token_row = ((int64_t)cu_seqlens[b] + t) * Hkv + g;
      else {
        int64_t pg = block_table[(int64_t)b * max_pages + t / page];
        token_row = (pg * Hkv + g) * page + t % page;
      }
      rows[t] = token_row * D;
    }
    const int64_t qo = ((int64_t)b * Hq + j) * D;
    attend(D, scale, kind, q + qo, k, v, rows, n, out + qo, lse ? lse + (int64_t)b * Hq + j : NULL);
    free(rows);
  }
  return bad ? -1 : 0;
}

int orc_decode_attn(int B, int Hq, int Hkv, int D, double scale, int kind, int layout,
                    int S, int page, int max_pages,
                    const uint16_t* q, const uint16_t* k, const uint16_t* v,
                    const int32_t* seqlens, const int32_t* cu_seqlens,
                    const int32_t* block_table, double* out, double* lse, int nthreads) {
  const kv_view kk = kv16(k, kind), vv = kv16(v, kind);
  return decode_attn_view(B, Hq, Hkv, D, scale, kind, layout, S, page, max_pages, q, &kk, &vv,
                          seqlens, cu_seqlens, block_table, out, lse, nthreads);
}

int orc_decode_attn_e4m3(int B, int Hq, int Hkv, int D, double scale, int kind, int layout,
                         int S, int page, int max_pages, const uint16_t* q, const uint8_t* k,
                         const uint8_t* v, double k_scale, double v_scale,
                         const int32_t* seqlens, const int32_t* cu_seqlens,
                         const int32_t* block_table, double* out, double* lse, int nthreads) {
  const kv_view kk = {k, 1, k_scale, NULL}, vv = {v, 1, v_scale, NULL};
  return decode_attn_view(B, Hq, Hkv, D, scale, kind, layout, S, page, max_pages, q, &kk, &vv,
                          seqlens, cu_seqlens, block_table, out, lse, nthreads);
}

/* ------------------------------------------------------------------------- */
/* CLO hybrid attention: cache buffer + persistent cache, read in place.      */
/* CLO page, section 7 (hybrid attention kernel) and section 2 (persistent    */
/* cache for hard-to-reuse heads).                                            */
/* ------------------------------------------------------------------------- */

static int hybrid_attn_view(int B, int Hq, int Hkv, int D, double scale, int kind,
                            int P_slots, int pers_cap, int buf_cap, const uint16_t* q,
                            const kv_view* pk, const kv_view* pv, const int32_t* pers_len,
                            const kv_view* bk, const kv_view* bv, const int32_t* buf_len,
                            const int32_t* head_map, double* out, double* lse, int nthreads) {
  if (B < 0 || Hq <= 0 || Hkv <= 0 || D <= 0 || Hq % Hkv != 0 || !head_map) return -1;
  const int G = Hq / Hkv;
  set_threads(nthreads);
  int bad = 0;
#pragma omp parallel for schedule(dynamic) reduction(| : bad)
  for (long pair = 0; pair < (long)B * Hq; ++pair) {
    const int b = (int)(pair / Hq), j = (int)(pair % Hq);
    const int g = j / G;
    const int slot = head_map[g];
    const kv_view *K, *V;
    int n;
    int64_t base;
    if (slot >= 0) {
      if (slot >= P_slots) { bad = 1; continue; }
      n = pers_len[b];
      if (n > pers_cap) { bad = 1; continue; }
      K = pk; V = pv;
      base = ((int64_t)b * P_slots + slot) * pers_cap;
    } else {
      n = buf_len[(int64_t)b * Hkv + g];
      if (n > buf_cap) { bad = 1; continue; }
      K = bk; V = bv;
      base = ((int64_t)b * Hkv + g) * buf_cap;
    }
    if (n < 0) { bad = 1; continue; }
    int64_t* rows = (int64_t*)malloc(sizeof(int64_t) * (size_t)(n > 0 ? n : 1));
    for (int t = 0; t < n; ++t) rows[t] = (base + t) * D;
    const int64_t qo = ((int64_t)b * Hq + j) * D;
    attend(D, scale, kind, q + qo, K, V, rows, n, out + qo, lse ? lse + (int64_t)b * Hq + j : NULL);
    free(rows);
  }
  return bad ? -1 : 0;
}

int orc_hybrid_attn(int B, int Hq, int Hkv, int D, double scale, int kind,
                    int P_slots, int pers_cap, int buf_cap,
                    const uint16_t* q, const uint16_t* pers_k, const uint16_t* pers_v,
                    const int32_t* pers_len, const uint16_t* buf_k, const uint16_t* buf_v,
                    const int32_t* buf_len, const int32_t* head_map,
                    double* out, double* lse, int nthreads) {
  const kv_view pk = kv16(pers_k, kind), pv = kv16(pers_v, kind);
  const kv_view bk = kv16(buf_k, kind), bv = kv16(buf_v, kind);
  return hybrid_attn_view(B, Hq, Hkv, D, scale, kind, P_slots, pers_cap, buf_cap, q, &pk, &pv,
                          pers_len, &bk, &bv, buf_len, head_map, out, lse, nthreads);
}

int orc_hybrid_attn_e4m3(int B, int Hq, int Hkv, int D, double scale, int kind,
                         int P_slots, int pers_cap, int buf_cap, const uint16_t* q,
                         const uint8_t* pers_k, const uint8_t* pers_v, const int32_t* pers_len,
                         const uint8_t* buf_k, const uint8_t* buf_v, const int32_t* buf_len,
                         const int32_t* head_map, double k_scale, double v_scale, double* out,
                         double* lse, int nthreads) {
  const kv_view pk = {pers_k, 1, k_scale, NULL}, pv = {pers_v, 1, v_scale, NULL};
  const kv_view bk = {buf_k, 1, k_scale, NULL}, bv = {buf_v, 1, v_scale, NULL};
  return hybrid_attn_view(B, Hq, Hkv, D, scale, kind, P_slots, pers_cap, buf_cap, q, &pk, &pv,
                          pers_len, &bk, &bv, buf_len, head_map, out, lse, nthreads);
}

/* ------------------------------------------------------------------------- */
/* Index-gather sparse attention over a GPU-resident full cache.              */
/* CLO page: top-k sparse attention (10% of the tokens) with HATA's hashed     */
/* retrieval; here the exact scores stand in for the hashes.  Eq. 6: q.k =    */
/* |q| |k| cos(q, k), so the ranking of the keys does not depend on |q|.      */
/* Reading: one selection per KV head, ranking its tokens by the sum over its */
/* query heads of q_j . K_t; ties go to the smaller token index; the selected */
/* indices are returned in ascending order.                                   */
/* ------------------------------------------------------------------------- */

int orc_topk_scores(int B, int Hq, int Hkv, int D, int kind, int S, const uint16_t* q,
                    const uint16_t* k, const int32_t* seqlens, double* scores, double* mags,
                    int nthreads) {
  if (B < 0 || Hq <= 0 || Hkv <= 0 || D <= 0 || Hq % Hkv != 0 || S < 0) return -1;
  const int G = Hq / Hkv;
  const double* L = lut(kind);
  set_threads(nthreads);
#pragma omp parallel for schedule(dynamic)
  for (long pair = 0; pair < (long)B * Hkv; ++pair) {
    const int b = (int)(pair / Hkv), g = (int)(pair % Hkv);
    int n = seqlens ? seqlens[b] : S;
    if (n > S) n = S;
    for (int t = 0; t < S; ++t) {
      double acc = 0.0, mag = 0.0;
      if (t < n) {
        const uint16_t* kr = k + (((int64_t)b * S + t) * Hkv + g) * D;
        for (int j = g * G; j < (g + 1) * G; ++j) {
          const uint16_t* qr = q + ((int64_t)b * Hq + j) * D;
          for (int d = 0; d < D; ++d) {
            acc += L[qr[d]] * L[kr[d]];
            mag += fabs(L[qr[d]] * L[kr[d]]);
          }
        }
      }
      scores[pair * S + t] = acc;
      if (mags) mags[pair * S + t] = mag;
    }
  }
  return 0;
}

typedef struct {
  double s;
  int t;
} scored_token;

/* Larger score first; equal scores: smaller token first. */
static int by_score_desc(const void* pa, const void* pb) {
  const scored_token* a = (const scored_token*)pa;
  const scored_token* b = (const scored_token*)pb;
  if (a->s > b->s) return -1;
  if (a->s < b->s) return 1;
  return (a->t > b->t) - (a->t < b->t);
}

static int by_index(const void* pa, const void* pb) {
  const int32_t a = *(const int32_t*)pa, b = *(const int32_t*)pb;
  return (a > b) - (a < b);
}

int orc_topk_select(int B, int Hq, int Hkv, int D, int kind, int S, const uint16_t* q,
                    const uint16_t* k, const int32_t* seqlens, int kk, int32_t* idx,
                    int32_t* idx_len, int nthreads) {
  if (kk < 0 || B < 0 || Hkv <= 0 || S < 0) return -1;
  double* sc = (double*)malloc(sizeof(double) * (size_t)((int64_t)B * Hkv * (S > 0 ? S : 1)));
  if (!sc) return -1;
  if (orc_topk_scores(B, Hq, Hkv, D, kind, S, q, k, seqlens, sc, NULL, nthreads) != 0) {
    free(sc);
    return -1;
  }
#pragma omp parallel for schedule(dynamic)
  for (long pair = 0; pair < (long)B * Hkv; ++pair) {
    const int b = (int)(pair / Hkv);
    int n = seqlens ? seqlens[b] : S;
    if (n > S) n = S;
    if (n < 0) n = 0;
    scored_token* v = (scored_token*)malloc(sizeof(scored_token) * (size_t)(n > 0 ? n : 1));
    for (int t = 0; t < n; ++t) {
      v[t].s = sc[pair * S + t];
      v[t].t = t;
    }
    qsort(v, (size_t)n, sizeof *v, by_score_desc);
    const int m = n < kk ? n : kk;
    int32_t* out = idx + pair * (int64_t)kk;
    for (int i = 0; i < m; ++i) out[i] = v[i].t;
    qsort(out, (size_t)m, sizeof *out, by_index);
    idx_len[pair] = m;
    free(v);
  }
  free(sc);
  return 0;
}

int orc_gather_attn(int B, int Hq, int Hkv, int D, double scale, int kind, int S,
                    const uint16_t* q, const uint16_t* k, const uint16_t* v, const int32_t* idx,
                    const int32_t* idx_len, int max_k, double* out, double* lse, int nthreads) {
  if (B < 0 || Hq <= 0 || Hkv <= 0 || D <= 0 || Hq % Hkv != 0 || max_k < 0) return -1;
  const int G = Hq / Hkv;
  const kv_view kk = kv16(k, kind), vv = kv16(v, kind);
  set_threads(nthreads);
  int bad = 0;
#pragma omp parallel for schedule(dynamic) reduction(| : bad)
  for (long pair = 0; pair < (long)B * Hq; ++pair) {
    const int b = (int)(pair / Hq), j = (int)(pair % Hq);
    const int g = j / G;
    const int n = idx_len[(int64_t)b * Hkv + g];
    if (n < 0 || n > max_k) {
      bad = 1;
      continue;
    }
    int64_t* rows = (int64_t*)malloc(sizeof(int64_t) * (size_t)(n > 0 ? n : 1));
    const int32_t* ix = idx + ((int64_t)b * Hkv + g) * max_k;
    for (int t = 0; t < n; ++t) {
      if (ix[t] < 0 || ix[t] >= S) bad = 1;
      rows[t] = (((int64_t)b * S + ix[t]) * Hkv + g) * D;
    }
    if (bad) {
      free(rows);
      continue;
    }
    const int64_t qo = ((int64_t)b * Hq + j) * D;
    attend(D, scale, kind, q + qo, &kk, &vv, rows, n, out + qo, lse ? lse + (int64_t)b * Hq + j : NULL);
    free(rows);
  }
  return bad ? -1 : 0;
}

/* ------------------------------------------------------------------------- */
/* CLO threshold chain, Eqs. 7-9.                                             */
/* ------------------------------------------------------------------------- */

void orc_thresholds(int n, const double* s, double eta, double n_exp, double* tau) {
  const double pi = acos(-1.0);
  const double theta_star = acos(eta);                      /* Eq. 7 */
  for (int i = 0; i < n; ++i) {
    const double lambda = pow(s[i], n_exp);                 /* Eq. 8 */
    const double theta = lambda * theta_star + (1.0 - lambda) * pi; /* Eq. 9 */
    tau[i] = cos(theta);
  }
}

/* ------------------------------------------------------------------------- */
/* CLO head-wise approximate cache: lookup + label update.                    */
/* Section 2 (one query label per head; hit iff cos >= tau_i, else the whole  */
/* head is replaced), section 3 (a miss replaces the label with the incoming  */
/* query), Eq. 10 (importance-weighted mean of a KV head's query cosines).   */
/* ------------------------------------------------------------------------- */

int orc_headcache_lookup(int B, int Hq, int Hkv, int D, int kind, const uint16_t* q,
                         uint16_t* labels, const float* w, const float* tau,
                         uint8_t* hit, double* agg, double* cosv,
                         int32_t* miss_list, int32_t* miss_count) {
  if (B < 0 || Hq <= 0 || Hkv <= 0 || D <= 0 || Hq % Hkv != 0 || !hit) return -1;
  const double* L = lut(kind);
  const int G = Hq / Hkv;
  int32_t misses = 0;
  for (int b = 0; b < B; ++b) {
    for (int g = 0; g < Hkv; ++g) {
      int degenerate = 0;
      double num = 0.0, wsum = 0.0, csum = 0.0;
      for (int jj = 0; jj < G; ++jj) {
        const int j = g * G + jj;
        const uint16_t* qr = q + ((int64_t)b * Hq + j) * D;
        const uint16_t* lr = labels + ((int64_t)b * Hq + j) * D;
        double dot = 0.0, qq = 0.0, ll = 0.0;
        for (int d = 0; d < D; ++d) {
          const double a = L[qr[d]], c = L[lr[d]];
          dot += a * c;
          qq += a * a;
          ll += c * c;
        }
        double c = 0.0;
        if (qq == 0.0 || ll == 0.0) degenerate = 1;
        else c = dot / (sqrt(qq) * sqrt(ll));
        if (cosv) cosv[(int64_t)b * Hq + j] = c;
        num += (double)w[j] * c;
        wsum += (double)w[j];
        csum += c;
      }
      const double a = wsum != 0.0 ? num / wsum : csum / G;
      const int h = !degenerate && a >= (double)tau[g];
      hit[(int64_t)b * Hkv + g] = (uint8_t)h;
      if (agg) agg[(int64_t)b * Hkv + g] = a;
      if (!h) {
        for (int jj = 0; jj < G; ++jj) {
          const int64_t o = ((int64_t)b * Hq + g * G + jj) * D;
          memcpy(labels + o, q + o, sizeof(uint16_t) * (size_t)D);
        }
        if (miss_list) miss_list[misses] = b * Hkv + g;
        ++misses;
      }
    }
  }
  if (miss_count) *miss_count = misses;
  return 0;
}

/* ------------------------------------------------------------------------- */
/* KVPR partial recompute, section A2: K[0:l] = X[0:l] W_K, V[0:l] = X[0:l] W_V. */
/* ------------------------------------------------------------------------- */

int orc_kv_recompute(int b, int l, int h, int kind, const uint16_t* x, int64_t x_bstride,
                     const uint16_t* wk, const uint16_t* wv, const int32_t* rows, int nrows,
                     double* k_out, double* v_out, int nthreads) {
  if (b < 0 || l < 0 || h <= 0) return -1;
  if (!rows) nrows = b * l;
  const double* L = lut(kind);
  set_threads(nthreads);
  int bad = 0;
#pragma omp parallel for schedule(dynamic) reduction(| : bad)
  for (int r = 0; r < nrows; ++r) {
    const int flat = rows ? rows[r] : r;
    if (flat < 0 || flat >= b * l) { bad = 1; continue; }
    const int bi = flat / l, t = flat % l;
    const uint16_t* xr = x + (int64_t)bi * x_bstride + (int64_t)t * h;
    double* kr = k_out + (int64_t)r * h;
    double* vr = v_out + (int64_t)r * h;
    for (int n = 0; n < h; ++n) { kr[n] = 0.0; vr[n] = 0.0; }
    for (int i = 0; i < h; ++i) {
      const double xi = L[xr[i]];
      const uint16_t* wki = wk + (int64_t)i * h;
      const uint16_t* wvi = wv + (int64_t)i * h;
      for (int n = 0; n < h; ++n) {
        kr[n] += xi * L[wki[n]];
        vr[n] += xi * L[wvi[n]];
      }
    }
  }
  return bad ? -1 : 0;
}

/* KVPR page, section A2: M_X = b l h p, M_KV = 2 b (s' - l) h p, N = 4 b l h^2. */
void orc_kvpr_cost(double b, double l, double s_prime, double h, double p,
                   double* m_x, double* m_kv, double* n_flops) {
  *m_x = b * l * h * p;
  *m_kv = 2.0 * b * (s_prime - l) * h * p;
  *n_flops = 4.0 * b * l * h * h;
}

/* KVPR page, section A2, total time of one layer with split point l:
 * t(l) = M_X / v_com + max(N / v_gpu, M_KV / v_com). */
double orc_kvpr_time(double b, double l, double s_prime, double h, double p, double v_com,
                     double v_gpu) {
  double m_x, m_kv, n;
  orc_kvpr_cost(b, l, s_prime, h, p, &m_x, &m_kv, &n);
  const double t_rec = n / v_gpu, t_kv = m_kv / v_com;
  return m_x / v_com + (t_rec > t_kv ? t_rec : t_kv);
}

/* The split point of least t(l) over every integer l in [0, l_max], by
 * trying each one; the first (smallest) l wins ties. */
int orc_kvpr_best_split(double b, int s_prime, int l_max, double h, double p, double v_com,
                        double v_gpu, double* t_best) {
  int best = 0;
  double tb = orc_kvpr_time(b, 0.0, s_prime, h, p, v_com, v_gpu);
  for (int l = 1; l <= l_max; ++l) {
    const double t = orc_kvpr_time(b, (double)l, s_prime, h, p, v_com, v_gpu);
    if (t < tb) {
      tb = t;
      best = l;
    }
  }
  if (t_best) *t_best = tb;
  return best;
}

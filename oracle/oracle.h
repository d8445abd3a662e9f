/*
 * oracle.h -- plain fp64 CPU reference for the long-KV-cache decode path.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product library calls, links or
 * includes this code; only the test suite, the smoke check and the CPU-baseline
 * leg of the benchmark load it.  It shares no code, header, table or constant
 * with the GPU path.
 *
 * Every routine reads the same 16-bit host arrays the GPU reads and widens each
 * element exactly to double before any arithmetic.  Nothing is blocked, fused or
 * reordered beyond what the cited definition states.
 *
 * Element types: 0 = IEEE binary16 (fp16), 1 = bfloat16.
 * Return value of the int routines: 0 on success, -1 on a bad argument.
 */
#ifndef LKV_ORACLE_H
#define LKV_ORACLE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Exact widening of one 16-bit value to double (fp16: kind 0, bf16: kind 1). */
double orc_widen(uint16_t bits, int kind);

/* Widen n values (used by the pins that check the widening against numpy). */
void orc_widen_array(const uint16_t* src, double* dst, size_t n, int kind);

/* Exact value of an OCP e4m3 ("fn") code: bias 7, subnormal f * 2^-9, the
 * all-ones exponent-and-fraction pattern is NaN, largest magnitude 448. */
double orc_widen_e4m3(uint8_t code);
void orc_widen_e4m3_array(const uint8_t* src, double* dst, size_t n);

/*
 * Decode attention, one query token per sequence, grouped KV heads.
 * Definition: KVPR page, section A3, the MHA equation softmax(Q K^T / sqrt(d)) V,
 * applied at the decode step where one token attends to every cached token.
 *
 * layout 0 (dense) : k, v [B, S, Hkv, D]; seqlens[B] (NULL => every length is S)
 * layout 1 (ragged): k, v [T, Hkv, D] packed by sequence; cu_seqlens[B+1]
 * layout 2 (paged) : k, v [P, Hkv, page, D]; block_table[B, max_pages]; seqlens[B]
 * q [B, Hq, D]; query head j reads KV head j / (Hq / Hkv).
 * out [B, Hq, D] fp64; lse [B, Hq] fp64 natural-log log-sum-exp (may be NULL).
 * An empty sequence yields out = 0 and lse = -inf.
 */
int orc_decode_attn(int B, int Hq, int Hkv, int D, double scale, int kind, int layout,
                    int S, int page, int max_pages,
                    const uint16_t* q, const uint16_t* k, const uint16_t* v,
                    const int32_t* seqlens, const int32_t* cu_seqlens,
                    const int32_t* block_table, double* out, double* lse, int nthreads);

/*
 * The same with K and V stored as e4m3 codes (one byte per element, same
 * layouts): element = code value * k_scale (K) or * v_scale (V).  q and the
 * output keep `kind`.  (CLO page, open questions: FP8 KV caches.)
 */
int orc_decode_attn_e4m3(int B, int Hq, int Hkv, int D, double scale, int kind, int layout,
                         int S, int page, int max_pages, const uint16_t* q, const uint8_t* k,
                         const uint8_t* v, double k_scale, double v_scale,
                         const int32_t* seqlens, const int32_t* cu_seqlens,
                         const int32_t* block_table, double* out, double* lse, int nthreads);

/*
 * Attention of one query over an explicit list of rows (element offsets into
 * k and v).  Returns the unnormalised sum o = sum_t exp(s_t - m) v_t, the max m
 * and the sum l = sum_t exp(s_t - m).  Used by the split/merge pins.
 */
void orc_attend_rows(int D, double scale, int kind, const uint16_t* q,
                     const uint16_t* k, const uint16_t* v, const int64_t* rows, int n,
                     double* o_unnorm, double* m, double* l);

/*
 * CLO cache buffer + persistent cache attention (CLO page, section 7: the hybrid
 * kernel reads both buffers in place).  For KV head g:
 *   head_map[g] >= 0 : rows pers[b, head_map[g], 0:pers_len[b]]
 *   head_map[g] <  0 : rows buf [b, g,           0:buf_len[b*Hkv+g]]
 * pers_k/v [B, P_slots, pers_cap, D]; buf_k/v [B, Hkv, buf_cap, D].
 */
int orc_hybrid_attn(int B, int Hq, int Hkv, int D, double scale, int kind,
                    int P_slots, int pers_cap, int buf_cap,
                    const uint16_t* q, const uint16_t* pers_k, const uint16_t* pers_v,
                    const int32_t* pers_len, const uint16_t* buf_k, const uint16_t* buf_v,
                    const int32_t* buf_len, const int32_t* head_map,
                    double* out, double* lse, int nthreads);

/* The hybrid attention with e4m3 K and V (element = code * k_scale / v_scale). */
int orc_hybrid_attn_e4m3(int B, int Hq, int Hkv, int D, double scale, int kind,
                         int P_slots, int pers_cap, int buf_cap, const uint16_t* q,
                         const uint8_t* pers_k, const uint8_t* pers_v, const int32_t* pers_len,
                         const uint8_t* buf_k, const uint8_t* buf_v, const int32_t* buf_len,
                         const int32_t* head_map, double k_scale, double v_scale, double* out,
                         double* lse, int nthreads);

/*
 * Index-gather sparse attention (CLO page: top-k sparse attention over a
 * fraction of the tokens, HATA's hashes replaced by exact scores; Eq. 6).
 * K, V: the dense cache [B, S, Hkv, D]; seqlens[B] (NULL => S).
 * orc_topk_scores: s[b, g, t] = sum over the group's query heads of q_j . K_t
 *   (t < len_b; 0 beyond), and mags = sum |q_jd K_td| (may be NULL).
 * orc_topk_select: per (b, g) the min(kk, len_b) tokens of largest s (ties:
 *   smaller t), ascending, into idx[b, g, 0:kk]; counts into idx_len[b*Hkv+g].
 * orc_gather_attn: attention of each query head over the rows idx[b, g,
 *   0:idx_len[b*Hkv+g]] (row stride max_k) of its KV head.
 */
int orc_topk_scores(int B, int Hq, int Hkv, int D, int kind, int S, const uint16_t* q,
                    const uint16_t* k, const int32_t* seqlens, double* scores, double* mags,
                    int nthreads);
int orc_topk_select(int B, int Hq, int Hkv, int D, int kind, int S, const uint16_t* q,
                    const uint16_t* k, const int32_t* seqlens, int kk, int32_t* idx,
                    int32_t* idx_len, int nthreads);
int orc_gather_attn(int B, int Hq, int Hkv, int D, double scale, int kind, int S,
                    const uint16_t* q, const uint16_t* k, const uint16_t* v, const int32_t* idx,
                    const int32_t* idx_len, int max_k, double* out, double* lse, int nthreads);

/*
 * Eqs. 7-9 of the CLO page (threshold chain), in fp64:
 *   theta* = arccos(eta); lambda_i = s_i^n; theta_i = lambda_i theta* + (1-lambda_i) pi;
 *   tau_i = cos(theta_i).
 */
void orc_thresholds(int n, const double* s, double eta, double n_exp, double* tau);

/*
 * Head-wise approximate cache lookup and label update (CLO page, sections 2-4:
 * cosine hit test against the stored query label, Eq. 10 importance-weighted
 * GQA aggregation, whole-head replacement on a miss).
 * q, labels [B, Hq, D] (kind 0/1); labels is updated in place.
 * w [Hq] importance weights; tau [Hkv] thresholds (the fp32 values the GPU uses).
 * Outputs: hit [B*Hkv]; agg [B*Hkv]; cosv [B*Hq]; miss_list [B*Hkv] ascending
 * b*Hkv+g; *miss_count.  Any output pointer except hit may be NULL.
 * A group with a zero-norm query or label misses.  Zero total weight uses the
 * unweighted mean.
 */
int orc_headcache_lookup(int B, int Hq, int Hkv, int D, int kind, const uint16_t* q,
                         uint16_t* labels, const float* w, const float* tau,
                         uint8_t* hit, double* agg, double* cosv,
                         int32_t* miss_list, int32_t* miss_count);

/*
 * KVPR partial recompute (KVPR page, section A2: K[0:l] = X[0:l] W_K and
 * V[0:l] = X[0:l] W_V, W in R^{h x h} applied as X.W).
 * x: bf16/fp16 [b, *, h] with x_bstride elements between batches (row t at
 * b*x_bstride + t*h).  wk, wv: [h, h] row-major (input index first).
 * Computes the rows listed in rows[] (flat index r = bi*l + t) into
 * k_out, v_out [nrows, h] fp64.  rows == NULL computes every row (nrows = b*l).
 */
int orc_kv_recompute(int b, int l, int h, int kind, const uint16_t* x, int64_t x_bstride,
                     const uint16_t* wk, const uint16_t* wv, const int32_t* rows, int nrows,
                     double* k_out, double* v_out, int nthreads);

/*
 * KVPR cost model (KVPR page, section A2): bytes of X[0:l], bytes of KV[l:s'],
 * and the recompute FLOP count 4 b l h^2.
 */
void orc_kvpr_cost(double b, double l, double s_prime, double h, double p,
                   double* m_x, double* m_kv, double* n_flops);

/* KVPR page, section A2: t(l) = M_X / v_com + max(N / v_gpu, M_KV / v_com). */
double orc_kvpr_time(double b, double l, double s_prime, double h, double p, double v_com,
                     double v_gpu);

/* Split point of least t(l) by trying every l in [0, l_max] (smallest l on
 * ties); *t_best (may be NULL) gets its time. */
int orc_kvpr_best_split(double b, int s_prime, int l_max, double h, double p, double v_com,
                        double v_gpu, double* t_best);

/* Threads the OpenMP runtime would use for nthreads <= 0. */
int orc_max_threads(void);

#ifdef __cplusplus
}
#endif
#endif

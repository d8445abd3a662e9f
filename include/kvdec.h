/*
 * kvdec.h -- libkvdec, long-KV-cache decode kernels for AMD MI355X (gfx950).
 *
 * C ABI.  Plain pointers and sizes only.  Every pointer is a DEVICE pointer
 * unless its comment says (host).  Every compute call is asynchronous on the
 * given HIP stream and returns after enqueueing.
 *
 * Ownership: the caller owns and allocates every buffer, including the
 * workspaces whose sizes the *_workspace queries return.  Compute calls never
 * allocate, free, synchronise or create streams.  Buffers documented as
 * in/out (labels, k_cache, v_cache) are updated in place.
 *
 * Errors: arguments are validated on the host before anything is enqueued.  On
 * a bad argument nothing is launched, the call returns a non-zero status and
 * kvdec_last_error() describes it (thread-local).  A failed launch returns
 * KVDEC_ERR_HIP.  Faults inside a kernel surface at the caller's next
 * synchronisation.  No call throws.
 *
 * Thread safety: calls may be made from several threads.  Two calls that share
 * a workspace must not run concurrently (they use it as scratch).
 *
 * Element types: KVDEC_F16 = IEEE binary16, KVDEC_BF16 = bfloat16.  All
 * accumulation is fp32; 16-bit outputs are rounded to nearest even once.
 */
#ifndef KVDEC_H
#define KVDEC_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define KVDEC_ABI_VERSION 11

typedef enum {
  KVDEC_OK = 0,
  KVDEC_ERR_INVALID = 1,     /* a null pointer, a negative size, inconsistent shapes */
  KVDEC_ERR_UNSUPPORTED = 2, /* valid but not implemented (e.g. head_dim != 128) */
  KVDEC_ERR_WORKSPACE = 3,   /* workspace missing or smaller than the query said */
  KVDEC_ERR_HIP = 4          /* a HIP runtime call failed */
} kvdec_status;

typedef enum { KVDEC_F16 = 0, KVDEC_BF16 = 1 } kvdec_dtype;
typedef enum { KVDEC_DENSE = 0, KVDEC_RAGGED = 1, KVDEC_PAGED = 2 } kvdec_layout;
/* Storage of K and V: the query's dtype, or e4m3 codes (OCP 8-bit float,
 * "fn" variant: bias 7, no infinities, largest magnitude 448), one byte per
 * element in the same layouts, each tensor with one scale (element = code
 * value * scale).  The CLO page raises FP8 KV caches as its natural next step:
 * they halve the bytes each token and head moves. */
typedef enum { KVDEC_KV_SAME = 0, KVDEC_KV_E4M3 = 1 } kvdec_kv_format;

/*
 * Decode attention descriptor.
 *
 * The operation (KVPR page, section A3, MHA equation, at the decode step where
 * each sequence contributes one query token; Neo page, method details, for the
 * paged pool and the split-then-aggregate parallelisation of one request):
 *
 *   for every sequence b and query head j, with KV head g = j / (Hq / Hkv):
 *     s_t   = softmax_scale * q[b, j, :] . K_g[b, t, :]      t < len_b
 *     out[b, j, :] = sum_t softmax(s)_t * V_g[b, t, :]
 *     lse[b, j]    = ln sum_t exp(s_t)          (natural log; -inf if len_b = 0)
 *
 * An empty sequence (len_b = 0) gives out = 0 and lse = -inf.
 *
 * Fields:
 *   batch          B >= 0
 *   num_q_heads    Hq >= 1; num_kv_heads Hkv >= 1; Hq % Hkv == 0; Hq / Hkv <= 8
 *   head_dim       must be 128
 *   softmax_scale  any finite value (1/sqrt(head_dim) in the usual case)
 *   dtype          kvdec_dtype of q, K, V and out
 *   layout         kvdec_layout (below)
 *   max_seqlen     DENSE: the allocated token count S of each sequence (the
 *                  row stride); RAGGED / PAGED: an upper bound on every len_b.
 *                  It sizes the grid and the workspace; lengths above it are
 *                  an error the kernel cannot report (they are clamped).
 *   page_size      PAGED only: tokens per page, a multiple of 16
 *   max_pages_per_seq PAGED only: row stride of block_table
 *   split_tokens   0 = balanced schedule: every tile of every sequence is
 *                  spread evenly over a persistent grid sized to the device,
 *                  so the length mix does not leave compute units idle;
 *                  otherwise each work item covers split_tokens tokens (a
 *                  multiple of 64) of one sequence, and a sequence's result
 *                  does not depend on the other sequences of the batch.
 *   kv_rows        RAGGED: the token rows T in k and v; PAGED: the pages P in
 *                  the pool; DENSE: ignored.  The kernel clamps cu_seqlens into
 *                  [0, T] and page ids into [0, P), so malformed metadata reads
 *                  wrong rows instead of faulting.
 *   kv_format      kvdec_kv_format of K and V (0: the dtype above)
 *   k_scale, v_scale  KVDEC_KV_E4M3 only: finite and > 0; K = k_scale * code,
 *                  V = v_scale * code.  k_scale enters the scores
 *                  (softmax_scale * k_scale * q . code), v_scale the output
 *                  (applied with the final normalisation).  Codes that are NaN
 *                  give NaN outputs.
 */
typedef struct {
  int32_t batch, num_q_heads, num_kv_heads, head_dim;
  float softmax_scale;
  int32_t dtype;
  int32_t layout;
  int32_t max_seqlen;
  int32_t page_size, max_pages_per_seq;
  int32_t split_tokens;
  int64_t kv_rows;
  int32_t kv_format;
  float k_scale, v_scale;
} kvdec_attn_desc;

/* Workspace bytes kvdec_decode_attn needs for this descriptor on the current
 * device (0 only with split_tokens > 0 when every sequence fits one work
 * item).  The workspace holds the per-call partial results; its contents need
 * no initialisation and are dead after the call's kernels finish.  It must be
 * 16-byte aligned (KVDEC_ERR_WORKSPACE otherwise).  The size
 * depends on the device's compute-unit count: query it on the device that
 * will run the call. */
kvdec_status kvdec_decode_attn_workspace(const kvdec_attn_desc* desc, size_t* bytes /*(host)*/);

/*
 * Decode attention.
 *   q   [B, Hq, 128]; out [B, Hq, 128] (dtype); lse [B, Hq] fp32 (may be NULL);
 *   k and v may be NULL when there are no rows to read (RAGGED with
 *   kv_rows = 0, DENSE with max_seqlen = 0): every sequence is then empty
 *   DENSE : k, v [B, max_seqlen, Hkv, 128]; seqlens [B] int32 (NULL => all max_seqlen)
 *   RAGGED: k, v [T, Hkv, 128] packed by sequence; cu_seqlens [B+1] int32,
 *           cu_seqlens[0] = 0, nondecreasing; seqlens ignored
 *   PAGED : k, v [P, Hkv, page_size, 128]; block_table [B, max_pages_per_seq]
 *           int32 page ids in [0, P); seqlens [B] int32 (required).  Token t of
 *           sequence b is slot t % page_size of page block_table[b][t / page_size].
 *           Slots past a sequence's end and table entries past its last page
 *           are never read.
 *   workspace / ws_bytes: see kvdec_decode_attn_workspace.
 */
kvdec_status kvdec_decode_attn(const kvdec_attn_desc* desc, const void* q, const void* k,
                               const void* v, const int32_t* seqlens, const int32_t* cu_seqlens,
                               const int32_t* block_table, void* out, float* lse,
                               void* workspace, size_t ws_bytes, hipStream_t stream);

/*
 * kvdec_decode_attn without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc).  The same operation, kernels and results
 * (bit for bit) as kvdec_decode_attn; the partials live in a library-owned
 * device array of KVDEC_NOALLOC_SCRATCH_BYTES per GPU, set up on the call's
 * first use on a device and held until the process ends.  The call allocates
 * nothing.  A descriptor whose workspace (kvdec_decode_attn_workspace) exceeds
 * that size returns KVDEC_ERR_WORKSPACE with nothing launched.  Every call on
 * one GPU shares its array: calls that may overlap on one GPU (two streams,
 * two threads) race on it and give wrong results; serialise them, or use
 * kvdec_decode_attn with a workspace each.
 */
#define KVDEC_NOALLOC_SCRATCH_BYTES (32u << 20)
kvdec_status kvdec_decode_attn_noalloc(const kvdec_attn_desc* desc, const void* q, const void* k,
                                       const void* v, const int32_t* seqlens,
                                       const int32_t* cu_seqlens, const int32_t* block_table,
                                       void* out, float* lse, hipStream_t stream);

/*
 * CLO cache buffer + persistent cache attention (CLO page, section 7: the
 * hybrid attention kernel reads both buffers in place, with no gather into one
 * buffer; section 2: hard-to-reuse heads keep their full KV resident).
 *
 * base: batch, heads, head_dim, softmax_scale, dtype, split_tokens, kv_format
 * and the scales as for kvdec_attn_desc (layout, max_seqlen, page fields are
 * ignored); with KVDEC_KV_E4M3 both the persistent and the buffer K/V are
 * codes under the same two scales.
 *   pers_k, pers_v [B, num_pers_slots, pers_cap, 128]; pers_len [B] int32
 *   buf_k,  buf_v  [B, Hkv, buf_cap, 128];             buf_len [B * Hkv] int32
 *   head_map [Hkv] int32: slot >= 0 reads persistent slot `slot` (rows
 *   0..pers_len[b]-1), -1 reads the cache buffer of that KV head (rows
 *   0..buf_len[b*Hkv+g]-1, the selected tokens compacted in any order).
 *   The metadata lives on the device, so the host cannot check it before the
 *   launch.  The kernels clamp instead of faulting: a slot >= num_pers_slots
 *   makes that head empty (out = 0, lse = -inf), and lengths are clamped into
 *   [0, pers_cap] and [0, buf_cap].  With KVDEC_CHECK=1 in the environment the
 *   call copies the metadata to the host first and rejects such values with
 *   KVDEC_ERR_INVALID, launching nothing (see kvdec_check_enabled).
 * The result for each KV head equals kvdec_decode_attn over the rows it reads.
 */
typedef struct {
  kvdec_attn_desc base;
  int32_t num_pers_slots, pers_cap, buf_cap;
} kvdec_hybrid_desc;

kvdec_status kvdec_sparse_hybrid_attn_workspace(const kvdec_hybrid_desc* desc,
                                                size_t* bytes /*(host)*/);
kvdec_status kvdec_sparse_hybrid_attn(const kvdec_hybrid_desc* desc, const void* q,
                                      const void* pers_k, const void* pers_v,
                                      const int32_t* pers_len, const void* buf_k,
                                      const void* buf_v, const int32_t* buf_len,
                                      const int32_t* head_map, void* out, float* lse,
                                      void* workspace, size_t ws_bytes, hipStream_t stream);

/*
 * Index-gather sparse attention (CLO page: decoding attends to a top-k
 * selection of each head's tokens, 10% of them; the selection's indices point
 * into the full cache, read in place with no compacted copy).
 *
 * base: batch, heads, head_dim, softmax_scale, dtype, split_tokens, kv_format
 * and scales as for kvdec_attn_desc; max_seqlen is the cache's rows per
 * sequence S (layout, page fields and kv_rows are ignored).
 *   k, v     the dense cache [B, S, Hkv, 128] (dtype, or e4m3 codes)
 *   idx      [B, Hkv, max_k] int32 token rows of each (sequence, KV head);
 *            entries past idx_len are never read; rows are clamped into
 *            [0, S), so malformed indices read wrong rows instead of faulting
 *   idx_len  [B * Hkv] int32 in [0, max_k]
 * For each query head j of KV head g:
 *   out[b, j] = softmax_t(softmax_scale * q[b, j] . K[b, idx_t, g]) V[b, idx_t, g]
 * over t < idx_len[b * Hkv + g] (out = 0, lse = -inf when empty).  The order
 * of the indices does not matter.  Requires S * Hkv * 128 * (bytes per
 * element) <= 2^31.
 */
typedef struct {
  kvdec_attn_desc base;
  int32_t max_k;
} kvdec_gather_desc;

kvdec_status kvdec_gather_attn_workspace(const kvdec_gather_desc* desc, size_t* bytes /*(host)*/);
kvdec_status kvdec_gather_attn(const kvdec_gather_desc* desc, const void* q, const void* k,
                               const void* v, const int32_t* idx, const int32_t* idx_len,
                               void* out, float* lse, void* workspace, size_t ws_bytes,
                               hipStream_t stream);

/*
 * Exact top-k token selection for kvdec_gather_attn (CLO page: top-k sparse
 * attention with HATA's hashed retrieval; the exact scores stand in for the
 * hashes.  Eq. 6: q.k = |q| |k| cos(q, k), so the selection does not depend
 * on |q|).  For each sequence b and KV head g, tokens t < len_b are ranked by
 *   s_t = sum over g's query heads j of q[b, j] . K[b, t, g]   (fp32)
 * and the min(top_k, len_b) largest are written to idx[b, g, :] in ascending
 * token order (ties go to the smaller t), their count to idx_len[b*Hkv+g].
 *   q [B, Hq, 128], k [B, S, Hkv, 128] (dtype); seqlens [B] int32 or NULL (all S)
 *   idx [B, Hkv, top_k] int32 (entries past idx_len are not written)
 * Requires S <= 262144, top_k >= 0, 16-bit K.  The workspace (16-byte
 * aligned, size from kvdec_topk_select_workspace, no initialisation needed)
 * holds the scores, B * Hkv rows of S rounded up to 4 floats, and then the
 * selection's per-pair histograms and counters.
 */
typedef struct {
  int32_t batch, num_q_heads, num_kv_heads, head_dim;
  int32_t dtype;
  int32_t max_seqlen;
  int32_t top_k;
} kvdec_topk_desc;

kvdec_status kvdec_topk_select_workspace(const kvdec_topk_desc* desc, size_t* bytes /*(host)*/);
kvdec_status kvdec_topk_select(const kvdec_topk_desc* desc, const void* q, const void* k,
                               const int32_t* seqlens, int32_t* idx, int32_t* idx_len,
                               void* workspace, size_t ws_bytes, hipStream_t stream);

/*
 * CLO head-wise approximate cache lookup fused with the query-label update
 * (CLO page, section 2: one query label per head, hit iff the cosine to the
 * label reaches tau, else the whole head is replaced; Eq. 10: a KV head's
 * cosine is the importance-weighted mean over its query heads; section 7: the
 * lookup and the label update share one read of q and the labels).
 *
 * For each sequence b and KV head g (query heads j = g*G .. g*G+G-1):
 *   c[b,j]   = q[b,j].label[b,j] / (|q[b,j]| |label[b,j]|)           (fp32)
 *   agg[b,g] = sum_j w[j] c[b,j] / sum_j w[j]    (unweighted mean if sum w = 0)
 *   hit[b,g] = agg[b,g] >= tau[g]; a group holding a zero-norm q or label misses
 *   on a miss: label[b,j] <- q[b,j] (bit copy) for every j of the group
 *   miss_list: the b*Hkv+g of every miss in ascending order; miss_count: their number
 *
 *   q, labels [B, Hq, D] (dtype; labels in/out); weights [Hq] fp32; tau [Hkv] fp32
 *   hit [B*Hkv] uint8; agg [B*Hkv] fp32, cos [B*Hq] fp32, miss_list [B*Hkv]
 *   int32, miss_count [1] int32 -- all four may be NULL (miss_list and
 *   miss_count together).  D must be 128.  Hq % Hkv == 0, Hq / Hkv <= 16.
 */
kvdec_status kvdec_headcache_lookup(int32_t B, int32_t Hq, int32_t Hkv, int32_t D, int32_t dtype,
                                    const void* q, void* labels, const float* weights,
                                    const float* tau, uint8_t* hit, float* agg, float* cos,
                                    int32_t* miss_list, int32_t* miss_count, hipStream_t stream);

/*
 * Head-cache lookup one layer ahead (CLO page, section 3, decoding flow,
 * Figure 9: at the start of layer l-1 the query of layer l is approximated by
 * q_approx = x_{l-1} W_Q^l and the lookup runs on it, so the heads it misses
 * can be fetched while layer l-1 still computes).  Computes
 *   q_approx[b][n] = sum_i x_prev[b][i] * w_q[n][i]   (fp32 sums, one rounding)
 * and then runs kvdec_headcache_lookup on q_approx (labels of missed groups
 * get q_approx).  The miss list is the prefetch queue.
 *   x_prev   [B, h] (dtype), the previous layer's hidden states
 *   w_q      [Hq * D, h] (dtype), output index first as torch.nn.Linear stores
 *            it (the query projection of the next layer)
 *   q_approx [B, Hq, D] (dtype), written
 *   the other arguments as kvdec_headcache_lookup.
 * Requires h a multiple of 8 in [8, 8192] and x_prev, w_q 16-byte aligned,
 * plus the kvdec_headcache_lookup rules.  W_Q is read once per group of four
 * batch rows; the two launches (projection, then lookup) go on `stream`.
 */
kvdec_status kvdec_headcache_lookup_ahead(int32_t B, int32_t Hq, int32_t Hkv, int32_t D,
                                          int32_t h, int32_t dtype, const void* x_prev,
                                          const void* w_q, void* q_approx, void* labels,
                                          const float* weights, const float* tau, uint8_t* hit,
                                          float* agg, float* cos, int32_t* miss_list,
                                          int32_t* miss_count, hipStream_t stream);

/*
 * Miss-driven prefetch into the cache buffer (CLO page, section 3, decoding
 * flow, Figure 9: the heads the lookup misses are fetched while the previous
 * layer computes; Figure 7: an update writes the new KV rows straight to
 * their final place in the cache buffer, with no staging copy).  The GPU
 * reads the selected rows from the offloaded KV pool in pinned host memory
 * itself, over PCIe: there is no host-side gather.
 *
 * For each of the first *miss_count entries p = b * Hkv + g of miss_list (as
 * kvdec_headcache_lookup writes them), skipping entries outside [0, B*Hkv)
 * and KV heads with head_map[g] >= 0 (persistent heads, always resident):
 *   n = clamp(idx_len[p], 0, min(max_k, buf_cap))
 *   buf[b, g, i, :] = pool[b, clamp(idx[p * max_k + i], 0, S-1), g, :]  for i < n
 *   buf_len[p] = n
 * for K and V alike.  Rows i >= n of the buffer, and pairs not in the list,
 * are left untouched.  The result does not depend on the order of the list.
 *
 *   desc           sizes (below)
 *   miss_list, miss_count  [B * Hkv], [1] int32 (device)
 *   head_map       [Hkv] int32 or NULL (every head is a buffer head)
 *   idx, idx_len   [B * Hkv, max_k], [B * Hkv] int32: the selected token rows
 *                  of each pair (any order; kvdec_topk_select writes them)
 *   pool_k, pool_v (host) the full KV in pinned host memory (hipHostMalloc or
 *                  a pinned torch tensor; pageable memory is refused, since
 *                  the GPU cannot read it), 16-byte aligned: token t of
 *                  sequence b, head g starts at element
 *                  b * pool_stride_b + t * pool_stride_s + g * pool_stride_h
 *                  ([B, S, Hkv, 128]: S*Hkv*128, Hkv*128, 128)
 *   buf_k, buf_v   [B, Hkv, buf_cap, 128] (device), 16-byte aligned
 *   buf_len        [B * Hkv] int32 (device), written for the listed pairs
 *   ready_flag     NULL, or a 32-bit sequence number in host-mapped memory
 *                  (kvdec_host_flag_alloc) that the host raises once the pool
 *                  rows are in place.  The copy then waits on the GPU until
 *                  (int32)(*ready_flag - ready_value) >= 0, for at most
 *                  timeout_us microseconds (<= 1000000): the host enqueues the
 *                  whole step without blocking on the transfer (CLO page,
 *                  section 2: GPU-centric synchronisation through an
 *                  identifier variable in shared memory).
 *   status         with ready_flag: [1] int32 (device or host-mapped), set to
 *                  0 when the flag was reached, 1 when the wait gave up; after
 *                  a give-up nothing is copied and buf_len is unchanged.
 *                  Ignored without ready_flag.
 * elem_bytes is 2 for fp16 / bf16 K/V and 1 for e4m3 codes.  All the checks
 * (including that the whole pool range lies in one pinned allocation) run
 * before anything is enqueued.
 */
typedef struct {
  int32_t batch, num_kv_heads, head_dim;  /* head_dim == 128 */
  int32_t elem_bytes;                     /* 2 or 1 */
  int32_t max_seqlen;                     /* S: token rows per (b, g) in the pool, >= 1 */
  int64_t pool_stride_b, pool_stride_s, pool_stride_h;  /* elements, >= 0, 16-byte multiples */
  int32_t max_k;                          /* row stride of idx */
  int32_t buf_cap;                        /* rows per (b, g) in the cache buffer */
} kvdec_prefetch_desc;

kvdec_status kvdec_headcache_prefetch(const kvdec_prefetch_desc* desc, const int32_t* miss_list,
                                      const int32_t* miss_count, const int32_t* head_map,
                                      const int32_t* idx, const int32_t* idx_len,
                                      const void* pool_k, const void* pool_v, void* buf_k,
                                      void* buf_v, int32_t* buf_len, const uint32_t* ready_flag,
                                      uint32_t ready_value, uint32_t timeout_us, int32_t* status,
                                      hipStream_t stream);

/*
 * GPU-centric synchronisation (CLO page, section 2, and its argument chain,
 * row 8: the GPU polls an identifier variable in host-shared memory instead
 * of the host blocking on the stream, so kernel launches and data transfer
 * run on separate host threads).
 *
 * kvdec_host_flag_alloc: a 32-bit flag (initially 0) in fine-grained pinned
 * host memory that the GPU reads and writes coherently while kernels run;
 * free it with kvdec_host_flag_free.  These two allocate and free; they are
 * set-up calls, never made inside a step.
 *
 * kvdec_flag_wait: enqueues a one-wave kernel that waits until
 * (int32)(*flag - value) >= 0 or timeout_us microseconds (<= 1000000) have
 * passed, then writes *status = 0 (reached) or 1 (gave up).  Work queued
 * after it on `stream` starts only then, and sees host writes made before
 * the flag was raised.  The wait always ends: the GPU never spins unbounded.
 * flag and status: host-mapped or device memory HIP knows, 4-byte aligned.
 *
 * kvdec_flag_signal: enqueues a kernel that sets *flag = value after the work
 * queued before it on `stream` has finished (a system-scope release), so a
 * host thread can poll the flag instead of synchronising the stream.
 */
kvdec_status kvdec_host_flag_alloc(uint32_t** flag /*(host) out*/);
kvdec_status kvdec_host_flag_free(uint32_t* flag);
kvdec_status kvdec_flag_wait(const uint32_t* flag, uint32_t value, uint32_t timeout_us,
                             int32_t* status, hipStream_t stream);
kvdec_status kvdec_flag_signal(uint32_t* flag, uint32_t value, hipStream_t stream);

/*
 * CLO threshold chain, Eqs. 7-9 (host only, fp64, rounded to fp32 once):
 *   theta* = arccos(eta); lambda_i = s_i^n_exp;
 *   tau_i = cos(lambda_i theta* + (1 - lambda_i) pi).
 * s: n importance scores in [0, 1] (host); tau: n outputs (host).
 * eta in [-1, 1]; n_exp > 0.
 */
kvdec_status kvdec_headcache_thresholds(int32_t n, const float* s /*(host)*/, double eta,
                                        double n_exp, float* tau /*(host)*/);

/*
 * KVPR partial recompute (KVPR page, section A2: K[0:l] = X[0:l] W_K,
 * V[0:l] = X[0:l] W_V with W in R^{h x h}; the recomputed rows join the rows
 * already resident before attention runs over [0, s')).
 *
 *   x        [b, *, h] bf16, row t of batch i at x + i*x_batch_stride + t*h (elements)
 *   w_k, w_v [h, h] bf16 row-major; w_layout KVDEC_W_IN_OUT: input index
 *            first, W[i][n] (the product is x . W); KVDEC_W_OUT_IN: output
 *            index first, W[n][i], as a torch.nn.Linear weight stores it (the
 *            same product with W read transposed; the faster layout here, as
 *            its rows are contiguous along the contraction)
 *   k_cache, v_cache [b, s_cap, H, head_dim] fp16 with h = H * head_dim; batch i
 *            starts cache_batch_stride elements after batch i-1.  Rows [0, l)
 *            are overwritten with fp16(x . W) (fp32 accumulation, one rounding);
 *            every other byte is left untouched.
 *   Requires l >= 0, b >= 0, head_dim == 128, h % 256 == 0 (covers the 40-head
 *   OPT-13B width 5120), x_batch_stride >= l*h, cache_batch_stride >= l*h.
 */
typedef enum { KVDEC_W_IN_OUT = 0, KVDEC_W_OUT_IN = 1 } kvdec_w_layout;

kvdec_status kvdec_kv_recompute(int32_t b, int32_t l, int32_t h, int32_t num_heads,
                                int32_t head_dim, const void* x, int64_t x_batch_stride,
                                const void* w_k, const void* w_v, int32_t w_layout,
                                void* k_cache, void* v_cache, int64_t cache_batch_stride,
                                hipStream_t stream);

/*
 * KVPR split point (KVPR page, section A2, the scheduler's choice of l): the
 * integer l in [0, l_max] that minimises the layer time
 *   t(l) = M_X(l) / v_com + max(N(l) / v_gpu, M_KV(l) / v_com),
 *   M_X = b l h p,  M_KV = 2 b (s' - l) h p,  N = 4 b l h^2,
 * with p = elem_bytes, v_com the host-to-device rate in bytes/s and v_gpu the
 * recompute rate in FLOP/s.  t falls while the transfer of the rows left
 * dominates and rises after, so the minimum is at one of the two integers
 * around the crossing (clamped to [0, l_max]); ties go to the smaller l.
 * Host only; *t_out (may be NULL) gets t(l) in seconds.
 * Requires b >= 0, 0 <= l_max <= s_prime, h >= 1, elem_bytes >= 1 and
 * finite v_com, v_gpu > 0.
 */
kvdec_status kvdec_kvpr_split(int64_t b, int64_t s_prime, int64_t l_max, int64_t h,
                              int32_t elem_bytes, double v_com, double v_gpu, int32_t* l_out,
                              double* t_out);

/*
 * One KVPR layer load (KVPR page, section A2, runtime module: the activations
 * of the first l tokens cross PCIe first and the GPU recomputes their K/V
 * while the K/V rows [l, s') are still in transfer).  Enqueues
 *   on copy_stream:    host-to-device copies of X[0:l] into x_dev, then of
 *                      the K and V rows [l, s') into k_cache, v_cache;
 *   on compute_stream: once X has arrived, the recompute of rows [0, l)
 *                      (as kvdec_kv_recompute), then a wait for the K/V
 *                      copies, so work queued on compute_stream after this
 *                      call sees cache rows [0, s') complete.
 *   x_host   [b, *, h] bf16, pinned host memory, batch stride x_host_bstride
 *            elements (>= l*h)
 *   x_dev    [b, l, h] bf16 device staging buffer (written)
 *   k_host, v_host  [b, *, H, head_dim] fp16 pinned host memory, batch stride
 *            kv_host_bstride elements (>= s_prime*h); rows [l, s_prime) are read
 *   w_k, w_v, w_layout, k_cache, v_cache, cache_bstride (>= s_prime*h): as in
 *            kvdec_kv_recompute
 * compute_stream and copy_stream must differ.  The call orders only its own
 * work: x_dev and the cache rows it writes must not be in use by work already
 * queued on either stream.  Without page-locked host memory the copies are
 * not asynchronous.  Requires 0 <= l <= s_prime and the kvdec_kv_recompute
 * shape rules; l == 0 copies everything, l == s_prime recomputes everything.
 */
kvdec_status kvdec_kvpr_load_layer(int32_t b, int32_t l, int32_t s_prime, int32_t h,
                                   int32_t num_heads, int32_t head_dim, const void* x_host,
                                   int64_t x_host_bstride, void* x_dev, const void* k_host,
                                   const void* v_host, int64_t kv_host_bstride, const void* w_k,
                                   const void* w_v, int32_t w_layout, void* k_cache, void* v_cache,
                                   int64_t cache_bstride, hipStream_t compute_stream,
                                   hipStream_t copy_stream);

/* Kernel timing, a profiling aid.  While enabled on the calling thread, every
 * call above launches its main kernel with a pair of HIP events that the
 * runtime stamps from that kernel's own dispatch (hipExtLaunchKernel): its
 * start and its end, with no extra packets on the stream.  Main kernels: the
 * split kernel of an attention call (not the merge kernel), the lookup kernel
 * of kvdec_headcache_lookup (not the compaction kernel), the projection of
 * kvdec_headcache_lookup_ahead, each of the six kernels of
 * kvdec_topk_select (the score pass, three radix-digit passes, the threshold
 * and the compaction), the GEMM of kvdec_kv_recompute and of
 * kvdec_kvpr_load_layer.
 * kvdec_kernel_timing(1) starts a new measurement (the library keeps and
 * reuses its events); kvdec_kernel_timing(0) stops recording.
 * kvdec_kernel_timing_read waits for the recorded events and returns the
 * summed kernel time in milliseconds and the number of launches timed since
 * the last kvdec_kernel_timing(1).  An event that could not be created or
 * recorded stops further recording and is reported here as KVDEC_ERR_HIP. */
kvdec_status kvdec_kernel_timing(int enable);
kvdec_status kvdec_kernel_timing_read(double* total_ms, int64_t* launches);

/* Streaming-read reference, a measurement aid (no part of the method).
 * Reads `bytes` bytes at device pointer `src` once, with 16-byte loads, and
 * may write one uint32 at device pointer `sink` (a value that depends on all
 * the words read; the write happens only for one value of it).  Its rate on a
 * buffer larger than the caches (L2, 256 MB MALL) is the HBM read bandwidth
 * one kernel reaches on this GPU, the second denominator reported beside the
 * published peak.  bytes > 0 and a multiple of 16; src 16-byte aligned; both
 * pointers non-NULL.  Asynchronous on `stream`; it is a main kernel for
 * kvdec_kernel_timing.  KVDEC_ERR_INVALID on bad arguments (nothing launched). */
kvdec_status kvdec_stream_read(const void* src, size_t bytes, uint32_t* sink, hipStream_t stream);

/* Debug validation of metadata that lives on the device.  The kernels never
 * fault on malformed metadata: they clamp it (see the kv_rows, head_map, idx
 * and miss_list notes above), which reads wrong rows or drops work without a
 * status.  With KVDEC_CHECK=1 in the environment (read at every call), each
 * call first copies its metadata to the host, after the work already queued
 * on its stream, synchronising that stream, and returns KVDEC_ERR_INVALID,
 * with nothing launched and a message naming the entry, for:
 *   kvdec_decode_attn (and _noalloc): cu_seqlens[0] != 0, cu_seqlens
 *     decreasing, a length above max_seqlen, cu_seqlens[B] > kv_rows,
 *     seqlens outside [0, max_seqlen], a used block-table entry outside
 *     [0, kv_rows);
 *   kvdec_sparse_hybrid_attn: a head_map entry that is neither -1 nor a slot
 *     in [0, num_pers_slots), pers_len outside [0, pers_cap], a buffer head's
 *     buf_len outside [0, buf_cap];
 *   kvdec_gather_attn: idx_len outside [0, max_k], a listed row outside [0, S);
 *   kvdec_topk_select: seqlens outside [0, max_seqlen];
 *   kvdec_headcache_prefetch: miss_count outside [0, B*Hkv], a listed pair
 *     outside [0, B*Hkv), and for listed buffer heads idx_len outside
 *     [0, min(max_k, buf_cap)] or a listed row outside [0, S).
 * Returns 1 when the mode is on for the next call, else 0.  For debugging
 * only: the copies and the synchronisation cost far more than the kernels. */
int kvdec_check_enabled(void);

const char* kvdec_status_string(kvdec_status status);
const char* kvdec_last_error(void);
int kvdec_abi_version(void);

#ifdef __cplusplus
}
#endif
#endif /* KVDEC_H */

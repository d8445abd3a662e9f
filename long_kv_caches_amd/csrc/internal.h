// internal.h -- declarations shared by the libkvdec host layer and its kernels.
#pragma once

#include <stdint.h>

#include <hip/hip_runtime.h>
#include <hip/hip_ext.h>

#include "kvdec.h"

namespace kvdec {

// Records a thread-local message for kvdec_last_error() and returns `st`.
kvdec_status fail(kvdec_status st, const char* fmt, ...);

constexpr int kHeadDim = 128;     // the one supported head_dim
constexpr int kTile = 16;         // tokens per wave tile (one MFMA row block)
constexpr int kWaves = 4;         // waves per attention workgroup
constexpr int kMaxGroup = 8;      // query heads per KV head handled by one workgroup
constexpr int kMaxUnits = 4096;   // tile-line units (sequences, or hybrid pairs) of the balanced schedule
constexpr int kMinTilesPerWave = 8;
constexpr int kFirstRoundWeight = 113;  // balanced: per 100, share of a first-round column

// Tile schedules of the attention kernels.
enum Mode : int { MODE_CHUNKS = 0, MODE_BALANCED = 1 };

// Where the K/V rows of one (sequence, KV head) pair live.
enum Source : int { SRC_DENSE = 0, SRC_RAGGED = 1, SRC_PAGED = 2, SRC_HYBRID = 3, SRC_GATHER = 4 };

struct AttnArgs {
  const uint16_t* q;
  const void* k;                // dense / ragged / paged pool; hybrid: persistent slots
  const void* v;
  const void* k2;               // hybrid: cache buffer
  const void* v2;
  const int32_t* seqlens;
  const int32_t* cu_seqlens;
  const int32_t* block_table;
  const int32_t* pers_len;
  const int32_t* buf_len;
  const int32_t* head_map;
  const int32_t* idx;           // gather: [B, Hkv, max_k] token rows of each pair
  const int32_t* idx_len;       // gather: [B * Hkv]
  uint16_t* out;
  float* lse;
  float* ws_o;                  // [slots, G, 128] unnormalised partial outputs
  float* ws_ml;                 // [slots, G, 2] partial (max, sum) in log2 units
  int32_t* ws_cols;             // balanced: [n_units][2] first and last column of each unit
                                // ((1, 0) for an empty unit), written by the main kernel
  int B, Hq, Hkv, G;
  int S;                        // dense: rows per sequence; ragged: token rows T;
                                // paged: pages P in the pool
  int page, max_pages;          // paged
  int P_slots, pers_cap, buf_cap;  // hybrid
  int max_k;                    // gather: index row stride (and the longest pair)
  int mode;                     // Mode
  int max_len;                  // lengths are clamped to this (the grid's coverage)
  int chunk;                    // chunks: tokens per work item, a multiple of kTile * kWaves
  int n_chunks;                 // chunks: work items per (sequence, KV head) in the grid
  int n_blocks;                 // balanced: persistent workgroups
  int n_cu;                     // balanced: CUs of the device (workgroups of the first round)
  int n_units;                  // balanced: units of the tile line
  int xcd_cols;                 // balanced: each column's workgroups on one XCD (column c on XCD c % 8)
  int xcd_w;                    // balanced, xcd_cols: per 100, the share of a column on an odd XCD
  float scale_log2;             // softmax_scale * log2(e) (* k_scale for e4m3 K)
  float out_scale;              // e4m3 V: v_scale, applied with the final normalisation
  int src;
  int dtype;
  int kv8;                      // K and V are e4m3 codes, one byte per element
};

// Bytes of workspace for `slots` partials of group size G plus n_cols ints.
size_t attn_workspace_bytes(int64_t slots, int G, int64_t n_cols);
// Carves ws into the partial-output, partial-(max, sum) and column-range
// regions; returns false if ws_bytes is too small.
bool attn_workspace_carve(void* ws, size_t ws_bytes, int64_t slots, int G, int64_t n_cols,
                          AttnArgs* a);
// Whether the balanced schedule puts each column's waves on one XCD, with
// column c on XCD c % 8: n_blocks <= max_blocks (the CUs times the dispatch
// rounds allowed) and either
// line_heads = 4m, m >= 2, with n_blocks a multiple of 8m, or line_heads 1
// (a column per wave) with n_blocks a multiple of 8.
inline bool balanced_xcd_cols(int line_heads, int n_blocks, int max_blocks) {
  if (n_blocks > max_blocks) return false;
  if (line_heads == 1) return n_blocks % 8 == 0;
  const int m = line_heads / kWaves;
  return line_heads % kWaves == 0 && m >= 2 && n_blocks % (8 * m) == 0;
}
// With columns on one XCD, per 100, the share of a column on an odd XCD:
// 0.95 for columns of two workgroups (8 KV heads), 0.87 for eight or more
// workgroups reading pages (32 KV heads, paged), else 0.90 (eight or more
// workgroups reading runs, or one wave).  Measured on MI355X, one process,
// interleaved, main kernel: the paged 1024 x 32-head batch 3342 / 3326 /
// 3312 us at 0.96 / 0.93 / 0.90, and at 0.88 / 0.87 / 0.86 / 0.84 10 / 15 /
// 19 / 12 us shorter than at 0.90 (whole calls at 0.87: 18 us), where the
// same batch laid out ragged was 3 / 8-12 / 23 us longer at 0.88 / 0.87 /
// 0.86; the 16 x 16K-32K batch with 8 KV heads 1.9-2.6 us
// shorter at 0.95 than with columns across XCDs, on three boxes, and 0.3 us
// longer to 0.3 us shorter with one XCD per column and equal weights; the CLO
// hybrids (a column per wave) 0.2-1.4 us shorter at 0.90 (whole calls
// 0.7-1.1 us) on three boxes, and about 0.5 us longer with equal weights.
inline int balanced_odd_xcd_weight(int line_heads, int src) {
  if (line_heads == 2 * kWaves) return 95;
  return line_heads >= 4 * kWaves && src == SRC_PAGED ? 87 : 90;
}
// Persistent workgroups for the balanced schedule on the current device:
// CUs x resident workgroups per CU, fewer when est_tiles is small.
int balanced_blocks(int dtype, int kv8, int G, int src, int64_t est_tiles);
// Compute units of the current device (cached per device).
int device_cu_count();

hipError_t launch_decode_attn(const AttnArgs& a, hipStream_t stream);

// Exact top-k selection (topk.hip).
constexpr int kTopkMaxLen = 262144;  // rows per sequence the selection handles
struct TopkArgs {
  const uint16_t* q;       // [B, Hq, 128]
  const uint16_t* k;       // [B, S, Hkv, 128]
  const int32_t* seqlens;  // [B] or NULL (all S)
  float* scores;           // [B * Hkv, S4] workspace, S4 = S rounded up to 4
  int32_t* idx;            // [B * Hkv, top_k]
  int32_t* idx_len;        // [B * Hkv]
  uint32_t* sel;           // [B * Hkv, topk_sel_words(C)] workspace after the scores
  int B, Hq, Hkv, G, S, S4, top_k;
  int C;                   // selection chunks per pair, topk_chunks(S)
  int dtype;
};
constexpr int kSelChunk = 16384;  // tokens per selection workgroup
constexpr int kSelHist = 2048;    // bins of a radix digit's histogram
inline int topk_chunks(int S) { return S > 0 ? (S + kSelChunk - 1) / kSelChunk : 1; }
__host__ __device__ constexpr int topk_sel_words(int chunks) { return 2048 + 2048 + 1024 + 8 + chunks * 1028; }
size_t topk_workspace_bytes(int pairs, int S);
hipError_t launch_topk(const TopkArgs& a, hipStream_t stream);

hipError_t launch_stream_read(const void* src, size_t bytes, uint32_t* sink, hipStream_t stream);

// Profiling events of the next main-kernel launch of a call: a start/stop
// pair from the calling thread's pool when kvdec_kernel_timing is enabled on
// it, else two nulls.
void timing_events(hipEvent_t* start, hipEvent_t* stop);

// Launches a call's main kernel.  With timing enabled, HIP stamps the events
// from the kernel's own dispatch (its start and its end), so they add no
// packets to the stream and read the kernel's execution time.
template <typename... KArgs, typename... Args>
inline void launch_timed(void (*kernel)(KArgs...), dim3 grid, dim3 block, uint32_t lds,
                         hipStream_t stream, const Args&... args) {
  hipEvent_t e0 = nullptr, e1 = nullptr;
  timing_events(&e0, &e1);
  hipExtLaunchKernelGGL(kernel, grid, block, lds, stream, e0, e1, 0u, args...);
}

struct LookupArgs {
  const uint16_t* q;
  uint16_t* labels;
  const float* w;
  const float* tau;
  uint8_t* hit;
  float* agg;
  float* cos;
  int32_t* miss_list;
  int32_t* miss_count;
  int B, Hq, Hkv, G;
  int dtype;
};
hipError_t launch_headcache_lookup(const LookupArgs& a, hipStream_t stream);

// q = x . W_q^T for a batch of rows (W_q stored [N, h], output index first).
struct QProjArgs {
  const uint16_t* x;  // [B, h]
  const uint16_t* w;  // [N, h]
  uint16_t* q;        // [B, N]
  int B, h, N;
  int dtype;
};
hipError_t launch_qproj(const QProjArgs& a, hipStream_t stream);

// Miss-driven prefetch into the cache buffer (prefetch.hip).
struct PrefetchArgs {
  const int32_t* miss_list;   // [B * Hkv] pairs b * Hkv + g, the first *miss_count valid
  const int32_t* miss_count;  // [1]
  const int32_t* head_map;    // [Hkv] or NULL: heads with a slot >= 0 are persistent, skipped
  const int32_t* idx;         // [B * Hkv, max_k] selected token rows of each pair
  const int32_t* idx_len;     // [B * Hkv]
  const void* pool_k;         // device address of the pinned host pool (K)
  const void* pool_v;
  void* buf_k;                // [B, Hkv, buf_cap, 128] cache buffer
  void* buf_v;
  int32_t* buf_len;           // [B * Hkv], set for every missed pair
  int32_t* status;            // NULL, or the flag wait's result: nonzero = copy nothing
  int64_t stride_b, stride_s, stride_h;  // pool strides in elements
  int B, Hkv, S, max_k, buf_cap;
  int max_rows;               // min(max_k, buf_cap)
  int elem_bytes;             // 2 (fp16, bf16) or 1 (e4m3 codes)
};
hipError_t launch_prefetch(const PrefetchArgs& a, hipStream_t stream);
hipError_t launch_flag_wait(const uint32_t* flag, uint32_t target, uint64_t ticks,
                            uint32_t max_polls, int32_t* status, hipStream_t stream);
hipError_t launch_flag_signal(uint32_t* flag, uint32_t value, hipStream_t stream);

struct RecomputeArgs {
  const uint16_t* x;
  const uint16_t* wk;
  const uint16_t* wv;
  uint16_t* kc;
  uint16_t* vc;
  int64_t x_bstride;
  int64_t c_bstride;
  int b, l, h;
  int w_layout;  // kvdec_w_layout
};
hipError_t launch_kv_recompute(const RecomputeArgs& a, hipStream_t stream);

}  // namespace kvdec

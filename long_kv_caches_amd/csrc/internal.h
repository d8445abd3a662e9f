// internal.h -- declarations shared by the libkvdec host layer and its kernels.
#pragma once

#include <stdint.h>

#include <hip/hip_runtime.h>

#include "kvdec.h"

namespace kvdec {

// Records a thread-local message for kvdec_last_error() and returns `st`.
kvdec_status fail(kvdec_status st, const char* fmt, ...);

constexpr int kHeadDim = 128;     // the one supported head_dim
constexpr int kTile = 16;         // tokens per wave tile (one MFMA row block)
constexpr int kWaves = 4;         // waves per attention workgroup
constexpr int kMaxGroup = 8;      // query heads per KV head handled by one workgroup
constexpr int kMaxChunks = 512;   // work items per (sequence, KV head) at most

// Where the K/V rows of one (sequence, KV head) pair live.
enum Source : int { SRC_DENSE = 0, SRC_RAGGED = 1, SRC_PAGED = 2, SRC_HYBRID = 3 };

struct AttnArgs {
  const uint16_t* q;
  const uint16_t* k;            // dense / ragged / paged pool; hybrid: persistent slots
  const uint16_t* v;
  const uint16_t* k2;           // hybrid: cache buffer
  const uint16_t* v2;
  const int32_t* seqlens;
  const int32_t* cu_seqlens;
  const int32_t* block_table;
  const int32_t* pers_len;
  const int32_t* buf_len;
  const int32_t* head_map;
  uint16_t* out;
  float* lse;
  float* ws_o;                  // [items, G, 128] unnormalised partial outputs
  float* ws_ml;                 // [items, G, 2] partial (max, sum) in log2 units
  int B, Hq, Hkv, G;
  int S;                        // dense: rows per sequence; ragged: token rows T;
                                // paged: pages P in the pool
  int page, max_pages;          // paged
  int P_slots, pers_cap, buf_cap;  // hybrid
  int chunk;                    // tokens per work item, a multiple of kTile * kWaves
  int n_chunks;                 // work items per (sequence, KV head) in the grid
  float scale_log2;             // softmax_scale * log2(e)
  int src;
  int dtype;
};

// Bytes of workspace for `items` partials of group size G.
size_t attn_workspace_bytes(int64_t items, int G);
// Carves ws into the partial-output and partial-(max, sum) regions; returns
// false if ws_bytes is too small.
bool attn_workspace_carve(void* ws, size_t ws_bytes, int64_t items, int G, AttnArgs* a);

hipError_t launch_decode_attn(const AttnArgs& a, hipStream_t stream);

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

struct RecomputeArgs {
  const uint16_t* x;
  const uint16_t* wk;
  const uint16_t* wv;
  uint16_t* kc;
  uint16_t* vc;
  int64_t x_bstride;
  int64_t c_bstride;
  int b, l, h;
};
hipError_t launch_kv_recompute(const RecomputeArgs& a, hipStream_t stream);

}  // namespace kvdec

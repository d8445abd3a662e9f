// headcache.hip -- CLO head-wise approximate cache lookup fused with the
// query-label update, for gfx950.
//
// CLO page, section 2: each head keeps one query label; the incoming query
// hits when its cosine to the label reaches the head's threshold tau, and a
// miss replaces the whole head.  Eq. 10: under GQA a KV head decides on the
// importance-weighted mean of its query heads' cosines.  Section 7: lookup and
// label update share one read of the query and the labels, in one kernel.
//
// One wave owns one (sequence, KV head) group: each lane holds two of the 128
// elements of every query head of the group, so the query and label rows are
// read once (coalesced 256-byte rows) and, on a miss, the query still in
// registers is written over the labels.  Reductions are fp32 DPP row sums
// and permlane swaps in a fixed order, so results are deterministic.
//
// The ascending miss list needs a scan over all groups.  Small problems
// (<= kOneBlockGroups groups) run in one workgroup: decisions go to LDS and the
// same workgroup compacts them, one launch in total.  Larger problems run one
// wave per group over many workgroups, then a one-workgroup compaction kernel.
#include "device_common.h"
#include "internal.h"

namespace kvdec {
namespace {

constexpr int kOneBlockGroups = 512;
constexpr int kScanThreads = 1024;

// Sum over the 64 lanes (every lane gets it): DPP steps within each 16-lane
// row, then permlane swaps across the rows; all on the VALU, fixed order.
__device__ __forceinline__ float lanes_sum(float x) { return rowgroup_sum(row_sum16(x)); }

// Processes group `grp` = b * Hkv + g with the 64 lanes of the calling wave.
// Returns the hit decision (uniform across the wave).  Every global load is
// issued before the first store, so none waits behind a possibly aliasing
// store, and the 3 G reductions are independent of each other.
template <int KIND>
__device__ bool lookup_group(const LookupArgs& a, int grp, int lane) {
  const int b = grp / a.Hkv, g = grp - b * a.Hkv;
  const int G = a.G;
  constexpr int kMaxG = 16;
  const int64_t row0 = ((int64_t)b * a.Hq + (int64_t)g * G) * kHeadDim;
  const uint32_t* __restrict__ q32 = reinterpret_cast<const uint32_t*>(a.q + row0);
  uint32_t* __restrict__ l32 = reinterpret_cast<uint32_t*>(a.labels + row0);
  const float* __restrict__ wg = a.w + g * G;
  uint32_t qv[kMaxG], lv[kMaxG];
  float w[kMaxG];
#pragma unroll
  for (int j = 0; j < kMaxG; ++j) {
    if (j < G) {
      qv[j] = q32[j * (kHeadDim / 2) + lane];
      lv[j] = l32[j * (kHeadDim / 2) + lane];
      w[j] = wg[j];
    }
  }
  const float tau = a.tau[g];
  float dot[kMaxG], qq[kMaxG], ll[kMaxG];
#pragma unroll
  for (int j = 0; j < kMaxG; ++j) {
    if (j < G) {
      const float q0 = lo_f32<KIND>(qv[j]), q1 = hi_f32<KIND>(qv[j]);
      const float l0 = lo_f32<KIND>(lv[j]), l1 = hi_f32<KIND>(lv[j]);
      dot[j] = lanes_sum(__builtin_fmaf(q0, l0, q1 * l1));
      qq[j] = lanes_sum(__builtin_fmaf(q0, q0, q1 * q1));
      ll[j] = lanes_sum(__builtin_fmaf(l0, l0, l1 * l1));
    }
  }
  float num = 0.f, wsum = 0.f, csum = 0.f;
  bool degenerate = false;
#pragma unroll
  for (int j = 0; j < kMaxG; ++j) {
    if (j < G) {
      float c = 0.f;
      if (qq[j] == 0.f || ll[j] == 0.f) degenerate = true;
      else c = dot[j] / (__builtin_sqrtf(qq[j]) * __builtin_sqrtf(ll[j]));
      if (a.cos && lane == j) a.cos[(int64_t)b * a.Hq + g * G + j] = c;
      num = __builtin_fmaf(w[j], c, num);
      wsum += w[j];
      csum += c;
    }
  }
  const float agg = wsum != 0.f ? num / wsum : csum / (float)G;
  const bool hit = !degenerate && agg >= tau;
  if (lane == 0) {
    a.hit[grp] = hit ? 1 : 0;
    if (a.agg) a.agg[grp] = agg;
  }
  if (!hit) {
#pragma unroll
    for (int j = 0; j < kMaxG; ++j)
      if (j < G) l32[j * (kHeadDim / 2) + lane] = qv[j];
  }
  return hit;
}

// Exclusive prefix sum of `x` over the kScanThreads threads of the block.
__device__ int block_exclusive_scan(int x, int* s_wave, int* total) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  int incl = x;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int y = __shfl_up(incl, d, 64);
    if (lane >= d) incl += y;
  }
  if (lane == 63) s_wave[wave] = incl;
  __syncthreads();
  if (tid == 0) {
    int run = 0;
    for (int w = 0; w < kScanThreads / 64; ++w) {
      const int t = s_wave[w];
      s_wave[w] = run;
      run += t;
    }
    *total = run;
  }
  __syncthreads();
  return s_wave[wave] + incl - x;
}

// Writes the ascending miss list from per-group decisions read by `is_hit`.
template <typename HitFn>
__device__ void compact_misses(int N, HitFn is_hit, int32_t* miss_list, int32_t* miss_count) {
  __shared__ int s_wave[kScanThreads / 64];
  __shared__ int s_total;
  const int per = (N + kScanThreads - 1) / kScanThreads;
  const int lo = min(N, (int)threadIdx.x * per), hi = min(N, lo + per);
  int cnt = 0;
  for (int i = lo; i < hi; ++i) cnt += is_hit(i) ? 0 : 1;
  int off = block_exclusive_scan(cnt, s_wave, &s_total);
  for (int i = lo; i < hi; ++i)
    if (!is_hit(i)) miss_list[off++] = i;
  if (threadIdx.x == 0) *miss_count = s_total;
}

template <int KIND>
__global__ __launch_bounds__(kScanThreads) void lookup_one_block_kernel(LookupArgs a) {
  __shared__ unsigned char s_hit[kOneBlockGroups];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int N = a.B * a.Hkv;
  for (int grp = wave; grp < N; grp += kScanThreads / 64) {
    const bool h = lookup_group<KIND>(a, grp, lane);
    if (lane == 0) s_hit[grp] = h ? 1 : 0;
  }
  __syncthreads();
  if (a.miss_list)
    compact_misses(N, [&](int i) { return s_hit[i] != 0; }, a.miss_list, a.miss_count);
}

template <int KIND>
__global__ __launch_bounds__(256) void lookup_grid_kernel(LookupArgs a) {
  const int lane = threadIdx.x & 63;
  const int grp = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (grp < a.B * a.Hkv) lookup_group<KIND>(a, grp, lane);
}

__global__ __launch_bounds__(kScanThreads) void compact_kernel(const uint8_t* hit, int N,
                                                               int32_t* miss_list,
                                                               int32_t* miss_count) {
  compact_misses(N, [&](int i) { return hit[i] != 0; }, miss_list, miss_count);
}

template <int KIND>
hipError_t launch_lookup_kind(const LookupArgs& a, hipStream_t stream) {
  const int N = a.B * a.Hkv;
  if (N <= kOneBlockGroups) {
    timing_begin(stream);
    lookup_one_block_kernel<KIND><<<1, kScanThreads, 0, stream>>>(a);
    timing_end(stream);
    return hipGetLastError();
  }
  timing_begin(stream);
  lookup_grid_kernel<KIND><<<(N + 3) / 4, 256, 0, stream>>>(a);
  timing_end(stream);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || !a.miss_list) return e;
  compact_kernel<<<1, kScanThreads, 0, stream>>>(a.hit, N, a.miss_list, a.miss_count);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_headcache_lookup(const LookupArgs& a, hipStream_t stream) {
  return a.dtype == KIND_F16 ? launch_lookup_kind<KIND_F16>(a, stream)
                             : launch_lookup_kind<KIND_BF16>(a, stream);
}

}  // namespace kvdec

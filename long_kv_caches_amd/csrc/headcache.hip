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

// A group's inputs as one wave holds them.  Each 16-lane row of the wave takes
// one query head at a time (row r: heads r, r + 4, ... of the group, one head
// per pass, P passes for G <= 4 P); lane n of a row holds elements 8n .. 8n+7
// of that head's q and label (one 16-byte load each), so a head's three sums
// need only reductions within its row.  P = 1, 2 or 4 (G <= 4, 8, 16).
template <int P>
struct GroupRegs {
  u32x4 qv[P], lv[P];
  float w[P];  // the weight of this row's head in each pass (0 past G)
  float tau;
};

// Issues the loads of group `grp` = b * Hkv + g (uniform across the wave).
template <int P>
__device__ __forceinline__ void lookup_load(const LookupArgs& a, int grp, int lane,
                                            GroupRegs<P>& r) {
  grp = uniform_i32(grp);
  const int b = grp / a.Hkv, g = grp - b * a.Hkv;
  const int G = a.G, row = lane >> 4, piece = lane & 15;
  const int64_t row0 = ((int64_t)b * a.Hq + (int64_t)g * G) * kHeadDim + piece * 8;
#pragma unroll
  for (int p = 0; p < P; ++p) {
    const int j = row + 4 * p;
    if (j < G) {
      r.qv[p] = load_b128(a.q + row0 + (int64_t)j * kHeadDim);
      r.lv[p] = load_b128(a.labels + row0 + (int64_t)j * kHeadDim);
      r.w[p] = a.w[g * G + j];
    } else {
      r.qv[p] = r.lv[p] = u32x4{0, 0, 0, 0};
      r.w[p] = 0.f;
    }
  }
  r.tau = a.tau[g];
}

// Decides group `grp` from its loaded inputs and writes its outputs; returns
// the hit decision (uniform across the wave).
template <int KIND, int P>
__device__ bool lookup_finish(const LookupArgs& a, int grp, int lane, const GroupRegs<P>& r) {
  grp = uniform_i32(grp);
  const int b = grp / a.Hkv, g = grp - b * a.Hkv;
  const int G = a.G, row = lane >> 4, piece = lane & 15;
  float num = 0.f, wsum = 0.f, csum = 0.f;
  bool degenerate = false;
#pragma unroll
  for (int p = 0; p < P; ++p) {
    const uint32_t qa[4] = {r.qv[p].x, r.qv[p].y, r.qv[p].z, r.qv[p].w};
    const uint32_t la[4] = {r.lv[p].x, r.lv[p].y, r.lv[p].z, r.lv[p].w};
    float dot = 0.f, qq = 0.f, ll = 0.f;
#pragma unroll
    for (int e = 0; e < 4; ++e) {  // v_dot2: two exact products and an fp32 add
      dot = dot2<KIND>(qa[e], la[e], dot);
      qq = dot2<KIND>(qa[e], qa[e], qq);
      ll = dot2<KIND>(la[e], la[e], ll);
    }
    dot = row_sum16(dot);
    qq = row_sum16(qq);
    ll = row_sum16(ll);
    const int j = row + 4 * p;
    if (j < G) {
      float c = 0.f;
      // hardware reciprocal square roots (about one unit in the last place
      // each), one per norm so no product of the squared norms can overflow
      if (qq == 0.f || ll == 0.f) degenerate = true;
      else c = dot * __builtin_amdgcn_rsqf(qq) * __builtin_amdgcn_rsqf(ll);
      if (a.cos && piece == 0) a.cos[(int64_t)b * a.Hq + g * G + j] = c;
      num = __builtin_fmaf(r.w[p], c, num);
      wsum += r.w[p];
      csum += c;
    }
  }
  // every lane of a row holds its row's partial sums; add the four rows
  num = rowgroup_sum(num);
  wsum = rowgroup_sum(wsum);
  csum = rowgroup_sum(csum);
  degenerate = __ballot(degenerate) != 0;
  const float agg = wsum != 0.f ? num / wsum : csum / (float)G;
  const bool hit = !degenerate && agg >= r.tau;
  if (lane == 0) {
    a.hit[grp] = hit ? 1 : 0;
    if (a.agg) a.agg[grp] = agg;
  }
  if (!hit) {
    const int64_t row0 = ((int64_t)b * a.Hq + (int64_t)g * G) * kHeadDim + piece * 8;
#pragma unroll
    for (int p = 0; p < P; ++p) {
      const int j = row + 4 * p;
      if (j < G) store_b128(a.labels + row0 + (int64_t)j * kHeadDim, r.qv[p]);
    }
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

// All groups in one workgroup, the miss list written by the same launch.  A
// wave takes groups wave, wave + 16, ...; the next group's loads are issued
// before the current group's outputs are stored (memory operations complete in
// issue order, so a load issued after a store would wait for it).  Wave 0 then
// compacts the decisions with ballots, 64 groups per step.
template <int KIND, int P>
__global__ __launch_bounds__(kScanThreads) void lookup_one_block_kernel(LookupArgs a) {
  constexpr int kW = kScanThreads / 64;
  __shared__ unsigned char s_hit[kOneBlockGroups];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int N = a.B * a.Hkv;
  GroupRegs<P> ra, rb;
  if (wave < N) lookup_load(a, wave, lane, ra);
  for (int grp = wave; grp < N; grp += 2 * kW) {
    if (grp + kW < N) lookup_load(a, grp + kW, lane, rb);
    bool h = lookup_finish<KIND, P>(a, grp, lane, ra);
    if (lane == 0) s_hit[grp] = h ? 1 : 0;
    if (grp + 2 * kW < N) lookup_load(a, grp + 2 * kW, lane, ra);
    if (grp + kW < N) {
      h = lookup_finish<KIND, P>(a, grp + kW, lane, rb);
      if (lane == 0) s_hit[grp + kW] = h ? 1 : 0;
    }
  }
  if (!a.miss_list) return;
  __syncthreads();
  if (wave != 0) return;
  int base = 0;
  for (int i0 = 0; i0 < N; i0 += 64) {
    const int i = i0 + lane;
    const bool miss = i < N && s_hit[i] == 0;
    const uint64_t m = __ballot(miss);
    const int before = __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32),
                                                 __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
    if (miss) a.miss_list[base + before] = i;
    base += __popcll(m);
  }
  if (lane == 0) *a.miss_count = base;
}

template <int KIND, int P>
__global__ __launch_bounds__(256) void lookup_grid_kernel(LookupArgs a) {
  const int lane = threadIdx.x & 63;
  const int grp = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (grp < a.B * a.Hkv) {
    GroupRegs<P> r;
    lookup_load(a, grp, lane, r);
    lookup_finish<KIND, P>(a, grp, lane, r);
  }
}

__global__ __launch_bounds__(kScanThreads) void compact_kernel(const uint8_t* hit, int N,
                                                               int32_t* miss_list,
                                                               int32_t* miss_count) {
  compact_misses(N, [&](int i) { return hit[i] != 0; }, miss_list, miss_count);
}

template <int KIND, int P>
hipError_t launch_lookup_kind(const LookupArgs& a, hipStream_t stream) {
  const int N = a.B * a.Hkv;
  if (N <= kOneBlockGroups) {
    launch_timed(lookup_one_block_kernel<KIND, P>, dim3(1), dim3(kScanThreads), 0u, stream, a);
    return hipGetLastError();
  }
  launch_timed(lookup_grid_kernel<KIND, P>, dim3((N + 3) / 4), dim3(256), 0u, stream, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || !a.miss_list) return e;
  compact_kernel<<<1, kScanThreads, 0, stream>>>(a.hit, N, a.miss_list, a.miss_count);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Approximate query one layer ahead (CLO page, section 3, decoding flow,
// Figure 9: at the start of layer l-1 the query of layer l is approximated by
// x_{l-1} W_Q^l, so the lookup, and the prefetch of the heads it misses, can
// run a layer early).
// q[b][n] = sum_i x[b][i] W[n][i]: a GEMV per batch row, bound by reading W
// once per group of kQBatch rows.  Workgroups of WAVES waves (8 for h <= 4096,
// two per CU; 16 above, one per CU) each take an equal run of
// R = ceil(N / workgroups) rows of W, so every CU streams the same bytes
// whatever N is.  Within a workgroup the h axis is split in WAVES slices, one
// per wave, of at most 64 16-byte pieces, so a lane holds one piece of its
// slice: of each x row of the batch group (registers, loaded once per group)
// and of kQRC rows of W at a time.  W chunks go through a ring of kQRing
// buffers; every load is issued unconditionally (rows past the run read zero
// through the buffer descriptor), so the compiler's waits cover exactly the
// chunk in use while the next ones stay in flight.  Products are v_dot2 with
// fp32 sums; a chunk's kQRC x kQBatch sums are reduced over the wave in one
// transposed reduction, the slice sums added in wave order; one rounding per
// output.
// ---------------------------------------------------------------------------
constexpr int kQBatch = 4, kQRC = 4, kQRing = 3, kQMaxR = 64, kQMaxWaves = 16;
constexpr uint32_t kQOutside = 0x80000000u;  // an offset past every descriptor

template <int KIND, int WAVES>
__global__ __launch_bounds__(WAVES * 64) __attribute__((amdgpu_waves_per_eu(4)))
void qproj_kernel(QProjArgs a, int R) {
  __shared__ float s_part[kQMaxWaves][kQMaxR][kQBatch];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int n0 = blockIdx.x * R;
  const int rows = min(R, a.N - n0);  // >= 1
  const int nch = a.h / 8;            // 16-byte pieces per row
  const int pw = (nch + WAVES - 1) / WAVES;
  const int p = wave * pw + lane;
  const uint32_t poff = (lane < pw && p < nch) ? (uint32_t)p * 16 : kQOutside;
  const uint32_t row_bytes = (uint32_t)a.h * 2;
  const __amdgpu_buffer_rsrc_t wr = make_rsrc(a.w + (int64_t)n0 * a.h, (uint32_t)rows * row_bytes);
  const int nchunks = (rows + kQRC - 1) / kQRC;

  for (int bg = 0; bg < a.B; bg += kQBatch) {
    const int nb = min(kQBatch, a.B - bg);
    const __amdgpu_buffer_rsrc_t xr = make_rsrc(a.x + (int64_t)bg * a.h, (uint32_t)nb * row_bytes);
    u32x4 xs[kQBatch];
#pragma unroll
    for (int b = 0; b < kQBatch; ++b)
      xs[b] = __builtin_amdgcn_raw_buffer_load_b128(
          xr, poff == kQOutside ? kQOutside : b * row_bytes + poff, 0, 0);
    auto load = [&](u32x4 (&wv)[kQRC], int ci) {
#pragma unroll
      for (int r = 0; r < kQRC; ++r)
        wv[r] = buffer_load_b128_nt(
            wr, poff == kQOutside ? kQOutside : (uint32_t)(ci * kQRC + r) * row_bytes + poff);
    };
    auto use = [&](const u32x4 (&wv)[kQRC], int ci) {
      // this lane's products for the chunk's rows x the group's batch rows
      // (zero past either), then one transposed wave reduction
      float v[kQRC * kQBatch];
#pragma unroll
      for (int r = 0; r < kQRC; ++r) {
#pragma unroll
        for (int b = 0; b < kQBatch; ++b) {
          float t = dot2<KIND>(wv[r].x, xs[b].x, 0.f);
          t = dot2<KIND>(wv[r].y, xs[b].y, t);
          t = dot2<KIND>(wv[r].z, xs[b].z, t);
          v[r * kQBatch + b] = dot2<KIND>(wv[r].w, xs[b].w, t);
        }
      }
      const float sum = transpose_reduce<kQRC * kQBatch>(v, lane);
      constexpr int kSpread = 64 / (kQRC * kQBatch);  // lanes holding each sum
      const int idx = lane / kSpread, r = idx / kQBatch, b = idx - r * kQBatch;
      const int row = ci * kQRC + r;
      if (lane % kSpread == 0 && row < rows && b < nb) s_part[wave][row][b] = sum;
    };
    u32x4 wbuf[kQRing][kQRC];
#pragma unroll
    for (int k = 0; k < kQRing - 1; ++k) load(wbuf[k], k);
    for (int ci = 0; ci < nchunks; ci += kQRing) {
#pragma unroll
      for (int k = 0; k < kQRing; ++k) {
        load(wbuf[(k + kQRing - 1) % kQRing], ci + k + kQRing - 1);
        if (ci + k < nchunks) use(wbuf[k], ci + k);
      }
    }
    __syncthreads();
    for (int i = threadIdx.x; i < rows * nb; i += WAVES * 64) {
      const int r = i / nb, b = i - r * nb;
      float sum = s_part[0][r][b];
#pragma unroll
      for (int w = 1; w < WAVES; ++w) sum += s_part[w][r][b];
      a.q[(int64_t)(bg + b) * a.N + n0 + r] = to_bits<KIND>(sum);
    }
    __syncthreads();  // s_part is rewritten by the next batch group
  }
}

template <int KIND>
void launch_qproj_kind(const QProjArgs& a, hipStream_t stream) {
  const bool wide = a.h > 4096;  // 16 slices keep each at <= 64 pieces
  const int groups = (wide ? 1 : 2) * device_cu_count();
  int R = (a.N + groups - 1) / groups;
  R = R < 1 ? 1 : (R > kQMaxR ? kQMaxR : R);
  const unsigned blocks = (unsigned)((a.N + R - 1) / R);
  if (wide) launch_timed(qproj_kernel<KIND, 16>, dim3(blocks), dim3(16 * 64), 0u, stream, a, R);
  else launch_timed(qproj_kernel<KIND, 8>, dim3(blocks), dim3(8 * 64), 0u, stream, a, R);
}

}  // namespace

hipError_t launch_qproj(const QProjArgs& a, hipStream_t stream) {
  if (a.dtype == KIND_F16) launch_qproj_kind<KIND_F16>(a, stream);
  else launch_qproj_kind<KIND_BF16>(a, stream);
  return hipGetLastError();
}

hipError_t launch_headcache_lookup(const LookupArgs& a, hipStream_t stream) {
  // passes of four heads per wave: G <= 4, <= 8, <= 16
  if (a.dtype == KIND_F16) {
    return a.G <= 4 ? launch_lookup_kind<KIND_F16, 1>(a, stream)
         : a.G <= 8 ? launch_lookup_kind<KIND_F16, 2>(a, stream)
                    : launch_lookup_kind<KIND_F16, 4>(a, stream);
  }
  return a.G <= 4 ? launch_lookup_kind<KIND_BF16, 1>(a, stream)
       : a.G <= 8 ? launch_lookup_kind<KIND_BF16, 2>(a, stream)
                  : launch_lookup_kind<KIND_BF16, 4>(a, stream);
}

}  // namespace kvdec

// topk.hip -- exact top-k token selection for index-gather sparse attention.
//
// CLO page: decoding attends to a top-k selection of each head's tokens (10%
// of them), retrieved with HATA's hash codes; here the exact scores stand in
// for the hashes.  Eq. 6 (q.k = |q| |k| cos(q, k)) is why the selection of a
// query can be reused by the next one: the ranking does not depend on |q|.
// One selection per (sequence b, KV head g): tokens t < len_b are ranked by
//   s_t = sum over the group's query heads j of q_j . K_t,
// computed as (sum_j q_j) . K_t in fp32; the min(top_k, len_b) largest are
// kept, ties going to the smaller token index, and written in ascending
// token order.
//
// Kernels:
//   topk_score_rows_kernel -- streams K once (HBM-bound) in memory order: each
//     wave takes 16 consecutive 256-byte (token, head) pieces per step, lane l
//     8 dims of piece 4 i + l / 16 in load i; the group query sums of every KV
//     head are in LDS (fp32), FMAs and a DPP row sum per piece.  Used up to 64
//     KV heads.
//   topk_score_kernel  -- the same scores one KV head at a time (more heads):
//     one wave per 16-token tile, lane l holds piece l % 16 (8 dims) of rows
//     4 * (l / 16) .. +3, the query sum in fp32 for its piece.
//   topk_select_kernel -- one 1024-thread workgroup per pair over the pair's
//     scores (L2-resident): a radix select of the k-th largest key in three
//     passes of 11, 11 and 10 bits (LDS histograms), then an ordered
//     compaction: per 256-token segment (lane l: tokens 4l .. 4l+3), ballots
//     count the keys above the threshold and those equal to it, a scan over
//     the segments gives each its output offset and its ties before it, and
//     a second sweep writes the selected indices in order.  Every sweep reads
//     the scores with 16-byte loads, four in flight per thread.
#include "device_common.h"
#include "internal.h"

namespace kvdec {
namespace {

constexpr int kSelThreads = 1024;
constexpr int kSelBatch = 4;  // 16-byte loads each thread keeps in flight in a sweep
constexpr int kSelWaves = kSelThreads / 64;
constexpr int kMaxSegments = kTopkMaxLen / 256;
constexpr int kRowSteps = 16;     // 16-segment steps each wave of the whole-row score kernel takes
constexpr int kRowMaxHkv = 64;    // KV heads whose query sums the whole-row kernel keeps in LDS

// Orderable key of a float: larger float <=> larger unsigned key.
__device__ __forceinline__ uint32_t order_key(float f) {
  const uint32_t u = __builtin_bit_cast(uint32_t, f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

template <int KIND>
__global__ __launch_bounds__(256) void topk_score_kernel(TopkArgs a) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int n = lane & 15, lg = lane >> 4;
  const int pair = blockIdx.y, b = pair / a.Hkv, g = pair - b * a.Hkv;
  const int len = uniform_i32(min(max(a.seqlens ? a.seqlens[b] : a.S, 0), a.S));
  const int t0 = (blockIdx.x * 4 + wave) * kTile;
  if (t0 >= len) return;
  // the group's query sum for this lane's 8 dims, fp32 in head order
  float qs[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  for (int j = 0; j < a.G; ++j) {
    const u32x4 qv = load_b128(a.q + ((int64_t)b * a.Hq + (int64_t)g * a.G + j) * kHeadDim + 8 * n);
    const uint32_t w[4] = {qv.x, qv.y, qv.z, qv.w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      qs[2 * e] += lo_f32<KIND>(w[e]);
      qs[2 * e + 1] += hi_f32<KIND>(w[e]);
    }
  }
  const uint32_t row_bytes = (uint32_t)a.Hkv * kHeadDim * 2;
  const int rows = min(len - t0, kTile);
  const uint16_t* kb = a.k + (((int64_t)b * a.S + t0) * a.Hkv + g) * kHeadDim;
  const __amdgpu_buffer_rsrc_t rk = make_rsrc(uniform_ptr(kb), uniform_u32((uint32_t)rows * row_bytes));
  u32x4 kv[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) kv[i] = buffer_load_b128_nt(rk, (4 * lg + i) * row_bytes + 16 * n);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t w[4] = {kv[i].x, kv[i].y, kv[i].z, kv[i].w};
    float acc = 0.f;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      acc = __builtin_fmaf(qs[2 * e], lo_f32<KIND>(w[e]), acc);
      acc = __builtin_fmaf(qs[2 * e + 1], hi_f32<KIND>(w[e]), acc);
    }
    acc = row_sum16(acc);
    const int t = t0 + 4 * lg + i;
    if (n == 0 && t < len) a.scores[(int64_t)pair * a.S4 + t] = acc;
  }
}

// Whole-row variant: the K rows of sequence b are read in memory order, all KV
// heads of a token together.  Piece (token t, head h) of 256 bytes is segment
// s = t * Hkv + h of the sequence; wave w of the block takes 16 segments per
// step, lane l piece l % 16 of segment 4 i + l / 16 in load i, so each load
// is 1 KB of contiguous memory.  The group query sums of all Hkv heads sit in
// LDS (fp32, head-major), summed and multiplied in the same order as above,
// so the scores are the same numbers.  The first step's loads are issued
// before the sums are formed, and each step's loads before the previous
// step's arithmetic.  The block's scores are staged in LDS in segment order
// and written out per head as runs of consecutive tokens (nontemporal): on
// MI355X single scattered 4-byte stores into the score rows made the pass
// 23% slower than the same reads alone (310 against 241 us on 1.7 GB), the
// staged runs 12% (270 us).
template <int KIND>
__global__ __launch_bounds__(256) void topk_score_rows_kernel(TopkArgs a) {
  constexpr int kBlockSegs = 4 * kRowSteps * kTile;
  __shared__ float s_sc[kBlockSegs];               // the block's scores, segment order
  extern __shared__ __align__(16) float s_qsum[];  // [Hkv, 128]
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int n = lane & 15, lg = lane >> 4;
  const int b = blockIdx.y, Hkv = a.Hkv;
  const int len = uniform_i32(min(max(a.seqlens ? a.seqlens[b] : a.S, 0), a.S));
  const int nseg = len * Hkv;
  const int blk0 = blockIdx.x * kBlockSegs;
  if (blk0 >= nseg) return;
  const uint16_t* kseq = a.k + (int64_t)b * a.S * Hkv * kHeadDim;
  // 16 segments from seg0 (those past the sequence read as zeros, unfetched)
  auto load_step = [&](int seg0, u32x4 (&kv)[4]) {
    const int segs = min(max(nseg - seg0, 0), kTile);
    const uint16_t* base = kseq + (int64_t)(segs > 0 ? seg0 : 0) * kHeadDim;
    const __amdgpu_buffer_rsrc_t rk = make_rsrc(uniform_ptr(base), uniform_u32((uint32_t)segs * 2 * kHeadDim));
#pragma unroll
    for (int i = 0; i < 4; ++i) kv[i] = buffer_load_b128_nt(rk, (4 * i + lg) * 2 * kHeadDim + 16 * n);
  };
  u32x4 cur[4], nxt[4];
  load_step(blk0 + wave * kTile, cur);
  for (int e = tid; e < Hkv * 16; e += 256) {
    const int h = e >> 4, p = e & 15;
    float qs[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    for (int j = 0; j < a.G; ++j) {
      const u32x4 qv = load_b128(a.q + ((int64_t)b * a.Hq + (int64_t)h * a.G + j) * kHeadDim + 8 * p);
      const uint32_t w[4] = {qv.x, qv.y, qv.z, qv.w};
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        qs[2 * q] += lo_f32<KIND>(w[q]);
        qs[2 * q + 1] += hi_f32<KIND>(w[q]);
      }
    }
    float4* dst = reinterpret_cast<float4*>(s_qsum + h * kHeadDim + 8 * p);
    dst[0] = make_float4(qs[0], qs[1], qs[2], qs[3]);
    dst[1] = make_float4(qs[4], qs[5], qs[6], qs[7]);
  }
  __syncthreads();
  // this lane's head for load 0 of step 0; 4 segments further per load,
  // 48 more per step (remainders by Hkv)
  int h = (blk0 + wave * kTile + lg) % Hkv;
  const int r4 = 4 % Hkv, r48 = 48 % Hkv;
#pragma unroll
  for (int step = 0; step < kRowSteps; ++step) {
    const int loc0 = (step * 4 + wave) * kTile;
    if (blk0 + loc0 >= nseg) break;
    if (step + 1 < kRowSteps) load_step(blk0 + loc0 + 4 * kTile, nxt);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float4* qp = reinterpret_cast<const float4*>(s_qsum + h * kHeadDim + 8 * n);
      const float4 x0 = qp[0], x1 = qp[1];
      const float qs[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
      const uint32_t w[4] = {cur[i].x, cur[i].y, cur[i].z, cur[i].w};
      float acc = 0.f;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        acc = __builtin_fmaf(qs[2 * e], lo_f32<KIND>(w[e]), acc);
        acc = __builtin_fmaf(qs[2 * e + 1], hi_f32<KIND>(w[e]), acc);
      }
      acc = row_sum16(acc);
      if (n == 0) s_sc[loc0 + 4 * i + lg] = acc;
      h += r4;
      if (h >= Hkv) h -= Hkv;
    }
    h += r48;
    if (h >= Hkv) h -= Hkv;
#pragma unroll
    for (int i = 0; i < 4; ++i) cur[i] = nxt[i];
  }
  __syncthreads();
  // segments [blk0, end) hold tokens t0 .. t1 (the first and last possibly
  // for some heads only); head h's scores go to its row as one run of tokens
  const int end = min(nseg, blk0 + kBlockSegs);
  const int t0 = blk0 / Hkv, ntok = (end - 1) / Hkv - t0 + 1;
  float* sc = a.scores + (int64_t)b * Hkv * a.S4;
  for (int e = tid; e < Hkv * ntok; e += 256) {
    const int hh = e / ntok, t = t0 + e - hh * ntok;
    const int seg = t * Hkv + hh;
    if (seg >= blk0 && seg < end) __builtin_nontemporal_store(s_sc[seg - blk0], sc + (int64_t)hh * a.S4 + t);
  }
}

// Exclusive scan of one int per thread over the workgroup; *total gets the sum.
__device__ int sel_scan(int x, int* s_wave, int* total) {
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
    for (int w = 0; w < kSelWaves; ++w) {
      const int t = s_wave[w];
      s_wave[w] = run;
      run += t;
    }
    *total = run;
  }
  __syncthreads();
  const int r = s_wave[wave] + incl - x;
  __syncthreads();  // s_wave is reused by the next scan
  return r;
}

// Ranks of this lane's four tokens (4 * lane + c) among the flagged tokens of
// a 256-token segment, in token order.
__device__ __forceinline__ void seg_ranks(const bool (&f)[4], int lane, int (&rank)[4], int* total) {
  int before = 0, all = 0;
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    const uint64_t m = __ballot(f[c]);
    before += (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
    all += __popcll(m);
  }
  int own = 0;
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    rank[c] = before + own;
    own += f[c] ? 1 : 0;
  }
  *total = all;
}

__global__ __launch_bounds__(kSelThreads) void topk_select_kernel(TopkArgs a) {
  __shared__ uint32_t s_hist[2048];
  __shared__ int s_seg_gt[kMaxSegments], s_seg_eq[kMaxSegments];
  __shared__ int s_wave[kSelWaves];
  __shared__ int s_total;
  __shared__ uint32_t s_sel[2];  // selected digit, remaining count
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int pair = blockIdx.x, b = pair / a.Hkv;
  const int len = min(max(a.seqlens ? a.seqlens[b] : a.S, 0), a.S);
  const int need = min(a.top_k, len);
  int32_t* out = a.idx + (int64_t)pair * a.top_k;
  if (tid == 0) a.idx_len[pair] = need;
  if (need == 0) return;
  if (need == len) {  // everything is kept
    for (int t = tid; t < len; t += kSelThreads) out[t] = t;
    return;
  }
  // the pair's scores (rows of S4 = S rounded up to 4 floats, so a 16-byte
  // read never leaves the row); reads past the row's valid groups return zeros,
  // and tokens at or past len are masked below
  const __amdgpu_buffer_rsrc_t rs = make_rsrc(uniform_ptr(a.scores + (int64_t)pair * a.S4),
                                              uniform_u32((uint32_t)((len + 3) & ~3) * 4u));
  auto load4 = [&](int t) -> f32x4 {  // tokens t .. t+3
    return __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, 4 * t, 0, 0));
  };
  // Radix select of the need-th largest key: digits of 11, 11, 10 bits.
  uint32_t prefix = 0, mask = 0;
  uint32_t remaining = (uint32_t)need;
  const int shifts[3] = {21, 10, 0}, widths[3] = {11, 11, 10};
  for (int p = 0; p < 3; ++p) {
    const int shift = shifts[p], nbins = 1 << widths[p];
    for (int i = tid; i < nbins; i += kSelThreads) s_hist[i] = 0;
    __syncthreads();
    for (int t0 = 4 * tid; t0 < len; t0 += 4 * kSelBatch * kSelThreads) {
      f32x4 v[kSelBatch];
#pragma unroll
      for (int u = 0; u < kSelBatch; ++u) v[u] = load4(t0 + 4 * u * kSelThreads);
#pragma unroll
      for (int u = 0; u < kSelBatch; ++u) {
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          const uint32_t k = order_key(v[u][c]);
          if (t0 + 4 * u * kSelThreads + c < len && (k & mask) == prefix)
            atomicAdd(&s_hist[(k >> shift) & (nbins - 1)], 1u);
        }
      }
    }
    __syncthreads();
    if (wave == 0) {
      // lane l sums bins [nbins - per (l + 1), nbins - per l) (from the top)
      const int per = nbins / 64;
      uint32_t c = 0;
      for (int i = 0; i < per; ++i) c += s_hist[nbins - per * (lane + 1) + i];
      uint32_t incl = c;
#pragma unroll
      for (int d = 1; d < 64; d <<= 1) {
        const uint32_t y = __shfl_up(incl, d, 64);
        if (lane >= d) incl += y;
      }
      const uint32_t before = incl - c;  // keys in higher bins
      if (before < remaining && remaining <= incl) {
        uint32_t run = before;
        for (int i = per - 1; i >= 0; --i) {
          const int bin = nbins - per * (lane + 1) + i;
          const uint32_t h = s_hist[bin];
          if (run + h >= remaining) {
            s_sel[0] = (uint32_t)bin;
            s_sel[1] = remaining - run;
            break;
          }
          run += h;
        }
      }
    }
    __syncthreads();
    prefix |= s_sel[0] << shift;
    mask |= (uint32_t)(nbins - 1) << shift;
    remaining = s_sel[1];
    __syncthreads();
  }
  const uint32_t T = prefix;                 // the need-th largest key
  const int take_eq = (int)remaining;        // keys equal to T to keep, lowest tokens first
  // Ordered compaction over 256-token segments (lane l: tokens 4l .. 4l+3).
  const int nseg = (len + 255) / 256;
  auto flags = [&](const f32x4& v, int t, bool (&gt)[4], bool (&eq)[4]) {
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const uint32_t k = order_key(v[c]);
      gt[c] = t + c < len && k > T;
      eq[c] = t + c < len && k == T;
    }
  };
  for (int s0 = wave; s0 < nseg; s0 += kSelBatch * kSelWaves) {
    f32x4 v[kSelBatch];
#pragma unroll
    for (int u = 0; u < kSelBatch; ++u) v[u] = load4(256 * (s0 + u * kSelWaves) + 4 * lane);
#pragma unroll
    for (int u = 0; u < kSelBatch; ++u) {
      const int s = s0 + u * kSelWaves;
      if (s >= nseg) break;  // the same in every lane
      bool gt[4], eq[4];
      flags(v[u], 256 * s + 4 * lane, gt, eq);
      int r[4], ngt, neq;
      seg_ranks(gt, lane, r, &ngt);
      seg_ranks(eq, lane, r, &neq);
      if (lane == 0) {
        s_seg_gt[s] = ngt;
        s_seg_eq[s] = neq;
      }
    }
  }
  __syncthreads();
  // scan the segments in order: each thread takes a contiguous run of them
  const int per = (nseg + kSelThreads - 1) / kSelThreads;
  const int s0 = min(nseg, tid * per), s1 = min(nseg, s0 + per);
  int my_gt = 0, my_eq = 0;
  for (int s = s0; s < s1; ++s) {
    my_gt += s_seg_gt[s];
    my_eq += s_seg_eq[s];
  }
  int gt_run = sel_scan(my_gt, s_wave, &s_total);
  int eq_run = sel_scan(my_eq, s_wave, &s_total);
  for (int s = s0; s < s1; ++s) {
    const int g_ = s_seg_gt[s], e_ = s_seg_eq[s];
    s_seg_gt[s] = gt_run + min(eq_run, take_eq);  // output offset of the segment
    s_seg_eq[s] = eq_run;                          // ties before the segment
    gt_run += g_;
    eq_run += e_;
  }
  __syncthreads();
  for (int s0b = wave; s0b < nseg; s0b += kSelBatch * kSelWaves) {
    f32x4 v[kSelBatch];
#pragma unroll
    for (int u = 0; u < kSelBatch; ++u) v[u] = load4(256 * (s0b + u * kSelWaves) + 4 * lane);
#pragma unroll
    for (int u = 0; u < kSelBatch; ++u) {
      const int s = s0b + u * kSelWaves;
      if (s >= nseg) break;  // the same in every lane
      const int t = 256 * s + 4 * lane;
      bool gt[4], eq[4], sel[4];
      flags(v[u], t, gt, eq);
      int er[4], sr[4], dummy;
      seg_ranks(eq, lane, er, &dummy);
#pragma unroll
      for (int c = 0; c < 4; ++c) sel[c] = gt[c] || (eq[c] && s_seg_eq[s] + er[c] < take_eq);
      seg_ranks(sel, lane, sr, &dummy);
#pragma unroll
      for (int c = 0; c < 4; ++c)
        if (sel[c]) out[s_seg_gt[s] + sr[c]] = t + c;
    }
  }
}

}  // namespace

hipError_t launch_topk(const TopkArgs& a, hipStream_t stream) {
  const int pairs = a.B * a.Hkv;
  if (a.S > 0) {  // with no rows every selection is empty: only the counts are written
    if (a.Hkv <= kRowMaxHkv) {
      const int per_block = 4 * kRowSteps * kTile;
      const dim3 rgrid((unsigned)((a.S * a.Hkv + per_block - 1) / per_block), (unsigned)a.B);
      const unsigned lds = (unsigned)(a.Hkv * kHeadDim * sizeof(float));
      if (a.dtype == KIND_F16) launch_timed(topk_score_rows_kernel<KIND_F16>, rgrid, dim3(256), lds, stream, a);
      else launch_timed(topk_score_rows_kernel<KIND_BF16>, rgrid, dim3(256), lds, stream, a);
    } else {
      const dim3 sgrid((unsigned)((a.S + 4 * kTile - 1) / (4 * kTile)), (unsigned)pairs);
      if (a.dtype == KIND_F16) launch_timed(topk_score_kernel<KIND_F16>, sgrid, dim3(256), 0u, stream, a);
      else launch_timed(topk_score_kernel<KIND_BF16>, sgrid, dim3(256), 0u, stream, a);
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  launch_timed(topk_select_kernel, dim3((unsigned)pairs), dim3(kSelThreads), 0u, stream, a);
  return hipGetLastError();
}

}  // namespace kvdec

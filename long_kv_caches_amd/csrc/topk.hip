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
//   topk_radix_kernel<0..2> -- a radix select of the k-th largest orderable
//     key in three digits of 11, 11 and 10 bits, one 1024-thread workgroup per
//     16K-token chunk of a pair: an LDS histogram of the chunk's keys that match
//     the prefix so far, added to the pair's merged histogram with atomics; the
//     next kernel's first wave picks the digit from it.  The low pass also keeps
//     each chunk's own histogram and its keys above the 22-bit prefix.
//   topk_final_kernel -- per pair: the threshold key T, the count of keys equal
//     to it to keep, and each chunk's keys above and equal to T before it.
//   topk_write_kernel -- the ordered compaction of each chunk: per 256-token
//     segment (lane l: tokens 4l .. 4l+3) ballots count the keys above the
//     threshold and those equal to it, a scan over the chunk's segments gives
//     each its output offset and its ties before it, and the selected indices
//     are written in order.  Every pass reads the chunk's scores with 16-byte
//     loads, 16 keys per thread.
// No workgroup waits for another: each read of other workgroups' counts is in
// a later kernel.
#include "device_common.h"
#include "internal.h"

namespace kvdec {
namespace {

constexpr int kSelThreads = 1024;
constexpr int kSelWaves = kSelThreads / 64;
constexpr int kSelSegs = kSelChunk / 256;  // 256-token segments per chunk: one per lane of a wave
static_assert(kSelSegs == 64 && kSelChunk == 4 * 4 * kSelThreads, "a thread holds 16 keys of its chunk");
static_assert(kTopkMaxLen / kSelChunk <= kSelWaves, "one wave per chunk when the last pass splits counts");
constexpr int kRowSteps = 4;      // 16-segment steps each wave of the whole-row score kernel takes
                                  // (measured on MI355X, batch 8 x 128K: the whole selection 3.6-4.2 us
                                  // shorter than with 16 steps, 4.5 / 14.5 us longer with 32 / 64)
constexpr int kRowMaxHkv = 64;    // KV heads whose query sums the whole-row kernel keeps in LDS

// A pair's slice of the selection workspace (after the score rows).  The
// merged histograms are atomic targets; each kernel reads what the previous
// ones left (a kernel boundary between every write and read of another
// workgroup's data).
struct SelPair {
  uint32_t* h0;      // [2048] keys per top digit (bits 21..31)
  uint32_t* h1;      // [2048] per middle digit (bits 10..20), keys under the chosen top digit
  uint32_t* h2;      // [1024] per low digit (bits 0..9), keys under the chosen 22-bit prefix
  uint32_t* state;   // [8]: after the middle pass prefix, mask, remaining, then T; after the
                     // low pass prefix, mask, remaining, then the keys equal to T to keep
  uint32_t* chunks;  // [chunks, 1028]: each chunk's low-digit histogram, its keys above the
                     // 22-bit prefix, then the keys above T and equal to T before the chunk
};

__device__ __forceinline__ SelPair sel_pair(const TopkArgs& a, int pair) {
  uint32_t* base = a.sel + (size_t)pair * topk_sel_words(a.C);
  return {base, base + 2048, base + 4096, base + 5120, base + 5128};
}

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
  // the selection's top-digit histogram of this pair starts at zero
  for (int w = blockIdx.x * 256 + threadIdx.x; w < 2048; w += gridDim.x * 256) sel_pair(a, pair).h0[w] = 0;
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
  // the selection's top-digit histograms of this sequence's pairs start at zero
  for (int w = blockIdx.x * 256 + tid; w < Hkv * 2048; w += gridDim.x * 256)
    sel_pair(a, b * Hkv + (w >> 11)).h0[w & 2047] = 0;
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

__device__ __forceinline__ uint32_t wave_sum_u32(uint32_t x) {
#pragma unroll
  for (int d = 32; d > 0; d >>= 1) x += __shfl_xor(x, d, 64);
  return x;
}

// This thread's 16 keys of chunk c: segment wave + 16 u (256 tokens each) of
// the chunk, tokens 4 lane .. 4 lane + 3 of it.  Reads past the row's valid
// 16-byte groups return zeros; tokens at or past len are masked by the caller.
__device__ __forceinline__ void load_chunk(const TopkArgs& a, int pair, int len, int c, int wave, int lane,
                                           f32x4 (&v)[4]) {
  const __amdgpu_buffer_rsrc_t rs = make_rsrc(uniform_ptr(a.scores + (int64_t)pair * a.S4),
                                              uniform_u32((uint32_t)((len + 3) & ~3) * 4u));
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int t = c * kSelChunk + 256 * (wave + kSelWaves * u) + 4 * lane;
    v[u] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, 4 * t, 0, 0));
  }
}

// The digit of a merged histogram (nbins bins, h 16-byte aligned) that holds
// the remaining-th largest key: *digit, and in *rem the rank of that key among
// the keys of the digit.  Run by one whole wave; lane l reads the bins
// [nbins - per (l + 1), nbins - per l), counted from the top.
template <int NBINS>
__device__ __forceinline__ void find_digit(const uint32_t* h, uint32_t remaining, int lane, uint32_t* digit,
                                           uint32_t* rem) {
  constexpr int per = NBINS / 64;
  const int first = NBINS - per * (lane + 1);
  uint32_t cnt[per];
#pragma unroll
  for (int i = 0; i < per; i += 4) {
    const u32x4 x = load_b128(h + first + i);
    cnt[i] = x.x;
    cnt[i + 1] = x.y;
    cnt[i + 2] = x.z;
    cnt[i + 3] = x.w;
  }
  uint32_t total = 0;
#pragma unroll
  for (int i = 0; i < per; ++i) total += cnt[i];
  uint32_t incl = total;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const uint32_t y = __shfl_up(incl, d, 64);
    if (lane >= d) incl += y;
  }
  const uint32_t before = incl - total;  // keys in higher bins
  if (before < remaining && remaining <= incl) {
    uint32_t run = before;
    bool found = false;
#pragma unroll
    for (int i = per - 1; i >= 0; --i) {
      if (!found && run + cnt[i] >= remaining) {
        *digit = (uint32_t)(first + i);
        *rem = remaining - run;
        found = true;
      }
      run += cnt[i];
    }
  }
}

// One digit of the radix select of the need-th largest key (P = 0, 1, 2:
// bits 21..31, 10..20, 0..9), one workgroup per chunk of a pair: the prefix
// chosen so far comes from the previous passes (P = 1: the top digit from the
// merged top histogram; P = 2: the stored prefix and the middle digit), then
// the chunk's keys that match it are counted in an LDS histogram of the next
// digit, whose bins are added to the pair's merged histogram.  The low pass
// also keeps each chunk's own histogram and its count of keys above the
// 22-bit prefix for the compaction's offsets.
template <int P>
__global__ __launch_bounds__(kSelThreads) void topk_radix_kernel(TopkArgs a) {
  constexpr int shift = P == 0 ? 21 : P == 1 ? 10 : 0;
  constexpr int nbins = P == 2 ? 1024 : 2048;
  __shared__ uint32_t s_hist[kSelHist];
  __shared__ uint32_t s_sel[2];  // digit, remaining
  __shared__ uint32_t s_above;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int c = blockIdx.x, pair = blockIdx.y, b = pair / a.Hkv;
  const int len = min(max(a.seqlens ? a.seqlens[b] : a.S, 0), a.S);
  const int need = min(a.top_k, len);
  if (P == 0 && c == 0 && tid == 0) a.idx_len[pair] = need;
  if (need == 0) return;
  if (need == len) {  // everything is kept: each chunk writes its own tokens
    if (P == 0) {
      int32_t* out = a.idx + (int64_t)pair * a.top_k;
      for (int t = c * kSelChunk + tid; t < min(len, (c + 1) * kSelChunk); t += kSelThreads) out[t] = t;
    }
    return;
  }
  const int nchunks = (len + kSelChunk - 1) / kSelChunk;
  if (c >= nchunks) return;
  const SelPair sp = sel_pair(a, pair);
  f32x4 v[4];
  load_chunk(a, pair, len, c, wave, lane, v);  // in flight while the prefix is found
  uint32_t prefix = 0, mask = 0;
  if (P == 0) {
    if (c == 0)  // the later passes' merged histograms start at zero
      for (int i = tid; i < 2048 + 1024; i += kSelThreads) sp.h1[i] = 0;
  } else {
    if (wave == 0) {
      if (P == 1) find_digit<2048>(sp.h0, (uint32_t)need, lane, &s_sel[0], &s_sel[1]);
      else find_digit<2048>(sp.h1, sp.state[2], lane, &s_sel[0], &s_sel[1]);
    }
    if (P == 2) {
      prefix = sp.state[0];
      mask = sp.state[1];
    }
  }
  for (int i = tid; i < nbins; i += kSelThreads) s_hist[i] = 0;
  if (tid == 0) s_above = 0;
  __syncthreads();
  if (P > 0) {  // the digit just found extends the prefix
    constexpr int pshift = P == 1 ? 21 : 10;
    prefix |= s_sel[0] << pshift;
    mask |= 2047u << pshift;
    if (c == 0 && tid == 0) {
      uint32_t* st = sp.state + 4 * (P - 1);
      st[0] = prefix;
      st[1] = mask;
      st[2] = s_sel[1];
    }
  }
  uint32_t above = 0;
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int t = c * kSelChunk + 256 * (wave + kSelWaves * u) + 4 * lane;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const uint32_t k = order_key(v[u][e]);
      if (t + e < len) {
        if ((k & mask) == prefix) atomicAdd(&s_hist[(k >> shift) & (nbins - 1)], 1u);
        else if (P == 2 && (k & mask) > prefix) ++above;
      }
    }
  }
  if (P == 2) {
    above = wave_sum_u32(above);
    if (lane == 0 && above) atomicAdd(&s_above, above);
  }
  __syncthreads();
  uint32_t* merged = P == 0 ? sp.h0 : P == 1 ? sp.h1 : sp.h2;
  for (int i = tid; i < nbins; i += kSelThreads) {
    const uint32_t n = s_hist[i];
    if (n) atomicAdd(&merged[i], n);
    if (P == 2) sp.chunks[c * 1028 + i] = n;
  }
  if (P == 2 && tid == 0) sp.chunks[c * 1028 + 1024] = s_above;
}

// The threshold of a pair, after the three digit passes: its low digit from
// the merged low histogram gives T, the need-th largest key, and the count of
// keys equal to T to keep; the chunks' own low histograms give each chunk's
// keys above T and equal to T, whose exclusive sums over the chunks before it
// the compaction needs.  One workgroup per pair.
__global__ __launch_bounds__(kSelThreads) void topk_final_kernel(TopkArgs a) {
  __shared__ uint32_t s_sel[2];
  __shared__ uint32_t s_cnt[kSelWaves][2];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int pair = blockIdx.x, b = pair / a.Hkv;
  const int len = min(max(a.seqlens ? a.seqlens[b] : a.S, 0), a.S);
  const int need = min(a.top_k, len);
  if (need == 0 || need == len) return;  // written by the first pass
  const int nchunks = (len + kSelChunk - 1) / kSelChunk;
  const SelPair sp = sel_pair(a, pair);
  if (wave == 0) find_digit<1024>(sp.h2, sp.state[6], lane, &s_sel[0], &s_sel[1]);
  __syncthreads();
  const uint32_t d = s_sel[0];
  if (wave < nchunks) {  // wave w: chunk w's keys above T and equal to T
    const uint32_t* h = sp.chunks + wave * 1028;
    uint32_t gt = 0;
    for (int i = (int)d + 1 + lane; i < 1024; i += 64) gt += h[i];
    gt = wave_sum_u32(gt);
    if (lane == 0) {
      s_cnt[wave][0] = gt + h[1024];
      s_cnt[wave][1] = h[d];
    }
  }
  __syncthreads();
  if (tid == 0) {
    uint32_t gt_run = 0, eq_run = 0;
    for (int c = 0; c < nchunks; ++c) {
      sp.chunks[c * 1028 + 1025] = gt_run;
      sp.chunks[c * 1028 + 1026] = eq_run;
      gt_run += s_cnt[c][0];
      eq_run += s_cnt[c][1];
    }
    sp.state[3] = sp.state[4] | d;  // T
    sp.state[7] = s_sel[1];         // keys equal to T to keep
  }
}

// Ordered compaction of one chunk: the keys above T, and the first keys equal
// to T in token order up to the count to keep, written in ascending token
// order at the chunk's offset.  Per 256-token segment, ballots count both
// kinds; a scan over the chunk's 64 segments (one per lane of wave 0) gives
// each its output offset and its ties before it.
__global__ __launch_bounds__(kSelThreads) void topk_write_kernel(TopkArgs a) {
  __shared__ int s_seg_gt[kSelSegs], s_seg_eq[kSelSegs];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int c = blockIdx.x, pair = blockIdx.y, b = pair / a.Hkv;
  const int len = min(max(a.seqlens ? a.seqlens[b] : a.S, 0), a.S);
  const int need = min(a.top_k, len);
  if (need == 0 || need == len) return;  // written by the first pass
  const int nchunks = (len + kSelChunk - 1) / kSelChunk;
  if (c >= nchunks) return;
  const SelPair sp = sel_pair(a, pair);
  f32x4 v[4];
  load_chunk(a, pair, len, c, wave, lane, v);  // in flight while the threshold is read
  const uint32_t T = sp.state[3];          // the need-th largest key
  const int take_eq = (int)sp.state[7];     // keys equal to T to keep, lowest tokens first
  const int gt_before = (int)sp.chunks[c * 1028 + 1025];  // keys above T in the chunks before
  const int eq_before = (int)sp.chunks[c * 1028 + 1026];  // keys equal to T in the chunks before
  int32_t* out = a.idx + (int64_t)pair * a.top_k;
  bool gt[4][4], eq[4][4];
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int s = wave + kSelWaves * u;
    const int t = c * kSelChunk + 256 * s + 4 * lane;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const uint32_t k = order_key(v[u][e]);
      gt[u][e] = t + e < len && k > T;
      eq[u][e] = t + e < len && k == T;
    }
    int r[4], ngt, neq;
    seg_ranks(gt[u], lane, r, &ngt);
    seg_ranks(eq[u], lane, r, &neq);
    if (lane == 0) {
      s_seg_gt[s] = ngt;
      s_seg_eq[s] = neq;
    }
  }
  __syncthreads();
  if (wave == 0) {  // lane l: segment l
    const int g = s_seg_gt[lane], e = s_seg_eq[lane];
    int ig = g, ie = e;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
      const int yg = __shfl_up(ig, d, 64), ye = __shfl_up(ie, d, 64);
      if (lane >= d) {
        ig += yg;
        ie += ye;
      }
    }
    const int eq_run = eq_before + ie - e;
    s_seg_gt[lane] = gt_before + ig - g + min(eq_run, take_eq);  // output offset of the segment
    s_seg_eq[lane] = eq_run;                                       // ties before the segment
  }
  __syncthreads();
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int s = wave + kSelWaves * u;
    const int t = c * kSelChunk + 256 * s + 4 * lane;
    int er[4], sr[4], dummy;
    bool sel[4];
    seg_ranks(eq[u], lane, er, &dummy);
#pragma unroll
    for (int e = 0; e < 4; ++e) sel[e] = gt[u][e] || (eq[u][e] && s_seg_eq[s] + er[e] < take_eq);
    seg_ranks(sel, lane, sr, &dummy);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int pos = s_seg_gt[s] + sr[e];  // < need by construction; checked so no write leaves the row
      if (sel[e] && pos < need) out[pos] = t + e;
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
  const dim3 cgrid((unsigned)a.C, (unsigned)pairs);
  launch_timed(topk_radix_kernel<0>, cgrid, dim3(kSelThreads), 0u, stream, a);
  launch_timed(topk_radix_kernel<1>, cgrid, dim3(kSelThreads), 0u, stream, a);
  launch_timed(topk_radix_kernel<2>, cgrid, dim3(kSelThreads), 0u, stream, a);
  launch_timed(topk_final_kernel, dim3((unsigned)pairs), dim3(kSelThreads), 0u, stream, a);
  launch_timed(topk_write_kernel, cgrid, dim3(kSelThreads), 0u, stream, a);
  return hipGetLastError();
}

size_t topk_workspace_bytes(int pairs, int S) {
  const size_t S4 = (size_t)((S + 3) & ~3);
  return (size_t)pairs * (S4 * sizeof(float) + (size_t)topk_sel_words(topk_chunks(S)) * sizeof(uint32_t));
}

}  // namespace kvdec

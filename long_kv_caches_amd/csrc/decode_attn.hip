// decode_attn.hip -- split-K decode attention for gfx950 (dense, ragged, paged,
// and the CLO cache-buffer + persistent-cache hybrid).
//
// Operation: for one query token per sequence, out = softmax(scale q K^T) V
// with grouped KV heads (KVPR page, section A3, MHA equation at the decode
// step).  One request's tokens are split into independent work items whose
// partial results are aggregated afterwards (Neo page, method details: the
// Flash-Decoding style split along a request, then aggregation of partial
// outputs), and paged KV follows the page pool + block table of the same page.
//
// Work decomposition (one workgroup = 4 waves = one work item):
//   item = (sequence b, KV head g, chunk c of `chunk` tokens).
//   Each wave walks 16-token tiles c*chunk + 16*(wave + 4i) of the item and
//   keeps its own online-softmax state (running max m, sum l, output o) for
//   the G query heads of KV head g.
//   Lane l owns the 16-byte piece n = l % 16 (8 of the 128 elements) of rows
//   4*(l/16) .. 4*(l/16)+3 of a tile, so every load instruction reads four
//   whole 256-byte rows (fully coalesced) for K and for V alike.  Per tile:
//     scores  v_dot2_f32_f16 (or _bf16) partial dots of the lane's piece with
//             q, summed over the 16 pieces of a row by four DPP row steps;
//     softmax tile max across the four row groups by permlane16/32 swaps,
//             exp2 in log2 units (scores are pre-scaled by scale*log2 e);
//     P.V     the probabilities are already in the lanes that hold the V
//             rows: fp32 FMAs on the lane's 8 V elements.
//   This op is HBM-bound (4-8 flops per byte), so the score dots stay on the
//   vector ALU, where they need no operand reshuffle; no LDS is touched in
//   the loop.
//   The 4 waves merge through LDS.  A sequence covered by one item writes the
//   normalised output directly; otherwise each item writes its partial
//   (o, m, l) to the workspace and a second, small kernel merges the partials
//   of each (b, g) in chunk order (so the result does not depend on which item
//   finished first).  The kernel boundary orders the partial writes before the
//   merge reads; no grid-wide fence or atomic is needed.
#include <type_traits>

#include "device_common.h"
#include "internal.h"

namespace kvdec {
namespace {

constexpr float kLn2 = 0.69314718055994530942f;

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

struct SeqView {
  int len;
  const uint16_t* kb;  // strided sources: row of token t at kb + t * stride
  const uint16_t* vb;
  int64_t stride;
};

template <int SRC>
__device__ __forceinline__ SeqView locate(const AttnArgs& a, int b, int g) {
  SeqView s;
  s.stride = (int64_t)a.Hkv * kHeadDim;
  if constexpr (SRC == SRC_DENSE) {
    s.len = a.seqlens ? min(a.seqlens[b], a.S) : a.S;
    const int64_t base = ((int64_t)b * a.S * a.Hkv + g) * kHeadDim;
    s.kb = a.k + base;
    s.vb = a.v + base;
  } else if constexpr (SRC == SRC_RAGGED) {
    // a.S holds the number of token rows T; offsets are clamped into [0, T].
    const int start = min(max(a.cu_seqlens[b], 0), a.S);
    const int end = min(max(a.cu_seqlens[b + 1], start), a.S);
    s.len = end - start;
    const int64_t base = ((int64_t)start * a.Hkv + g) * kHeadDim;
    s.kb = a.k + base;
    s.vb = a.v + base;
  } else if constexpr (SRC == SRC_PAGED) {
    s.len = min(a.seqlens[b], a.max_pages * a.page);
    s.kb = a.k;
    s.vb = a.v;
  } else {  // SRC_HYBRID
    const int slot = __builtin_amdgcn_readfirstlane(a.head_map[g]);
    s.stride = kHeadDim;
    if (slot >= 0) {
      s.len = slot < a.P_slots ? min(a.pers_len[b], a.pers_cap) : 0;
      const int64_t base = ((int64_t)b * a.P_slots + slot) * a.pers_cap * kHeadDim;
      s.kb = a.k + base;
      s.vb = a.v + base;
    } else {
      s.len = min(a.buf_len[b * a.Hkv + g], a.buf_cap);
      const int64_t base = ((int64_t)b * a.Hkv + g) * a.buf_cap * kHeadDim;
      s.kb = a.k2 + base;
      s.vb = a.v2 + base;
    }
  }
  // Values loaded from memory are the same for the whole workgroup; say so,
  // so that buffer descriptors built from them stay in scalar registers.
  s.len = __builtin_amdgcn_readfirstlane(max(0, min(s.len, a.n_chunks * a.chunk)));
  return s;
}

template <int KIND, int G, int SRC>
__global__ __launch_bounds__(256) void decode_attn_kernel(AttnArgs a) {
  static_assert(G >= 1 && G <= kMaxGroup, "group size");
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform per wave
  const int n = lane & 15, lg = lane >> 4;

  int bid = blockIdx.x;
  const int g = bid % a.Hkv;
  bid /= a.Hkv;
  const int c = bid % a.n_chunks;
  const int b = bid / a.n_chunks;

  const SeqView sq = locate<SRC>(a, b, g);
  const int len = sq.len;
  const int n_c = (len + a.chunk - 1) / a.chunk;
  const int64_t head0 = (int64_t)b * a.Hq + (int64_t)g * G;  // first query head row

  if (len == 0) {
    if (c == 0) {
      for (int idx = tid; idx < G * kHeadDim; idx += 256) {
        a.out[(head0 + (idx >> 7)) * kHeadDim + (idx & 127)] = 0;
        if ((idx & 127) == 0 && a.lse) a.lse[head0 + (idx >> 7)] = -INFINITY;
      }
    }
    return;
  }
  if (c >= n_c) return;

  // q piece n of each query head of the group (8 elements, 4 packed words).
  u32x4 qf[G];
#pragma unroll
  for (int j = 0; j < G; ++j) qf[j] = load_b128(a.q + (head0 + j) * kHeadDim + 8 * n);

  const int t_lo = c * a.chunk;
  const int t_hi = min(len, t_lo + a.chunk);
  const int n_tiles = (t_hi - t_lo + kTile - 1) / kTile;

  // K/V rows of one 16-token tile come through buffer resources whose base is
  // the tile's first row (scalar registers) and whose size covers only the
  // rows below len: rows past the end of the sequence, and whole tiles past
  // the wave's last one, read as zeros with no memory traffic.  Per-lane
  // offsets are the same for every tile.
  const uint32_t row_bytes = (SRC == SRC_PAGED) ? kHeadDim * 2 : (uint32_t)(sq.stride * 2);
  uint32_t row_off[4];  // this lane's rows 4*lg + i, piece n
#pragma unroll
  for (int i = 0; i < 4; ++i) row_off[i] = (4 * lg + i) * row_bytes + 16 * n;

  auto load_tile = [&](int kt, u32x4 (&kf)[4], u32x4 (&vf)[4]) {
    const int t0 = t_lo + kTile * kt;
    const int rows = kt < n_tiles ? min(len - t0, kTile) : 0;
    int64_t row0;  // element offset of the tile's first row
    if constexpr (SRC == SRC_PAGED) {
      int pg = kt < n_tiles ? a.block_table[(int64_t)b * a.max_pages + t0 / a.page] : 0;
      pg = __builtin_amdgcn_readfirstlane(min(max(pg, 0), a.S - 1));  // a.S: pages in the pool
      row0 = (((int64_t)pg * a.Hkv + g) * a.page + t0 % a.page) * kHeadDim;  // tiles never straddle pages
    } else {
      row0 = (int64_t)t0 * sq.stride;
    }
    const uint32_t nbytes = uniform_u32(rows > 0 ? (uint32_t)rows * row_bytes : 0u);
    const __amdgpu_buffer_rsrc_t rk = make_rsrc(uniform_ptr(sq.kb + row0), nbytes);
    const __amdgpu_buffer_rsrc_t rv = make_rsrc(uniform_ptr(sq.vb + row0), nbytes);
#pragma unroll
    for (int i = 0; i < 4; ++i) kf[i] = buffer_load_b128_nt(rk, row_off[i]);
#pragma unroll
    for (int i = 0; i < 4; ++i) vf[i] = buffer_load_b128_nt(rv, row_off[i]);
  };

  // Online-softmax state; every lane holds the same m and l (per head).
  float m_run[G], l_run[G], o[G][8];
#pragma unroll
  for (int j = 0; j < G; ++j) {
    m_run[j] = -INFINITY;
    l_run[j] = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) o[j][e] = 0.f;
  }

  // One 16-token tile: scores, online softmax, P.V accumulation.
  auto process = [&](const u32x4 (&kf)[4], const u32x4 (&vf)[4], int kt) {
    const int t0 = t_lo + kTile * kt;
    float sc[4][G];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const bool valid = t0 + 4 * lg + i < len;
#pragma unroll
      for (int j = 0; j < G; ++j) {
        float part = 0.f;
#pragma unroll
        for (int e = 0; e < 4; ++e) part = dot2<KIND>(kf[i][e], qf[j][e], part);
        const float full = row_sum16(part);
        sc[i][j] = valid ? full * a.scale_log2 : -INFINITY;
      }
    }
    bool grew = false;
    float alpha[G];
#pragma unroll
    for (int j = 0; j < G; ++j) {
      float tmax = fmaxf(fmaxf(sc[0][j], sc[1][j]), fmaxf(sc[2][j], sc[3][j]));
      tmax = rowgroup_max(tmax);
      const float m_new = fmaxf(m_run[j], tmax);  // finite: every tile has a valid token
      alpha[j] = fast_exp2(m_run[j] - m_new);
      grew |= m_new > m_run[j];
      m_run[j] = m_new;
    }
    float p[4][G];
#pragma unroll
    for (int j = 0; j < G; ++j) {
#pragma unroll
      for (int i = 0; i < 4; ++i) p[i][j] = fast_exp2(sc[i][j] - m_run[j]);
      l_run[j] = l_run[j] * alpha[j] + ((p[0][j] + p[1][j]) + (p[2][j] + p[3][j]));
    }
    if (__builtin_amdgcn_readfirstlane((int)grew)) {  // the same in every lane
#pragma unroll
      for (int j = 0; j < G; ++j)
#pragma unroll
        for (int e = 0; e < 8; ++e) o[j][e] *= alpha[j];
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float vv[8];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        vv[2 * e] = lo_f32<KIND>(vf[i][e]);
        vv[2 * e + 1] = hi_f32<KIND>(vf[i][e]);
      }
#pragma unroll
      for (int j = 0; j < G; ++j)
#pragma unroll
        for (int e = 0; e < 8; ++e) o[j][e] = __builtin_fmaf(p[i][j], vv[e], o[j][e]);
    }
  };

  // Two register buffers in ping-pong: the next tile's loads are in flight
  // while the current one is processed.  Loads are unconditional (a tile past
  // the wave's last one reads nothing), so no branch or register copy forces
  // an early wait.
  if (wave < n_tiles) {
    u32x4 ka[4], va[4], kb[4], vb[4];
    load_tile(wave, ka, va);
    for (int kt = wave;; kt += 2 * kWaves) {
      load_tile(kt + kWaves, kb, vb);
      process(ka, va, kt);
      if (kt + kWaves >= n_tiles) break;
      load_tile(kt + 2 * kWaves, ka, va);
      process(kb, vb, kt + kWaves);
      if (kt + 2 * kWaves >= n_tiles) break;
    }
  }

  // Sum the four row groups (they hold different rows of the same pieces).
#pragma unroll
  for (int j = 0; j < G; ++j) {
    l_run[j] = rowgroup_sum(l_run[j]);
#pragma unroll
    for (int e = 0; e < 8; ++e) o[j][e] = rowgroup_sum(o[j][e]);
  }

  // Merge the four waves through LDS.
  __shared__ float sm_o[kWaves][G][kHeadDim];
  __shared__ float sm_m[kWaves][G], sm_l[kWaves][G];
  if (lg == 0) {
#pragma unroll
    for (int j = 0; j < G; ++j)
#pragma unroll
      for (int e = 0; e < 8; ++e) sm_o[wave][j][8 * n + e] = o[j][e];
  }
  if (lane == 0) {
#pragma unroll
    for (int j = 0; j < G; ++j) {
      sm_m[wave][j] = m_run[j];
      sm_l[wave][j] = l_run[j];
    }
  }
  __syncthreads();

  const int64_t item = ((int64_t)b * a.Hkv + g) * a.n_chunks + c;
  for (int idx = tid; idx < G * kHeadDim; idx += 256) {
    const int j = idx >> 7, d = idx & 127;
    float M = sm_m[0][j];
#pragma unroll
    for (int w = 1; w < kWaves; ++w) M = fmaxf(M, sm_m[w][j]);
    float num = 0.f, den = 0.f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      const float wt = fast_exp2(sm_m[w][j] - M);
      num = __builtin_fmaf(wt, sm_o[w][j][d], num);
      den = __builtin_fmaf(wt, sm_l[w][j], den);
    }
    if (n_c == 1) {
      a.out[(head0 + j) * kHeadDim + d] = to_bits<KIND>(num / den);
      if (d == 0 && a.lse) a.lse[head0 + j] = (M + __builtin_log2f(den)) * kLn2;
    } else {
      a.ws_o[(item * G + j) * kHeadDim + d] = num;
      if (d == 0) {
        a.ws_ml[(item * G + j) * 2] = M;
        a.ws_ml[(item * G + j) * 2 + 1] = den;
      }
    }
  }
  if (n_c == 1) return;
}

// Merges the partials of one (sequence, KV head) pair: out = sum_c w_c o_c /
// sum_c w_c l_c with w_c = 2^(m_c - M), M = max_c m_c, chunks in order.
template <int KIND, int G, int SRC>
__global__ __launch_bounds__(256) void decode_merge_kernel(AttnArgs a) {
  __shared__ float s_w[kMaxChunks * G];  // m_c, then the weights 2^(m_c - M)
  __shared__ float s_l[kMaxChunks * G];
  __shared__ float s_M[G], s_L[G];
  const int tid = threadIdx.x;
  const int g = blockIdx.x % a.Hkv, b = blockIdx.x / a.Hkv;
  const int len = locate<SRC>(a, b, g).len;
  const int n_c = (len + a.chunk - 1) / a.chunk;
  if (n_c <= 1) return;  // written by the split kernel
  const int64_t item0 = ((int64_t)b * a.Hkv + g) * a.n_chunks;
  const int64_t head0 = (int64_t)b * a.Hq + (int64_t)g * G;

  for (int i = tid; i < n_c * G; i += 256) {
    s_w[i] = a.ws_ml[(item0 * G + i) * 2];
    s_l[i] = a.ws_ml[(item0 * G + i) * 2 + 1];
  }
  __syncthreads();
  if (tid < G) {
    float M = -INFINITY;
    for (int c = 0; c < n_c; ++c) M = fmaxf(M, s_w[c * G + tid]);
    s_M[tid] = M;
  }
  __syncthreads();
  for (int i = tid; i < n_c * G; i += 256) s_w[i] = fast_exp2(s_w[i] - s_M[i % G]);
  __syncthreads();
  if (tid < G) {
    float L = 0.f;
    for (int c = 0; c < n_c; ++c) L = __builtin_fmaf(s_w[c * G + tid], s_l[c * G + tid], L);
    s_L[tid] = L;
  }
  __syncthreads();
  for (int idx = tid; idx < G * kHeadDim; idx += 256) {
    const int j = idx >> 7, d = idx & 127;
    const float* po = a.ws_o + (item0 * G + j) * kHeadDim + d;
    float num = 0.f;
#pragma unroll 8
    for (int c = 0; c < n_c; ++c) num = __builtin_fmaf(s_w[c * G + j], po[(int64_t)c * G * kHeadDim], num);
    a.out[(head0 + j) * kHeadDim + d] = to_bits<KIND>(num / s_L[j]);
    if (d == 0 && a.lse) a.lse[head0 + j] = (s_M[j] + __builtin_log2f(s_L[j])) * kLn2;
  }
}

template <int KIND, int G, int SRC>
hipError_t launch_src(const AttnArgs& a, hipStream_t stream) {
  const dim3 grid((unsigned)((int64_t)a.B * a.n_chunks * a.Hkv)), block(256);
  decode_attn_kernel<KIND, G, SRC><<<grid, block, 0, stream>>>(a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || a.n_chunks <= 1) return e;
  decode_merge_kernel<KIND, G, SRC><<<dim3((unsigned)(a.B * a.Hkv)), block, 0, stream>>>(a);
  return hipGetLastError();
}

template <int KIND, int G>
hipError_t launch_g(const AttnArgs& a, hipStream_t stream) {
  switch (a.src) {
    case SRC_DENSE: return launch_src<KIND, G, SRC_DENSE>(a, stream);
    case SRC_RAGGED: return launch_src<KIND, G, SRC_RAGGED>(a, stream);
    case SRC_PAGED: return launch_src<KIND, G, SRC_PAGED>(a, stream);
    default: return launch_src<KIND, G, SRC_HYBRID>(a, stream);
  }
}

template <int KIND>
hipError_t launch_kind(const AttnArgs& a, hipStream_t stream) {
  switch (a.G) {
    case 1: return launch_g<KIND, 1>(a, stream);
    case 2: return launch_g<KIND, 2>(a, stream);
    case 3: return launch_g<KIND, 3>(a, stream);
    case 4: return launch_g<KIND, 4>(a, stream);
    case 5: return launch_g<KIND, 5>(a, stream);
    case 6: return launch_g<KIND, 6>(a, stream);
    case 7: return launch_g<KIND, 7>(a, stream);
    case 8: return launch_g<KIND, 8>(a, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

size_t attn_workspace_bytes(int64_t items, int G) {
  auto up = [](size_t x) { return (x + 255) & ~size_t(255); };
  return up((size_t)items * G * kHeadDim * 4) + up((size_t)items * G * 2 * 4);
}

bool attn_workspace_carve(void* ws, size_t ws_bytes, int64_t items, int G, AttnArgs* a) {
  auto up = [](size_t x) { return (x + 255) & ~size_t(255); };
  if (ws_bytes < attn_workspace_bytes(items, G) || ws == nullptr) return false;
  char* p = static_cast<char*>(ws);
  a->ws_o = reinterpret_cast<float*>(p);
  a->ws_ml = reinterpret_cast<float*>(p + up((size_t)items * G * kHeadDim * 4));
  return true;
}

hipError_t launch_decode_attn(const AttnArgs& a, hipStream_t stream) {
  return a.dtype == KIND_F16 ? launch_kind<KIND_F16>(a, stream) : launch_kind<KIND_BF16>(a, stream);
}

}  // namespace kvdec

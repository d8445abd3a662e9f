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
//   Per tile:
//     K tile -> registers in the MFMA A layout (lane l holds token l%16 and
//               four 16-byte pieces of its 256-byte row), Q^T in the B layout;
//               four v_mfma_f32_16x16x32 give the 16 x G score block.
//     online softmax in log2 units (scores are pre-scaled by scale*log2 e).
//     V tile -> registers (lane l holds 16 bytes of one of four tokens), the
//               probabilities reach it by a DPP row broadcast, fp32 FMAs.
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
    const int slot = a.head_map[g];
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
  s.len = max(0, min(s.len, a.n_chunks * a.chunk));
  return s;
}

template <int KIND, int G, int SRC>
__global__ __launch_bounds__(256) void decode_attn_kernel(AttnArgs a) {
  static_assert(G >= 1 && G <= kMaxGroup, "group size");
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
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

  // Q^T fragment in the MFMA B layout: column n = query head, rows = the same
  // 8-element d pieces the K fragment uses.  Heads n >= G are zero.
  u32x4 qf[4];
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    qf[s] = u32x4{0u, 0u, 0u, 0u};
    if (n < G) qf[s] = load_b128(a.q + (head0 + n) * kHeadDim + 32 * s + 8 * lg);
  }

  const int t_lo = c * a.chunk;
  const int t_hi = min(len, t_lo + a.chunk);
  const int n_tiles = (t_hi - t_lo + kTile - 1) / kTile;

  // Element offsets of the K/V rows this lane reads for the tile at t0.
  auto tile_rows = [&](int t0, int64_t& rk, int64_t (&rv)[4]) {
    const int tk = min(t0 + n, len - 1);
    if constexpr (SRC == SRC_PAGED) {
      int pg = a.block_table[(int64_t)b * a.max_pages + t0 / a.page];
      pg = min(max(pg, 0), a.S - 1);  // a.S holds the pool's page count
      const int64_t pbase = ((int64_t)pg * a.Hkv + g) * a.page;
      const int in0 = t0 % a.page;  // tiles never straddle pages
      rk = (pbase + in0 + (tk - t0)) * kHeadDim;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int tv = min(t0 + 4 * lg + i, len - 1);
        rv[i] = (pbase + in0 + (tv - t0)) * kHeadDim;
      }
    } else {
      rk = (int64_t)tk * sq.stride;
#pragma unroll
      for (int i = 0; i < 4; ++i) rv[i] = (int64_t)min(t0 + 4 * lg + i, len - 1) * sq.stride;
    }
  };
  auto load_tile = [&](int t0, u32x4 (&kf)[4], u32x4 (&vf)[4]) {
    int64_t rk, rv[4];
    tile_rows(t0, rk, rv);
#pragma unroll
    for (int s = 0; s < 4; ++s) kf[s] = load_b128<true>(sq.kb + rk + 32 * s + 8 * lg);
#pragma unroll
    for (int i = 0; i < 4; ++i) vf[i] = load_b128<true>(sq.vb + rv[i] + 8 * n);
  };

  float m_run = -INFINITY, l_run = 0.f;
  float o[G][8];
#pragma unroll
  for (int j = 0; j < G; ++j)
#pragma unroll
    for (int e = 0; e < 8; ++e) o[j][e] = 0.f;

  // One 16-token tile: MFMA scores, online softmax, P.V accumulation.
  auto process = [&](const u32x4 (&kf)[4], const u32x4 (&vf)[4], int kt) {
    // scores: acc[r] = S[token 4*lg + r][head n]
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < 4; ++s) acc = mfma16x16x32<KIND>(kf[s], qf[s], acc);

    const int t0 = t_lo + kTile * kt;
    float sc[4];
#pragma unroll
    for (int r = 0; r < 4; ++r)
      sc[r] = (t0 + 4 * lg + r < len) ? acc[r] * a.scale_log2 : -INFINITY;
    float tmax = fmaxf(fmaxf(sc[0], sc[1]), fmaxf(sc[2], sc[3]));
    tmax = fmaxf(tmax, xor_shfl(tmax, 16));
    tmax = fmaxf(tmax, xor_shfl(tmax, 32));
    const float m_new = fmaxf(m_run, tmax);  // finite: every tile has a valid token
    const float alpha = fast_exp2(m_run - m_new);
    float p[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) p[r] = fast_exp2(sc[r] - m_new);
    l_run = l_run * alpha + ((p[0] + p[1]) + (p[2] + p[3]));
    const bool grew = (n < G) && (m_new > m_run);
    m_run = m_new;

    if (__ballot(grew)) {
      static_for<0, G>([&](auto J) {
        const float aj = row_bcast<decltype(J)::value>(alpha);
#pragma unroll
        for (int e = 0; e < 8; ++e) o[J][e] *= aj;
      });
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float vv[8];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        vv[2 * e] = lo_f32<KIND>(vf[i][e]);
        vv[2 * e + 1] = hi_f32<KIND>(vf[i][e]);
      }
      static_for<0, G>([&](auto J) {
        const float pj = row_bcast<decltype(J)::value>(p[i]);
#pragma unroll
        for (int e = 0; e < 8; ++e) o[J][e] = __builtin_fmaf(pj, vv[e], o[J][e]);
      });
    }
  };

  // Two register buffers in ping-pong: the next tile's loads are in flight
  // while the current one is processed.  Prefetch addresses are clamped to the
  // wave's last tile, so loads are unconditional (no branch, no register copy
  // that would force an early wait); a clamped repeat re-reads lines just
  // fetched.
  if (wave < n_tiles) {
    const int last = wave + kWaves * ((n_tiles - 1 - wave) / kWaves);
    auto tile_t0 = [&](int kt) { return t_lo + kTile * min(kt, last); };
    u32x4 ka[4], va[4], kb[4], vb[4];
    load_tile(tile_t0(wave), ka, va);
    for (int kt = wave;; kt += 2 * kWaves) {
      load_tile(tile_t0(kt + kWaves), kb, vb);
      process(ka, va, kt);
      if (kt + kWaves > last) break;
      load_tile(tile_t0(kt + 2 * kWaves), ka, va);
      process(kb, vb, kt + kWaves);
      if (kt + 2 * kWaves > last) break;
    }
  }

  // Sum the four lane groups (they hold different tokens of the same heads).
  l_run += xor_shfl(l_run, 16);
  l_run += xor_shfl(l_run, 32);
#pragma unroll
  for (int j = 0; j < G; ++j)
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      o[j][e] += xor_shfl(o[j][e], 16);
      o[j][e] += xor_shfl(o[j][e], 32);
    }

  // Merge the four waves through LDS.
  __shared__ float sm_o[kWaves][G][kHeadDim];
  __shared__ float sm_m[kWaves][G], sm_l[kWaves][G];
  if (lg == 0) {
#pragma unroll
    for (int j = 0; j < G; ++j)
#pragma unroll
      for (int e = 0; e < 8; ++e) sm_o[wave][j][8 * n + e] = o[j][e];
    if (n < G) {
      sm_m[wave][n] = m_run;
      sm_l[wave][n] = l_run;
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

// decode_attn.hip -- split-K decode attention for gfx950 (dense, ragged, paged,
// and the CLO cache-buffer + persistent-cache hybrid).
//
// Operation: for one query token per sequence, out = softmax(scale q K^T) V
// with grouped KV heads (KVPR page, section A3, MHA equation at the decode
// step).  One request's tokens are split into independent pieces whose
// partial results are aggregated afterwards (Neo page, method details: the
// Flash-Decoding style split along a request, then aggregation of partial
// outputs), and paged KV follows the page pool + block table of the same page.
//
// The unit of work is a 16-token tile of one (sequence b, KV head g) pair.  A
// wave streams a run of tiles of one pair and keeps an online-softmax state
// (running max m, sum l, output o) for the G query heads of KV head g.
// Lane l owns the 16-byte piece n = l % 16 (8 of the 128 elements) of rows
// 4*(l/16) .. 4*(l/16)+3 of a tile, so every load instruction reads four whole
// 256-byte rows (fully coalesced) for K and for V alike.  Two register buffers
// alternate so the next tile's loads are in flight while the current one is
// processed.  This op is HBM-bound (4-8 flops per byte); two tile paths
// process a loaded tile:
//   VecPath (G <= 2): scores by v_dot2_f32_f16 (or _bf16) partial dots of the
//     lane's piece with q, summed over the 16 pieces of a row by four DPP row
//     steps; the tile max across the four row groups by permlane16/32 swaps;
//     exp2 in log2 units (scores are pre-scaled by scale * log2 e); P.V as
//     fp32 FMAs on the lane's 8 V elements, which sit in the lanes that hold
//     the probabilities.  No LDS in the tile loop.
//   MfmaPath (G >= 3): K passes through a small per-wave LDS slice into the
//     layout of the score MFMA; P.V runs on MFMAs too (below).  From G = 3 the
//     VALU path's per-tile work (G dots and 8G FMAs per row) costs time.
//
// Two schedules distribute the tiles:
//   balanced (default) -- a persistent grid of CUs x occupancy workgroups.
//     The tile line (one KV head of every sequence) is cut into columns;
//     column k is run for every head h by one wave each, so waves that run
//     together read all heads of the same token rows.  On a full grid a
//     column's waves share one XCD, and columns on the slower odd XCDs get
//     fewer tiles (column_of, item_line).  A wave streams its
//     column as one sequence of tiles (the next tile's loads are issued
//     across pair boundaries) and writes one partial per pair it touches, or
//     the final output when it covers a whole pair.  Its priority steps down
//     as its share gets done, which keeps the waves of a CU in step.
//   fixed chunks (split_tokens > 0) -- one workgroup per (b, g, chunk of
//     split_tokens tokens); its four waves interleave the chunk's tiles and
//     merge through LDS.  The partition then depends only on each sequence's
//     own length.
// In both, a second small kernel merges the partials of each pair in a fixed
// order (so results do not depend on timing); the kernel boundary orders the
// partial writes before the merge reads, with no grid-wide fence or atomic.
//
// K and V may also be e4m3 codes, one byte per element, each tensor with one
// scale (the CLO page's open question on FP8 KV caches).  The lane layout is
// the same, a lane's piece of a row is then 8 bytes, and a tile is half the
// bytes.  K codes are widened exactly to the query's 16-bit type for the
// scores (k_scale is folded into the score scale), V codes to fp32 for the
// VALU path's FMAs or to fp16 for the matrix-core P.V (v_scale is applied with
// the final normalisation).
#include <atomic>
#include <type_traits>

#include "device_common.h"
#include "internal.h"

namespace kvdec {
namespace {

constexpr float kLn2 = 0.69314718055994530942f;

// Attention kinds: bit 0 is the 16-bit type of q and out (KIND_F16 or
// KIND_BF16); bit 1 is set when K and V are e4m3 codes.
constexpr int KIND_KV8 = 2;
template <int KIND>
constexpr int kQKind = KIND & 1;
template <int KIND>
constexpr bool kKv8 = (KIND & KIND_KV8) != 0;
template <int KIND>
constexpr int kKvBytes = kKv8<KIND> ? 1 : 2;  // bytes per K/V element
// A lane's piece of one K or V row: 8 elements.
template <int KIND>
using KvPiece = std::conditional_t<kKv8<KIND>, u32x2, u32x4>;

// The matrix-core tile path (below) takes K/V of every format with three or
// more query heads per KV head; one or two heads keep the VALU path, whose
// per-tile work is small there and which holds more waves per SIMD.
// (Measured on MI355X on the 16 x 16K-32K fp16 batch: 241-242 vs 250-252 us at
// G = 4, 241 vs 246 at G = 3, 246 vs 440 at G = 8.)
constexpr int kMfmaMinG = 3;
template <int KIND, int G>
constexpr bool kUsesMfma = G >= kMfmaMinG;

// Address of K/V element `elems` of a tensor starting at base.
template <int KIND>
__device__ __forceinline__ const char* kv_at(const void* base, int64_t elems) {
  return static_cast<const char*>(base) + elems * kKvBytes<KIND>;
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

struct SeqView {
  int len;
  const char* kb;  // row of token t of the pair starts at kb (+ t rows)
  const char* vb;
};

// Length of pair (b, g), per thread (no uniformity assumed).
template <int SRC>
__device__ __forceinline__ int pair_len(const AttnArgs& a, int b, int g) {
  int len;
  if constexpr (SRC == SRC_DENSE) {
    len = a.seqlens ? min(a.seqlens[b], a.S) : a.S;
  } else if constexpr (SRC == SRC_RAGGED) {
    // a.S holds the number of token rows T; offsets are clamped into [0, T].
    const int start = min(max(a.cu_seqlens[b], 0), a.S);
    len = min(max(a.cu_seqlens[b + 1], start), a.S) - start;
  } else if constexpr (SRC == SRC_PAGED) {
    len = min(a.seqlens[b], a.max_pages * a.page);
  } else if constexpr (SRC == SRC_GATHER) {
    len = min(a.idx_len[b * a.Hkv + g], a.max_k);
  } else {  // SRC_HYBRID
    const int slot = a.head_map[g];
    if (slot >= 0) len = slot < a.P_slots ? min(a.pers_len[b], a.pers_cap) : 0;
    else len = min(a.buf_len[b * a.Hkv + g], a.buf_cap);
  }
  return max(0, min(len, a.max_len));
}

// Rows of pair (b, g), for a wave that handles this pair.
template <int KIND, int SRC>
__device__ __forceinline__ SeqView locate(const AttnArgs& a, int b, int g) {
  SeqView s;
  // Values loaded from memory are the same for the whole wave; say so, so
  // that buffer descriptors built from them stay in scalar registers.
  s.len = __builtin_amdgcn_readfirstlane(pair_len<SRC>(a, b, g));
  if constexpr (SRC == SRC_DENSE || SRC == SRC_GATHER) {
    const int64_t base = ((int64_t)b * a.S * a.Hkv + g) * kHeadDim;
    s.kb = kv_at<KIND>(a.k, base);
    s.vb = kv_at<KIND>(a.v, base);
  } else if constexpr (SRC == SRC_RAGGED) {
    const int start = __builtin_amdgcn_readfirstlane(min(max(a.cu_seqlens[b], 0), a.S));
    const int64_t base = ((int64_t)start * a.Hkv + g) * kHeadDim;
    s.kb = kv_at<KIND>(a.k, base);
    s.vb = kv_at<KIND>(a.v, base);
  } else if constexpr (SRC == SRC_PAGED) {
    s.kb = kv_at<KIND>(a.k, 0);
    s.vb = kv_at<KIND>(a.v, 0);
  } else {  // SRC_HYBRID
    const int slot = __builtin_amdgcn_readfirstlane(a.head_map[g]);
    if (slot >= 0) {
      const int64_t base = ((int64_t)b * a.P_slots + min(slot, max(a.P_slots - 1, 0))) *
                           a.pers_cap * kHeadDim;
      s.kb = kv_at<KIND>(a.k, base);
      s.vb = kv_at<KIND>(a.v, base);
    } else {
      const int64_t base = ((int64_t)b * a.Hkv + g) * a.buf_cap * kHeadDim;
      s.kb = kv_at<KIND>(a.k2, base);
      s.vb = kv_at<KIND>(a.v2, base);
    }
  }
  return s;
}

// Online-softmax state of one wave for G query heads; every lane holds the
// same m and l, and o for its own 8-element piece (per row group until
// finish() sums the row groups).
template <int G>
struct WaveState {
  float m[G], l[G], o[G][8];
  __device__ __forceinline__ void init() {
#pragma unroll
    for (int j = 0; j < G; ++j) {
      m[j] = -INFINITY;
      l[j] = 0.f;
#pragma unroll
      for (int e = 0; e < 8; ++e) o[j][e] = 0.f;
    }
  }
  __device__ __forceinline__ void finish() {
#pragma unroll
    for (int j = 0; j < G; ++j) {
      l[j] = rowgroup_sum(l[j]);
#pragma unroll
      for (int e = 0; e < 8; ++e) o[j][e] = rowgroup_sum(o[j][e]);
    }
  }
};

// q piece n of each query head of the group (8 elements, 4 packed words).
template <int G>
__device__ __forceinline__ void load_q(const AttnArgs& a, int64_t head0, int n, u32x4 (&qf)[G]) {
#pragma unroll
  for (int j = 0; j < G; ++j) qf[j] = load_b128(a.q + (head0 + j) * kHeadDim + 8 * n);
}

// Byte offsets, within a tile, of the four rows of this lane: rows 4*lg + i,
// piece n (8 elements).
template <int KIND>
__device__ __forceinline__ void tile_row_offsets(uint32_t row_bytes, int lane, uint32_t (&row_off)[4]) {
  const int n = lane & 15, lg = lane >> 4;
#pragma unroll
  for (int i = 0; i < 4; ++i) row_off[i] = (4 * lg + i) * row_bytes + 8 * kKvBytes<KIND> * n;
}

// Bytes from one token row of a pair to the next.
template <int KIND, int SRC>
__device__ __forceinline__ uint32_t tile_row_bytes(const AttnArgs& a) {
  return (SRC == SRC_PAGED || SRC == SRC_HYBRID ? 1u : (uint32_t)a.Hkv) * kHeadDim * kKvBytes<KIND>;
}

// Gather source: token indices t0 + first .. t0 + first + count - 1 of pair
// (b, g)'s index row (count 1 or 4), those at or past `rows` read as 0.
__device__ __forceinline__ u32x4 gather_rows(const AttnArgs& a, int b, int g, int t0, int rows,
                                            int first, int count) {
  const int32_t* ix = a.idx + ((int64_t)b * a.Hkv + g) * a.max_k + t0;
  const __amdgpu_buffer_rsrc_t ri = make_rsrc(uniform_ptr(ix), uniform_u32((uint32_t)max(rows, 0) * 4u));
  if (count == 4) return __builtin_amdgcn_raw_buffer_load_b128(ri, 4 * first, 0, 0);
  return u32x4{(uint32_t)__builtin_amdgcn_raw_buffer_load_b32(ri, 4 * first, 0, 0), 0u, 0u, 0u};
}

// Byte offset of a gathered row's piece: the token index clamped into the
// cache, or an offset past the descriptor (zeros) for an invalid row.
constexpr uint32_t kOutsideRows = 0x80000000u;
__device__ __forceinline__ uint32_t gather_offset(const AttnArgs& a, uint32_t token, bool valid,
                                                  uint32_t row_bytes, uint32_t piece) {
  const int t = min(max((int)token, 0), a.S - 1);
  return valid ? (uint32_t)t * row_bytes + piece : kOutsideRows;
}

// Page of the tile whose first row is t0 of sequence b (0 when !active),
// clamped into the pool.  A scalar load: the entry is the same for the whole
// wave, and waiting for a scalar load does not wait for the K/V loads the
// wave has in flight, which waiting for a vector load would (vector loads
// complete in issue order).
__device__ __forceinline__ int tile_page(const AttnArgs& a, int b, int t0, bool active) {
  using ConstI32 = const __attribute__((address_space(4))) int32_t*;
  int pg = 0;
  if (active) pg = ((ConstI32)a.block_table)[(int64_t)b * a.max_pages + t0 / a.page];
  return uniform_i32(min(max(pg, 0), a.S - 1));  // a.S: pages in the pool
}

// Bytes of the valid rows of the tile whose first row is t0 (0 when !active
// or past the end), from wave-uniform values: scalar arithmetic, with no
// vector register taken for it while the wave's loads are in flight.
__device__ __forceinline__ uint32_t tile_bytes(int len, int t0, bool active, uint32_t row_bytes) {
  const int rem = uniform_i32(len - t0);
  if (!active || rem <= 0) return 0u;
  return (uint32_t)(rem < kTile ? rem : kTile) * row_bytes;
}

// Loads K and V of the tile whose first row is t0 of pair (b, g) into kf, vf.
// The rows come through buffer resources whose base is the tile's first row
// (scalar registers) and whose size covers only rows below len, so rows past
// the end of the sequence, and a tile with active == false, read as zeros with
// no memory traffic.
template <int KIND, int SRC>
__device__ __forceinline__ void load_kv_tile(const AttnArgs& a, int b, int g, const char* kb,
                                             const char* vb, int len, int t0, bool active,
                                             const uint32_t (&row_off)[4], KvPiece<KIND> (&kf)[4],
                                             KvPiece<KIND> (&vf)[4]) {
  const uint32_t row_bytes = tile_row_bytes<KIND, SRC>(a);
  const int rows = active ? min(len - t0, kTile) : 0;
  if constexpr (SRC == SRC_GATHER) {
    // Rows of the tile come from the pair's index row; the descriptors cover
    // the pair's whole cache (a.S rows), and a row past the tile's valid ones
    // gets an offset outside them, so it reads zeros.
    const int lane = threadIdx.x & 63, lg = lane >> 4;
    const u32x4 tix = gather_rows(a, b, g, t0, rows, 4 * lg, 4);
    const __amdgpu_buffer_rsrc_t rk = make_rsrc(kb, uniform_u32((uint32_t)a.S * row_bytes));
    const __amdgpu_buffer_rsrc_t rv = make_rsrc(vb, uniform_u32((uint32_t)a.S * row_bytes));
    uint32_t off[4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
      off[i] = gather_offset(a, tix[i], 4 * lg + i < rows, row_bytes, 8 * kKvBytes<KIND> * (lane & 15));
    if constexpr (kKv8<KIND>) {
#pragma unroll
      for (int i = 0; i < 4; ++i) kf[i] = buffer_load_b64_nt(rk, off[i]);
#pragma unroll
      for (int i = 0; i < 4; ++i) vf[i] = buffer_load_b64_nt(rv, off[i]);
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i) kf[i] = buffer_load_b128_nt(rk, off[i]);
#pragma unroll
      for (int i = 0; i < 4; ++i) vf[i] = buffer_load_b128_nt(rv, off[i]);
    }
    return;
  }
  int64_t row0;  // byte offset of the tile's first row
  if constexpr (SRC == SRC_PAGED) {
    const int pg = tile_page(a, b, t0, active);
    // never straddles pages
    row0 = (((int64_t)pg * a.Hkv + g) * a.page + t0 % a.page) * kHeadDim * kKvBytes<KIND>;
  } else {
    row0 = (int64_t)t0 * row_bytes;
  }
  const uint32_t nbytes = tile_bytes(len, t0, active, row_bytes);
  const __amdgpu_buffer_rsrc_t rk = make_rsrc(uniform_ptr(kb + row0), nbytes);
  const __amdgpu_buffer_rsrc_t rv = make_rsrc(uniform_ptr(vb + row0), nbytes);
  if constexpr (kKv8<KIND>) {
#pragma unroll
    for (int i = 0; i < 4; ++i) kf[i] = buffer_load_b64_nt(rk, row_off[i]);
#pragma unroll
    for (int i = 0; i < 4; ++i) vf[i] = buffer_load_b64_nt(rv, row_off[i]);
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i) kf[i] = buffer_load_b128_nt(rk, row_off[i]);
#pragma unroll
    for (int i = 0; i < 4; ++i) vf[i] = buffer_load_b128_nt(rv, row_off[i]);
  }
}

// The 8 K elements of a lane's piece as four packed 16-bit pairs of the
// query's type (e4m3 widens exactly to fp16 and to bf16).
template <int KIND>
__device__ __forceinline__ void k_pairs(const KvPiece<KIND>& k, uint32_t (&w)[4]) {
  if constexpr (kKv8<KIND>) {
    if constexpr (kQKind<KIND> == KIND_F16) {
      w[0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(k.x, 1.0f, false));
      w[1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(k.x, 1.0f, true));
      w[2] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(k.y, 1.0f, false));
      w[3] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(k.y, 1.0f, true));
    } else {
      w[0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(k.x, 1.0f, false));
      w[1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(k.x, 1.0f, true));
      w[2] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(k.y, 1.0f, false));
      w[3] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(k.y, 1.0f, true));
    }
  } else {
    w[0] = k.x;
    w[1] = k.y;
    w[2] = k.z;
    w[3] = k.w;
  }
}

// The 8 V elements of a lane's piece in fp32 (exact for every storage type).
template <int KIND>
__device__ __forceinline__ void v_floats(const KvPiece<KIND>& v, float (&vv)[8]) {
  if constexpr (kKv8<KIND>) {
    typedef float f2 __attribute__((ext_vector_type(2)));
    const f2 a0 = __builtin_amdgcn_cvt_pk_f32_fp8(v.x, false), a1 = __builtin_amdgcn_cvt_pk_f32_fp8(v.x, true);
    const f2 a2 = __builtin_amdgcn_cvt_pk_f32_fp8(v.y, false), a3 = __builtin_amdgcn_cvt_pk_f32_fp8(v.y, true);
    vv[0] = a0.x; vv[1] = a0.y; vv[2] = a1.x; vv[3] = a1.y;
    vv[4] = a2.x; vv[5] = a2.y; vv[6] = a3.x; vv[7] = a3.y;
  } else {
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      vv[2 * e] = lo_f32<kQKind<KIND>>(w[e]);
      vv[2 * e + 1] = hi_f32<kQKind<KIND>>(w[e]);
    }
  }
}

// Online-softmax update of st with the tile whose first row is t0 (rows at or
// past len are masked out; the tile holds at least one row below len).
template <int KIND, int G>
__device__ __forceinline__ void process_tile(const AttnArgs& a, const u32x4 (&qf)[G],
                                             const KvPiece<KIND> (&kf)[4],
                                             const KvPiece<KIND> (&vf)[4], int t0, int len, int lg,
                                             WaveState<G>& st) {
  constexpr int QK = kQKind<KIND>;
  float sc[4][G];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const bool valid = t0 + 4 * lg + i < len;
    uint32_t kw[4];
    k_pairs<KIND>(kf[i], kw);
#pragma unroll
    for (int j = 0; j < G; ++j) {
      float part = 0.f;
#pragma unroll
      for (int e = 0; e < 4; ++e) part = dot2<QK>(kw[e], qf[j][e], part);
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
    const float m_new = fmaxf(st.m[j], tmax);  // finite: every tile has a valid token
    alpha[j] = fast_exp2(st.m[j] - m_new);
    grew |= m_new > st.m[j];
    st.m[j] = m_new;
  }
  float p[4][G];
#pragma unroll
  for (int j = 0; j < G; ++j) {
#pragma unroll
    for (int i = 0; i < 4; ++i) p[i][j] = fast_exp2(sc[i][j] - st.m[j]);
    st.l[j] = st.l[j] * alpha[j] + ((p[0][j] + p[1][j]) + (p[2][j] + p[3][j]));
  }
  if (__builtin_amdgcn_readfirstlane((int)grew)) {  // the same in every lane
#pragma unroll
    for (int j = 0; j < G; ++j)
#pragma unroll
      for (int e = 0; e < 8; ++e) st.o[j][e] *= alpha[j];
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    float vv[8];
    v_floats<KIND>(vf[i], vv);
#pragma unroll
    for (int j = 0; j < G; ++j)
#pragma unroll
      for (int e = 0; e < 8; ++e) st.o[j][e] = __builtin_fmaf(p[i][j], vv[e], st.o[j][e]);
  }
}

// Final output of G heads from a finished wave state (lanes of row group 0).
template <int KIND, int G>
__device__ __forceinline__ void store_output(const AttnArgs& a, int64_t head0, const WaveState<G>& st,
                                             int lane) {
  if (lane < 16) {
#pragma unroll
    for (int j = 0; j < G; ++j) {
      const float inv = kKv8<KIND> ? a.out_scale / st.l[j] : 1.f / st.l[j];
      uint32_t w[4];
#pragma unroll
      for (int e = 0; e < 4; ++e)
        w[e] = (uint32_t)to_bits<kQKind<KIND>>(st.o[j][2 * e] * inv) |
               ((uint32_t)to_bits<kQKind<KIND>>(st.o[j][2 * e + 1] * inv) << 16);
      store_b128(a.out + (head0 + j) * kHeadDim + 8 * lane, u32x4{w[0], w[1], w[2], w[3]});
    }
  }
  if (lane == 0 && a.lse) {
#pragma unroll
    for (int j = 0; j < G; ++j) a.lse[head0 + j] = (st.m[j] + __builtin_log2f(st.l[j])) * kLn2;
  }
}

// Unnormalised partial of G heads into workspace slot `slot`.
template <int G>
__device__ __forceinline__ void store_partial(const AttnArgs& a, int64_t slot, const WaveState<G>& st,
                                              int lane) {
  if (lane < 16) {
#pragma unroll
    for (int j = 0; j < G; ++j) {
      float* dst = a.ws_o + (slot * G + j) * kHeadDim + 8 * lane;
      store_b128(dst, u32x4{__builtin_bit_cast(uint32_t, st.o[j][0]), __builtin_bit_cast(uint32_t, st.o[j][1]),
                            __builtin_bit_cast(uint32_t, st.o[j][2]), __builtin_bit_cast(uint32_t, st.o[j][3])});
      store_b128(dst + 4, u32x4{__builtin_bit_cast(uint32_t, st.o[j][4]), __builtin_bit_cast(uint32_t, st.o[j][5]),
                                __builtin_bit_cast(uint32_t, st.o[j][6]), __builtin_bit_cast(uint32_t, st.o[j][7])});
    }
  }
  if (lane == 0) {
#pragma unroll
    for (int j = 0; j < G; ++j) {
      a.ws_ml[(slot * G + j) * 2] = st.m[j];
      a.ws_ml[(slot * G + j) * 2 + 1] = st.l[j];
    }
  }
}

template <int KIND, int G>
__device__ __forceinline__ void store_empty(const AttnArgs& a, int64_t head0) {
  for (int idx = threadIdx.x; idx < G * kHeadDim; idx += 256) {
    a.out[(head0 + (idx >> 7)) * kHeadDim + (idx & 127)] = 0;
    if ((idx & 127) == 0 && a.lse) a.lse[head0 + (idx >> 7)] = -INFINITY;
  }
}

// Partial rows a merge workgroup folds at once (32 lanes per row, 4 elements
// each): more rows shorten each row's chain of loads when a few heads have many
// partials, fewer rows keep large grids of heads with few partials cheap to
// dispatch (measured on MI355X: 32768 heads of a paged batch took 74 us with
// 16 rows and 21 us with 4; 128 hybrid heads 6.9 us with 8 rows and 6.2 with 16).
__host__ __device__ constexpr int merge_rows(int heads) { return heads <= 1024 ? 16 : heads <= 8192 ? 8 : 4; }

// Merges n_p >= 1 partials of query head j of a group (slots slot0 +
// i * slot_step, i < n_p) into the final output and lse of head head0 + j:
// out = sum_i w_i o_i / sum_i w_i l_i with w_i = 2^(m_i - M), M = max_i m_i.
// Thread (c, r) of the 32 * ROWS takes elements 4c .. 4c+3 of the partials
// i = r, r + ROWS, ... in order, with a running maximum, so
// each partial is read once; the rows are then scaled to the common maximum
// and added in the order r = 0, 1, ..., so the result does not depend on timing.
template <int KIND, int G, int ROWS>
__device__ void merge_head(const AttnArgs& a, int64_t head0, int j, int64_t slot0, int slot_step,
                           int n_p) {
  __shared__ float s_m[ROWS];
  __shared__ f32x4 s_acc[ROWS][32];
  __shared__ float s_l[ROWS];
  const int tid = threadIdx.x, c = tid & 31, r = tid >> 5;
  // row r folds partials r, r + ROWS, ... with a running maximum (one
  // pass over the partials: their maxima and outputs are read together)
  float m = -INFINITY;
  float acc0 = 0.f, acc1 = 0.f, acc2 = 0.f, acc3 = 0.f, lsum = 0.f;
#pragma unroll 4
  for (int i = r; i < n_p; i += ROWS) {
    const int64_t sj = (slot0 + (int64_t)i * slot_step) * G + j;
    const float mi = a.ws_ml[sj * 2], li = a.ws_ml[sj * 2 + 1];
    const f32x4 o = *reinterpret_cast<const f32x4*>(a.ws_o + sj * kHeadDim + 4 * c);
    const float mn = fmaxf(m, mi);
    // m = -inf at first: sc = 0 (equal maxima need no scaling, -inf included)
    const float sc = m == mn ? 1.f : fast_exp2(m - mn), w = mi == mn ? 1.f : fast_exp2(mi - mn);
    acc0 = __builtin_fmaf(w, o.x, acc0 * sc);
    acc1 = __builtin_fmaf(w, o.y, acc1 * sc);
    acc2 = __builtin_fmaf(w, o.z, acc2 * sc);
    acc3 = __builtin_fmaf(w, o.w, acc3 * sc);
    lsum = __builtin_fmaf(w, li, lsum * sc);
    m = mn;
  }
  s_acc[r][c] = f32x4{acc0, acc1, acc2, acc3};
  if (c == 0) {
    s_m[r] = m;
    s_l[r] = lsum;
  }
  __syncthreads();
  if (r == 0) {
    float M = s_m[0];
#pragma unroll
    for (int rr = 1; rr < ROWS; ++rr) M = fmaxf(M, s_m[rr]);
    float o0 = 0.f, o1 = 0.f, o2 = 0.f, o3 = 0.f, L = 0.f;
#pragma unroll
    for (int rr = 0; rr < ROWS; ++rr) {
      const float sr = fast_exp2(s_m[rr] - M);  // rows with no partial: -inf, weight 0
      const f32x4 v = s_acc[rr][c];
      o0 = __builtin_fmaf(sr, v.x, o0);
      o1 = __builtin_fmaf(sr, v.y, o1);
      o2 = __builtin_fmaf(sr, v.z, o2);
      o3 = __builtin_fmaf(sr, v.w, o3);
      L = __builtin_fmaf(sr, s_l[rr], L);
    }
    constexpr int QK = kQKind<KIND>;
    const float inv = kKv8<KIND> ? a.out_scale / L : 1.f / L;
    const uint32_t w0 = (uint32_t)to_bits<QK>(o0 * inv) | ((uint32_t)to_bits<QK>(o1 * inv) << 16);
    const uint32_t w1 = (uint32_t)to_bits<QK>(o2 * inv) | ((uint32_t)to_bits<QK>(o3 * inv) << 16);
    *reinterpret_cast<uint2*>(a.out + (head0 + j) * kHeadDim + 4 * c) = make_uint2(w0, w1);
    if (c == 0 && a.lse) a.lse[head0 + j] = (M + __builtin_log2f(L)) * kLn2;
  }
}

// ---------------------------------------------------------------------------
// Tile paths.  A path is how a wave holds q, a tile and its softmax state:
//   VecPath  -- the VALU path above (lanes own row pieces of K and V);
//   MfmaPath -- matrix cores for the scores and P.V (any K/V format), below.
// Both present the same functions to the schedules.
// ---------------------------------------------------------------------------

template <int KIND, int G>
struct VecPath {
  using Q = u32x4[G];
  using State = WaveState<G>;
  struct Tile {
    KvPiece<KIND> k[4], v[4];
  };
  struct Offs {
    uint32_t row[4];
  };
  template <int SRC>
  __device__ static void offsets(const AttnArgs& a, int lane, Offs& o) {
    tile_row_offsets<KIND>(tile_row_bytes<KIND, SRC>(a), lane, o.row);
  }
  __device__ static void load_q(const AttnArgs& a, int64_t head0, int lane, Q& q) {
    kvdec::load_q<G>(a, head0, lane & 15, q);
  }
  template <int SRC>
  __device__ static void load(const AttnArgs& a, int b, int g, const char* kb, const char* vb, int len,
                              int t0, bool active, const Offs& o, Tile& t) {
    load_kv_tile<KIND, SRC>(a, b, g, kb, vb, len, t0, active, o.row, t.k, t.v);
  }
  __device__ static void process(const AttnArgs& a, const Q& q, const Tile& t, int t0, int len,
                                 int lane, State& st) {
    process_tile<KIND, G>(a, q, t.k, t.v, t0, len, lane >> 4, st);
  }
  __device__ static void store_output(const AttnArgs& a, int64_t head0, const State& st, int lane) {
    kvdec::store_output<KIND, G>(a, head0, st, lane);
  }
  __device__ static void store_partial(const AttnArgs& a, int64_t slot, const State& st, int lane) {
    kvdec::store_partial<G>(a, slot, st, lane);
  }
  // The finished state into the chunk kernel's LDS merge arrays.
  __device__ static void to_lds(const State& st, int lane, float (*so)[kHeadDim], float* sm,
                                float* sl) {
    if (lane < 16) {
#pragma unroll
      for (int j = 0; j < G; ++j)
#pragma unroll
        for (int e = 0; e < 8; ++e) so[j][8 * lane + e] = st.o[j][e];
    }
    if (lane == 0) {
#pragma unroll
      for (int j = 0; j < G; ++j) {
        sm[j] = st.m[j];
        sl[j] = st.l[j];
      }
    }
  }
};

// Matrix-core path, for every K/V format (fp16, bf16, e4m3) at 3 <= G <= 8
// query heads, padded to 16.
//   Scores: S[token][head] by four v_mfma_f32_16x16x32 (f16 or bf16, the
//   query's type): A = K (lane l: token l%16, dims 32*(l/16) .. +31 of the
//   row, widened from its 32 codes), B = q (lane l: head l%16, the same
//   dims).  The dot product only needs K and q to agree on which dim each
//   k index is, so each lane reads 32 contiguous bytes of one row.
//   Result: lane l holds head n = l%16 for tokens 4*(l/16) + i.
//   Softmax: per lane for its head's four tokens; the max across the four
//   lane groups by permlane swaps; P is rounded to fp16 once and the running
//   sum adds the rounded values, so the output stays a convex combination of
//   V rows.
//   P.V: eight v_mfma_f32_16x16x16_f16: A = P exactly as the scores left it
//   (lane l: head l%16, tokens 4*(l/16) + i), B = V (lane l: tokens
//   4*(l/16) + i, dim 8*(l%16) + c for product c): V is loaded as in the VALU
//   path (rows 4*(l/16) .. +3, 8-byte piece l%16) and its 4 x 8 codes are
//   transposed with byte permutes, then widened to fp16 (exact).
//   Output: o[c][i] is head 4*(l/16) + i, dim 8*(l%16) + c.
template <int QK>
__device__ __forceinline__ f32x4 mfma_scores(u32x4 k, u32x4 q, f32x4 c) {
  typedef _Float16 h8 __attribute__((ext_vector_type(8)));
  typedef __bf16 b8 __attribute__((ext_vector_type(8)));
  if constexpr (QK == KIND_F16)
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(h8, k), __builtin_bit_cast(h8, q), c,
                                                  0, 0, 0);
  else
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(b8, k), __builtin_bit_cast(b8, q),
                                                   c, 0, 0, 0);
}

// Two e4m3 codes (bytes 0-1, or 2-3 with hi) widened to a packed pair of the
// 16-bit type QK (exact).
template <int QK>
__device__ __forceinline__ uint32_t e4m3_pair(uint32_t w, bool hi) {
  if constexpr (QK == KIND_F16)
    return hi ? __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, true))
              : __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, false));
  else
    return hi ? __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, true))
              : __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, false));
}

struct MState {
  float m, l;    // this lane's head (lane % 16): running max (log2 units), sum of its tokens
  f32x4 o[8];    // o[c][i]: head 4*(lane/16) + i, dim 8*(lane%16) + c
  __device__ __forceinline__ void init() {
    m = -INFINITY;
    l = 0.f;
#pragma unroll
    for (int c = 0; c < 8; ++c) o[c] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  __device__ __forceinline__ void finish() { l = rowgroup_sum(l); }
};

template <int KIND, int G>
struct MfmaPath {
  static_assert(G <= 8, "matrix-core path: at most 8 heads per KV head");
  // bf16 V: P.V runs on bf16 MFMAs, and one bf16 rounding of a weight (2^-9
  // relative) would be too coarse for the output tolerance on short sequences,
  // so each weight is split into two bf16 parts, hi + lo (about 2^-17
  // relative), with two P.V MFMAs per dim block.  fp16 and e4m3 V take one
  // fp16 rounding (2^-12).
  static constexpr bool kSplitP = !kKv8<KIND> && kQKind<KIND> == KIND_BF16;
  // Registers (accumulators in 36 AGPRs): 128 VGPRs for e4m3 K/V, three
  // waves per SIMD (capping it at four spills); 160-166 for 16-bit K/V, two
  // waves per SIMD.
  using Q = u32x4[4];
  using State = MState;
  // K and V are both loaded as the VALU path loads them: lane l takes the
  // piece l % 16 (8 elements: 8 bytes of e4m3, 16 of fp16) of rows
  // 4*(l/16) + i, so each load instruction reads four whole rows.  (The score
  // MFMA wants row l % 16 in lane l: loading K that way touches 16 rows per
  // instruction, part of each, and streamed about 9-12% slower on MI355X.)  K
  // then goes through a small LDS slice of the wave to reach the MFMA layout.
  struct Tile {
    KvPiece<KIND> k[4];  // rows 4*(l/16) + i, 8 elements each
    KvPiece<KIND> v[4];
  };
  __device__ static KvPiece<KIND> load_piece(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    if constexpr (kKv8<KIND>) return buffer_load_b64_nt(r, off);
    else return buffer_load_b128_nt(r, off);
  }
  struct Offs {
    uint32_t row[4];  // this lane's pieces within a tile
  };
  template <int SRC>
  __device__ static void offsets(const AttnArgs& a, int lane, Offs& o) {
    tile_row_offsets<KIND>(tile_row_bytes<KIND, SRC>(a), lane, o.row);
  }
  __device__ static void load_q(const AttnArgs& a, int64_t head0, int lane, Q& q) {
    const int n = lane & 15;
#pragma unroll
    for (int c = 0; c < 4; ++c)
      q[c] = n < G ? load_b128(a.q + (head0 + n) * kHeadDim + 32 * (lane >> 4) + 8 * c)
                   : u32x4{0, 0, 0, 0};
  }
  template <int SRC>
  __device__ static void load(const AttnArgs& a, int b, int g, const char* kb, const char* vb, int len,
                              int t0, bool active, const Offs& o, Tile& t) {
    const uint32_t row_bytes = tile_row_bytes<KIND, SRC>(a);
    const int rows = active ? min(len - t0, kTile) : 0;
    if constexpr (SRC == SRC_GATHER) {
      const int lane = threadIdx.x & 63, n = lane & 15, grp = lane >> 4;
      const u32x4 vt = gather_rows(a, b, g, t0, rows, 4 * grp, 4);
      const __amdgpu_buffer_rsrc_t rk = make_rsrc(kb, uniform_u32((uint32_t)a.S * row_bytes));
      const __amdgpu_buffer_rsrc_t rv = make_rsrc(vb, uniform_u32((uint32_t)a.S * row_bytes));
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const uint32_t off = gather_offset(a, vt[i], 4 * grp + i < rows, row_bytes, 8 * kKvBytes<KIND> * n);
        t.k[i] = load_piece(rk, off);
        t.v[i] = load_piece(rv, off);
      }
      return;
    }
    int64_t row0;  // byte offset of the tile's first row
    if constexpr (SRC == SRC_PAGED) {
      const int pg = tile_page(a, b, t0, active);
      row0 = (((int64_t)pg * a.Hkv + g) * a.page + t0 % a.page) * kHeadDim * kKvBytes<KIND>;
    } else {
      row0 = (int64_t)t0 * row_bytes;
    }
    const uint32_t nbytes = tile_bytes(len, t0, active, row_bytes);
    const __amdgpu_buffer_rsrc_t rk = make_rsrc(uniform_ptr(kb + row0), nbytes);
    const __amdgpu_buffer_rsrc_t rv = make_rsrc(uniform_ptr(vb + row0), nbytes);
#pragma unroll
    for (int i = 0; i < 4; ++i) t.k[i] = load_piece(rk, o.row[i]);
#pragma unroll
    for (int i = 0; i < 4; ++i) t.v[i] = load_piece(rv, o.row[i]);
  }
  __device__ static void process(const AttnArgs& a, const Q& q, const Tile& t, int t0, int len,
                                 int lane, State& st) {
    constexpr int QK = kQKind<KIND>;
    const int n = lane & 15, grp = lane >> 4;
    // K through the wave's LDS slice: rows of 128 + 16 (e4m3) or 256 + 16
    // (fp16) bytes, conflict-free for the writes of whole rows and for the
    // 16-byte reads of 8 rows at one offset; lane l reads elements
    // 32*(l/16) .. +31 of row l % 16.
    constexpr int kPieceWords = 2 * kKvBytes<KIND>;                // one lane's piece
    constexpr int kRowWords = 16 * kPieceWords + 4;
    __shared__ __attribute__((aligned(16))) uint32_t s_k[kWaves][kTile * kRowWords];
    uint32_t* kl = s_k[__builtin_amdgcn_readfirstlane(threadIdx.x >> 6)];
#pragma unroll
    for (int i = 0; i < 4; ++i)
      *reinterpret_cast<KvPiece<KIND>*>(&kl[(4 * grp + i) * kRowWords + kPieceWords * n]) = t.k[i];
    constexpr int kRuns = 2 * kKvBytes<KIND>;  // 16-byte reads of a lane's 32 elements
    u32x4 kr[kRuns];
#pragma unroll
    for (int r = 0; r < kRuns; ++r) kr[r] = *reinterpret_cast<const u32x4*>(&kl[n * kRowWords + 4 * kRuns * grp + 4 * r]);
    f32x4 s = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      if constexpr (kKv8<KIND>) {
        const uint32_t w0 = kr[c >> 1][2 * (c & 1)], w1 = kr[c >> 1][2 * (c & 1) + 1];
        const u32x4 kk = {e4m3_pair<QK>(w0, false), e4m3_pair<QK>(w0, true), e4m3_pair<QK>(w1, false),
                          e4m3_pair<QK>(w1, true)};
        s = mfma_scores<QK>(kk, q[c], s);
      } else {
        s = mfma_scores<QK>(kr[c], q[c], s);  // fp16 elements 8c .. 8c+7 of the lane's run
      }
    }
    float sc[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) sc[i] = t0 + 4 * grp + i < len ? s[i] * a.scale_log2 : -INFINITY;
    const float tmax = rowgroup_max(fmaxf(fmaxf(sc[0], sc[1]), fmaxf(sc[2], sc[3])));
    const float m_new = fmaxf(st.m, tmax);  // finite: every tile has a valid token
    const float alpha = fast_exp2(st.m - m_new);
    const bool grew = n < G && m_new > st.m;
    st.m = m_new;
    typedef _Float16 h4 __attribute__((ext_vector_type(4)));
    typedef short s4 __attribute__((ext_vector_type(4)));
    h4 ph;
    s4 pb_hi, pb_lo;
    float pw[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float p = n < G ? fast_exp2(sc[i] - m_new) : 0.f;
      if constexpr (kSplitP) {
        const uint16_t hb = to_bits<KIND_BF16>(p);
        const float hf = __builtin_bit_cast(float, (uint32_t)hb << 16);
        const uint16_t lb = to_bits<KIND_BF16>(p - hf);  // p - hf is exact in fp32
        pb_hi[i] = (short)hb;
        pb_lo[i] = (short)lb;
        pw[i] = hf + __builtin_bit_cast(float, (uint32_t)lb << 16);
      } else {
        ph[i] = (_Float16)p;
        pw[i] = (float)ph[i];
      }
    }
    // the running sum adds the weights exactly as P.V uses them
    st.l = st.l * alpha + ((pw[0] + pw[1]) + (pw[2] + pw[3]));
    if (__ballot(grew)) {
      // rows of o are heads 4 * grp + i; their factors sit in lanes 4 * grp + i
      float ai[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) ai[i] = __shfl(alpha, 4 * grp + i, 64);
#pragma unroll
      for (int c = 0; c < 8; ++c)
#pragma unroll
        for (int i = 0; i < 4; ++i) st.o[c][i] *= ai[i];
    }
    typedef unsigned int u2 __attribute__((ext_vector_type(2)));
    if constexpr (!kKv8<KIND>) {
      // 16-bit V: for dim 8n + c, rows 0..3 are half c of the lane's 4 pieces
#pragma unroll
      for (int c = 0; c < 8; ++c) {
        const uint32_t sel = (c & 1) ? 0x07060302u : 0x05040100u;
        const u2 vb = {__builtin_amdgcn_perm(t.v[1][c >> 1], t.v[0][c >> 1], sel),
                       __builtin_amdgcn_perm(t.v[3][c >> 1], t.v[2][c >> 1], sel)};
        if constexpr (kSplitP) {
          st.o[c] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(pb_hi, __builtin_bit_cast(s4, vb), st.o[c], 0, 0, 0);
          st.o[c] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(pb_lo, __builtin_bit_cast(s4, vb), st.o[c], 0, 0, 0);
        } else {
          st.o[c] = __builtin_amdgcn_mfma_f32_16x16x16f16(ph, __builtin_bit_cast(h4, vb), st.o[c], 0, 0, 0);
        }
      }
      return;
    }
    // V codes of dim 8n + c for rows 0..3, one dword per c (byte i = row i)
    uint32_t col[8];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const uint32_t r0 = t.v[0][h], r1 = t.v[1][h], r2 = t.v[2][h], r3 = t.v[3][h];
      const uint32_t t01a = __builtin_amdgcn_perm(r1, r0, 0x05010400u);  // r0.b0 r1.b0 r0.b1 r1.b1
      const uint32_t t01b = __builtin_amdgcn_perm(r1, r0, 0x07030602u);  // r0.b2 r1.b2 r0.b3 r1.b3
      const uint32_t t23a = __builtin_amdgcn_perm(r3, r2, 0x05010400u);
      const uint32_t t23b = __builtin_amdgcn_perm(r3, r2, 0x07030602u);
      col[4 * h + 0] = __builtin_amdgcn_perm(t23a, t01a, 0x05040100u);
      col[4 * h + 1] = __builtin_amdgcn_perm(t23a, t01a, 0x07060302u);
      col[4 * h + 2] = __builtin_amdgcn_perm(t23b, t01b, 0x05040100u);
      col[4 * h + 3] = __builtin_amdgcn_perm(t23b, t01b, 0x07060302u);
    }
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      const u2 vb = {e4m3_pair<KIND_F16>(col[c], false), e4m3_pair<KIND_F16>(col[c], true)};
      st.o[c] = __builtin_amdgcn_mfma_f32_16x16x16f16(ph, __builtin_bit_cast(h4, vb), st.o[c], 0, 0, 0);
    }
  }
  // Normaliser of each of this lane's output rows (heads 4 * grp + i).
  __device__ static void row_sums(const State& st, int lane, float (&li)[4]) {
#pragma unroll
    for (int i = 0; i < 4; ++i) li[i] = __shfl(st.l, 4 * (lane >> 4) + i, 64);
  }
  __device__ static void store_output(const AttnArgs& a, int64_t head0, const State& st, int lane) {
    constexpr int QK = kQKind<KIND>;
    const int n = lane & 15, grp = lane >> 4;
    float li[4];
    row_sums(st, lane, li);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int j = 4 * grp + i;
      if (j < G) {
        const float inv = a.out_scale / li[i];
        uint32_t w[4];
#pragma unroll
        for (int e = 0; e < 4; ++e)
          w[e] = (uint32_t)to_bits<QK>(st.o[2 * e][i] * inv) |
                 ((uint32_t)to_bits<QK>(st.o[2 * e + 1][i] * inv) << 16);
        store_b128(a.out + (head0 + j) * kHeadDim + 8 * n, u32x4{w[0], w[1], w[2], w[3]});
      }
    }
    if (grp == 0 && n < G && a.lse) a.lse[head0 + n] = (st.m + __builtin_log2f(st.l)) * kLn2;
  }
  __device__ static void store_partial(const AttnArgs& a, int64_t slot, const State& st, int lane) {
    const int n = lane & 15, grp = lane >> 4;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int j = 4 * grp + i;
      if (j < G) {
        float* dst = a.ws_o + (slot * G + j) * kHeadDim + 8 * n;
#pragma unroll
        for (int c = 0; c < 8; ++c) dst[c] = st.o[c][i];
      }
    }
    if (grp == 0 && n < G) {
      a.ws_ml[(slot * G + n) * 2] = st.m;
      a.ws_ml[(slot * G + n) * 2 + 1] = st.l;
    }
  }
  __device__ static void to_lds(const State& st, int lane, float (*so)[kHeadDim], float* sm,
                                float* sl) {
    const int n = lane & 15, grp = lane >> 4;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int j = 4 * grp + i;
      if (j < G)
#pragma unroll
        for (int c = 0; c < 8; ++c) so[j][8 * n + c] = st.o[c][i];
    }
    if (grp == 0 && n < G) {
      sm[n] = st.m;
      sl[n] = st.l;
    }
  }
};

template <int KIND, int G>
using PathOf = std::conditional_t<kUsesMfma<KIND, G>, MfmaPath<KIND, G>, VecPath<KIND, G>>;

// Streams tiles tile_first + k * tile_step (k < count) of pair (b, g) into st.
template <class P, int SRC>
__device__ __forceinline__ void run_tiles(const AttnArgs& a, int b, int g, const SeqView& sq,
                                          const typename P::Q& q, int tile_first, int count,
                                          int tile_step, typename P::State& st) {
  const int lane = threadIdx.x & 63;
  typename P::Offs offs;
  P::template offsets<SRC>(a, lane, offs);
  using T = typename P::Tile;
  auto load = [&](int k, T& t) {
    P::template load<SRC>(a, b, g, sq.kb, sq.vb, sq.len, (tile_first + k * tile_step) * kTile,
                          k < count, offs, t);
  };
  auto process = [&](const T& t, int k) {
    P::process(a, q, t, (tile_first + k * tile_step) * kTile, sq.len, lane, st);
  };

  // Ping-pong: loads are unconditional (a tile past the run reads nothing), so
  // no branch or register copy forces an early wait on the prefetch.
  if (count <= 0) return;
  T ta, tb;
  load(0, ta);
  for (int k = 0;; k += 2) {
    load(k + 1, tb);
    process(ta, k);
    if (k + 1 >= count) break;
    load(k + 2, ta);
    process(tb, k + 1);
    if (k + 2 >= count) break;
  }
}

// ---------------------------------------------------------------------------
// Fixed-chunk schedule: one workgroup per (b, g, chunk).
// ---------------------------------------------------------------------------

template <int KIND, int G, int SRC>
__global__ __launch_bounds__(256) void decode_chunk_kernel(AttnArgs a) {
  static_assert(G >= 1 && G <= kMaxGroup, "group size");
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);

  int bid = blockIdx.x;
  const int g = bid % a.Hkv;
  bid /= a.Hkv;
  const int c = bid % a.n_chunks;
  const int b = bid / a.n_chunks;

  const SeqView sq = locate<KIND, SRC>(a, b, g);
  const int len = sq.len;
  const int n_c = (len + a.chunk - 1) / a.chunk;
  const int64_t head0 = (int64_t)b * a.Hq + (int64_t)g * G;
  if (len == 0) {
    if (c == 0) store_empty<KIND, G>(a, head0);
    return;
  }
  if (c >= n_c) return;

  using P = PathOf<KIND, G>;
  typename P::Q qf;
  P::load_q(a, head0, lane, qf);
  const int tile0 = c * (a.chunk / kTile);
  const int n_tiles = (min(len, (c + 1) * a.chunk) - c * a.chunk + kTile - 1) / kTile;
  const int mine = n_tiles > wave ? (n_tiles - 1 - wave) / kWaves + 1 : 0;
  typename P::State st;
  st.init();
  run_tiles<P, SRC>(a, b, g, sq, qf, tile0 + wave, mine, kWaves, st);
  st.finish();

  // Merge the four waves through LDS.
  __shared__ float sm_o[kWaves][G][kHeadDim];
  __shared__ float sm_m[kWaves][G], sm_l[kWaves][G];
  P::to_lds(st, lane, sm_o[wave], sm_m[wave], sm_l[wave]);
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
      const float wt = fast_exp2(sm_m[w][j] - M);  // 0 for a wave with no tiles
      num = __builtin_fmaf(wt, sm_o[w][j][d], num);
      den = __builtin_fmaf(wt, sm_l[w][j], den);
    }
    if (n_c == 1) {
      a.out[(head0 + j) * kHeadDim + d] =
          to_bits<kQKind<KIND>>(kKv8<KIND> ? num * (a.out_scale / den) : num / den);
      if (d == 0 && a.lse) a.lse[head0 + j] = (M + __builtin_log2f(den)) * kLn2;
    } else {
      a.ws_o[(item * G + j) * kHeadDim + d] = num;
      if (d == 0) {
        a.ws_ml[(item * G + j) * 2] = M;
        a.ws_ml[(item * G + j) * 2 + 1] = den;
      }
    }
  }
}

// One workgroup per (pair, query head of the group).
template <int KIND, int G, int SRC, int ROWS>
__global__ __launch_bounds__(32 * ROWS) void decode_chunk_merge_kernel(AttnArgs a) {
  const int j = blockIdx.x % G, p = blockIdx.x / G;
  const int g = p % a.Hkv, b = p / a.Hkv;
  const int len = __builtin_amdgcn_readfirstlane(pair_len<SRC>(a, b, g));
  const int n_c = (len + a.chunk - 1) / a.chunk;
  if (n_c <= 1) return;  // written by the chunk kernel
  merge_head<KIND, G, ROWS>(a, (int64_t)b * a.Hq + (int64_t)g * G, j, (int64_t)p * a.n_chunks, 1, n_c);
}

// ---------------------------------------------------------------------------
// Balanced schedule: persistent waves taking items of the tile line.
// ---------------------------------------------------------------------------

// Tile line: the tiles of one KV head of every unit, units in order; unit
// u = sequence b, whose Hkv heads share one length, or, for the hybrid
// source, pair u (lengths differ per KV head).  Item k of the line is run
// for every line head h < LH (LH = Hkv, or 1 for the hybrid source) as item
// k * LH + h, so waves that run at the same time read all heads of the same
// token rows: each 2 KB row of the [tokens, Hkv, 128] cache is then read
// whole within a short time, where one head's 256 B pieces read alone leave
// most of each DRAM row unused (measured on MI355X: a line of whole pairs
// was about 20% slower).  The first tile of unit u is pref[u], pref[n_units]
// is the line length; the unit's length and, for the ragged source, its
// first token row (for the hybrid source, its persistent slot) are kept
// beside it, so that finding a unit needs no global load.
template <int SRC>
__device__ __forceinline__ int line_heads(const AttnArgs& a) {
  return SRC == SRC_HYBRID || SRC == SRC_GATHER ? 1 : a.Hkv;
}

// Sources whose units are single (sequence, KV head) pairs, as their lengths
// differ per KV head.
template <int SRC>
constexpr bool kPairUnits = SRC == SRC_HYBRID || SRC == SRC_GATHER;

struct UnitTable {
  int* pref;  // [n_units + 1]
  int* len;   // [n_units]
  int* aux;   // [n_units]
};

template <int SRC>
__device__ void build_units(const AttnArgs& a, const UnitTable& ut) {
  __shared__ int s_wave[kWaves];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int nu = a.n_units;
  const int per = (nu + 255) / 256;
  const int u0 = min(nu, tid * per), u1 = min(nu, u0 + per);
  int local = 0;
  for (int u = u0; u < u1; ++u) {
    const int b = kPairUnits<SRC> ? u / a.Hkv : u;
    const int g = kPairUnits<SRC> ? u % a.Hkv : 0;
    const int len = pair_len<SRC>(a, b, g);
    ut.len[u] = len;
    if constexpr (SRC == SRC_RAGGED) ut.aux[u] = min(max(a.cu_seqlens[b], 0), a.S);
    else if constexpr (SRC == SRC_HYBRID) ut.aux[u] = a.head_map[g];
    else ut.aux[u] = 0;
    local += (len + kTile - 1) / kTile;
  }
  int incl = local;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int y = __shfl_up(incl, d, 64);
    if (lane >= d) incl += y;
  }
  if (lane == 63) s_wave[wave] = incl;
  __syncthreads();
  int base = 0;
  for (int w = 0; w < wave; ++w) base += s_wave[w];
  int run = base + incl - local;
  for (int u = u0; u < u1; ++u) {
    ut.pref[u] = run;
    run += (ut.len[u] + kTile - 1) / kTile;
  }
  if (tid == 255) ut.pref[nu] = base + incl;
  __syncthreads();
}

// Items of the line: columns k < Wc <= (persistent waves) / LH; item
// k * LH + h (column k, line head h) belongs to the wave that runs column k
// for line head h.  Column k holds line tiles [first(k), first(k + 1)),
// first(k) = N * cum(k) / total, cum(k) the sum of the weights of columns
// below k: a column run by workgroups of the first dispatch round (one per
// CU: blocks below the CU count) weighs w0, the others w1, and where the
// columns alternate between even and odd XCDs (xcd_cols), an odd column that
// times wo / 100.  The main and the merge kernel cut the line the same way
// from its length N.
struct ItemLine {
  int N, Wc, C0;          // C0: columns of the first round
  int w0, w1, wo;
  bool xcd_cols;
  int64_t total;          // cum(Wc)
  // sum over columns c < n of 100, or wo for the odd ones
  __device__ int64_t xsum(int n) const { return 100 * (int64_t)n - (int64_t)(100 - wo) * (n >> 1); }
  __device__ int64_t cum(int k) const {
    if (!xcd_cols)  // (all columns of one XCD weight; the common case, kept short)
      return k <= C0 ? (int64_t)w0 * k : (int64_t)w0 * C0 + (int64_t)w1 * (k - C0);
    return k <= C0 ? (int64_t)w0 * xsum(k)
                   : (int64_t)w0 * xsum(C0) + (int64_t)w1 * (xsum(k) - xsum(C0));
  }
  __device__ int first(int k) const { return (int)((int64_t)N * cum(k) / total); }
  // the largest n with xsum(n) <= u (xsum grows by 100 + wo every two columns)
  __device__ int xsum_inv(int64_t u) const {
    const int64_t pair = 100 + wo, p = u / pair;
    return (int)(2 * p + (u - p * pair >= 100 ? 1 : 0));
  }
  // the column that holds tile x (x < N): the largest k with first(k) <= x
  __device__ int of_tile(int x) const {
    const int64_t lim = (int64_t)(x + 1) * total;  // first(k) <= x  <=>  N * cum(k) < lim
    if (!xcd_cols) {
      if (C0 >= Wc || (int64_t)N * w0 * C0 >= lim)
        return (int)((lim - 1) / ((int64_t)N * w0));
      return C0 + (int)((lim - 1 - (int64_t)N * w0 * C0) / ((int64_t)N * w1));
    }
    const int64_t t = (lim - 1) / N;  // the largest cum(k) allowed
    const int64_t c0 = (int64_t)w0 * xsum(C0);
    const int k = C0 >= Wc || c0 > t ? xsum_inv(t / w0) : xsum_inv(xsum(C0) + (t - c0) / w1);
    return min(k, Wc - 1);
  }
};

// Which column and line head a wave runs.  With a.xcd_cols set (the host sets
// it when a column's LH waves fill m >= 2 whole workgroups, LH = 4m as with 8
// or 32 KV heads, and the grid holds at most one workgroup per CU, two for
// bf16 K/V read from runs, in whole groups of 8m workgroups) the m workgroups
// of a column are on one XCD (workgroups go to the 8 XCDs in turn): block b = 8t + x runs
// column 8 (t / m) + x for heads 4 (t % m) ...; with one head per column
// (LH = 1: the hybrid and gather sources, or a single KV head) wave i of
// block b = 8t + x runs column 8 (4t + i) + x.  Otherwise wave w = 4b + i
// runs column w / LH for head w % LH.  (Measured on MI355X: on the paged
// 1024 x 32-head batch, one XCD per column 3376 -> 3361 us, and with odd XCDs
// weighted 0.90, 3312 us; e4m3, at three workgroups per CU, lost 1-2 us.)
struct ColumnOf {
  int col, head;
};
__device__ __forceinline__ ColumnOf column_of(const AttnArgs& a, int LH) {
  ColumnOf c;
  const int b = (int)blockIdx.x, wave = (int)(threadIdx.x >> 6);
  if (a.xcd_cols && LH == 1) {  // four columns per workgroup: 8 (4t + i) + x
    const int x = b % 8, t = b / 8;
    c.col = (t * kWaves + wave) * 8 + x;
    c.head = 0;
  } else if (a.xcd_cols) {
    const int m = LH / kWaves, x = b % 8, t = b / 8;
    c.col = (t / m) * 8 + x;
    c.head = (t % m) * kWaves + wave;
  } else {
    const int w = b * kWaves + wave;
    c.col = w / LH;
    c.head = w - c.col * LH;
  }
  return c;
}

// Waves of a first-round workgroup stream faster than the others (measured on
// MI355X with the priority steps below: 1.086 times the rate of the later
// waves on the 16 x 16K-32K ragged batch and the CLO hybrid, on three boxes),
// so their columns get more: 1.13 times as much, which also lightens the
// later waves, among them the slowest (a later-round wave on a slow XCD ends
// the kernel; weighting by the rate ratio alone left it 1-3 us later in a
// simulation on the measured per-wave rates).  Waves on odd-numbered XCDs
// stream slower than those on even ones (measured on MI355X with one
// workgroup per CU: 0.94-0.98 against 1.00-1.06 of the mean on the CLO
// hybrid, and on the 16 x 16K-32K batch whatever heads they run), so where a
// column's waves share one XCD (a.xcd_cols, column_of), columns on odd XCDs
// get a.xcd_w / 100 as much.  At
// most N columns, and equal weights below 2 tiles per column, so that no
// column is empty.
__device__ __forceinline__ ItemLine item_line(const AttnArgs& a, int N, int LH) {
  ItemLine L;
  L.N = N;
  L.Wc = min(a.n_blocks * kWaves / LH, N);
  L.C0 = min(L.Wc, (a.n_cu * kWaves + LH - 1) / LH);  // columns whose first wave is dispatched first
  const bool weighted = N >= 2 * L.Wc;
  L.w0 = weighted ? kFirstRoundWeight : 100;
  L.w1 = 100;
  // the XCD weight where a column's waves share one XCD (with more than one
  // dispatch round it multiplies the first-round weight)
  L.xcd_cols = a.xcd_cols != 0;  // column c on XCD c % 8
  L.wo = weighted && L.xcd_cols ? a.xcd_w : 100;
  L.total = L.cum(L.Wc);
  return L;
}

// Waves of the workgroups that reach a CU first win most arbitration
// (oldest first), so with equal shares they end far ahead of the others
// (measured on MI355X: mean end 238 vs 265 us on the 16 x 16K-32K ragged
// batch even with the steps below, 199 vs 261 us without).  A wave starts its
// share at the highest priority and steps down a level at each quarter done,
// so the waves that are behind get served first.
__device__ __forceinline__ void set_progress_priority(int level) {
  switch (level) {
    case 3: __builtin_amdgcn_s_setprio(3); break;
    case 2: __builtin_amdgcn_s_setprio(2); break;
    case 1: __builtin_amdgcn_s_setprio(1); break;
    default: __builtin_amdgcn_s_setprio(0); break;
  }
}

// A run of tiles of one pair inside one item: tiles [x0, x1) of the line,
// the first of them tile t of the pair.  All fields are wave-uniform.
struct Seg {
  int x0, x1, t;
  int b, g, len;
  int slot;    // partial slot: (column + unit) * LH + line head
  bool whole;  // the run is the whole pair
  const char* kb;
  const char* vb;
};

// The run that starts at line tile x of column `item` (ending at hi), head h.
template <int KIND, int SRC>
__device__ __forceinline__ Seg seg_at(const AttnArgs& a, const UnitTable& ut, int x, int item, int hi,
                                      int h) {
  int lo_u = 0, hi_u = a.n_units;  // largest u with pref[u] <= x
  while (hi_u - lo_u > 1) {
    const int mid = (lo_u + hi_u) >> 1;
    if (uniform_i32(ut.pref[mid]) <= x) lo_u = mid;
    else hi_u = mid;
  }
  const int u = uniform_i32(lo_u);
  const int ubase = uniform_i32(ut.pref[u]);
  const int uend = uniform_i32(ut.pref[u + 1]);
  const int LH = line_heads<SRC>(a);
  Seg sg;
  sg.x0 = x;
  sg.x1 = uniform_i32(min(hi, uend));
  sg.t = x - ubase;
  sg.b = kPairUnits<SRC> ? u / a.Hkv : u;
  sg.g = kPairUnits<SRC> ? u % a.Hkv : h;
  sg.len = uniform_i32(ut.len[u]);
  sg.slot = (item + u) * LH + h;
  sg.whole = x == ubase && sg.x1 == uend;
  const int aux = uniform_i32(ut.aux[u]);
  if constexpr (SRC == SRC_DENSE || SRC == SRC_GATHER) {
    const int64_t base = ((int64_t)sg.b * a.S * a.Hkv + sg.g) * kHeadDim;
    sg.kb = kv_at<KIND>(a.k, base);
    sg.vb = kv_at<KIND>(a.v, base);
  } else if constexpr (SRC == SRC_RAGGED) {
    const int64_t base = ((int64_t)aux * a.Hkv + sg.g) * kHeadDim;
    sg.kb = kv_at<KIND>(a.k, base);
    sg.vb = kv_at<KIND>(a.v, base);
  } else if constexpr (SRC == SRC_PAGED) {
    sg.kb = kv_at<KIND>(a.k, 0);
    sg.vb = kv_at<KIND>(a.v, 0);
  } else {  // SRC_HYBRID: aux is the persistent slot, or < 0 for the cache buffer
    if (aux >= 0) {
      const int64_t base = ((int64_t)sg.b * a.P_slots + min(aux, max(a.P_slots - 1, 0))) *
                           a.pers_cap * kHeadDim;
      sg.kb = kv_at<KIND>(a.k, base);
      sg.vb = kv_at<KIND>(a.v, base);
    } else {
      const int64_t base = ((int64_t)sg.b * a.Hkv + sg.g) * a.buf_cap * kHeadDim;
      sg.kb = kv_at<KIND>(a.k2, base);
      sg.vb = kv_at<KIND>(a.v2, base);
    }
  }
  return sg;
}

// Persistent waves stream the tiles of their items as one sequence: the
// loads for the next tile are issued while the current one is processed,
// also where the next tile starts another pair or another item, so a wave's
// loads stay in flight across item boundaries.  When the processed tile ends
// its run, the state goes out (as the pair's output when the run is the whole
// pair, else as the partial of slot item + pair) and the next run begins.
template <int KIND, int G, int SRC>
__global__ __launch_bounds__(256) void decode_balanced_kernel(AttnArgs a) {
  extern __shared__ int s_units[];
  const UnitTable ut{s_units, s_units + a.n_units + 1, s_units + 2 * a.n_units + 1};
  build_units<SRC>(a, ut);

  const int lane = threadIdx.x & 63;
  const int LH = line_heads<SRC>(a);
  const ColumnOf co = column_of(a, LH);
  const ItemLine L = item_line(a, uniform_i32(ut.pref[a.n_units]), LH);
  const int lk = uniform_i32(co.col), lh = uniform_i32(co.head);
  // Each unit's first and last column, (1, 0) for an empty unit, for the
  // merge kernel (which would otherwise need the unit table and 64-bit
  // divisions in each of its many workgroups); unit u goes to lane
  // u / n_blocks of block u % n_blocks, before any wave leaves.
  for (int u = (int)threadIdx.x * a.n_blocks + (int)blockIdx.x; u < a.n_units;
       u += 256 * a.n_blocks) {
    const int ub = ut.pref[u], ue = ut.pref[u + 1];
    *reinterpret_cast<int2*>(&a.ws_cols[2 * u]) =
        ue > ub ? make_int2(L.of_tile(ub), L.of_tile(ue - 1)) : make_int2(1, 0);
  }
  if (lk >= L.Wc) return;
  const int x_end = uniform_i32(L.first(lk + 1));
  const int share = x_end - uniform_i32(L.first(lk));
  if (share <= 0) return;
  int done = 0;
  set_progress_priority(3);

  using P = PathOf<KIND, G>;
  using T = typename P::Tile;
  typename P::Offs offs;
  P::template offsets<SRC>(a, lane, offs);

  // Load side: run ls, next tile to load lx; `more` is false once the share
  // is loaded.
  Seg ls = seg_at<KIND, SRC>(a, ut, L.first(lk), lk, x_end, lh);
  int lx = ls.x0;
  bool more = true;
  // Process side: run ps, next tile to process px.
  Seg ps = ls;
  int px = lx;
  typename P::Q qf, qn;
  constexpr int kQWords = sizeof(typename P::Q) / sizeof(u32x4);
  P::load_q(a, (int64_t)ps.b * a.Hq + (int64_t)ps.g * G, lane, qf);
  typename P::State st;
  st.init();

  auto advance = [&]() {
    if (!more) return;
    if (++lx < ls.x1) return;
    if (lx >= x_end) {
      more = false;
      return;
    }
    ls = seg_at<KIND, SRC>(a, ut, lx, lk, x_end, lh);  // the next unit
    P::load_q(a, (int64_t)ls.b * a.Hq + (int64_t)ls.g * G, lane, qn);
  };
  auto load = [&](T& t) {
    P::template load<SRC>(a, ls.b, ls.g, ls.kb, ls.vb, ls.len, (ls.t + lx - ls.x0) * kTile, more,
                          offs, t);
  };
  // Processes tile px; returns false when nothing is left to process.
  auto step = [&](const T& t) -> bool {
    P::process(a, qf, t, (ps.t + px - ps.x0) * kTile, ps.len, lane, st);
    ++done;
    if ((4 * done) / share != (4 * (done - 1)) / share) set_progress_priority(3 - (4 * done) / share);
    if (++px < ps.x1) return true;
    st.finish();
    // A fresh copy of the lane index: address arithmetic that depends on it
    // is then done here, instead of being hoisted and kept live in the loop.
    int lane_s = lane;
    asm volatile("" : "+v"(lane_s));
    const int64_t head0 = (int64_t)ps.b * a.Hq + (int64_t)ps.g * G;
    if (ps.whole) P::store_output(a, head0, st, lane_s);
    else P::store_partial(a, ps.slot, st, lane_s);
    st.init();
    if (!more) return false;
    // The loaded tile after the finished run starts run ls.
    ps = ls;
    px = ps.x0;
#pragma unroll
    for (int j = 0; j < kQWords; ++j) qf[j] = qn[j];
    return true;
  };

  T ta, tb;
  load(ta);
  for (;;) {
    advance();
    load(tb);
    if (!step(ta)) break;
    advance();
    load(ta);
    if (!step(tb)) break;
  }
}

// One workgroup per (pair, query head of the group).  The partial of item k
// and unit u for line head h is slot (k + u) * LH + h: items grow along the
// line and units follow it, so no two runs share a slot, and the slots of
// one pair are LH apart.
template <int KIND, int G, int SRC, int ROWS>
__global__ __launch_bounds__(32 * ROWS) void decode_balanced_merge_kernel(AttnArgs a) {
  const int j = blockIdx.x % G, p = blockIdx.x / G;
  const int b = p / a.Hkv, g = p % a.Hkv;
  const int LH = line_heads<SRC>(a);
  const int u = kPairUnits<SRC> ? p : b, h = kPairUnits<SRC> ? 0 : g;
  // first and last column, each non-empty; (1, 0) for an empty unit
  const int2 kc = *reinterpret_cast<const int2*>(&a.ws_cols[2 * u]);
  const int k0 = kc.x, k1 = kc.y;
  const int64_t head0 = (int64_t)b * a.Hq + (int64_t)g * G;
  if (k1 < k0) {
    if (threadIdx.x < kHeadDim) a.out[(head0 + j) * kHeadDim + threadIdx.x] = 0;
    if (threadIdx.x == 0 && a.lse) a.lse[head0 + j] = -INFINITY;
    return;
  }
  if (k0 == k1) return;  // one item covered the pair and wrote the output
  merge_head<KIND, G, ROWS>(a, head0, j, (int64_t)(k0 + u) * LH + h, LH, k1 - k0 + 1);
}


// ---------------------------------------------------------------------------
// Launch
// ---------------------------------------------------------------------------

// One merge workgroup per query head, with merge_rows(heads) rows.
template <void (*K16)(AttnArgs), void (*K8)(AttnArgs), void (*K4)(AttnArgs)>
hipError_t launch_merge(int heads, const AttnArgs& a, hipStream_t stream) {
  const int rows = merge_rows(heads);
  const dim3 grid((unsigned)heads), block((unsigned)(32 * rows));
  if (rows == 16) K16<<<grid, block, 0, stream>>>(a);
  else if (rows == 8) K8<<<grid, block, 0, stream>>>(a);
  else K4<<<grid, block, 0, stream>>>(a);
  return hipGetLastError();
}

template <int KIND, int G, int SRC>
hipError_t launch_src(const AttnArgs& a, hipStream_t stream) {
  const dim3 block(256);
  if (a.mode == MODE_BALANCED) {
    const size_t lds = (size_t)(3 * a.n_units + 1) * sizeof(int);
    launch_timed(decode_balanced_kernel<KIND, G, SRC>, dim3((unsigned)a.n_blocks), block, (uint32_t)lds,
                 stream, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    return launch_merge<decode_balanced_merge_kernel<KIND, G, SRC, 16>, decode_balanced_merge_kernel<KIND, G, SRC, 8>,
                        decode_balanced_merge_kernel<KIND, G, SRC, 4>>(a.B * a.Hkv * G, a, stream);
  }
  const dim3 grid((unsigned)((int64_t)a.B * a.n_chunks * a.Hkv));
  launch_timed(decode_chunk_kernel<KIND, G, SRC>, grid, block, 0u, stream, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || a.n_chunks <= 1) return e;
  return launch_merge<decode_chunk_merge_kernel<KIND, G, SRC, 16>, decode_chunk_merge_kernel<KIND, G, SRC, 8>,
                      decode_chunk_merge_kernel<KIND, G, SRC, 4>>(a.B * a.Hkv * G, a, stream);
}

template <int KIND, int G, int SRC>
int balanced_occupancy() {
  static std::atomic<int> cached{0};
  int v = cached.load(std::memory_order_relaxed);
  if (v > 0) return v;
  int occ = 0;
  const size_t lds = (size_t)(3 * kMaxUnits + 1) * sizeof(int);
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(
          &occ, reinterpret_cast<const void*>(decode_balanced_kernel<KIND, G, SRC>), 256, lds) !=
          hipSuccess ||
      occ < 1) {
    (void)hipGetLastError();
    occ = 2;
  }
  cached.store(occ, std::memory_order_relaxed);
  return occ;
}

template <int KIND, int G>
hipError_t launch_g(const AttnArgs& a, hipStream_t stream) {
  switch (a.src) {
    case SRC_DENSE: return launch_src<KIND, G, SRC_DENSE>(a, stream);
    case SRC_RAGGED: return launch_src<KIND, G, SRC_RAGGED>(a, stream);
    case SRC_PAGED: return launch_src<KIND, G, SRC_PAGED>(a, stream);
    case SRC_GATHER: return launch_src<KIND, G, SRC_GATHER>(a, stream);
    default: return launch_src<KIND, G, SRC_HYBRID>(a, stream);
  }
}

template <int KIND, int G>
int occupancy_g(int src) {
  switch (src) {
    case SRC_DENSE: return balanced_occupancy<KIND, G, SRC_DENSE>();
    case SRC_RAGGED: return balanced_occupancy<KIND, G, SRC_RAGGED>();
    case SRC_PAGED: return balanced_occupancy<KIND, G, SRC_PAGED>();
    case SRC_GATHER: return balanced_occupancy<KIND, G, SRC_GATHER>();
    default: return balanced_occupancy<KIND, G, SRC_HYBRID>();
  }
}

template <int KIND, template <int, int> class F, typename... Args>
auto dispatch_g(int G, Args... args) {
  switch (G) {
    case 1: return F<KIND, 1>::run(args...);
    case 2: return F<KIND, 2>::run(args...);
    case 3: return F<KIND, 3>::run(args...);
    case 4: return F<KIND, 4>::run(args...);
    case 5: return F<KIND, 5>::run(args...);
    case 6: return F<KIND, 6>::run(args...);
    case 7: return F<KIND, 7>::run(args...);
    default: return F<KIND, 8>::run(args...);
  }
}

template <int KIND, int G>
struct LaunchF {
  static hipError_t run(const AttnArgs& a, hipStream_t s) { return launch_g<KIND, G>(a, s); }
};
template <int KIND, int G>
struct OccF {
  static int run(int src) { return occupancy_g<KIND, G>(src); }
};

}  // namespace

int device_cu_count() {
  static std::atomic<int> cached[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) {
    (void)hipGetLastError();
    return 256;
  }
  int v = cached[dev].load(std::memory_order_relaxed);
  if (v > 0) return v;
  int cus = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      cus < 1) {
    (void)hipGetLastError();
    cus = 256;
  }
  cached[dev].store(cus, std::memory_order_relaxed);
  return cus;
}

int balanced_blocks(int dtype, int kv8, int G, int src, int64_t est_tiles) {
  if (G < 1 || G > kMaxGroup) return 1;
  int occ;
  switch ((dtype == KIND_F16 ? KIND_F16 : KIND_BF16) | (kv8 ? KIND_KV8 : 0)) {
    case KIND_F16: occ = dispatch_g<KIND_F16, OccF>(G, src); break;
    case KIND_BF16: occ = dispatch_g<KIND_BF16, OccF>(G, src); break;
    case KIND_F16 | KIND_KV8: occ = dispatch_g<KIND_F16 | KIND_KV8, OccF>(G, src); break;
    default: occ = dispatch_g<KIND_BF16 | KIND_KV8, OccF>(G, src); break;
  }
  // fp16 K/V read from runs (not gathered rows): one workgroup per CU.  Its
  // four waves, one per SIMD, read faster than two or three workgroups' worth
  // (measured on MI355X, one process, interleaved: the 16 x 16K-32K ragged
  // batch 237.1 -> 236.1 us, the CLO hybrid 111.1 -> 107.0, the 1024-sequence
  // MHA batch 3377 -> 3348; a read probe with the same tiles: 6.9 TB/s at
  // two workgroups per CU, 7.1 at one), and every column then starts in the
  // first dispatch round.  bf16 (P.V in two halves), e4m3 (decoding) and
  // gathered rows (index loads) have more to do per byte and lose with one
  // (+1, +17 and +8 us), so they keep the resident maximum.
  if (dtype == KIND_F16 && !kv8 && src != SRC_GATHER) occ = 1;
  const int64_t cap = (int64_t)device_cu_count() * occ;
  // at least kMinTilesPerWave tiles per wave when the work is small
  const int64_t need = (est_tiles + (int64_t)kWaves * kMinTilesPerWave - 1) / ((int64_t)kWaves * kMinTilesPerWave);
  return (int)std::max<int64_t>(1, std::min(cap, need));
}

size_t attn_workspace_bytes(int64_t slots, int G, int64_t n_cols) {
  auto up = [](size_t x) { return (x + 255) & ~size_t(255); };
  return up((size_t)slots * G * kHeadDim * 4) + up((size_t)slots * G * 2 * 4) + up((size_t)n_cols * 4);
}

bool attn_workspace_carve(void* ws, size_t ws_bytes, int64_t slots, int G, int64_t n_cols,
                          AttnArgs* a) {
  auto up = [](size_t x) { return (x + 255) & ~size_t(255); };
  if (ws_bytes < attn_workspace_bytes(slots, G, n_cols) || ws == nullptr) return false;
  char* p = static_cast<char*>(ws);
  a->ws_o = reinterpret_cast<float*>(p);
  p += up((size_t)slots * G * kHeadDim * 4);
  a->ws_ml = reinterpret_cast<float*>(p);
  p += up((size_t)slots * G * 2 * 4);
  a->ws_cols = n_cols > 0 ? reinterpret_cast<int32_t*>(p) : nullptr;  // 256-byte aligned
  return true;
}

hipError_t launch_decode_attn(const AttnArgs& a, hipStream_t stream) {
  switch ((a.dtype == KIND_F16 ? KIND_F16 : KIND_BF16) | (a.kv8 ? KIND_KV8 : 0)) {
    case KIND_F16: return dispatch_g<KIND_F16, LaunchF>(a.G, a, stream);
    case KIND_BF16: return dispatch_g<KIND_BF16, LaunchF>(a.G, a, stream);
    case KIND_F16 | KIND_KV8: return dispatch_g<KIND_F16 | KIND_KV8, LaunchF>(a.G, a, stream);
    default: return dispatch_g<KIND_BF16 | KIND_KV8, LaunchF>(a.G, a, stream);
  }
}

}  // namespace kvdec

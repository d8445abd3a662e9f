// kv_recompute.hip -- KVPR partial K/V recompute as an MFMA GEMM for gfx950.
//
// KVPR page, section A2: the first l tokens' keys and values are recomputed on
// the GPU from the saved activations, K[0:l] = X[0:l] W_K and V[0:l] = X[0:l]
// W_V with W in R^{h x h}, and then join the resident rows [l, s') before
// attention.  Here both products form one GEMM
//     C[M = b*l, N = 2h] = X[M, K = h] . [W_K | W_V][K, N]
// with bf16 inputs, fp32 MFMA accumulation and an epilogue that rounds to
// fp16 and writes row (batch i, token t) straight into k_cache / v_cache
// [b, s_cap, H, 128] at rows t < l (every other byte untouched).
//
// Three kernels:
//   kv_recompute_kernel_wide<layout>: grids of at least 256 tiles of 256 x 256
//     (one workgroup per CU, four 128 x 128 waves, a hand-pipelined loop);
//     either W layout, [in, out] through LDS transpose reads.
//   kv_recompute_kernel_k64 / kv_recompute_kernel: smaller grids, 256 x 128
//     tiles (two workgroups per CU), W [out, in] / W [in, out].
// In the 256 x 128 kernels a 256-thread workgroup's four waves each own a
// 128 x 64 quarter as 4 x 2 v_mfma_f32_32x32x16_bf16 blocks (accumulators in
// VGPRs, two waves per SIMD).  X rows are K-contiguous.  W stored [out, in]
// (as a torch.nn.Linear weight) is K-contiguous too and is staged exactly like
// X, in 64-wide K steps.  W stored [in, out] is N-contiguous: there each thread
// transposes a 4 x 4 block of it in registers (byte permutes) before storing
// it K-contiguous in LDS, in 32-wide K steps with loads two steps ahead and
// double-buffered LDS.  Its transposed 8-byte stores put rows 4 apart on the
// same LDS banks (measured on MI355X: that kernel runs at about 40% of the
// MFMA rate with no global loads at all, 85% with no LDS operand traffic).
#include "device_common.h"
#include "internal.h"

namespace kvdec {
namespace {

constexpr int BM = 256, BN = 128, BK = 32;
constexpr int LDS_STRIDE = BK + 8;  // bf16 elements per LDS row (80 bytes: spreads banks)

typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ uint32_t pack_lo(uint32_t a, uint32_t b) {
  // (a.lo, b.lo) -> low half from a, high half from b
  return __builtin_amdgcn_perm(b, a, 0x05040100u);
}
__device__ __forceinline__ uint32_t pack_hi(uint32_t a, uint32_t b) {
  return __builtin_amdgcn_perm(b, a, 0x07060302u);
}

// One K step's global data of this thread: four 16-byte pieces of X rows and
// a 4 x 4 block of W.
struct Stage {
  u32x4 a[4];
  u32x2 b[4];
};

// [in, out] weights.
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2))) void kv_recompute_kernel(RecomputeArgs a) {
  __shared__ __attribute__((aligned(16))) uint16_t As[2][BM * LDS_STRIDE];
  __shared__ __attribute__((aligned(16))) uint16_t Bs[2][BN * LDS_STRIDE];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int M = a.b * a.l, N = 2 * a.h, K = a.h;
  const int n_tiles_n = N / BN;
  const int tile_m = blockIdx.x / n_tiles_n, tile_n = blockIdx.x % n_tiles_n;
  const int m0 = tile_m * BM, n0 = tile_n * BN;

  // W source for this N tile (never straddles the K|V boundary: h % BN == 0).
  const bool is_v = n0 >= a.h;
  const uint16_t* W = is_v ? a.wv : a.wk;
  const int wn0 = is_v ? n0 - a.h : n0;

  // A loads: thread -> 16-byte piece ak of rows am + 64 i (i < 4); rows past
  // M read row M - 1 (their results are not stored).
  const int am = tid >> 2, ak = (tid & 3) * 8;
  const uint16_t* xrow[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = min(m0 + am + 64 * i, M - 1);
    const int bi = r / a.l, t = r - bi * a.l;
    xrow[i] = a.x + (int64_t)bi * a.x_bstride + (int64_t)t * a.h + ak;
  }
  // B loads: thread -> 4 k-rows (bk .. bk+3) x 4 n-columns (bn .. bn+3); 32
  // lanes read one 256-byte W row piece.  (Measured: a k-fastest mapping,
  // which avoids the LDS bank conflicts of the transposed stores, was slower
  // overall because of its scattered global reads.)
  const int bn = (tid & 31) * 4, bk = (tid >> 5) * 4;
  const uint16_t* wsrc = W + (int64_t)bk * a.h + wn0 + bn;

  auto gload = [&](int k0, Stage& st) {
#pragma unroll
    for (int i = 0; i < 4; ++i) st.a[i] = load_b128(xrow[i] + k0);
#pragma unroll
    for (int i = 0; i < 4; ++i) st.b[i] = *reinterpret_cast<const u32x2*>(wsrc + (int64_t)(k0 + i) * a.h);
  };
  auto lstore = [&](int buf, const Stage& st) {
#pragma unroll
    for (int i = 0; i < 4; ++i) store_b128(&As[buf][(am + 64 * i) * LDS_STRIDE + ak], st.a[i]);
    // st.b[i] = W[bk+i][bn .. bn+3] as two dwords; transpose to columns.
    u32x2 col[4];
    col[0] = u32x2{pack_lo(st.b[0].x, st.b[1].x), pack_lo(st.b[2].x, st.b[3].x)};
    col[1] = u32x2{pack_hi(st.b[0].x, st.b[1].x), pack_hi(st.b[2].x, st.b[3].x)};
    col[2] = u32x2{pack_lo(st.b[0].y, st.b[1].y), pack_lo(st.b[2].y, st.b[3].y)};
    col[3] = u32x2{pack_hi(st.b[0].y, st.b[1].y), pack_hi(st.b[2].y, st.b[3].y)};
#pragma unroll
    for (int j = 0; j < 4; ++j) *reinterpret_cast<u32x2*>(&Bs[buf][(bn + j) * LDS_STRIDE + bk]) = col[j];
  };

  // Wave quarter: rows wm .. wm+127, cols wn .. wn+63.
  const int wm = (wave >> 1) * 128, wn = (wave & 1) * 64;
  f32x16 acc[4][2];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;

  auto compute = [&](int buf) {
#pragma unroll
    for (int ks = 0; ks < BK / 16; ++ks) {
      u32x4 fa[4], fb[2];
      const int kk = 16 * ks + 8 * (lane >> 5);
#pragma unroll
      for (int i = 0; i < 4; ++i)
        fa[i] = *reinterpret_cast<const u32x4*>(&As[buf][(wm + 32 * i + (lane & 31)) * LDS_STRIDE + kk]);
#pragma unroll
      for (int j = 0; j < 2; ++j)
        fb[j] = *reinterpret_cast<const u32x4*>(&Bs[buf][(wn + 32 * j + (lane & 31)) * LDS_STRIDE + kk]);
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
              __builtin_bit_cast(bf16x8, fa[i]), __builtin_bit_cast(bf16x8, fb[j]), acc[i][j], 0, 0, 0);
    }
  };

  // K step kt computes from LDS[kt & 1]; the registers of stage kt & 1 are
  // refilled with step kt + 2 as soon as step kt has been stored, and step
  // kt + 1 (loaded during step kt - 1) is stored after the compute.
  const int nk = K / BK;  // a multiple of 8 (h % 256 == 0)
  Stage s0, s1;
  gload(0, s0);
  gload(BK, s1);
  lstore(0, s0);
  __syncthreads();
  for (int kt = 0; kt < nk; kt += 2) {
    // even step: LDS[0] holds kt, s1 holds kt + 1
    if (kt + 2 < nk) gload((kt + 2) * BK, s0);
    compute(0);
    lstore(1, s1);
    __syncthreads();
    // odd step: LDS[1] holds kt + 1, s0 holds kt + 2
    if (kt + 3 < nk) gload((kt + 3) * BK, s1);
    compute(1);
    if (kt + 2 < nk) lstore(0, s0);
    __syncthreads();
  }

  // Epilogue: acc[i][j][e] = C[row wm + 32i + 8*(e/4) + 4*(lane/32) + e%4][col wn + 32j + lane%32]
  uint16_t* C = is_v ? a.vc : a.kc;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const int r = m0 + wm + 32 * i + 8 * (e >> 2) + 4 * (lane >> 5) + (e & 3);
      if (r >= M) continue;
      const int bi = r / a.l, t = r - bi * a.l;
      uint16_t* crow = C + (int64_t)bi * a.c_bstride + (int64_t)t * a.h + wn0 + wn + (lane & 31);
#pragma unroll
      for (int j = 0; j < 2; ++j) crow[32 * j] = to_bits<KIND_F16>(acc[i][j][e]);
    }
  }
}

// [out, in] weights: W rows are K-contiguous like X rows and are staged the
// same way.  64-wide K steps, so each wave issues 32 MFMAs between barriers;
// the next step's loads are in flight in registers during the compute, and
// one LDS buffer with two barriers per step keeps two workgroups on a CU
// (measured on MI355X: 0.99-1.03 PFLOP/s on the OPT-13B shape, against
// 0.92 with 32-wide steps and double-buffered LDS).  144-byte LDS rows:
// fragment reads of 32 consecutive rows hit distinct banks.
constexpr int BK2 = 64, LDS2 = BK2 + 8;
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2))) void kv_recompute_kernel_k64(RecomputeArgs a) {
  __shared__ __attribute__((aligned(16))) uint16_t As[BM * LDS2];
  __shared__ __attribute__((aligned(16))) uint16_t Bs[BN * LDS2];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int M = a.b * a.l, N = 2 * a.h, K = a.h;
  const int n_tiles_n = N / BN;
  const int tile_m = blockIdx.x / n_tiles_n, tile_n = blockIdx.x % n_tiles_n;
  const int m0 = tile_m * BM, n0 = tile_n * BN;
  const bool is_v = n0 >= a.h;
  const uint16_t* W = is_v ? a.wv : a.wk;
  const int wn0 = is_v ? n0 - a.h : n0;
  const int am = tid >> 3, ak = (tid & 7) * 8;
  const uint16_t* xrow[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int r = min(m0 + am + 32 * i, M - 1);
    const int bi = r / a.l, t = r - bi * a.l;
    xrow[i] = a.x + (int64_t)bi * a.x_bstride + (int64_t)t * a.h + ak;
  }
  const uint16_t* wsrc = W + (int64_t)(wn0 + am) * a.h + ak;
  u32x4 sa[8], sb[4];
  auto gload = [&](int k0) {
#pragma unroll
    for (int i = 0; i < 8; ++i) sa[i] = load_b128(xrow[i] + k0);
#pragma unroll
    for (int i = 0; i < 4; ++i) sb[i] = load_b128(wsrc + (int64_t)32 * i * a.h + k0);
  };
  auto lstore = [&]() {
#pragma unroll
    for (int i = 0; i < 8; ++i) store_b128(&As[(am + 32 * i) * LDS2 + ak], sa[i]);
#pragma unroll
    for (int i = 0; i < 4; ++i) store_b128(&Bs[(am + 32 * i) * LDS2 + ak], sb[i]);
  };
  const int wm = (wave >> 1) * 128, wn = (wave & 1) * 64;
  f32x16 acc[4][2];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;
  const int nk = K / BK2;
  gload(0);
  lstore();
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    if (kt + 1 < nk) gload((kt + 1) * BK2);
#pragma unroll
    for (int ks = 0; ks < BK2 / 16; ++ks) {
      u32x4 fa[4], fb[2];
      const int kk = 16 * ks + 8 * (lane >> 5);
#pragma unroll
      for (int i = 0; i < 4; ++i)
        fa[i] = *reinterpret_cast<const u32x4*>(&As[(wm + 32 * i + (lane & 31)) * LDS2 + kk]);
#pragma unroll
      for (int j = 0; j < 2; ++j)
        fb[j] = *reinterpret_cast<const u32x4*>(&Bs[(wn + 32 * j + (lane & 31)) * LDS2 + kk]);
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
              __builtin_bit_cast(bf16x8, fa[i]), __builtin_bit_cast(bf16x8, fb[j]), acc[i][j], 0, 0, 0);
    }
    __syncthreads();
    if (kt + 1 < nk) {
      lstore();
      __syncthreads();
    }
  }
  uint16_t* C = is_v ? a.vc : a.kc;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const int r = m0 + wm + 32 * i + 8 * (e >> 2) + 4 * (lane >> 5) + (e & 3);
      if (r >= M) continue;
      const int bi = r / a.l, t = r - bi * a.l;
      uint16_t* crow = C + (int64_t)bi * a.c_bstride + (int64_t)t * a.h + wn0 + wn + (lane & 31);
#pragma unroll
      for (int j = 0; j < 2; ++j) crow[32 * j] = to_bits<KIND_F16>(acc[i][j][e]);
    }
  }
}

// [out, in] weights, large grids: 256 x 256 tiles, one workgroup of four waves
// per CU, each wave a 128 x 128 quarter as 4 x 4 MFMA blocks accumulating in
// AGPRs (one wave per SIMD, 512 registers).  Per FLOP that reads 2/3 of the
// LDS operand bytes of the 128 x 64 quarters and stages 2/3 of the global
// bytes.  With a single wave per SIMD nothing hides latency for it, so the
// loop is software-pipelined by hand and the order pinned with scheduling
// groups:
//   - the fragments of slice s + 1 are read from LDS while slice s's 16
//     MFMAs issue;
//   - the next step's data (loaded during the previous step) is written into
//     the other LDS buffer, and the loads of the step after it issued into the
//     freed registers, a quarter per slice between MFMAs;
//   - the one barrier per step sits before the last slice's MFMAs, whose
//     operands are already in registers, so the next step's first fragments
//     are read across it.
// The body is branch-free: loads past the last step re-read the last step
// (in bounds, never used).  The epilogue stages each wave's fp16 quarter in
// LDS and writes whole 16-byte row pieces.  Measured on MI355X (OPT-13B
// shape): 1.19 PFLOP/s against 0.91 for kv_recompute_kernel_k64 on the same
// data, with the clock at 1.6-1.7 GHz under this load; 2600 cycles per
// 64-wide K step against a 2048-cycle MFMA floor.
constexpr int WT = 256;                  // tile rows and columns
constexpr int WS = 64 + 8;               // LDS row stride of K-contiguous rows (bf16 elements)
constexpr int WP = WT + 16;              // LDS row stride of [in, out] W rows (N-contiguous)
constexpr int WBUF = 2 * WT * WS;        // one buffer: X rows, then W rows in either layout
constexpr int WLOADS = 2 * WT * 8 / 256; // 16-byte pieces per thread per step (8 X, 8 W)
constexpr int WES = 128 + 8;             // epilogue row stride (fp16 elements)
static_assert(WT * WS + 64 * WP <= WBUF, "an [in, out] W step fits in a buffer");
static_assert(4 * 128 * WES <= 2 * WBUF, "epilogue staging fits in the LDS buffers");

template <int N>
__device__ __forceinline__ void sched_mfma_lds_read() {
  if constexpr (N > 0) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one MFMA
    __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // one LDS read
    sched_mfma_lds_read<N - 1>();
  }
}
template <int N>
__device__ __forceinline__ void sched_mfma_stage() {
  if constexpr (N > 0) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
    __builtin_amdgcn_sched_group_barrier(0x200, 1, 0);  // LDS write
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
    __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);  // global load
    sched_mfma_stage<N - 1>();
  }
}
template <int N>
__device__ __forceinline__ void sched_mfma_stage_tight() {
  if constexpr (N > 0) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
    __builtin_amdgcn_sched_group_barrier(0x200, 1, 0);  // LDS write
    __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);  // global load
    sched_mfma_stage_tight<N - 1>();
  }
}
template <int N>
__device__ __forceinline__ void sched_mfma() {
  if constexpr (N > 0) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    sched_mfma<N - 1>();
  }
}

// gfx950 LDS transpose read of 16-bit data.  In each group of 16 lanes, lane j
// gets, as its element i, element j % 4 of the 8 bytes addressed by lane
// 4 * i + j / 4 of the group (checked with an in-bounds probe on MI355X).  So
// with lane s of a group pointing at row k0 + s / 4, columns n0 + 4 * (s % 4)
// of an N-contiguous tile, lane j receives rows k0 .. k0 + 3 of column n0 + j:
// four consecutive k of one column, as a K-contiguous MFMA operand wants.
__device__ __forceinline__ u32x2 lds_read_tr16(const uint16_t* p) {
  typedef __attribute__((__vector_size__(4 * sizeof(__bf16)))) __bf16 bf16x4_t;
  typedef __attribute__((address_space(3))) bf16x4_t* lds_ptr;
  return __builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_ptr)(const_cast<uint16_t*>(p))));
}

// Tile order: each XCD (workgroups are dealt to the 8 XCDs round robin) takes
// a contiguous run of tiles, ordered down columns of 4 tile-columns, so the
// workgroups resident on one XCD share X and W panels in its L2.
__device__ __forceinline__ void wide_tile(int blk, int tiles_m, int tiles_n, int& tm, int& tn) {
  const int T = tiles_m * tiles_n, q = T / 8, r = T % 8, x = blk % 8;
  const int L = x * q + min(x, r) + blk / 8;
  const int g = L / (tiles_m * 4), cb = g * 4, w = min(4, tiles_n - cb);
  const int in = L - g * tiles_m * 4;
  tm = in / w;
  tn = cb + in % w;
}

// 256 x 256 tiles for large grids, both W layouts.  [out, in] W rows are
// K-contiguous and are staged like X rows.  [in, out] W is staged as it lies,
// 64 rows (one K step) of 256 contiguous outputs, and each B fragment is two
// transpose reads of it (4 consecutive k each).
template <int WL>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1))) void kv_recompute_kernel_wide(RecomputeArgs a) {
  constexpr bool kInOut = WL == KVDEC_W_IN_OUT;
  constexpr int kBReads = kInOut ? 8 : 4;  // LDS reads of one slice's B fragments
  __shared__ __attribute__((aligned(16))) uint16_t S[2 * WBUF];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int M = a.b * a.l;
  int tm, tn;
  wide_tile(blockIdx.x, (M + WT - 1) / WT, 2 * a.h / WT, tm, tn);
  const int m0 = tm * WT, n0 = tn * WT;
  const bool is_v = n0 >= a.h;  // h % 256 == 0: a tile never straddles K | V
  const uint16_t* W = is_v ? a.wv : a.wk;
  const int wn0 = is_v ? n0 - a.h : n0;

  // X: thread -> 16-byte piece ak of tile rows ar + 32 i (rows past M re-read
  // row M - 1).  W [out, in]: the same for W rows (outputs) wn0 + ar + 32 i.
  // W [in, out]: piece wc of rows (inputs) wr + 8 i of the step.
  const int ar = tid >> 3, ak = (tid & 7) * 8;
  const int wr = tid >> 5, wc = (tid & 31) * 8;
  const uint16_t* src[WLOADS];
#pragma unroll
  for (int i = 0; i < WLOADS / 2; ++i) {
    const int r = min(m0 + ar + 32 * i, M - 1);
    const int bi = r / a.l, t = r - bi * a.l;
    src[i] = a.x + (int64_t)bi * a.x_bstride + (int64_t)t * a.h + ak;
    src[WLOADS / 2 + i] = kInOut ? W + (int64_t)(wr + 8 * i) * a.h + wn0 + wc
                                 : W + (int64_t)(wn0 + ar + 32 * i) * a.h + ak;
  }
  // element offset of step k0 for piece i
  auto koff = [&](int i, int k0) -> int64_t { return kInOut && i >= WLOADS / 2 ? (int64_t)k0 * a.h : k0; };
  auto dst = [&](int i) {
    if (i < WLOADS / 2) return (ar + 32 * i) * WS + ak;
    return kInOut ? WT * WS + (wr + 8 * (i - WLOADS / 2)) * WP + wc : (WT + ar + 32 * (i - WLOADS / 2)) * WS + ak;
  };

  const int wm = (wave >> 1) * 128, wn = (wave & 1) * 128;
  const int fa_off = (wm + (lane & 31)) * WS + 8 * (lane >> 5);
  const int g16 = lane >> 4, s16 = lane & 15;
  const int fb_off = kInOut ? WT * WS + (8 * (g16 >> 1) + (s16 >> 2)) * WP + wn + 16 * (g16 & 1) + 4 * (s16 & 3)
                            : (WT + wn + (lane & 31)) * WS + 8 * (lane >> 5);
  // A fragment i and B fragment j of K slice ks (16 k) from buffer `buf`.
  auto frag_a = [&](const uint16_t* buf, int ks, int i) {
    return *reinterpret_cast<const u32x4*>(&buf[fa_off + 32 * i * WS + 16 * ks]);
  };
  auto frag_b = [&](const uint16_t* buf, int ks, int j) {
    if constexpr (kInOut) {
      const uint16_t* p = buf + fb_off + 16 * ks * WP + 32 * j;
      const u32x2 lo = lds_read_tr16(p), hi = lds_read_tr16(p + 4 * WP);
      return u32x4{lo.x, lo.y, hi.x, hi.y};
    } else {
      return *reinterpret_cast<const u32x4*>(&buf[fb_off + 32 * j * WS + 16 * ks]);
    }
  };
  f32x16 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;

  const int nk = a.h / 64;  // >= 4
  u32x4 st[WLOADS];
#pragma unroll
  for (int i = 0; i < WLOADS; ++i) st[i] = load_b128(src[i]);
#pragma unroll
  for (int i = 0; i < WLOADS; ++i) store_b128(&S[dst(i)], st[i]);
#pragma unroll
  for (int i = 0; i < WLOADS; ++i) st[i] = load_b128(src[i] + koff(i, 64));
  __syncthreads();
  u32x4 fa[2][4], fb[2][4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    fa[0][i] = frag_a(S, 0, i);
    fb[0][i] = frag_b(S, 0, i);
  }
  for (int kt = 0; kt < nk; ++kt) {
    const uint16_t* cur = S + (kt & 1) * WBUF;
    uint16_t* nxt = S + ((kt + 1) & 1) * WBUF;
    const int k2 = min(kt + 2, nk - 1) * 64;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      const int c = ks & 1;
      if (ks < 3) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          fa[c ^ 1][i] = frag_a(cur, ks + 1, i);
          fb[c ^ 1][i] = frag_b(cur, ks + 1, i);
        }
      }
#pragma unroll
      for (int p = 0; p < WLOADS / 4; ++p) {
        const int i = ks * (WLOADS / 4) + p;
        store_b128(&nxt[dst(i)], st[i]);
        st[i] = load_b128(src[i] + koff(i, k2));
      }
      if (ks == 3) {
        // every wave's writes of nxt are done and its reads of cur issued
        __syncthreads();
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          fa[0][i] = frag_a(nxt, 0, i);
          fb[0][i] = frag_b(nxt, 0, i);
        }
      }
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
              __builtin_bit_cast(bf16x8, fa[c][i]), __builtin_bit_cast(bf16x8, fb[c][j]), acc[i][j], 0, 0, 0);
      if (ks < 3) {
        if constexpr (kInOut) {
          sched_mfma_lds_read<4 + kBReads>();
          sched_mfma_stage_tight<WLOADS / 4>();
        } else {
          sched_mfma_lds_read<4 + kBReads>();
          sched_mfma_stage<WLOADS / 4>();
        }
      } else {
        sched_mfma_lds_read<4 + kBReads>();
        sched_mfma<16 - 4 - kBReads>();
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  }

  // Epilogue: acc[i][j][e] = C[row wm + 32i + 8*(e/4) + 4*(lane/32) + e%4][col wn + 32j + lane%32];
  // each wave stages its quarter as fp16 rows in LDS, then writes 16-byte row pieces
  // with non-temporal stores: nothing reads them back in this kernel, while the X
  // and W panels in L2 are read again by the next round's tiles, and every CU
  // writes its 128 KB at the same moment at the end of a round (measured on
  // MI355X, one process, interleaved, bit-identical output: [out, in] W 5.3-8.1 us
  // shorter per call, [in, out] 2.8-2.9 us).
  __syncthreads();
  uint16_t* E = S + wave * (128 * WES);
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e)
        E[(32 * i + 8 * (e >> 2) + 4 * (lane >> 5) + (e & 3)) * WES + 32 * j + (lane & 31)] =
            to_bits<KIND_F16>(acc[i][j][e]);
  __syncthreads();
  uint16_t* C = is_v ? a.vc : a.kc;
#pragma unroll 4
  for (int c = 0; c < 32; ++c) {
    const int q = c * 64 + lane, row = q >> 4, col = (q & 15) * 8;
    const int r = m0 + wm + row;
    if (r < M) {
      const int bi = r / a.l, t = r - bi * a.l;
      store_b128<true>(C + (int64_t)bi * a.c_bstride + (int64_t)t * a.h + wn0 + wn + col,
                       *reinterpret_cast<const u32x4*>(&E[row * WES + col]));
    }
  }
}

}  // namespace

// The 256 x 256 kernel runs one workgroup per CU: below a chip's worth of
// tiles the 256 x 128 kernel (two per CU, twice the tiles) keeps more CUs busy.
constexpr int64_t kWideMinBlocks = 256;

hipError_t launch_kv_recompute(const RecomputeArgs& a, hipStream_t stream) {
  const int M = a.b * a.l, N = 2 * a.h;
  const int64_t blocks = (int64_t)((M + BM - 1) / BM) * (N / BN);
  const int64_t wide_blocks = (int64_t)((M + WT - 1) / WT) * (N / WT);
  if (wide_blocks >= kWideMinBlocks) {
    if (a.w_layout == KVDEC_W_OUT_IN)
      launch_timed(kv_recompute_kernel_wide<KVDEC_W_OUT_IN>, dim3((unsigned)wide_blocks), dim3(256), 0u, stream, a);
    else
      launch_timed(kv_recompute_kernel_wide<KVDEC_W_IN_OUT>, dim3((unsigned)wide_blocks), dim3(256), 0u, stream, a);
  } else if (a.w_layout == KVDEC_W_OUT_IN)
    launch_timed(kv_recompute_kernel_k64, dim3((unsigned)blocks), dim3(256), 0u, stream, a);
  else
    launch_timed(kv_recompute_kernel, dim3((unsigned)blocks), dim3(256), 0u, stream, a);
  return hipGetLastError();
}

}  // namespace kvdec

// device_common.h -- small gfx950 device helpers shared by the libkvdec kernels.
#pragma once

#include <stdint.h>

#include <hip/hip_runtime.h>

namespace kvdec {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

enum Kind : int { KIND_F16 = 0, KIND_BF16 = 1 };

// 16-byte global load.  `nt` marks streamed data (read once) as non-temporal.
template <bool NT = false>
__device__ __forceinline__ u32x4 load_b128(const void* p) {
  if constexpr (NT) return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
  else return *reinterpret_cast<const u32x4*>(p);
}

// Values the caller knows are equal across the wave (kept in scalar registers).
__device__ __forceinline__ uint32_t uniform_u32(uint32_t x) {
  return (uint32_t)__builtin_amdgcn_readfirstlane((int)x);
}
__device__ __forceinline__ int uniform_i32(int x) { return __builtin_amdgcn_readfirstlane(x); }
template <typename T>
__device__ __forceinline__ const T* uniform_ptr(const T* p) {
  const uint64_t u = reinterpret_cast<uint64_t>(p);
  const uint64_t lo = uniform_u32((uint32_t)u), hi = uniform_u32((uint32_t)(u >> 32));
  return reinterpret_cast<const T*>(lo | (hi << 32));
}

// Raw buffer resource over [base, base + nbytes): loads at offsets >= nbytes
// return zero and touch no memory.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t nbytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, (int)nbytes, 0x00020000);
}

// 16-byte buffer load marked non-temporal (streamed once).
__device__ __forceinline__ u32x4 buffer_load_b128_nt(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, 2);
}

// 8-byte buffer load marked non-temporal.
__device__ __forceinline__ u32x2 buffer_load_b64_nt(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b64(r, (int)off, 0, 2);
}

// 16-byte global store.  `nt` marks data no kernel of the call reads back
// as non-temporal.
template <bool NT = false>
__device__ __forceinline__ void store_b128(void* p, u32x4 v) {
  if constexpr (NT) __builtin_nontemporal_store(v, reinterpret_cast<u32x4*>(p));
  else *reinterpret_cast<u32x4*>(p) = v;
}

// Low / high 16-bit element of a packed pair, widened to fp32.
template <int KIND>
__device__ __forceinline__ float lo_f32(uint32_t w) {
  if constexpr (KIND == KIND_F16) {
    return (float)__builtin_bit_cast(_Float16, (uint16_t)(w & 0xffffu));
  } else {
    return __builtin_bit_cast(float, w << 16);
  }
}
template <int KIND>
__device__ __forceinline__ float hi_f32(uint32_t w) {
  if constexpr (KIND == KIND_F16) {
    return (float)__builtin_bit_cast(_Float16, (uint16_t)(w >> 16));
  } else {
    return __builtin_bit_cast(float, w & 0xffff0000u);
  }
}

// fp32 -> 16-bit, round to nearest even.
template <int KIND>
__device__ __forceinline__ uint16_t to_bits(float x) {
  if constexpr (KIND == KIND_F16) {
    return __builtin_bit_cast(uint16_t, (_Float16)x);
  } else {
    uint32_t u = __builtin_bit_cast(uint32_t, x);
    if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40u);  // quiet NaN
    u += 0x7fffu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
  }
}

// acc + a.lo * b.lo + a.hi * b.hi on packed 16-bit pairs, fp32 accumulate.
template <int KIND>
__device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float acc) {
  typedef _Float16 h2 __attribute__((ext_vector_type(2)));
  typedef __bf16 b2 __attribute__((ext_vector_type(2)));
  if constexpr (KIND == KIND_F16) {
    return __builtin_amdgcn_fdot2(__builtin_bit_cast(h2, a), __builtin_bit_cast(h2, b), acc, false);
  } else {
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(b2, a), __builtin_bit_cast(b2, b), acc,
                                           false);
  }
}

template <int CTRL>
__device__ __forceinline__ float dpp_f32(float x) {
  return __builtin_bit_cast(
      float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL, 0xF, 0xF, false));
}

// Sum over the 16 lanes of each row; every lane of the row gets the sum.
// Steps: swap neighbours, swap pairs (quad permutes), then mirror within
// half-rows and within the row.  Fixed order, so the result is deterministic.
__device__ __forceinline__ float row_sum16(float x) {
  x += dpp_f32<0xB1>(x);   // quad_perm [1,0,3,2]
  x += dpp_f32<0x4E>(x);   // quad_perm [2,3,0,1]
  x += dpp_f32<0x141>(x);  // row_half_mirror
  x += dpp_f32<0x140>(x);  // row_mirror
  return x;
}

// Row exchanges: from a value x, a pair (a, b) holding (row r, row r^1) for
// permlane16 and (half h, half h^1) for permlane32 in every lane, so a op b
// combines the partners.  The copy into b happens inside the same asm
// statement, so the pair lives only for this exchange.  Inline assembly,
// because the compiler builtins for these swaps hand back the first result
// for both outputs.  The s_nop pads cover the VALU-write / permlane-read
// hazard on either side.
__device__ __forceinline__ void permlane16_pair(uint32_t x, uint32_t& a, uint32_t& b) {
  a = x;
  asm volatile("v_mov_b32 %1, %0\n\ts_nop 1\n\tv_permlane16_swap_b32 %0, %1\n\ts_nop 1"
               : "+v"(a), "=&v"(b));
}
__device__ __forceinline__ void permlane32_pair(uint32_t x, uint32_t& a, uint32_t& b) {
  a = x;
  asm volatile("v_mov_b32 %1, %0\n\ts_nop 1\n\tv_permlane32_swap_b32 %0, %1\n\ts_nop 1"
               : "+v"(a), "=&v"(b));
}

// Combine the four 16-lane rows of the wave (every lane gets the result):
// rows 0<->1 and 2<->3 by permlane16 swap, then halves by permlane32 swap.
__device__ __forceinline__ float rowgroup_max(float x) {
  uint32_t a, b;
  permlane16_pair(__builtin_bit_cast(uint32_t, x), a, b);
  x = fmaxf(__builtin_bit_cast(float, a), __builtin_bit_cast(float, b));
  permlane32_pair(__builtin_bit_cast(uint32_t, x), a, b);
  return fmaxf(__builtin_bit_cast(float, a), __builtin_bit_cast(float, b));
}
__device__ __forceinline__ float rowgroup_sum(float x) {
  uint32_t a, b;
  permlane16_pair(__builtin_bit_cast(uint32_t, x), a, b);
  x = __builtin_bit_cast(float, a) + __builtin_bit_cast(float, b);
  permlane32_pair(__builtin_bit_cast(uint32_t, x), a, b);
  return __builtin_bit_cast(float, a) + __builtin_bit_cast(float, b);
}

// In-place exchanges of two registers across row pairs / wave halves:
// permlane16: the odd rows of a trade places with the even rows of b;
// permlane32: the upper half of a trades places with the lower half of b.
// Afterwards a + b pairs row r (half h) of a with row r^1 (half h^1) of a in
// the rows (halves) where a's own lanes stayed, and likewise for b.
__device__ __forceinline__ void permlane16_swap2(float& a, float& b) {
  asm volatile("s_nop 1\n\tv_permlane16_swap_b32 %0, %1\n\ts_nop 1" : "+v"(a), "+v"(b));
}
__device__ __forceinline__ void permlane32_swap2(float& a, float& b) {
  asm volatile("s_nop 1\n\tv_permlane32_swap_b32 %0, %1\n\ts_nop 1" : "+v"(a), "+v"(b));
}

// One halving step of a transposed reduction over lane bit `bit` (0..3) inside
// 16-lane rows: the lane keeps `lo` if its bit is clear, `hi` if set, and adds
// the partner's copy of the same one.  Partners: bit 3 by rotating a row by 8,
// bit 2 by mirroring each half-row (the partner differs in bit 2 and agrees in
// bits 3 and up), bits 1 and 0 by quad permutes.
template <int BIT>
__device__ __forceinline__ float transpose_step(float lo, float hi, int lane) {
  const bool up = (lane >> BIT) & 1;
  const float keep = up ? hi : lo, send = up ? lo : hi;
  if constexpr (BIT == 3) return keep + dpp_f32<0x128>(send);       // row_ror:8
  else if constexpr (BIT == 2) return keep + dpp_f32<0x141>(send);  // row_half_mirror
  else if constexpr (BIT == 1) return keep + dpp_f32<0x4E>(send);   // quad_perm [2,3,0,1]
  else return keep + dpp_f32<0xB1>(send);                           // quad_perm [1,0,3,2]
}

// Sums each of V = 16 or 32 values over the 64 lanes of the wave at once.
// Each level halves the number of registers: the lanes of one side keep the
// first half of the values, the other side the second half, and each adds its
// partner's copy; levels run over lane bits 5, 4, 3, ... .  The last levels,
// once one register is left, are plain pair sums.  On return lane l holds the
// full sum of value l / (64 / V).  Fixed order, so deterministic.  v is
// clobbered.
template <int V>
__device__ __forceinline__ float transpose_reduce(float (&v)[V], int lane) {
  static_assert(V == 16 || V == 32, "V must be 16 or 32");
#pragma unroll
  for (int i = 0; i < V / 2; ++i) {  // bit 5
    permlane32_swap2(v[i], v[V / 2 + i]);
    v[i] += v[V / 2 + i];
  }
#pragma unroll
  for (int i = 0; i < V / 4; ++i) {  // bit 4
    permlane16_swap2(v[i], v[V / 4 + i]);
    v[i] += v[V / 4 + i];
  }
#pragma unroll
  for (int i = 0; i < V / 8; ++i) v[i] = transpose_step<3>(v[i], v[V / 8 + i], lane);
#pragma unroll
  for (int i = 0; i < V / 16; ++i) v[i] = transpose_step<2>(v[i], v[V / 16 + i], lane);
  float x = v[0];
  if constexpr (V == 32) x = transpose_step<1>(v[0], v[1], lane);
  else x += dpp_f32<0x4E>(x);  // bit 1, plain
  x += dpp_f32<0xB1>(x);       // bit 0, plain
  return x;
}

}  // namespace kvdec

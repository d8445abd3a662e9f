// device_common.h -- small gfx950 device helpers shared by the libkvdec kernels.
#pragma once

#include <stdint.h>

#include <hip/hip_runtime.h>

namespace kvdec {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
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

__device__ __forceinline__ void store_b128(void* p, u32x4 v) {
  *reinterpret_cast<u32x4*>(p) = v;
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

// 16x16x32 MFMA on 8 packed 16-bit values per lane (fp32 accumulate).
template <int KIND>
__device__ __forceinline__ f32x4 mfma16x16x32(u32x4 a, u32x4 b, f32x4 c) {
  if constexpr (KIND == KIND_F16) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a),
                                                  __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
  } else {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
  }
}

// Value of lane J of this lane's 16-lane row (DPP row broadcast).
template <int J>
__device__ __forceinline__ float row_bcast(float x) {
  return __builtin_bit_cast(
      float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x150 + J, 0xF, 0xF, false));
}

__device__ __forceinline__ float xor_shfl(float x, int mask) { return __shfl_xor(x, mask, 64); }

// Compile-time loop: f(std::integral_constant<int, I>) for I in [0, N).
template <int I, int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (I < N) {
    f(std::integral_constant<int, I>{});
    static_for<I + 1, N>(f);
  }
}

__device__ __forceinline__ float ld_agent(const float* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

}  // namespace kvdec

// prefetch.hip -- CLO's miss-driven prefetch into the cache buffer, and the
// flags in host-mapped memory that order GPU work against host-side work
// without a host stream synchronisation.
//
// CLO page, section 3 (decoding flow, Figure 9): the lookup of layer l runs
// at the start of layer l-1, and the heads it misses are fetched while layer
// l-1 computes; Figure 7: an update writes the new KV rows straight to their
// final place in the cache buffer.  Section 2 (GPU-centric synchronisation)
// and the argument chain's row 8: the GPU polls an identifier variable in
// memory that host and GPU share, instead of the host blocking on the stream.
//
// Here the GPU pulls the selected rows from the pinned host pool itself, over
// PCIe, with no host-side gather and no staging copy; the host's part is to
// raise a flag once the pool rows are in place.
#include <algorithm>

#include "device_common.h"
#include "internal.h"

namespace kvdec {

// Waits until the 32-bit sequence number at `flag` reaches `target`
// ((int32)(value - target) >= 0), for at most `ticks` of the constant-rate
// wall clock and at most max_polls + 1 reads, then writes 0 (reached) or 1
// (gave up) to *status.  One lane polls; each read is a system-scope acquire,
// so host writes made before the flag was raised are visible to the work
// queued after this kernel.  Between reads the wave sleeps (s_sleep 127, at
// least 3 us at the highest clock), so max_polls also bounds the time if the
// clock were not to advance.
__global__ __launch_bounds__(64) void flag_wait_kernel(const uint32_t* flag, uint32_t target,
                                                       uint64_t ticks, uint32_t max_polls,
                                                       int32_t* status) {
  if (threadIdx.x != 0) return;
  const uint64_t t0 = wall_clock64();
  int32_t st = 1;
  for (uint32_t i = 0; i <= max_polls; ++i) {
    const uint32_t v = __hip_atomic_load(flag, __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_SYSTEM);
    if ((int32_t)(v - target) >= 0) {
      st = 0;
      break;
    }
    if (wall_clock64() - t0 >= ticks) break;
    __builtin_amdgcn_s_sleep(127);
  }
  __hip_atomic_store(status, st, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_SYSTEM);
}

// Raises `flag` to `value` once the work queued before it on the stream has
// finished: a system-scope release store, so a host thread polling the flag
// sees it after that work's writes.
__global__ __launch_bounds__(64) void flag_signal_kernel(uint32_t* flag, uint32_t value) {
  if (threadIdx.x != 0) return;
  __hip_atomic_store(flag, value, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_SYSTEM);
}

// The copy.  Work unit: kUnitSteps load steps of one missed (sequence, KV
// head) pair, one wave each; waves stride over the units of all misses, so
// the work spreads evenly whichever heads missed.  A row (one token of one
// head, 128 elements) is ROW_BYTES / 16 lanes of 16 bytes; one load
// instruction covers 64 * 16 / ROW_BYTES rows, and all of a unit's K and V
// loads are issued before the first store, so a wave keeps
// 2 * kUnitSteps * 1 KiB in flight to cover the PCIe round trip.
constexpr int kUnitSteps = 8;

template <int ROW_BYTES>
__global__ __launch_bounds__(256) void prefetch_rows_kernel(PrefetchArgs a) {
  constexpr int LPR = ROW_BYTES / 16;  // lanes per row
  constexpr int RPI = 64 / LPR;        // rows per load instruction
  constexpr int UNIT = RPI * kUnitSteps;
  if (a.status && __hip_atomic_load(a.status, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != 0)
    return;  // the wait for the host's flag gave up: copy nothing
  // Pool rows the host wrote before raising the flag must not be served from
  // a line of this XCD's L2 that an earlier read left there: a system-scope
  // acquire drops those lines before this workgroup reads the pool.
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "");

  const int lane = threadIdx.x & 63;
  const int pairs = a.B * a.Hkv;
  const int n_miss = min(max(__hip_atomic_load(a.miss_count, __ATOMIC_RELAXED,
                                               __HIP_MEMORY_SCOPE_AGENT), 0), pairs);
  // units per pair; at least one, which also sets buf_len of an empty selection
  const int upp = max((a.max_rows + UNIT - 1) / UNIT, 1);
  const int64_t n_units = (int64_t)n_miss * upp;
  const int64_t n_waves = (int64_t)gridDim.x * 4;
  const char* pk = static_cast<const char*>(a.pool_k);
  const char* pv = static_cast<const char*>(a.pool_v);
  char* bk = static_cast<char*>(a.buf_k);
  char* bv = static_cast<char*>(a.buf_v);
  const int piece = lane % LPR;

  for (int64_t u = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6); u < n_units; u += n_waves) {
    const int m = (int)(u / upp), c = (int)(u % upp);
    const int pair = uniform_i32(a.miss_list[m]);
    if (pair < 0 || pair >= pairs) continue;  // not a (sequence, KV head) of this batch
    const int b = pair / a.Hkv, g = pair % a.Hkv;
    if (a.head_map && a.head_map[g] >= 0) continue;  // persistent head: always resident
    const int n = uniform_i32(min(max(a.idx_len[pair], 0), a.max_rows));
    if (c == 0 && lane == 0) a.buf_len[pair] = n;
    const int r0 = c * UNIT;
    if (r0 >= n) continue;

    const int32_t* idx = a.idx + (int64_t)pair * a.max_k;
    const int64_t head_off = (int64_t)b * a.stride_b + (int64_t)g * a.stride_h;
    const int64_t dst0 = (int64_t)pair * a.buf_cap;
    int64_t src[kUnitSteps];
    int row[kUnitSteps];
    // the index loads are unconditional (rows past n re-read row n - 1), so
    // all of them are in flight together
    int t[kUnitSteps];
#pragma unroll
    for (int s = 0; s < kUnitSteps; ++s) {
      row[s] = r0 + s * RPI + lane / LPR;
      t[s] = idx[min(row[s], n - 1)];
    }
#pragma unroll
    for (int s = 0; s < kUnitSteps; ++s)
      src[s] = (head_off + (int64_t)min(max(t[s], 0), a.S - 1) * a.stride_s) * a.elem_bytes +
               piece * 16;
    u32x4 kr[kUnitSteps], vr[kUnitSteps];
#pragma unroll
    for (int s = 0; s < kUnitSteps; ++s) {
      if (row[s] < n) {
        kr[s] = *reinterpret_cast<const u32x4*>(pk + src[s]);
        vr[s] = *reinterpret_cast<const u32x4*>(pv + src[s]);
      }
    }
#pragma unroll
    for (int s = 0; s < kUnitSteps; ++s) {
      if (row[s] < n) {
        const int64_t dst = (dst0 + row[s]) * ROW_BYTES + piece * 16;
        __builtin_nontemporal_store(kr[s], reinterpret_cast<u32x4*>(bk + dst));
        __builtin_nontemporal_store(vr[s], reinterpret_cast<u32x4*>(bv + dst));
      }
    }
  }
}

hipError_t launch_flag_wait(const uint32_t* flag, uint32_t target, uint64_t ticks,
                            uint32_t max_polls, int32_t* status, hipStream_t stream) {
  hipLaunchKernelGGL(flag_wait_kernel, dim3(1), dim3(64), 0, stream, flag, target, ticks,
                     max_polls, status);
  return hipGetLastError();
}

hipError_t launch_flag_signal(uint32_t* flag, uint32_t value, hipStream_t stream) {
  hipLaunchKernelGGL(flag_signal_kernel, dim3(1), dim3(64), 0, stream, flag, value);
  return hipGetLastError();
}

hipError_t launch_prefetch(const PrefetchArgs& a, hipStream_t stream) {
  const int row_bytes = kHeadDim * a.elem_bytes;
  const int unit = (64 * 16 / row_bytes) * kUnitSteps;
  const int64_t units = (int64_t)a.B * a.Hkv * std::max((a.max_rows + unit - 1) / unit, 1);
  const int64_t blocks = std::max<int64_t>(1, std::min<int64_t>((int64_t)device_cu_count() * 4,
                                                                (units + 3) / 4));
  hipEvent_t e0, e1;
  timing_events(&e0, &e1);
  if (row_bytes == 256)
    hipExtLaunchKernelGGL(prefetch_rows_kernel<256>, dim3((uint32_t)blocks), dim3(256), 0, stream,
                          e0, e1, 0u, a);
  else
    hipExtLaunchKernelGGL(prefetch_rows_kernel<128>, dim3((uint32_t)blocks), dim3(256), 0, stream,
                          e0, e1, 0u, a);
  return hipGetLastError();
}

}  // namespace kvdec

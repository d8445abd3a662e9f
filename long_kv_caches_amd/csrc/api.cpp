// api.cpp -- the libkvdec C ABI: argument validation, work planning and
// launches.  Every check runs on the host before anything is enqueued.
#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <stdlib.h>

#include <algorithm>
#include <atomic>
#include <cmath>
#include <mutex>
#include <utility>
#include <vector>

#include "internal.h"

namespace kvdec {

static thread_local char g_err[512] = "";

kvdec_status fail(kvdec_status st, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof g_err, fmt, ap);
  va_end(ap);
  return st;
}

static kvdec_status ok() {
  g_err[0] = '\0';
  return KVDEC_OK;
}

static kvdec_status hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return ok();
  return fail(KVDEC_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

// Work plan of the attention kernels.  With split_tokens = 0 the balanced
// schedule runs a persistent grid whose waves take items of the tile line
// (all tiles of all pairs, laid out on the device from the actual lengths)
// until none is left.  With split_tokens > 0, or when the tile line has more
// units than the balanced kernel keeps in LDS or more tiles than an int
// indexes, one workgroup handles each chunk of split_tokens tokens of a
// (sequence, KV head) pair.
struct Plan {
  int mode;
  int max_len;
  int chunk, n_chunks;    // chunks
  int n_blocks, n_units;  // balanced
  int n_cu;               // balanced
  int xcd_rounds;         // balanced: dispatch rounds (workgroups per CU) that allow XCD-local columns
  int xcd_w;              // balanced: per 100, the share of a column on an odd XCD, if XCD-local
  int64_t max_items;      // balanced: columns of the line
  int line_heads;         // balanced: heads run per line item
};

static constexpr int64_t kTargetItems = 2048;
static constexpr int kMinChunk = 128;
static constexpr int kChunkQuantum = kTile * kWaves;  // 64

static int round_up(int64_t x, int q) { return (int)(((x + q - 1) / q) * q); }

static Plan plan_attn(int dtype, int kv8, int G, int src, int64_t pairs, int64_t n_units,
                      int64_t est_tokens, int max_len, int split_tokens) {
  Plan p = {};
  p.max_len = std::max(max_len, 0);
  const int64_t est_tiles = pairs * ((std::max(max_len, 1) + kTile - 1) / kTile);
  if (split_tokens == 0 && n_units <= kMaxUnits && est_tiles < (int64_t(1) << 30)) {
    p.mode = MODE_BALANCED;
    p.n_units = (int)n_units;
    // at least one wave per line head: with fewer, no column exists and
    // some heads would never be run
    const int64_t LH = pairs / std::max<int64_t>(n_units, 1);
    p.n_blocks = (int)std::max<int64_t>(balanced_blocks(dtype, kv8, G, src, est_tiles),
                                        (LH + kWaves - 1) / kWaves);
    p.n_cu = device_cu_count();
    // XCD-local columns with one workgroup per CU, and with two for bf16 K/V
    // read from runs (measured on MI355X, one process, interleaved: the
    // 16 x 16K-32K batch in bf16, two workgroups per CU, 2.4-2.9 us shorter;
    // e4m3 and gathered rows, also at two, 0.7-1.5 us longer)
    p.xcd_rounds = dtype == KVDEC_BF16 && !kv8 && src != SRC_GATHER ? 2 : 1;
    // Wc = W / LH columns of the line, slots (column + unit) * LH + h.
    p.max_items = (int64_t)p.n_blocks * kWaves / std::max<int64_t>(LH, 1);
    p.line_heads = (int)LH;
    p.xcd_w = balanced_odd_xcd_weight(p.line_heads, src);
    return p;
  }
  p.mode = MODE_CHUNKS;
  const int full = std::max(kChunkQuantum, round_up(std::max(max_len, 1), kChunkQuantum));
  if (split_tokens > 0) {
    p.chunk = std::min(split_tokens, full);
  } else {
    int64_t c = (est_tokens + kTargetItems - 1) / kTargetItems;
    c = std::max<int64_t>(c, kMinChunk);
    p.chunk = std::min(round_up(c, kChunkQuantum), full);
  }
  p.n_chunks = (std::max(max_len, 1) + p.chunk - 1) / p.chunk;
  p.max_len = std::min<int64_t>((int64_t)p.n_chunks * p.chunk, std::max(max_len, 0));
  return p;
}

static kvdec_status check_common(const kvdec_attn_desc* d, bool check_layout) {
  if (!d) return fail(KVDEC_ERR_INVALID, "desc is NULL");
  if (d->batch < 0) return fail(KVDEC_ERR_INVALID, "batch < 0");
  if (d->num_q_heads < 1 || d->num_kv_heads < 1)
    return fail(KVDEC_ERR_INVALID, "num_q_heads and num_kv_heads must be >= 1");
  if (d->num_q_heads % d->num_kv_heads != 0)
    return fail(KVDEC_ERR_INVALID, "num_q_heads %% num_kv_heads != 0");
  if (d->num_q_heads / d->num_kv_heads > kMaxGroup)
    return fail(KVDEC_ERR_UNSUPPORTED, "query heads per KV head > %d", kMaxGroup);
  if (d->head_dim != kHeadDim) return fail(KVDEC_ERR_UNSUPPORTED, "head_dim must be 128");
  if (d->dtype != KVDEC_F16 && d->dtype != KVDEC_BF16)
    return fail(KVDEC_ERR_UNSUPPORTED, "dtype must be KVDEC_F16 or KVDEC_BF16");
  if (!isfinite(d->softmax_scale)) return fail(KVDEC_ERR_INVALID, "softmax_scale not finite");
  if (d->split_tokens < 0 || d->split_tokens % kChunkQuantum != 0)
    return fail(KVDEC_ERR_INVALID, "split_tokens must be 0 or a positive multiple of 64");
  if (d->kv_format != KVDEC_KV_SAME && d->kv_format != KVDEC_KV_E4M3)
    return fail(KVDEC_ERR_UNSUPPORTED, "unknown kv_format %d", d->kv_format);
  if (d->kv_format == KVDEC_KV_E4M3 &&
      !(isfinite(d->k_scale) && isfinite(d->v_scale) && d->k_scale > 0.f && d->v_scale > 0.f))
    return fail(KVDEC_ERR_INVALID, "e4m3 K/V need finite k_scale, v_scale > 0");
  if (check_layout) {
    if (d->layout != KVDEC_DENSE && d->layout != KVDEC_RAGGED && d->layout != KVDEC_PAGED)
      return fail(KVDEC_ERR_INVALID, "unknown layout %d", d->layout);
    if (d->max_seqlen < 0) return fail(KVDEC_ERR_INVALID, "max_seqlen < 0");
    if (d->layout == KVDEC_PAGED) {
      if (d->page_size < 16 || d->page_size % 16 != 0)
        return fail(KVDEC_ERR_UNSUPPORTED, "page_size must be a positive multiple of 16");
      if (d->max_pages_per_seq < 1) return fail(KVDEC_ERR_INVALID, "max_pages_per_seq < 1");
      if ((int64_t)d->max_pages_per_seq * d->page_size < d->max_seqlen)
        return fail(KVDEC_ERR_INVALID, "max_pages_per_seq * page_size < max_seqlen");
      if (d->kv_rows < 1 || d->kv_rows > INT32_MAX)
        return fail(KVDEC_ERR_INVALID, "kv_rows (pages in the pool) must be in [1, 2^31)");
    }
    if (d->layout == KVDEC_RAGGED && (d->kv_rows < 0 || d->kv_rows > INT32_MAX))
      return fail(KVDEC_ERR_INVALID, "kv_rows (token rows) must be in [0, 2^31)");
  }
  return ok();
}

static Plan plan_decode(const kvdec_attn_desc* d) {
  const int64_t pairs = (int64_t)d->batch * d->num_kv_heads;
  const int src = d->layout == KVDEC_DENSE ? SRC_DENSE : d->layout == KVDEC_RAGGED ? SRC_RAGGED : SRC_PAGED;
  return plan_attn(d->dtype, d->kv_format == KVDEC_KV_E4M3, d->num_q_heads / d->num_kv_heads, src,
                   pairs, d->batch, pairs * (int64_t)d->max_seqlen, d->max_seqlen, d->split_tokens);
}

static Plan plan_hybrid(const kvdec_hybrid_desc* h) {
  const kvdec_attn_desc* d = &h->base;
  const int64_t pairs = (int64_t)d->batch * d->num_kv_heads;
  const int64_t est = (int64_t)d->batch *
                      ((int64_t)h->num_pers_slots * h->pers_cap + (int64_t)d->num_kv_heads * h->buf_cap);
  return plan_attn(d->dtype, d->kv_format == KVDEC_KV_E4M3, d->num_q_heads / d->num_kv_heads,
                   SRC_HYBRID, pairs, pairs, est, std::max(h->pers_cap, h->buf_cap),
                   d->split_tokens);
}

// Partial slots and column-table entries the plan needs in the workspace.
static void ws_shape(const kvdec_attn_desc* d, const Plan& p, int64_t* slots, int64_t* n_cols) {
  const int64_t pairs = (int64_t)d->batch * d->num_kv_heads;
  if (p.mode == MODE_BALANCED) {
    // slot (item + unit) * LH + h; each unit's first and last column
    // [n_units][2]
    *slots = (p.max_items + p.n_units) * p.line_heads;
    *n_cols = 2 * (int64_t)p.n_units;
  } else {
    *slots = p.n_chunks > 1 ? pairs * p.n_chunks : 0;
    *n_cols = 0;
  }
}

static size_t attn_ws(const kvdec_attn_desc* d, const Plan& p) {
  if (d->batch == 0) return 0;
  int64_t slots, n_cols;
  ws_shape(d, p, &slots, &n_cols);
  if (slots == 0 && n_cols == 0) return 0;
  return attn_workspace_bytes(slots, d->num_q_heads / d->num_kv_heads, n_cols);
}

static void fill_common(const kvdec_attn_desc* d, const Plan& p, AttnArgs* a) {
  a->B = d->batch;
  a->Hq = d->num_q_heads;
  a->Hkv = d->num_kv_heads;
  a->G = d->num_q_heads / d->num_kv_heads;
  a->mode = p.mode;
  a->max_len = p.max_len;
  a->chunk = p.chunk;
  a->n_chunks = p.n_chunks;
  a->n_blocks = p.n_blocks;
  a->n_units = p.n_units;
  a->n_cu = p.n_cu;
  a->xcd_cols = p.mode == MODE_BALANCED &&
                balanced_xcd_cols(p.line_heads, p.n_blocks, p.n_cu * p.xcd_rounds);
  a->xcd_w = a->xcd_cols ? p.xcd_w : 100;
  a->kv8 = d->kv_format == KVDEC_KV_E4M3;
  // e4m3 K: scale * q . (k_scale * code) = (scale * k_scale) * q . code
  a->scale_log2 = (float)((double)d->softmax_scale * (a->kv8 ? (double)d->k_scale : 1.0) *
                          1.4426950408889634074);
  a->out_scale = a->kv8 ? d->v_scale : 1.f;
  a->dtype = d->dtype;
}

static kvdec_status run_attn(const kvdec_attn_desc* d, const Plan& p, AttnArgs& a, void* ws,
                             size_t ws_bytes, hipStream_t stream) {
  int64_t slots, n_cols;
  ws_shape(d, p, &slots, &n_cols);
  if (slots > 0 || n_cols > 0) {
    if (!attn_workspace_carve(ws, ws_bytes, slots, a.G, n_cols, &a))
      return fail(KVDEC_ERR_WORKSPACE, "workspace needs %zu bytes, got %zu%s", attn_ws(d, p),
                  ws_bytes, ws ? "" : " (NULL)");
    if (reinterpret_cast<uintptr_t>(ws) % 16 != 0)
      return fail(KVDEC_ERR_WORKSPACE, "workspace must be 16-byte aligned");
  }
  if (p.mode == MODE_CHUNKS && (int64_t)d->batch * p.n_chunks * d->num_kv_heads > INT32_MAX)
    return fail(KVDEC_ERR_UNSUPPORTED, "grid too large");
  return hip_status(launch_decode_attn(a, stream), "decode attention launch");
}

// Kernel timing: per thread, a pool of event pairs reused from one
// kvdec_kernel_timing(1) to the next.
struct TimingState {
  bool on = false;
  size_t used = 0;
  std::vector<std::pair<hipEvent_t, hipEvent_t>> pool;
  hipError_t err = hipSuccess;
};
static thread_local TimingState g_timing;

void timing_events(hipEvent_t* start, hipEvent_t* stop) {
  *start = *stop = nullptr;
  TimingState& t = g_timing;
  if (!t.on || t.err != hipSuccess) return;
  if (t.used == t.pool.size()) {
    hipEvent_t e0 = nullptr, e1 = nullptr;
    if ((t.err = hipEventCreate(&e0)) != hipSuccess) return;
    if ((t.err = hipEventCreate(&e1)) != hipSuccess) {
      (void)hipEventDestroy(e0);
      return;
    }
    t.pool.emplace_back(e0, e1);
  }
  *start = t.pool[t.used].first;
  *stop = t.pool[t.used].second;
  ++t.used;
}

// Checks the kvdec_headcache_lookup arguments and fills a.
static kvdec_status lookup_args(int32_t B, int32_t Hq, int32_t Hkv, int32_t D, int32_t dtype,
                                const void* q, void* labels, const float* weights,
                                const float* tau, uint8_t* hit, float* agg, float* cos,
                                int32_t* miss_list, int32_t* miss_count, LookupArgs* a) {
  if (B < 0 || Hq < 1 || Hkv < 1) return fail(KVDEC_ERR_INVALID, "bad B / Hq / Hkv");
  if (Hq % Hkv != 0) return fail(KVDEC_ERR_INVALID, "Hq %% Hkv != 0");
  if (Hq / Hkv > 16) return fail(KVDEC_ERR_UNSUPPORTED, "query heads per KV head > 16");
  if (D != kHeadDim) return fail(KVDEC_ERR_UNSUPPORTED, "D must be 128");
  if (dtype != KVDEC_F16 && dtype != KVDEC_BF16) return fail(KVDEC_ERR_UNSUPPORTED, "bad dtype");
  if ((int64_t)B * Hkv > INT32_MAX / 4 || (int64_t)B * Hq * D > INT32_MAX)
    return fail(KVDEC_ERR_UNSUPPORTED, "B * Hkv too large");
  if (B == 0) return ok();
  if (!q || !labels || !weights || !tau || !hit)
    return fail(KVDEC_ERR_INVALID, "q, labels, weights, tau and hit must be non-NULL");
  if ((miss_list == nullptr) != (miss_count == nullptr))
    return fail(KVDEC_ERR_INVALID, "miss_list and miss_count go together");
  a->q = static_cast<const uint16_t*>(q);
  a->labels = static_cast<uint16_t*>(labels);
  a->w = weights;
  a->tau = tau;
  a->hit = hit;
  a->agg = agg;
  a->cos = cos;
  a->miss_list = miss_list;
  a->miss_count = miss_count;
  a->B = B;
  a->Hq = Hq;
  a->Hkv = Hkv;
  a->G = Hq / Hkv;
  a->dtype = dtype;
  return ok();
}

// Checks the kvdec_kv_recompute arguments and fills a.
static kvdec_status recompute_args(int32_t b, int32_t l, int32_t h, int32_t num_heads,
                                   int32_t head_dim, const void* x, int64_t x_batch_stride,
                                   const void* w_k, const void* w_v, int32_t w_layout,
                                   void* k_cache, void* v_cache, int64_t cache_batch_stride,
                                   RecomputeArgs* a) {
  if (b < 0 || l < 0 || h < 1 || num_heads < 1) return fail(KVDEC_ERR_INVALID, "bad sizes");
  if (w_layout != KVDEC_W_IN_OUT && w_layout != KVDEC_W_OUT_IN)
    return fail(KVDEC_ERR_INVALID, "w_layout must be KVDEC_W_IN_OUT or KVDEC_W_OUT_IN");
  if (head_dim != kHeadDim) return fail(KVDEC_ERR_UNSUPPORTED, "head_dim must be 128");
  if ((int64_t)num_heads * head_dim != h) return fail(KVDEC_ERR_INVALID, "h != num_heads * head_dim");
  if (h % 256 != 0) return fail(KVDEC_ERR_UNSUPPORTED, "h must be a multiple of 256");
  if (x_batch_stride < (int64_t)l * h || cache_batch_stride < (int64_t)l * h)
    return fail(KVDEC_ERR_INVALID, "batch strides smaller than l * h");
  if (b == 0 || l == 0) return ok();
  if (!x || !w_k || !w_v || !k_cache || !v_cache)
    return fail(KVDEC_ERR_INVALID, "x, w_k, w_v, k_cache and v_cache must be non-NULL");
  a->x = static_cast<const uint16_t*>(x);
  a->wk = static_cast<const uint16_t*>(w_k);
  a->wv = static_cast<const uint16_t*>(w_v);
  a->kc = static_cast<uint16_t*>(k_cache);
  a->vc = static_cast<uint16_t*>(v_cache);
  a->x_bstride = x_batch_stride;
  a->c_bstride = cache_batch_stride;
  a->b = b;
  a->l = l;
  a->h = h;
  a->w_layout = w_layout;
  return ok();
}

// Library-owned scratch of kvdec_decode_attn_noalloc: the attention kernels'
// per-call partials, for callers that cannot allocate.  The array's name is a
// host-side stand-in in host code; kernels get the device address that
// hipGetSymbolAddress returns, fetched once per device with that device
// current.  Nothing in it needs to start at zero (the kernels write every
// partial before they read it).
static __device__ __align__(256) unsigned char scratch[KVDEC_NOALLOC_SCRATCH_BYTES];

static constexpr int kMaxDevices = 64;
static std::atomic<void*> g_scratch_addr[kMaxDevices];
static std::mutex g_scratch_mu;

static kvdec_status scratch_address(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_status(e, "hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices)
    return fail(KVDEC_ERR_UNSUPPORTED, "device index %d >= %d", dev, kMaxDevices);
  void* p = g_scratch_addr[dev].load(std::memory_order_acquire);
  if (!p) {
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    p = g_scratch_addr[dev].load(std::memory_order_relaxed);
    if (!p) {
      e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
      if (e != hipSuccess || !p) return hip_status(e, "hipGetSymbolAddress(scratch)");
      g_scratch_addr[dev].store(p, std::memory_order_release);
    }
  }
  *out = p;
  return ok();
}


// Memory the GPU reads or writes outside the caller's device buffers must be
// memory HIP knows: pinned host memory (hipHostMalloc, or torch's pinned
// tensors) or device memory.  A GPU access to pageable host memory faults,
// so it is refused here.  Checks that [p, p + bytes) lies in one such
// allocation and returns the address kernels use for p.
static kvdec_status mapped_range(const void* p, size_t bytes, bool host_only, const char* what,
                                 void** dev) {
  hipPointerAttribute_t at = {};
  hipError_t e = hipPointerGetAttributes(&at, p);
  if (e != hipSuccess) {
    (void)hipGetLastError();  // clear the runtime's last error: this failure is reported here
    return fail(KVDEC_ERR_INVALID,
                "%s is not memory HIP knows (host memory must be pinned, e.g. hipHostMalloc)", what);
  }
  const bool host = at.type == hipMemoryTypeHost;
  if (!host && (host_only || at.type != hipMemoryTypeDevice))
    return fail(KVDEC_ERR_INVALID, "%s must be pinned host memory%s (memory type %d)", what,
                host_only ? "" : " or device memory", (int)at.type);
  if (!at.devicePointer) return fail(KVDEC_ERR_INVALID, "%s has no device mapping", what);
  hipDeviceptr_t base = nullptr;
  size_t size = 0;
  e = hipMemGetAddressRange(&base, &size, const_cast<void*>(p));
  if (e == hipSuccess) {
    const uintptr_t lo = reinterpret_cast<uintptr_t>(base), at_p = reinterpret_cast<uintptr_t>(p);
    if (at_p < lo || at_p - lo + bytes > size)
      return fail(KVDEC_ERR_INVALID, "%s: %zu bytes from it run past its allocation (%zu bytes)",
                  what, bytes, size - (at_p - lo));
  } else {
    // no range query for this memory: the last byte must be mapped the same way
    (void)hipGetLastError();
    hipPointerAttribute_t end = {};
    if (bytes > 1) {
      e = hipPointerGetAttributes(&end, static_cast<const char*>(p) + bytes - 1);
      if (e != hipSuccess || end.type != at.type) {
        (void)hipGetLastError();
        return fail(KVDEC_ERR_INVALID, "%s: %zu bytes from it are not all in known memory", what,
                    bytes);
      }
    }
  }
  *dev = at.devicePointer;
  return ok();
}

// Ticks per microsecond of the constant-rate clock kernels read (wall_clock64).
static uint64_t wall_ticks_per_us() {
  static std::atomic<int> cached[kMaxDevices];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
    (void)hipGetLastError();
    return 100;
  }
  int khz = cached[dev].load(std::memory_order_relaxed);
  if (khz <= 0) {
    if (hipDeviceGetAttribute(&khz, hipDeviceAttributeWallClockRate, dev) != hipSuccess ||
        khz <= 0) {
      (void)hipGetLastError();
      khz = 100000;
    }
    cached[dev].store(khz, std::memory_order_relaxed);
  }
  return (uint64_t)std::max(khz / 1000, 1);
}

static constexpr uint32_t kMaxTimeoutUs = 1000000;

// Checks a flag wait's arguments and returns the device addresses of flag
// and status (each any HIP-known memory, 4-byte aligned).
static kvdec_status flag_wait_args(const uint32_t* flag, uint32_t timeout_us, int32_t* status,
                                   void** fdev, void** sdev) {
  if (!flag || !status) return fail(KVDEC_ERR_INVALID, "flag and status must be non-NULL");
  if (timeout_us > kMaxTimeoutUs)
    return fail(KVDEC_ERR_INVALID, "timeout_us must be <= %u", kMaxTimeoutUs);
  if (reinterpret_cast<uintptr_t>(flag) % 4 || reinterpret_cast<uintptr_t>(status) % 4)
    return fail(KVDEC_ERR_INVALID, "flag and status must be 4-byte aligned");
  kvdec_status st = mapped_range(flag, 4, false, "flag", fdev);
  if (st != KVDEC_OK) return st;
  return mapped_range(status, 4, false, "status", sdev);
}

static kvdec_status enqueue_flag_wait(void* fdev, uint32_t value, uint32_t timeout_us, void* sdev,
                                      hipStream_t stream) {
  const uint64_t ticks = (uint64_t)timeout_us * wall_ticks_per_us();
  return hip_status(launch_flag_wait(static_cast<const uint32_t*>(fdev), value, ticks,
                                     timeout_us + 1, static_cast<int32_t*>(sdev), stream),
                    "flag wait launch");
}


// ---------------------------------------------------------------------------
// Debug validation of device-resident metadata, on when the environment holds
// KVDEC_CHECK=1.  The kernels clamp malformed metadata so that it cannot make
// them fault; this mode copies the metadata to the host instead (after the
// work already queued on the stream, which may be what writes it), and
// rejects what the kernels would clamp, before anything is launched.
// ---------------------------------------------------------------------------
static bool check_mode() {
  const char* e = getenv("KVDEC_CHECK");
  return e && e[0] == '1' && e[1] == '\0';
}

template <typename T>
static kvdec_status fetch(std::vector<T>* h, const T* d, size_t n, hipStream_t stream,
                          const char* what) {
  h->assign(n, T());
  if (n == 0) return ok();
  if (!d) return fail(KVDEC_ERR_INVALID, "KVDEC_CHECK: %s is NULL", what);
  hipError_t e = hipMemcpyAsync(h->data(), d, n * sizeof(T), hipMemcpyDeviceToHost, stream);
  if (e == hipSuccess) e = hipStreamSynchronize(stream);
  if (e != hipSuccess) return hip_status(e, what);
  return ok();
}

static kvdec_status check_decode_meta(const kvdec_attn_desc* d, const int32_t* seqlens,
                                      const int32_t* cu, const int32_t* bt, hipStream_t stream) {
  const int B = d->batch;
  std::vector<int32_t> h;
  kvdec_status st;
  if (d->layout == KVDEC_RAGGED) {
    if ((st = fetch(&h, cu, (size_t)B + 1, stream, "cu_seqlens")) != KVDEC_OK) return st;
    if (h[0] != 0) return fail(KVDEC_ERR_INVALID, "KVDEC_CHECK: cu_seqlens[0] = %d, not 0", h[0]);
    for (int b = 0; b < B; ++b) {
      if (h[b + 1] < h[b])
        return fail(KVDEC_ERR_INVALID, "KVDEC_CHECK: cu_seqlens decreases at %d (%d after %d)",
                    b + 1, h[b + 1], h[b]);
      if (h[b + 1] - h[b] > d->max_seqlen)
        return fail(KVDEC_ERR_INVALID, "KVDEC_CHECK: sequence %d has %d tokens > max_seqlen %d",
                    b, h[b + 1] - h[b], d->max_seqlen);
    }
    if (h[B] > d->kv_rows)
      return fail(KVDEC_ERR_INVALID, "KVDEC_CHECK: cu_seqlens[%d] = %d > kv_rows %lld", B, h[B],
                  (long long)d->kv_rows);
    return ok();
  }
  if (!seqlens) return ok();  // dense: every length is max_seqlen
  if ((st = fetch(&h, seqlens, (size_t)B, stream, "seqlens")) != KVDEC_OK) return st;
  for (int b = 0; b < B; ++b)
    if (h[b] < 0 || h[b] > d->max_seqlen)
      return fail(KVDEC_ERR_INVALID, "KVDEC_CHECK: seqlens[%d] = %d outside [0, max_seqlen %d]",
                  b, h[b], d->max_seqlen);
  if (d->layout != KVDEC_PAGED) return ok();
  std::vector<int32_t> t;
  const int mp = d->max_pages_per_seq;
  if ((st = fetch(&t, bt, (size_t)B * mp, stream, "block_table")) != KVDEC_OK) return st;
  for (int b = 0; b < B; ++b)
    for (int p = 0; p < (h[b] + d->page_size - 1) / d->page_size; ++p) {
      const int id = t[(size_t)b * mp + p];
      if (id < 0 || id >= d->kv_rows)
        return fail(KVDEC_ERR_INVALID, "KVDEC_CHECK: block_table[%d][%d] = %d outside [0, %lld)",
                    b, p, id, (long long)d->kv_rows);
    }
  return ok();
}

static kvdec_status check_hybrid_meta(const kvdec_hybrid_desc* hd, const int32_t* pers_len,
                                      const int32_t* buf_len, const int32_t* head_map,
                                      hipStream_t stream) {
  const int B = hd->base.batch, Hkv = hd->base.num_kv_heads;
  std::vector<int32_t> hm, pl, bl;
  kvdec_status st;
  if ((st = fetch(&hm, head_map, (size_t)Hkv, stream, "head_map")) != KVDEC_OK) return st;
  bool pers = false;
  for (int g = 0; g < Hkv; ++g) {
    if (hm[g] < -1 || hm[g] >= hd->num_pers_slots)
      return fail(KVDEC_ERR_INVALID, "KVDEC_CHECK: head_map[%d] = %d is neither -1 nor a slot "
                  "in [0, %d)", g, hm[g], hd->num_pers_slots);
    pers |= hm[g] >= 0;
  }
  if (pers) {
    if ((st = fetch(&pl, pers_len, (size_t)B, stream, "pers_len")) != KVDEC_OK) return st;
    for (int b = 0; b < B; ++b)
      if (pl[b] < 0 || pl[b] > hd->pers_cap)
        return fail(KVDEC_ERR_INVALID, "KVDEC_CHECK: pers_len[%d] = %d outside [0, pers_cap %d]",
                    b, pl[b], hd->pers_cap);
  }
  if ((st = fetch(&bl, buf_len, (size_t)B * Hkv, stream, "buf_len")) != KVDEC_OK) return st;
  for (int b = 0; b < B; ++b)
    for (int g = 0; g < Hkv; ++g) {
      const int n = bl[(size_t)b * Hkv + g];
      if (hm[g] < 0 && (n < 0 || n > hd->buf_cap))
        return fail(KVDEC_ERR_INVALID, "KVDEC_CHECK: buf_len[%d] = %d outside [0, buf_cap %d]",
                    b * Hkv + g, n, hd->buf_cap);
    }
  return ok();
}

// Index lists of (sequence, KV head) pairs (row stride max_k): lengths in
// [0, len_cap], the listed rows in [0, S).  Only the pairs in `pairs` (all,
// when empty) are checked.
static kvdec_status check_index_lists(const int32_t* idx, const int32_t* idx_len, int n_pairs,
                                      int max_k, int len_cap, int S,
                                      const std::vector<int>& pairs, hipStream_t stream) {
  std::vector<int32_t> len, ix;
  kvdec_status st;
  if ((st = fetch(&len, idx_len, (size_t)n_pairs, stream, "idx_len")) != KVDEC_OK) return st;
  bool any = false;
  auto each = [&](auto&& fn) -> kvdec_status {
    if (pairs.empty()) {
      for (int p = 0; p < n_pairs; ++p)
        if ((st = fn(p)) != KVDEC_OK) return st;
    } else {
      for (int p : pairs)
        if ((st = fn(p)) != KVDEC_OK) return st;
    }
    return ok();
  };
  st = each([&](int p) -> kvdec_status {
    if (len[p] < 0 || len[p] > len_cap)
      return fail(KVDEC_ERR_INVALID, "KVDEC_CHECK: idx_len[%d] = %d outside [0, %d]", p, len[p],
                  len_cap);
    any |= len[p] > 0;
    return ok();
  });
  if (st != KVDEC_OK || !any) return st;
  if ((st = fetch(&ix, idx, (size_t)n_pairs * max_k, stream, "idx")) != KVDEC_OK) return st;
  return each([&](int p) -> kvdec_status {
    for (int i = 0; i < len[p]; ++i) {
      const int t = ix[(size_t)p * max_k + i];
      if (t < 0 || t >= S)
        return fail(KVDEC_ERR_INVALID, "KVDEC_CHECK: idx[%d][%d] = %d outside [0, %d)", p, i, t, S);
    }
    return ok();
  });
}
}  // namespace kvdec

using namespace kvdec;

extern "C" {

int kvdec_abi_version(void) { return KVDEC_ABI_VERSION; }

int kvdec_check_enabled(void) { return check_mode() ? 1 : 0; }

kvdec_status kvdec_kernel_timing(int enable) {
  TimingState& t = g_timing;
  t.on = enable != 0;
  if (t.on) {
    t.used = 0;
    t.err = hipSuccess;
  }
  return ok();
}

kvdec_status kvdec_stream_read(const void* src, size_t bytes, uint32_t* sink, hipStream_t stream) {
  if (!src || !sink) return fail(KVDEC_ERR_INVALID, "src and sink must be non-NULL");
  if (bytes == 0 || bytes % 16 != 0) return fail(KVDEC_ERR_INVALID, "bytes must be a positive multiple of 16");
  if (reinterpret_cast<uintptr_t>(src) % 16 != 0) return fail(KVDEC_ERR_INVALID, "src must be 16-byte aligned");
  return hip_status(launch_stream_read(src, bytes, sink, stream), "stream read launch");
}

kvdec_status kvdec_kernel_timing_read(double* total_ms, int64_t* launches) {
  if (!total_ms || !launches) return fail(KVDEC_ERR_INVALID, "total_ms and launches must be non-NULL");
  TimingState& t = g_timing;
  if (t.err != hipSuccess) return hip_status(t.err, "kernel timing event");
  double sum = 0.0;
  for (size_t i = 0; i < t.used; ++i) {
    hipError_t e = hipEventSynchronize(t.pool[i].second);
    float ms = 0.f;
    if (e == hipSuccess) e = hipEventElapsedTime(&ms, t.pool[i].first, t.pool[i].second);
    if (e != hipSuccess) return hip_status(e, "kernel timing event");
    sum += ms;
  }
  *total_ms = sum;
  *launches = (int64_t)t.used;
  return ok();
}

const char* kvdec_last_error(void) { return g_err; }

const char* kvdec_status_string(kvdec_status s) {
  switch (s) {
    case KVDEC_OK: return "KVDEC_OK";
    case KVDEC_ERR_INVALID: return "KVDEC_ERR_INVALID";
    case KVDEC_ERR_UNSUPPORTED: return "KVDEC_ERR_UNSUPPORTED";
    case KVDEC_ERR_WORKSPACE: return "KVDEC_ERR_WORKSPACE";
    case KVDEC_ERR_HIP: return "KVDEC_ERR_HIP";
  }
  return "unknown kvdec_status";
}

kvdec_status kvdec_decode_attn_noalloc(const kvdec_attn_desc* d, const void* q, const void* k,
                                       const void* v, const int32_t* seqlens,
                                       const int32_t* cu_seqlens, const int32_t* block_table,
                                       void* out, float* lse, hipStream_t stream) {
  kvdec_status st = check_common(d, true);
  if (st != KVDEC_OK) return st;
  if (d->batch == 0) return ok();
  const size_t need = attn_ws(d, plan_decode(d));
  if (need > KVDEC_NOALLOC_SCRATCH_BYTES)
    return fail(KVDEC_ERR_WORKSPACE,
                "this call needs %zu bytes of partials, the library's scratch holds %zu",
                need, (size_t)KVDEC_NOALLOC_SCRATCH_BYTES);
  void* ws = nullptr;
  if (need > 0) {
    st = scratch_address(&ws);
    if (st != KVDEC_OK) return st;
  }
  return kvdec_decode_attn(d, q, k, v, seqlens, cu_seqlens, block_table, out, lse, ws,
                           need > 0 ? (size_t)KVDEC_NOALLOC_SCRATCH_BYTES : 0, stream);
}

kvdec_status kvdec_decode_attn_workspace(const kvdec_attn_desc* d, size_t* bytes) {
  if (!bytes) return fail(KVDEC_ERR_INVALID, "bytes is NULL");
  kvdec_status st = check_common(d, true);
  if (st != KVDEC_OK) return st;
  *bytes = attn_ws(d, plan_decode(d));
  return ok();
}

kvdec_status kvdec_decode_attn(const kvdec_attn_desc* d, const void* q, const void* k,
                               const void* v, const int32_t* seqlens, const int32_t* cu_seqlens,
                               const int32_t* block_table, void* out, float* lse, void* ws,
                               size_t ws_bytes, hipStream_t stream) {
  kvdec_status st = check_common(d, true);
  if (st != KVDEC_OK) return st;
  if (d->batch == 0) return ok();
  if (!q || !out) return fail(KVDEC_ERR_INVALID, "q and out must be non-NULL");
  // k and v may be NULL only when no row can be read
  const bool no_rows = (d->layout == KVDEC_RAGGED && d->kv_rows == 0) ||
                       (d->layout == KVDEC_DENSE && d->max_seqlen == 0);
  if ((!k || !v) && !no_rows)
    return fail(KVDEC_ERR_INVALID, "k and v must be non-NULL (unless there are no K/V rows)");
  if (d->layout == KVDEC_RAGGED && !cu_seqlens)
    return fail(KVDEC_ERR_INVALID, "RAGGED needs cu_seqlens");
  if (d->layout == KVDEC_PAGED && (!seqlens || !block_table))
    return fail(KVDEC_ERR_INVALID, "PAGED needs seqlens and block_table");
  const Plan p = plan_decode(d);
  AttnArgs a = {};
  fill_common(d, p, &a);
  a.q = static_cast<const uint16_t*>(q);
  a.k = k;
  a.v = v;
  a.seqlens = seqlens;
  a.cu_seqlens = cu_seqlens;
  a.block_table = block_table;
  a.out = static_cast<uint16_t*>(out);
  a.lse = lse;
  if (d->layout == KVDEC_DENSE) {
    a.src = SRC_DENSE;
    a.S = d->max_seqlen;
  } else if (d->layout == KVDEC_RAGGED) {
    a.src = SRC_RAGGED;
    a.S = (int)d->kv_rows;
  } else {
    a.src = SRC_PAGED;
    a.S = (int)d->kv_rows;
    a.page = d->page_size;
    a.max_pages = d->max_pages_per_seq;
  }
  if (check_mode() && (st = check_decode_meta(d, seqlens, cu_seqlens, block_table, stream)) != KVDEC_OK)
    return st;
  return run_attn(d, p, a, ws, ws_bytes, stream);
}

static kvdec_status check_hybrid(const kvdec_hybrid_desc* h) {
  if (!h) return fail(KVDEC_ERR_INVALID, "desc is NULL");
  kvdec_status st = check_common(&h->base, false);
  if (st != KVDEC_OK) return st;
  if (h->num_pers_slots < 0 || h->pers_cap < 0 || h->buf_cap < 0)
    return fail(KVDEC_ERR_INVALID, "negative hybrid capacity");
  return ok();
}

kvdec_status kvdec_sparse_hybrid_attn_workspace(const kvdec_hybrid_desc* h, size_t* bytes) {
  if (!bytes) return fail(KVDEC_ERR_INVALID, "bytes is NULL");
  kvdec_status st = check_hybrid(h);
  if (st != KVDEC_OK) return st;
  *bytes = attn_ws(&h->base, plan_hybrid(h));
  return ok();
}

kvdec_status kvdec_sparse_hybrid_attn(const kvdec_hybrid_desc* h, const void* q,
                                      const void* pers_k, const void* pers_v,
                                      const int32_t* pers_len, const void* buf_k,
                                      const void* buf_v, const int32_t* buf_len,
                                      const int32_t* head_map, void* out, float* lse, void* ws,
                                      size_t ws_bytes, hipStream_t stream) {
  kvdec_status st = check_hybrid(h);
  if (st != KVDEC_OK) return st;
  const kvdec_attn_desc* d = &h->base;
  if (d->batch == 0) return ok();
  if (!q || !out || !head_map) return fail(KVDEC_ERR_INVALID, "q, out and head_map must be non-NULL");
  if (h->num_pers_slots > 0 && (!pers_k || !pers_v || !pers_len))
    return fail(KVDEC_ERR_INVALID, "persistent slots need pers_k, pers_v and pers_len");
  if (!buf_k || !buf_v || !buf_len)
    return fail(KVDEC_ERR_INVALID, "buf_k, buf_v and buf_len must be non-NULL");
  const Plan p = plan_hybrid(h);
  AttnArgs a = {};
  fill_common(d, p, &a);
  a.src = SRC_HYBRID;
  a.q = static_cast<const uint16_t*>(q);
  a.k = pers_k;
  a.v = pers_v;
  a.k2 = buf_k;
  a.v2 = buf_v;
  a.pers_len = pers_len;
  a.buf_len = buf_len;
  a.head_map = head_map;
  a.P_slots = h->num_pers_slots;
  a.pers_cap = h->pers_cap;
  a.buf_cap = h->buf_cap;
  a.out = static_cast<uint16_t*>(out);
  a.lse = lse;
  if (check_mode() && (st = check_hybrid_meta(h, pers_len, buf_len, head_map, stream)) != KVDEC_OK)
    return st;
  return run_attn(d, p, a, ws, ws_bytes, stream);
}

static kvdec_status check_gather(const kvdec_gather_desc* gd) {
  if (!gd) return fail(KVDEC_ERR_INVALID, "desc is NULL");
  kvdec_status st = check_common(&gd->base, false);
  if (st != KVDEC_OK) return st;
  const kvdec_attn_desc* d = &gd->base;
  if (d->max_seqlen < 0) return fail(KVDEC_ERR_INVALID, "max_seqlen < 0");
  if (gd->max_k < 0) return fail(KVDEC_ERR_INVALID, "max_k < 0");
  const int64_t elem = d->kv_format == KVDEC_KV_E4M3 ? 1 : 2;
  if ((int64_t)d->max_seqlen * d->num_kv_heads * kHeadDim * elem > (int64_t(1) << 31))
    return fail(KVDEC_ERR_UNSUPPORTED, "S * Hkv * 128 * element bytes must be <= 2^31");
  return ok();
}

static Plan plan_gather(const kvdec_gather_desc* gd) {
  const kvdec_attn_desc* d = &gd->base;
  const int64_t pairs = (int64_t)d->batch * d->num_kv_heads;
  return plan_attn(d->dtype, d->kv_format == KVDEC_KV_E4M3, d->num_q_heads / d->num_kv_heads,
                   SRC_GATHER, pairs, pairs, pairs * (int64_t)gd->max_k, gd->max_k, d->split_tokens);
}

kvdec_status kvdec_gather_attn_workspace(const kvdec_gather_desc* gd, size_t* bytes) {
  if (!bytes) return fail(KVDEC_ERR_INVALID, "bytes is NULL");
  kvdec_status st = check_gather(gd);
  if (st != KVDEC_OK) return st;
  *bytes = attn_ws(&gd->base, plan_gather(gd));
  return ok();
}

kvdec_status kvdec_gather_attn(const kvdec_gather_desc* gd, const void* q, const void* k,
                               const void* v, const int32_t* idx, const int32_t* idx_len,
                               void* out, float* lse, void* ws, size_t ws_bytes,
                               hipStream_t stream) {
  kvdec_status st = check_gather(gd);
  if (st != KVDEC_OK) return st;
  const kvdec_attn_desc* d = &gd->base;
  if (d->batch == 0) return ok();
  if (!q || !out || !idx_len) return fail(KVDEC_ERR_INVALID, "q, out and idx_len must be non-NULL");
  if (gd->max_k > 0 && d->max_seqlen > 0 && (!k || !v || !idx))
    return fail(KVDEC_ERR_INVALID, "k, v and idx must be non-NULL");
  const Plan p = plan_gather(gd);
  AttnArgs a = {};
  fill_common(d, p, &a);
  a.src = SRC_GATHER;
  a.q = static_cast<const uint16_t*>(q);
  a.k = k;
  a.v = v;
  a.idx = idx;
  a.idx_len = idx_len;
  a.max_k = gd->max_k;
  a.S = std::max(d->max_seqlen, 1);
  a.out = static_cast<uint16_t*>(out);
  a.lse = lse;
  // with no cache rows or no index slots every pair is empty: the kernels
  // then read neither k, v nor idx
  if (d->max_seqlen == 0 || gd->max_k == 0) a.max_k = 0;
  if (check_mode() &&
      (st = check_index_lists(idx, idx_len, d->batch * d->num_kv_heads, gd->max_k, gd->max_k,
                              std::max(d->max_seqlen, 1), {}, stream)) != KVDEC_OK)
    return st;
  return run_attn(d, p, a, ws, ws_bytes, stream);
}

static kvdec_status check_topk(const kvdec_topk_desc* d) {
  if (!d) return fail(KVDEC_ERR_INVALID, "desc is NULL");
  if (d->batch < 0 || d->num_q_heads < 1 || d->num_kv_heads < 1)
    return fail(KVDEC_ERR_INVALID, "bad batch / head counts");
  if (d->num_q_heads % d->num_kv_heads != 0)
    return fail(KVDEC_ERR_INVALID, "num_q_heads %% num_kv_heads != 0");
  if (d->head_dim != kHeadDim) return fail(KVDEC_ERR_UNSUPPORTED, "head_dim must be 128");
  if (d->dtype != KVDEC_F16 && d->dtype != KVDEC_BF16)
    return fail(KVDEC_ERR_UNSUPPORTED, "dtype must be KVDEC_F16 or KVDEC_BF16");
  if (d->max_seqlen < 0 || d->max_seqlen > kTopkMaxLen)
    return fail(KVDEC_ERR_UNSUPPORTED, "max_seqlen must be in [0, %d]", kTopkMaxLen);
  if (d->top_k < 0) return fail(KVDEC_ERR_INVALID, "top_k < 0");
  if ((int64_t)d->batch * d->num_kv_heads > 65535)
    return fail(KVDEC_ERR_UNSUPPORTED, "batch * num_kv_heads must be <= 65535");
  return ok();
}

kvdec_status kvdec_topk_select_workspace(const kvdec_topk_desc* d, size_t* bytes) {
  if (!bytes) return fail(KVDEC_ERR_INVALID, "bytes is NULL");
  kvdec_status st = check_topk(d);
  if (st != KVDEC_OK) return st;
  *bytes = topk_workspace_bytes(d->batch * d->num_kv_heads, d->max_seqlen);
  return ok();
}

kvdec_status kvdec_topk_select(const kvdec_topk_desc* d, const void* q, const void* k,
                               const int32_t* seqlens, int32_t* idx, int32_t* idx_len, void* ws,
                               size_t ws_bytes, hipStream_t stream) {
  kvdec_status st = check_topk(d);
  if (st != KVDEC_OK) return st;
  if (d->batch == 0) return ok();
  if (!idx_len) return fail(KVDEC_ERR_INVALID, "idx_len must be non-NULL");
  const size_t need = topk_workspace_bytes(d->batch * d->num_kv_heads, d->max_seqlen);
  if (d->max_seqlen > 0) {
    if (!q || !k) return fail(KVDEC_ERR_INVALID, "q and k must be non-NULL");
    if (d->top_k > 0 && !idx) return fail(KVDEC_ERR_INVALID, "idx must be non-NULL");
    if (!ws || ws_bytes < need)
      return fail(KVDEC_ERR_WORKSPACE, "workspace needs %zu bytes, got %zu", need, ws_bytes);
    if (reinterpret_cast<uintptr_t>(ws) & 15)
      return fail(KVDEC_ERR_WORKSPACE, "workspace must be 16-byte aligned");
  }
  TopkArgs a = {};
  a.q = static_cast<const uint16_t*>(q);
  a.k = static_cast<const uint16_t*>(k);
  a.seqlens = d->max_seqlen > 0 ? seqlens : nullptr;
  a.scores = static_cast<float*>(ws);
  a.idx = idx;
  a.idx_len = idx_len;
  a.B = d->batch;
  a.Hq = d->num_q_heads;
  a.Hkv = d->num_kv_heads;
  a.G = d->num_q_heads / d->num_kv_heads;
  a.S = d->max_seqlen;
  a.S4 = (d->max_seqlen + 3) & ~3;
  a.C = topk_chunks(d->max_seqlen);
  a.sel = ws ? reinterpret_cast<uint32_t*>(static_cast<char*>(ws) +
                                           (size_t)a.B * a.Hkv * a.S4 * sizeof(float))
             : nullptr;
  a.top_k = d->top_k;
  a.dtype = d->dtype;
  if (check_mode() && a.seqlens) {
    std::vector<int32_t> h;
    if ((st = fetch(&h, seqlens, (size_t)d->batch, stream, "seqlens")) != KVDEC_OK) return st;
    for (int b = 0; b < d->batch; ++b)
      if (h[b] < 0 || h[b] > d->max_seqlen)
        return fail(KVDEC_ERR_INVALID, "KVDEC_CHECK: seqlens[%d] = %d outside [0, max_seqlen %d]",
                    b, h[b], d->max_seqlen);
  }
  return hip_status(launch_topk(a, stream), "top-k selection launch");
}

kvdec_status kvdec_headcache_lookup(int32_t B, int32_t Hq, int32_t Hkv, int32_t D, int32_t dtype,
                                    const void* q, void* labels, const float* weights,
                                    const float* tau, uint8_t* hit, float* agg, float* cos,
                                    int32_t* miss_list, int32_t* miss_count, hipStream_t stream) {
  LookupArgs a = {};
  kvdec_status st = lookup_args(B, Hq, Hkv, D, dtype, q, labels, weights, tau, hit, agg, cos,
                                miss_list, miss_count, &a);
  if (st != KVDEC_OK || B == 0) return st;
  return hip_status(launch_headcache_lookup(a, stream), "head-cache lookup launch");
}

kvdec_status kvdec_host_flag_alloc(uint32_t** flag) {
  if (!flag) return fail(KVDEC_ERR_INVALID, "flag is NULL");
  *flag = nullptr;
  void* p = nullptr;
  hipError_t e = hipHostMalloc(&p, 64, hipHostMallocCoherent | hipHostMallocMapped);
  if (e != hipSuccess) return hip_status(e, "hipHostMalloc (flag)");
  static_cast<volatile uint32_t*>(p)[0] = 0;
  *flag = static_cast<uint32_t*>(p);
  return ok();
}

kvdec_status kvdec_host_flag_free(uint32_t* flag) {
  if (!flag) return ok();
  return hip_status(hipHostFree(flag), "hipHostFree (flag)");
}

kvdec_status kvdec_flag_wait(const uint32_t* flag, uint32_t value, uint32_t timeout_us,
                             int32_t* status, hipStream_t stream) {
  void *fdev = nullptr, *sdev = nullptr;
  kvdec_status st = flag_wait_args(flag, timeout_us, status, &fdev, &sdev);
  if (st != KVDEC_OK) return st;
  return enqueue_flag_wait(fdev, value, timeout_us, sdev, stream);
}

kvdec_status kvdec_flag_signal(uint32_t* flag, uint32_t value, hipStream_t stream) {
  if (!flag) return fail(KVDEC_ERR_INVALID, "flag must be non-NULL");
  if (reinterpret_cast<uintptr_t>(flag) % 4) return fail(KVDEC_ERR_INVALID, "flag must be 4-byte aligned");
  void* fdev = nullptr;
  kvdec_status st = mapped_range(flag, 4, false, "flag", &fdev);
  if (st != KVDEC_OK) return st;
  return hip_status(launch_flag_signal(static_cast<uint32_t*>(fdev), value, stream),
                    "flag signal launch");
}

kvdec_status kvdec_headcache_prefetch(const kvdec_prefetch_desc* d, const int32_t* miss_list,
                                      const int32_t* miss_count, const int32_t* head_map,
                                      const int32_t* idx, const int32_t* idx_len,
                                      const void* pool_k, const void* pool_v, void* buf_k,
                                      void* buf_v, int32_t* buf_len, const uint32_t* ready_flag,
                                      uint32_t ready_value, uint32_t timeout_us, int32_t* status,
                                      hipStream_t stream) {
  if (!d) return fail(KVDEC_ERR_INVALID, "desc is NULL");
  if (d->batch < 0 || d->num_kv_heads < 1) return fail(KVDEC_ERR_INVALID, "bad batch / num_kv_heads");
  if (d->head_dim != kHeadDim) return fail(KVDEC_ERR_UNSUPPORTED, "head_dim must be 128");
  if (d->elem_bytes != 1 && d->elem_bytes != 2)
    return fail(KVDEC_ERR_UNSUPPORTED, "elem_bytes must be 2 (fp16, bf16) or 1 (e4m3)");
  if (d->max_seqlen < 1 || d->max_k < 0 || d->buf_cap < 0)
    return fail(KVDEC_ERR_INVALID, "max_seqlen must be >= 1, max_k and buf_cap >= 0");
  if (d->pool_stride_b < 0 || d->pool_stride_s < 0 || d->pool_stride_h < 0)
    return fail(KVDEC_ERR_INVALID, "pool strides must be >= 0");
  const int64_t eb = d->elem_bytes;
  if ((d->pool_stride_b * eb) % 16 || (d->pool_stride_s * eb) % 16 || (d->pool_stride_h * eb) % 16)
    return fail(KVDEC_ERR_INVALID, "pool strides must be multiples of 16 bytes");
  if ((int64_t)d->batch * d->num_kv_heads > INT32_MAX / 2 ||
      (int64_t)d->batch * d->num_kv_heads * std::max(d->max_k, 1) > INT32_MAX)
    return fail(KVDEC_ERR_UNSUPPORTED, "batch * num_kv_heads * max_k too large");
  const int pairs = d->batch * d->num_kv_heads;
  const bool nothing = pairs == 0;
  if (nothing && !ready_flag) return ok();
  void *fdev = nullptr, *sdev = nullptr, *kdev = nullptr, *vdev = nullptr;
  kvdec_status st;
  if (ready_flag) {
    st = flag_wait_args(ready_flag, timeout_us, status, &fdev, &sdev);
    if (st != KVDEC_OK) return st;
  }
  if (!nothing) {
    if (!miss_list || !miss_count || !idx || !idx_len || !pool_k || !pool_v || !buf_k || !buf_v ||
        !buf_len)
      return fail(KVDEC_ERR_INVALID, "miss_list, miss_count, idx, idx_len, the pools, the "
                                     "buffers and buf_len must be non-NULL");
    if (reinterpret_cast<uintptr_t>(pool_k) % 16 || reinterpret_cast<uintptr_t>(pool_v) % 16 ||
        reinterpret_cast<uintptr_t>(buf_k) % 16 || reinterpret_cast<uintptr_t>(buf_v) % 16)
      return fail(KVDEC_ERR_INVALID, "pools and buffers must be 16-byte aligned");
    // every row the kernel can address: b < B, t < S, g < Hkv (indices are clamped)
    const int64_t last = (int64_t)(d->batch - 1) * d->pool_stride_b +
                         (int64_t)(d->max_seqlen - 1) * d->pool_stride_s +
                         (int64_t)(d->num_kv_heads - 1) * d->pool_stride_h + kHeadDim;
    st = mapped_range(pool_k, (size_t)(last * eb), true, "pool_k", &kdev);
    if (st != KVDEC_OK) return st;
    st = mapped_range(pool_v, (size_t)(last * eb), true, "pool_v", &vdev);
    if (st != KVDEC_OK) return st;
  }
  if (!nothing && check_mode()) {
    // before the flag wait is queued: a rejected call launches nothing
    std::vector<int32_t> mc, ml, hm;
    if ((st = fetch(&mc, miss_count, 1, stream, "miss_count")) != KVDEC_OK) return st;
    if (mc[0] < 0 || mc[0] > pairs)
      return fail(KVDEC_ERR_INVALID, "KVDEC_CHECK: miss_count = %d outside [0, %d]", mc[0], pairs);
    if ((st = fetch(&ml, miss_list, (size_t)mc[0], stream, "miss_list")) != KVDEC_OK) return st;
    if (head_map && (st = fetch(&hm, head_map, (size_t)d->num_kv_heads, stream, "head_map")) != KVDEC_OK)
      return st;
    std::vector<int> listed;
    for (int i = 0; i < mc[0]; ++i) {
      if (ml[i] < 0 || ml[i] >= pairs)
        return fail(KVDEC_ERR_INVALID, "KVDEC_CHECK: miss_list[%d] = %d outside [0, %d)", i,
                    ml[i], pairs);
      if (!head_map || hm[ml[i] % d->num_kv_heads] < 0) listed.push_back(ml[i]);
    }
    if (!listed.empty() &&
        (st = check_index_lists(idx, idx_len, pairs, d->max_k, std::min(d->max_k, d->buf_cap),
                                d->max_seqlen, listed, stream)) != KVDEC_OK)
      return st;
  }
  if (ready_flag) {
    st = enqueue_flag_wait(fdev, ready_value, timeout_us, sdev, stream);
    if (st != KVDEC_OK) return st;
  }
  if (nothing) return ok();
  PrefetchArgs a = {};
  a.miss_list = miss_list;
  a.miss_count = miss_count;
  a.head_map = head_map;
  a.idx = idx;
  a.idx_len = idx_len;
  a.pool_k = kdev;
  a.pool_v = vdev;
  a.buf_k = buf_k;
  a.buf_v = buf_v;
  a.buf_len = buf_len;
  a.status = static_cast<int32_t*>(sdev);
  a.stride_b = d->pool_stride_b;
  a.stride_s = d->pool_stride_s;
  a.stride_h = d->pool_stride_h;
  a.B = d->batch;
  a.Hkv = d->num_kv_heads;
  a.S = d->max_seqlen;
  a.max_k = d->max_k;
  a.buf_cap = d->buf_cap;
  a.max_rows = std::min(d->max_k, d->buf_cap);
  a.elem_bytes = d->elem_bytes;
  return hip_status(launch_prefetch(a, stream), "prefetch launch");
}

kvdec_status kvdec_headcache_lookup_ahead(int32_t B, int32_t Hq, int32_t Hkv, int32_t D,
                                          int32_t h, int32_t dtype, const void* x_prev,
                                          const void* w_q, void* q_approx, void* labels,
                                          const float* weights, const float* tau, uint8_t* hit,
                                          float* agg, float* cos, int32_t* miss_list,
                                          int32_t* miss_count, hipStream_t stream) {
  LookupArgs a = {};
  kvdec_status st = lookup_args(B, Hq, Hkv, D, dtype, q_approx, labels, weights, tau, hit, agg,
                                cos, miss_list, miss_count, &a);
  if (st != KVDEC_OK) return st;
  if (h < 8 || h % 8 != 0 || h > 8192)  // x of four batch rows fits the staging
    return fail(KVDEC_ERR_UNSUPPORTED, "h must be a multiple of 8 in [8, 8192]");
  if (B == 0) return ok();
  if (!x_prev || !w_q) return fail(KVDEC_ERR_INVALID, "x_prev and w_q must be non-NULL");
  if ((reinterpret_cast<uintptr_t>(x_prev) | reinterpret_cast<uintptr_t>(w_q)) & 15)
    return fail(KVDEC_ERR_INVALID, "x_prev and w_q must be 16-byte aligned");
  QProjArgs qa = {};
  qa.x = static_cast<const uint16_t*>(x_prev);
  qa.w = static_cast<const uint16_t*>(w_q);
  qa.q = static_cast<uint16_t*>(q_approx);
  qa.B = B;
  qa.h = h;
  qa.N = Hq * D;
  qa.dtype = dtype;
  hipError_t e = launch_qproj(qa, stream);
  if (e != hipSuccess) return hip_status(e, "query projection launch");
  return hip_status(launch_headcache_lookup(a, stream), "head-cache lookup launch");
}

kvdec_status kvdec_headcache_thresholds(int32_t n, const float* s, double eta, double n_exp,
                                        float* tau) {
  if (n < 0) return fail(KVDEC_ERR_INVALID, "n < 0");
  if (n > 0 && (!s || !tau)) return fail(KVDEC_ERR_INVALID, "s and tau must be non-NULL");
  if (!(eta >= -1.0 && eta <= 1.0)) return fail(KVDEC_ERR_INVALID, "eta outside [-1, 1]");
  if (!(n_exp > 0.0) || !isfinite(n_exp)) return fail(KVDEC_ERR_INVALID, "n_exp must be > 0");
  const double pi = 3.14159265358979323846;
  const double theta_star = acos(eta);  // Eq. 7
  for (int32_t i = 0; i < n; ++i) {
    const double si = (double)s[i];
    if (!(si >= 0.0 && si <= 1.0)) return fail(KVDEC_ERR_INVALID, "s[%d] outside [0, 1]", i);
    const double lambda = pow(si, n_exp);                          // Eq. 8
    tau[i] = (float)cos(lambda * theta_star + (1.0 - lambda) * pi);  // Eq. 9
  }
  return ok();
}

kvdec_status kvdec_kv_recompute(int32_t b, int32_t l, int32_t h, int32_t num_heads,
                                int32_t head_dim, const void* x, int64_t x_batch_stride,
                                const void* w_k, const void* w_v, int32_t w_layout,
                                void* k_cache, void* v_cache, int64_t cache_batch_stride,
                                hipStream_t stream) {
  RecomputeArgs a = {};
  kvdec_status st = recompute_args(b, l, h, num_heads, head_dim, x, x_batch_stride, w_k, w_v,
                                   w_layout, k_cache, v_cache, cache_batch_stride, &a);
  if (st != KVDEC_OK || b == 0 || l == 0) return st;
  return hip_status(launch_kv_recompute(a, stream), "kv recompute launch");
}

kvdec_status kvdec_kvpr_split(int64_t b, int64_t s_prime, int64_t l_max, int64_t h,
                              int32_t elem_bytes, double v_com, double v_gpu, int32_t* l_out,
                              double* t_out) {
  if (!l_out) return fail(KVDEC_ERR_INVALID, "l_out is NULL");
  if (b < 0 || s_prime < 0 || l_max < 0 || l_max > s_prime || s_prime > INT32_MAX || h < 1 ||
      elem_bytes < 1)
    return fail(KVDEC_ERR_INVALID, "need b >= 0, 0 <= l_max <= s_prime < 2^31, h >= 1, elem_bytes >= 1");
  if (!(std::isfinite(v_com) && v_com > 0.0 && std::isfinite(v_gpu) && v_gpu > 0.0))
    return fail(KVDEC_ERR_INVALID, "v_com and v_gpu must be finite and > 0");
  const double B = (double)b, S = (double)s_prime, H = (double)h, p = (double)elem_bytes;
  auto t_of = [&](double l) {
    const double t_x = B * l * H * p / v_com;
    const double t_rec = 4.0 * B * l * H * H / v_gpu;
    const double t_kv = 2.0 * B * (S - l) * H * p / v_com;
    return t_x + std::max(t_rec, t_kv);
  };
  // crossing of the recompute time c l and the remaining transfer d (s' - l)
  const double c = 4.0 * H * H / v_gpu, d = 2.0 * H * p / v_com;
  const double lc = d * S / (c + d);
  int64_t best = 0;
  double tb = t_of(0.0);
  const double cands[2] = {std::floor(lc), std::ceil(lc)};
  for (double x : cands) {
    const int64_t l = std::min<int64_t>(std::max<int64_t>((int64_t)x, 0), l_max);
    const double t = t_of((double)l);
    if (t < tb || (t == tb && l < best)) {
      tb = t;
      best = l;
    }
  }
  const double t_max = t_of((double)l_max);
  if (t_max < tb) {
    tb = t_max;
    best = l_max;
  }
  *l_out = (int32_t)best;
  if (t_out) *t_out = tb;
  return ok();
}

// Per-thread events that order the copies of a layer load against its
// recompute (reused from call to call: a wait always refers to the record
// just before it).
struct LoadEvents {
  hipEvent_t x_done = nullptr, kv_done = nullptr;
};
static thread_local LoadEvents g_load_events;

kvdec_status kvdec_kvpr_load_layer(int32_t b, int32_t l, int32_t s_prime, int32_t h,
                                   int32_t num_heads, int32_t head_dim, const void* x_host,
                                   int64_t x_host_bstride, void* x_dev, const void* k_host,
                                   const void* v_host, int64_t kv_host_bstride, const void* w_k,
                                   const void* w_v, int32_t w_layout, void* k_cache, void* v_cache,
                                   int64_t cache_bstride, hipStream_t compute_stream,
                                   hipStream_t copy_stream) {
  if (l < 0 || s_prime < l) return fail(KVDEC_ERR_INVALID, "need 0 <= l <= s_prime");
  if (compute_stream == copy_stream)
    return fail(KVDEC_ERR_INVALID, "compute_stream and copy_stream must differ");
  RecomputeArgs a = {};
  kvdec_status st = recompute_args(b, l, h, num_heads, head_dim, x_dev, (int64_t)l * h, w_k, w_v,
                                   w_layout, k_cache, v_cache, cache_bstride, &a);
  if (st != KVDEC_OK) return st;
  if (x_host_bstride < (int64_t)l * h) return fail(KVDEC_ERR_INVALID, "x_host_bstride < l * h");
  if (kv_host_bstride < (int64_t)s_prime * h || cache_bstride < (int64_t)s_prime * h)
    return fail(KVDEC_ERR_INVALID, "kv_host_bstride and cache_bstride must be >= s_prime * h");
  if (b == 0 || s_prime == 0) return ok();
  if ((s_prime > l && (!k_host || !v_host)) || (l > 0 && !x_host))
    return fail(KVDEC_ERR_INVALID, "x_host, k_host and v_host must be non-NULL where rows are read");
  LoadEvents& ev = g_load_events;
  if (!ev.x_done) {
    hipError_t e = hipEventCreateWithFlags(&ev.x_done, hipEventDisableTiming);
    if (e == hipSuccess) e = hipEventCreateWithFlags(&ev.kv_done, hipEventDisableTiming);
    if (e != hipSuccess) {
      if (ev.x_done) (void)hipEventDestroy(ev.x_done);
      ev.x_done = nullptr;
      return hip_status(e, "event create");
    }
  }
  const size_t e2 = sizeof(uint16_t);
  hipError_t e = hipSuccess;
  if (l > 0) {
    e = hipMemcpy2DAsync(x_dev, (size_t)l * h * e2, x_host, (size_t)x_host_bstride * e2,
                         (size_t)l * h * e2, (size_t)b, hipMemcpyHostToDevice, copy_stream);
    if (e == hipSuccess) e = hipEventRecord(ev.x_done, copy_stream);
    if (e == hipSuccess) e = hipStreamWaitEvent(compute_stream, ev.x_done, 0);
    if (e != hipSuccess) return hip_status(e, "activation copy");
    e = launch_kv_recompute(a, compute_stream);
    if (e != hipSuccess) return hip_status(e, "kv recompute launch");
  }
  if (s_prime > l) {
    const size_t off = (size_t)l * h * e2, width = (size_t)(s_prime - l) * h * e2;
    const void* srcs[2] = {k_host, v_host};
    void* dsts[2] = {k_cache, v_cache};
    for (int i = 0; i < 2 && e == hipSuccess; ++i)
      e = hipMemcpy2DAsync(static_cast<char*>(dsts[i]) + off, (size_t)cache_bstride * e2,
                           static_cast<const char*>(srcs[i]) + off, (size_t)kv_host_bstride * e2,
                           width, (size_t)b, hipMemcpyHostToDevice, copy_stream);
    if (e == hipSuccess) e = hipEventRecord(ev.kv_done, copy_stream);
    if (e == hipSuccess) e = hipStreamWaitEvent(compute_stream, ev.kv_done, 0);
    if (e != hipSuccess) return hip_status(e, "K/V copy");
  }
  return ok();
}


}  // extern "C"

"""ctypes binding of libkvdec (include/kvdec.h).

Argument marshalling only: tensors become device pointers, the current torch
stream becomes the hipStream_t, and a non-OK status raises KvdecError with the
library's message.  Every computation runs in the library's HIP kernels; if
libkvdec.so is missing this module raises at import (there is no fallback).
"""
from __future__ import annotations

import ctypes
import os

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libkvdec.so")

KVDEC_OK, KVDEC_ERR_INVALID, KVDEC_ERR_UNSUPPORTED, KVDEC_ERR_WORKSPACE, KVDEC_ERR_HIP = range(5)
KVDEC_F16, KVDEC_BF16 = 0, 1
KVDEC_DENSE, KVDEC_RAGGED, KVDEC_PAGED = 0, 1, 2
KVDEC_W_IN_OUT, KVDEC_W_OUT_IN = 0, 1
KVDEC_KV_SAME, KVDEC_KV_E4M3 = 0, 1

_DTYPES = {torch.float16: KVDEC_F16, torch.bfloat16: KVDEC_BF16}


class KvdecError(RuntimeError):
    def __init__(self, status, msg):
        super().__init__(f"{status_string(status)}: {msg}")
        self.status = status


class AttnDesc(ctypes.Structure):
    _fields_ = [
        ("batch", ctypes.c_int32), ("num_q_heads", ctypes.c_int32),
        ("num_kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
        ("softmax_scale", ctypes.c_float), ("dtype", ctypes.c_int32),
        ("layout", ctypes.c_int32), ("max_seqlen", ctypes.c_int32),
        ("page_size", ctypes.c_int32), ("max_pages_per_seq", ctypes.c_int32),
        ("split_tokens", ctypes.c_int32), ("kv_rows", ctypes.c_int64),
        ("kv_format", ctypes.c_int32), ("k_scale", ctypes.c_float), ("v_scale", ctypes.c_float),
    ]


class GatherDesc(ctypes.Structure):
    _fields_ = [("base", AttnDesc), ("max_k", ctypes.c_int32)]


class TopkDesc(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("num_q_heads", ctypes.c_int32),
                ("num_kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("dtype", ctypes.c_int32), ("max_seqlen", ctypes.c_int32), ("top_k", ctypes.c_int32)]


class PrefetchDesc(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("num_kv_heads", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("elem_bytes", ctypes.c_int32),
                ("max_seqlen", ctypes.c_int32), ("pool_stride_b", ctypes.c_int64),
                ("pool_stride_s", ctypes.c_int64), ("pool_stride_h", ctypes.c_int64),
                ("max_k", ctypes.c_int32), ("buf_cap", ctypes.c_int32)]


class HybridDesc(ctypes.Structure):
    _fields_ = [("base", AttnDesc), ("num_pers_slots", ctypes.c_int32),
                ("pers_cap", ctypes.c_int32), ("buf_cap", ctypes.c_int32)]


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built; run `python -m long_kv_caches_amd.build`")
    lib = ctypes.CDLL(LIB_PATH)
    P, i32, i64, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
    st = ctypes.c_int
    sig = {
        "kvdec_decode_attn_workspace": ([ctypes.POINTER(AttnDesc), ctypes.POINTER(sz)], st),
        "kvdec_decode_attn": ([ctypes.POINTER(AttnDesc), P, P, P, P, P, P, P, P, P, sz, P], st),
        "kvdec_decode_attn_noalloc": ([ctypes.POINTER(AttnDesc), P, P, P, P, P, P, P, P, P], st),
        "kvdec_sparse_hybrid_attn_workspace": ([ctypes.POINTER(HybridDesc), ctypes.POINTER(sz)], st),
        "kvdec_sparse_hybrid_attn": ([ctypes.POINTER(HybridDesc), P, P, P, P, P, P, P, P, P, P, P,
                                      sz, P], st),
        "kvdec_headcache_lookup": ([i32, i32, i32, i32, i32, P, P, P, P, P, P, P, P, P, P], st),
        "kvdec_headcache_lookup_ahead": ([i32] * 6 + [P] * 11 + [P], st),
        "kvdec_gather_attn_workspace": ([P, ctypes.POINTER(ctypes.c_size_t)], st),
        "kvdec_gather_attn": ([P, P, P, P, P, P, P, P, P, ctypes.c_size_t, P], st),
        "kvdec_topk_select_workspace": ([P, ctypes.POINTER(ctypes.c_size_t)], st),
        "kvdec_topk_select": ([P, P, P, P, P, P, P, ctypes.c_size_t, P], st),
        "kvdec_headcache_prefetch": ([ctypes.POINTER(PrefetchDesc)] + [P] * 11
                                     + [ctypes.c_uint32, ctypes.c_uint32, P, P], st),
        "kvdec_host_flag_alloc": ([ctypes.POINTER(P)], st),
        "kvdec_host_flag_free": ([P], st),
        "kvdec_flag_wait": ([P, ctypes.c_uint32, ctypes.c_uint32, P, P], st),
        "kvdec_flag_signal": ([P, ctypes.c_uint32, P], st),
        "kvdec_headcache_thresholds": ([i32, P, ctypes.c_double, ctypes.c_double, P], st),
        "kvdec_kv_recompute": ([i32, i32, i32, i32, i32, P, i64, P, P, i32, P, P, i64, P], st),
        "kvdec_kvpr_split": ([i64, i64, i64, i64, i32, ctypes.c_double, ctypes.c_double,
                              ctypes.POINTER(i32), ctypes.POINTER(ctypes.c_double)], st),
        "kvdec_kvpr_load_layer": ([i32, i32, i32, i32, i32, i32, P, i64, P, P, P, i64, P, P, i32, P,
                                   P, i64, P, P], st),
        "kvdec_kernel_timing": ([ctypes.c_int], st),
        "kvdec_stream_read": ([P, sz, P, P], st),
        "kvdec_kernel_timing_read": ([ctypes.POINTER(ctypes.c_double), ctypes.POINTER(i64)], st),
        "kvdec_status_string": ([st], ctypes.c_char_p),
        "kvdec_last_error": ([], ctypes.c_char_p),
        "kvdec_abi_version": ([], ctypes.c_int),
        "kvdec_check_enabled": ([], ctypes.c_int),
    }
    for name, (args, res) in sig.items():
        fn = getattr(lib, name)
        fn.argtypes = args
        fn.restype = res
    return lib


lib = _load()
NOALLOC_SCRATCH_BYTES = 32 << 20
EXPORTED = ("kvdec_decode_attn_workspace", "kvdec_decode_attn", "kvdec_decode_attn_noalloc",
            "kvdec_sparse_hybrid_attn_workspace",
            "kvdec_sparse_hybrid_attn", "kvdec_headcache_lookup", "kvdec_headcache_lookup_ahead",
            "kvdec_gather_attn_workspace", "kvdec_gather_attn", "kvdec_topk_select_workspace",
            "kvdec_topk_select",
            "kvdec_headcache_thresholds", "kvdec_headcache_prefetch", "kvdec_host_flag_alloc",
            "kvdec_host_flag_free", "kvdec_flag_wait", "kvdec_flag_signal",
            "kvdec_kv_recompute", "kvdec_kvpr_split", "kvdec_kvpr_load_layer", "kvdec_kernel_timing",
            "kvdec_kernel_timing_read", "kvdec_stream_read", "kvdec_status_string",
            "kvdec_last_error", "kvdec_abi_version", "kvdec_check_enabled")


def check_enabled() -> bool:
    """Whether KVDEC_CHECK=1 (debug validation of device metadata) is on."""
    return bool(lib.kvdec_check_enabled())


def status_string(status: int) -> str:
    return lib.kvdec_status_string(status).decode()


def last_error() -> str:
    return lib.kvdec_last_error().decode()


def _check(status):
    if status != KVDEC_OK:
        raise KvdecError(status, last_error())


def _ptr(t):
    if t is None:
        return None
    if not isinstance(t, torch.Tensor):
        raise TypeError("expected a torch.Tensor")
    if not t.is_contiguous():
        raise ValueError("tensors must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def attn_desc(*, batch, num_q_heads, num_kv_heads, dtype, layout, max_seqlen, head_dim=128,
              softmax_scale=None, page_size=0, max_pages_per_seq=0, split_tokens=0, kv_rows=0,
              kv_format=KVDEC_KV_SAME, k_scale=1.0, v_scale=1.0):
    """dtype: of q and out (and of K/V unless kv_format is KVDEC_KV_E4M3, where
    K and V are uint8 e4m3 codes times k_scale / v_scale)."""
    if softmax_scale is None:
        softmax_scale = head_dim ** -0.5
    return AttnDesc(batch, num_q_heads, num_kv_heads, head_dim, softmax_scale,
                    _DTYPES[dtype] if isinstance(dtype, torch.dtype) else int(dtype), layout,
                    max_seqlen, page_size, max_pages_per_seq, split_tokens, kv_rows,
                    int(kv_format), float(k_scale), float(v_scale))


def hybrid_desc(*, num_pers_slots, pers_cap, buf_cap, **kw):
    kw.setdefault("layout", KVDEC_DENSE)
    kw.setdefault("max_seqlen", 0)
    return HybridDesc(attn_desc(**kw), num_pers_slots, pers_cap, buf_cap)


def gather_desc(*, max_k, **kw):
    """base fields as attn_desc (max_seqlen = the cache's rows per sequence)."""
    kw.setdefault("layout", KVDEC_DENSE)
    return GatherDesc(attn_desc(**kw), max_k)


def topk_desc(*, batch, num_q_heads, num_kv_heads, dtype, max_seqlen, top_k, head_dim=128):
    return TopkDesc(batch, num_q_heads, num_kv_heads, head_dim,
                    _DTYPES[dtype] if isinstance(dtype, torch.dtype) else int(dtype), max_seqlen, top_k)


def kvdec_gather_attn_workspace(desc: GatherDesc) -> int:
    n = ctypes.c_size_t()
    _check(lib.kvdec_gather_attn_workspace(ctypes.byref(desc), ctypes.byref(n)))
    return n.value


def kvdec_gather_attn(desc, q, k, v, idx, idx_len, out, lse, workspace, stream=None):
    ws_ptr = None if workspace is None else ctypes.c_void_p(workspace.data_ptr())
    ws_n = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib.kvdec_gather_attn(ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v), _ptr(idx),
                                 _ptr(idx_len), _ptr(out), _ptr(lse), ws_ptr, ws_n, _stream(stream)))
    return out


def kvdec_topk_select_workspace(desc: TopkDesc) -> int:
    n = ctypes.c_size_t()
    _check(lib.kvdec_topk_select_workspace(ctypes.byref(desc), ctypes.byref(n)))
    return n.value


def kvdec_topk_select(desc, q, k, seqlens, idx, idx_len, workspace, stream=None):
    ws_ptr = None if workspace is None else ctypes.c_void_p(workspace.data_ptr())
    ws_n = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib.kvdec_topk_select(ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(seqlens), _ptr(idx),
                                 _ptr(idx_len), ws_ptr, ws_n, _stream(stream)))
    return idx


def kvdec_decode_attn_workspace(desc: AttnDesc) -> int:
    n = ctypes.c_size_t()
    _check(lib.kvdec_decode_attn_workspace(ctypes.byref(desc), ctypes.byref(n)))
    return n.value


def kvdec_sparse_hybrid_attn_workspace(desc: HybridDesc) -> int:
    n = ctypes.c_size_t()
    _check(lib.kvdec_sparse_hybrid_attn_workspace(ctypes.byref(desc), ctypes.byref(n)))
    return n.value


def kvdec_kvpr_split(b, s_prime, l_max, h, elem_bytes, v_com, v_gpu):
    """KVPR split point: (l, t(l) in seconds) minimising the section A2 layer time."""
    l, t = ctypes.c_int32(), ctypes.c_double()
    _check(lib.kvdec_kvpr_split(int(b), int(s_prime), int(l_max), int(h), int(elem_bytes),
                                float(v_com), float(v_gpu), ctypes.byref(l), ctypes.byref(t)))
    return l.value, t.value


def _host_ptr(t):
    if not isinstance(t, torch.Tensor) or t.is_cuda:
        raise TypeError("expected a host (CPU) torch.Tensor")
    if not t.is_contiguous():
        raise ValueError("tensors must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


def kvdec_kvpr_load_layer(x_host, x_dev, k_host, v_host, w_k, w_v, k_cache, v_cache, l, s_prime,
                          w_layout=0, compute_stream=None, copy_stream=None):
    """x_host [b, s_x, h] bf16 and k_host, v_host [b, s_cap_h, H, 128] fp16 in pinned host
    memory; x_dev [b, l, h] bf16 staging; caches [b, s_cap, H, 128] fp16 (rows [0, s') made
    complete on compute_stream)."""
    b, s_x, h = x_host.shape
    H, hd = k_cache.shape[2], k_cache.shape[3]
    if copy_stream is None:
        raise ValueError("copy_stream is required (a stream other than compute_stream)")
    _check(lib.kvdec_kvpr_load_layer(b, int(l), int(s_prime), h, H, hd, _host_ptr(x_host), s_x * h,
                                     _ptr(x_dev), _host_ptr(k_host), _host_ptr(v_host),
                                     k_host.shape[1] * H * hd, _ptr(w_k), _ptr(w_v), int(w_layout),
                                     _ptr(k_cache), _ptr(v_cache), k_cache.shape[1] * H * hd,
                                     _stream(compute_stream), _stream(copy_stream)))


def prefetch_desc(*, batch, num_kv_heads, elem_bytes, max_seqlen, pool_strides, max_k, buf_cap,
                  head_dim=128):
    """pool_strides: (b, s, h) element strides of the host pool."""
    sb, ss, sh = (int(x) for x in pool_strides)
    return PrefetchDesc(batch, num_kv_heads, head_dim, elem_bytes, max_seqlen, sb, ss, sh, max_k,
                        buf_cap)


class HostFlag:
    """A 32-bit flag in fine-grained pinned host memory (kvdec_host_flag_alloc).
    `value` reads and writes it from the host; `ptr` is its address."""

    def __init__(self):
        p = ctypes.c_void_p()
        _check(lib.kvdec_host_flag_alloc(ctypes.byref(p)))
        self.ptr = p.value
        self._word = ctypes.c_uint32.from_address(self.ptr)

    @property
    def value(self) -> int:
        return self._word.value

    @value.setter
    def value(self, v: int) -> None:
        self._word.value = int(v) & 0xFFFFFFFF

    def close(self) -> None:
        if self.ptr:
            _check(lib.kvdec_host_flag_free(ctypes.c_void_p(self.ptr)))
            self.ptr = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def _flag_ptr(f):
    if isinstance(f, HostFlag):
        return ctypes.c_void_p(f.ptr)
    return _ptr(f)


def _any_ptr(t):
    """Address of a contiguous tensor on the host or the device."""
    if t is None:
        return None
    if not t.is_contiguous():
        raise ValueError("tensors must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


def kvdec_headcache_prefetch(desc, miss_list, miss_count, head_map, idx, idx_len, pool_k, pool_v,
                             buf_k, buf_v, buf_len, ready_flag=None, ready_value=0, timeout_us=0,
                             status=None, stream=None):
    """pool_k, pool_v: pinned host tensors; the rest on the device (status may also be a
    HostFlag-like host-mapped word); ready_flag: HostFlag or None."""
    _check(lib.kvdec_headcache_prefetch(
        ctypes.byref(desc), _ptr(miss_list), _ptr(miss_count), _ptr(head_map), _ptr(idx),
        _ptr(idx_len), _any_ptr(pool_k), _any_ptr(pool_v), _ptr(buf_k), _ptr(buf_v), _ptr(buf_len),
        None if ready_flag is None else _flag_ptr(ready_flag), int(ready_value) & 0xFFFFFFFF,
        int(timeout_us), None if status is None else _flag_ptr(status), _stream(stream)))


def kvdec_flag_wait(flag, value, timeout_us, status, stream=None):
    """flag: HostFlag or device int32 tensor; status: device int32 tensor or HostFlag."""
    _check(lib.kvdec_flag_wait(_flag_ptr(flag), int(value) & 0xFFFFFFFF, int(timeout_us),
                               _flag_ptr(status), _stream(stream)))


def kvdec_flag_signal(flag, value, stream=None):
    _check(lib.kvdec_flag_signal(_flag_ptr(flag), int(value) & 0xFFFFFFFF, _stream(stream)))


def kvdec_kernel_timing(enable: bool) -> None:
    _check(lib.kvdec_kernel_timing(1 if enable else 0))


def kvdec_kernel_timing_read():
    """(summed main-kernel milliseconds, launches) since kvdec_kernel_timing(True)."""
    ms, n = ctypes.c_double(), ctypes.c_int64()
    _check(lib.kvdec_kernel_timing_read(ctypes.byref(ms), ctypes.byref(n)))
    return ms.value, n.value


def kvdec_stream_read(src, sink, stream=None) -> None:
    """Reads all of device tensor `src` once (the streaming-read reference); may
    write one uint32 into device tensor `sink` (at least 4 bytes)."""
    if sink.numel() * sink.element_size() < 4:
        raise ValueError("sink needs at least 4 bytes")
    _check(lib.kvdec_stream_read(_ptr(src), src.numel() * src.element_size(), _ptr(sink), _stream(stream)))


def alloc_workspace(nbytes: int, device="cuda"):
    """Workspace buffer (uint8, contents irrelevant); None when nbytes is 0."""
    if nbytes == 0:
        return None
    return torch.empty(nbytes, dtype=torch.uint8, device=device)


def kvdec_decode_attn(desc, q, k, v, seqlens, cu_seqlens, block_table, out, lse, workspace,
                      stream=None):
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib.kvdec_decode_attn(ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v), _ptr(seqlens),
                                 _ptr(cu_seqlens), _ptr(block_table), _ptr(out), _ptr(lse),
                                 _ptr(workspace), ws_bytes, _stream(stream)))
    return out


def kvdec_decode_attn_noalloc(desc, q, k, v, seqlens, cu_seqlens, block_table, out, lse,
                              stream=None):
    """kvdec_decode_attn with the library's own scratch in place of a workspace."""
    _check(lib.kvdec_decode_attn_noalloc(ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v),
                                         _ptr(seqlens), _ptr(cu_seqlens), _ptr(block_table),
                                         _ptr(out), _ptr(lse), _stream(stream)))
    return out


def kvdec_sparse_hybrid_attn(desc, q, pers_k, pers_v, pers_len, buf_k, buf_v, buf_len, head_map,
                             out, lse, workspace, stream=None):
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib.kvdec_sparse_hybrid_attn(ctypes.byref(desc), _ptr(q), _ptr(pers_k), _ptr(pers_v),
                                        _ptr(pers_len), _ptr(buf_k), _ptr(buf_v), _ptr(buf_len),
                                        _ptr(head_map), _ptr(out), _ptr(lse), _ptr(workspace),
                                        ws_bytes, _stream(stream)))
    return out


def kvdec_headcache_lookup(q, labels, weights, tau, hit, agg=None, cos=None, miss_list=None,
                           miss_count=None, stream=None):
    B, Hq, D = q.shape
    Hkv = tau.numel()
    _check(lib.kvdec_headcache_lookup(B, Hq, Hkv, D, _DTYPES[q.dtype], _ptr(q), _ptr(labels),
                                      _ptr(weights), _ptr(tau), _ptr(hit), _ptr(agg), _ptr(cos),
                                      _ptr(miss_list), _ptr(miss_count), _stream(stream)))
    return hit


def kvdec_headcache_lookup_ahead(x_prev, w_q, q_approx, labels, weights, tau, hit, agg=None,
                                 cos=None, miss_list=None, miss_count=None, stream=None):
    """x_prev [B, h]; w_q [Hq*D, h] as nn.Linear stores it; q_approx [B, Hq, D]
    (written); the rest as kvdec_headcache_lookup, run on q_approx."""
    B, Hq, D = q_approx.shape
    h = x_prev.shape[1]
    Hkv = tau.numel()
    _check(lib.kvdec_headcache_lookup_ahead(B, Hq, Hkv, D, h, _DTYPES[q_approx.dtype], _ptr(x_prev),
                                            _ptr(w_q), _ptr(q_approx), _ptr(labels), _ptr(weights),
                                            _ptr(tau), _ptr(hit), _ptr(agg), _ptr(cos),
                                            _ptr(miss_list), _ptr(miss_count), _stream(stream)))
    return hit


def kvdec_headcache_thresholds(s, eta=0.8, n_exp=3.0):
    """Host-side Eqs. 7-9; s is a CPU float32 tensor, returns a CPU float32 tensor."""
    s = torch.as_tensor(s, dtype=torch.float32).contiguous()
    tau = torch.empty_like(s)
    _check(lib.kvdec_headcache_thresholds(s.numel(), ctypes.c_void_p(s.data_ptr()), float(eta),
                                          float(n_exp), ctypes.c_void_p(tau.data_ptr())))
    return tau


def kvdec_kv_recompute(x, w_k, w_v, k_cache, v_cache, l, w_layout=0, stream=None):
    """x [b, s_x, h] bf16; w_k, w_v [h, h] bf16 ([in, out] for KVDEC_W_IN_OUT,
    [out, in] as nn.Linear stores them for KVDEC_W_OUT_IN); k_cache, v_cache
    [b, s_cap, H, 128] fp16 (rows [0, l) written)."""
    b, s_x, h = x.shape
    H, hd = k_cache.shape[2], k_cache.shape[3]
    _check(lib.kvdec_kv_recompute(b, l, h, H, hd, _ptr(x), s_x * h, _ptr(w_k), _ptr(w_v), int(w_layout),
                                  _ptr(k_cache), _ptr(v_cache), k_cache.shape[1] * H * hd,
                                  _stream(stream)))
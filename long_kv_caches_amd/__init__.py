"""libkvdec: long-KV-cache decode kernels for AMD MI355X (gfx950).

The compute lives in the HIP library ``libkvdec.so`` (C ABI in include/kvdec.h);
this package is its thin ctypes binding (``_lib``) and build script (``build``).
"""
from ._lib import (  # noqa: F401
    KVDEC_BF16, KVDEC_DENSE, KVDEC_F16, KVDEC_KV_E4M3, KVDEC_KV_SAME, KVDEC_PAGED, KVDEC_RAGGED,
    KVDEC_W_IN_OUT, KVDEC_W_OUT_IN,
    AttnDesc, HybridDesc,
    KvdecError, alloc_workspace, attn_desc, hybrid_desc, kvdec_decode_attn,
    kvdec_decode_attn_noalloc, NOALLOC_SCRATCH_BYTES,
    kvdec_decode_attn_workspace, kvdec_headcache_lookup, kvdec_headcache_lookup_ahead,
    kvdec_headcache_thresholds,
    kvdec_kernel_timing, kvdec_kernel_timing_read, kvdec_kv_recompute, kvdec_kvpr_load_layer,
    kvdec_kvpr_split, kvdec_sparse_hybrid_attn,
    kvdec_sparse_hybrid_attn_workspace, last_error, status_string,
    GatherDesc, TopkDesc, gather_desc, topk_desc, kvdec_gather_attn, kvdec_gather_attn_workspace,
    kvdec_topk_select, kvdec_topk_select_workspace, kvdec_stream_read,
    PrefetchDesc, prefetch_desc, HostFlag, kvdec_headcache_prefetch, kvdec_flag_wait,
    kvdec_flag_signal, check_enabled,
)

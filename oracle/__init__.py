"""fp64 CPU oracle for the long-KV-cache decode path -- TEST INFRASTRUCTURE ONLY.

Only the tests, the smoke check and the benchmark's CPU-baseline leg may import
this package.  The product library never calls it, and it shares no code with
the GPU path.  The arithmetic lives in ``oracle.c`` (plain loops in fp64); this
module only compiles it, loads it and marshals numpy arrays.

Parity status of each routine (what pins it) is listed in the docstrings; the
pins themselves are the ``tests/test_oracle_*.py`` files.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None

F16, BF16 = 0, 1
DENSE, RAGGED, PAGED = 0, 1, 2


def build(force: bool = True) -> str:
    """Compile liboracle.so with gcc (fp64, OpenMP)."""
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + ".tmp"
        subprocess.check_call(
            ["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared", "-Wall", "-Wextra",
             "-Wno-unused-parameter", _SRC, "-o", tmp, "-lm", "-lpthread"])
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        build(force=False)
    lib = ctypes.CDLL(_LIB_PATH)
    P = ctypes.c_void_p
    i32, i64, f64 = ctypes.c_int, ctypes.c_int64, ctypes.c_double
    lib.orc_widen.argtypes = [ctypes.c_uint16, i32]
    lib.orc_widen.restype = f64
    lib.orc_widen_array.argtypes = [P, P, ctypes.c_size_t, i32]
    lib.orc_widen_array.restype = None
    lib.orc_widen_e4m3_array.argtypes = [P, P, ctypes.c_size_t]
    lib.orc_widen_e4m3_array.restype = None
    lib.orc_decode_attn_e4m3.argtypes = [i32, i32, i32, i32, f64, i32, i32, i32, i32, i32,
                                         P, P, P, f64, f64, P, P, P, P, P, i32]
    lib.orc_decode_attn_e4m3.restype = i32
    lib.orc_hybrid_attn_e4m3.argtypes = [i32, i32, i32, i32, f64, i32, i32, i32, i32,
                                         P, P, P, P, P, P, P, P, f64, f64, P, P, i32]
    lib.orc_hybrid_attn_e4m3.restype = i32
    lib.orc_decode_attn.argtypes = [i32, i32, i32, i32, f64, i32, i32, i32, i32, i32,
                                    P, P, P, P, P, P, P, P, i32]
    lib.orc_decode_attn.restype = i32
    lib.orc_attend_rows.argtypes = [i32, f64, i32, P, P, P, P, i32, P, P, P]
    lib.orc_attend_rows.restype = None
    lib.orc_hybrid_attn.argtypes = [i32, i32, i32, i32, f64, i32, i32, i32, i32,
                                    P, P, P, P, P, P, P, P, P, P, i32]
    lib.orc_hybrid_attn.restype = i32
    lib.orc_thresholds.argtypes = [i32, P, f64, f64, P]
    lib.orc_thresholds.restype = None
    lib.orc_headcache_lookup.argtypes = [i32, i32, i32, i32, i32, P, P, P, P, P, P, P, P, P]
    lib.orc_headcache_lookup.restype = i32
    lib.orc_kv_recompute.argtypes = [i32, i32, i32, i32, P, i64, P, P, P, i32, P, P, i32]
    lib.orc_kv_recompute.restype = i32
    lib.orc_kvpr_cost.argtypes = [f64, f64, f64, f64, f64, P, P, P]
    lib.orc_kvpr_cost.restype = None
    lib.orc_kvpr_time.argtypes = [f64] * 7
    lib.orc_kvpr_time.restype = f64
    lib.orc_kvpr_best_split.argtypes = [f64, ctypes.c_int, ctypes.c_int, f64, f64, f64, f64, P]
    lib.orc_kvpr_best_split.restype = ctypes.c_int
    lib.orc_topk_scores.argtypes = [i32, i32, i32, i32, i32, i32, P, P, P, P, P, i32]
    lib.orc_topk_scores.restype = i32
    lib.orc_topk_select.argtypes = [i32, i32, i32, i32, i32, i32, P, P, P, i32, P, P, i32]
    lib.orc_topk_select.restype = i32
    lib.orc_gather_attn.argtypes = [i32, i32, i32, i32, f64, i32, i32, P, P, P, P, P, i32, P, P, i32]
    lib.orc_gather_attn.restype = i32
    lib.orc_max_threads.argtypes = []
    lib.orc_max_threads.restype = i32
    _lib = lib
    return lib


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _u16(a):
    """View a float16 / uint16 array as contiguous uint16 bits."""
    a = np.ascontiguousarray(a)
    if a.dtype == np.float16:
        return a.view(np.uint16)
    if a.dtype != np.uint16:
        raise TypeError(f"expected float16 or uint16 bits, got {a.dtype}")
    return a


def _i32(a):
    return None if a is None else np.ascontiguousarray(a, dtype=np.int32)


def max_threads() -> int:
    return int(_load().orc_max_threads())


def widen(bits, kind=F16):
    """Exact widening of 16-bit values (fp16 or bf16 bit patterns) to fp64."""
    b = _u16(bits)
    out = np.empty(b.shape, np.float64)
    _load().orc_widen_array(_ptr(b), _ptr(out), b.size, kind)
    return out


def widen_e4m3(codes):
    """Exact values of OCP e4m3 codes (uint8) as fp64."""
    c = np.ascontiguousarray(codes, dtype=np.uint8)
    out = np.empty(c.shape, np.float64)
    _load().orc_widen_e4m3_array(_ptr(c), _ptr(out), c.size)
    return out


def decode_attn(q, k, v, *, num_kv_heads, layout, scale, kind=F16, seqlens=None,
                cu_seqlens=None, block_table=None, page_size=16, nthreads=0, k_scale=None,
                v_scale=None):
    """Decode attention in fp64 (KVPR page, section A3 MHA equation, one query token).

    q [B, Hq, D]; k, v in the dense [B, S, Hkv, D], ragged [T, Hkv, D] or
    paged [P, Hkv, page, D] layout.  Returns (out [B, Hq, D], lse [B, Hq]).
    Pinned by: single key, identical keys, q = 0, two-key logistic closed form,
    shift/permutation invariance, torch fp64 SDPA, paged = ragged = dense.
    k and v as uint8 arrays are e4m3 codes: element = code value * k_scale
    (v_scale for V); q and the output keep `kind`.
    """
    fp8 = np.asarray(k).dtype == np.uint8
    q = _u16(q)
    if fp8:
        k = np.ascontiguousarray(k, dtype=np.uint8); v = np.ascontiguousarray(v, dtype=np.uint8)
        if k_scale is None or v_scale is None:
            raise ValueError("e4m3 K/V need k_scale and v_scale")
    else:
        k = _u16(k); v = _u16(v)
    B, Hq, D = q.shape
    S = k.shape[1] if layout == DENSE else 0
    max_pages = 0
    if layout == PAGED:
        block_table = _i32(block_table)
        max_pages = block_table.shape[1]
        page_size = k.shape[2]
    out = np.zeros((B, Hq, D), np.float64)
    lse = np.zeros((B, Hq), np.float64)
    if fp8:
        rc = _load().orc_decode_attn_e4m3(B, Hq, num_kv_heads, D, float(scale), kind, layout, S,
                                          page_size, max_pages, _ptr(q), _ptr(k), _ptr(v),
                                          float(k_scale), float(v_scale), _ptr(_i32(seqlens)),
                                          _ptr(_i32(cu_seqlens)), _ptr(block_table), _ptr(out),
                                          _ptr(lse), nthreads)
    else:
        rc = _load().orc_decode_attn(B, Hq, num_kv_heads, D, float(scale), kind, layout, S,
                                     page_size, max_pages, _ptr(q), _ptr(k), _ptr(v),
                                     _ptr(_i32(seqlens)), _ptr(_i32(cu_seqlens)),
                                     _ptr(block_table), _ptr(out), _ptr(lse), nthreads)
    if rc != 0:
        raise ValueError("orc_decode_attn: bad arguments")
    return out, lse


def attend_rows(q_row, k, v, rows, scale, kind=F16):
    """Unnormalised attention of one query over explicit rows -> (o, m, l)."""
    q_row = _u16(q_row); k = _u16(k); v = _u16(v)
    D = q_row.shape[-1]
    rows = np.ascontiguousarray(rows, dtype=np.int64) * D
    o = np.zeros(D, np.float64)
    m = ctypes.c_double(); l = ctypes.c_double()
    _load().orc_attend_rows(D, float(scale), kind, _ptr(q_row), _ptr(k), _ptr(v), _ptr(rows),
                            int(rows.size), _ptr(o), ctypes.byref(m), ctypes.byref(l))
    return o, m.value, l.value


def hybrid_attn(q, pers_k, pers_v, pers_len, buf_k, buf_v, buf_len, head_map, *, scale,
                kind=F16, nthreads=0, k_scale=None, v_scale=None):
    """CLO cache buffer + persistent cache attention in fp64 (CLO page, section 7).
    uint8 K/V arrays are e4m3 codes, as in decode_attn."""
    fp8 = np.asarray(pers_k).dtype == np.uint8
    q = _u16(q)
    if fp8:
        conv = lambda a: np.ascontiguousarray(a, dtype=np.uint8)
        if k_scale is None or v_scale is None:
            raise ValueError("e4m3 K/V need k_scale and v_scale")
    else:
        conv = _u16
    pers_k = conv(pers_k); pers_v = conv(pers_v)
    buf_k = conv(buf_k); buf_v = conv(buf_v)
    B, Hq, D = q.shape
    Hkv = buf_k.shape[1]
    P_slots, pers_cap = pers_k.shape[1], pers_k.shape[2]
    buf_cap = buf_k.shape[2]
    out = np.zeros((B, Hq, D), np.float64)
    lse = np.zeros((B, Hq), np.float64)
    if fp8:
        rc = _load().orc_hybrid_attn_e4m3(B, Hq, Hkv, D, float(scale), kind, P_slots, pers_cap,
                                          buf_cap, _ptr(q), _ptr(pers_k), _ptr(pers_v),
                                          _ptr(_i32(pers_len)), _ptr(buf_k), _ptr(buf_v),
                                          _ptr(_i32(buf_len)), _ptr(_i32(head_map)),
                                          float(k_scale), float(v_scale), _ptr(out), _ptr(lse),
                                          nthreads)
    else:
        rc = _load().orc_hybrid_attn(B, Hq, Hkv, D, float(scale), kind, P_slots, pers_cap,
                                     buf_cap, _ptr(q), _ptr(pers_k), _ptr(pers_v),
                                     _ptr(_i32(pers_len)), _ptr(buf_k), _ptr(buf_v),
                                     _ptr(_i32(buf_len)), _ptr(_i32(head_map)), _ptr(out),
                                     _ptr(lse), nthreads)
    if rc != 0:
        raise ValueError("orc_hybrid_attn: bad arguments")
    return out, lse


def topk_scores(q, k, *, num_kv_heads, seqlens=None, kind=F16, nthreads=0):
    """CLO top-k scores in fp64: s[b, g, t] = sum over KV head g's query heads
    of q_j . K_t (t < len_b, else 0), and m[b, g, t] = sum |q_jd K_td|.
    k is the dense cache [B, S, Hkv, D]."""
    q = _u16(q); k = _u16(k)
    B, Hq, D = q.shape
    S = k.shape[1]
    s = np.zeros((B, num_kv_heads, S), np.float64)
    m = np.zeros_like(s)
    rc = _load().orc_topk_scores(B, Hq, num_kv_heads, D, kind, S, _ptr(q), _ptr(k),
                                 _ptr(_i32(seqlens)), _ptr(s), _ptr(m), nthreads)
    if rc != 0:
        raise ValueError("orc_topk_scores: bad arguments")
    return s, m


def topk_select(q, k, top_k, *, num_kv_heads, seqlens=None, kind=F16, nthreads=0):
    """Exact top-k per (sequence, KV head) of the scores above (ties: smaller
    token), ascending.  Returns (idx [B, Hkv, top_k] int32, idx_len [B * Hkv])."""
    q = _u16(q); k = _u16(k)
    B, Hq, D = q.shape
    S = k.shape[1]
    idx = np.full((B, num_kv_heads, max(top_k, 0)), -1, np.int32)
    n = np.zeros(B * num_kv_heads, np.int32)
    rc = _load().orc_topk_select(B, Hq, num_kv_heads, D, kind, S, _ptr(q), _ptr(k),
                                 _ptr(_i32(seqlens)), int(top_k), _ptr(idx), _ptr(n), nthreads)
    if rc != 0:
        raise ValueError("orc_topk_select: bad arguments")
    return idx, n


def gather_attn(q, k, v, idx, idx_len, *, num_kv_heads, scale, kind=F16, nthreads=0):
    """Attention of each query head over the token rows idx[b, g, :idx_len] of
    the dense cache [B, S, Hkv, D] (CLO top-k sparse attention, gathered in place)."""
    q = _u16(q); k = _u16(k); v = _u16(v)
    idx = np.ascontiguousarray(idx, dtype=np.int32)
    B, Hq, D = q.shape
    S = k.shape[1]
    out = np.zeros((B, Hq, D), np.float64)
    lse = np.zeros((B, Hq), np.float64)
    rc = _load().orc_gather_attn(B, Hq, num_kv_heads, D, float(scale), kind, S, _ptr(q), _ptr(k),
                                 _ptr(v), _ptr(idx), _ptr(_i32(idx_len)), idx.shape[2], _ptr(out),
                                 _ptr(lse), nthreads)
    if rc != 0:
        raise ValueError("orc_gather_attn: bad arguments")
    return out, lse


def thresholds(s, eta=0.8, n_exp=3.0):
    """CLO Eqs. 7-9 in fp64: tau_i = cos(s_i^n arccos(eta) + (1 - s_i^n) pi)."""
    s = np.ascontiguousarray(s, dtype=np.float64)
    tau = np.empty_like(s)
    _load().orc_thresholds(int(s.size), _ptr(s), float(eta), float(n_exp), _ptr(tau))
    return tau


def headcache_lookup(q, labels, weights, tau, *, num_kv_heads, kind=F16):
    """CLO head-wise cache lookup + label update in fp64.

    Returns a dict with hit [B, Hkv] (uint8), agg [B, Hkv], cos [B, Hq],
    labels (updated copy), miss_list, miss_count.
    """
    q = _u16(q)
    lab = _u16(labels).copy()
    B, Hq, D = q.shape
    Hkv = num_kv_heads
    w = np.ascontiguousarray(weights, dtype=np.float32)
    t = np.ascontiguousarray(tau, dtype=np.float32)
    hit = np.zeros(B * Hkv, np.uint8)
    agg = np.zeros(B * Hkv, np.float64)
    cosv = np.zeros(B * Hq, np.float64)
    ml = np.full(B * Hkv, -1, np.int32)
    mc = ctypes.c_int32()
    rc = _load().orc_headcache_lookup(B, Hq, Hkv, D, kind, _ptr(q), _ptr(lab), _ptr(w), _ptr(t),
                                      _ptr(hit), _ptr(agg), _ptr(cosv), _ptr(ml), ctypes.byref(mc))
    if rc != 0:
        raise ValueError("orc_headcache_lookup: bad arguments")
    n = mc.value
    return dict(hit=hit.reshape(B, Hkv), agg=agg.reshape(B, Hkv), cos=cosv.reshape(B, Hq),
                labels=lab, miss_list=ml[:n].copy(), miss_count=n)


def approx_query(x_prev, w_q, *, kind=F16):
    """CLO one-layer-ahead query (CLO page, section 3, decoding flow, Figure 9):
    q_approx = x_{l-1} W_Q^l in fp64, with W_Q stored output index first
    ([N, h], as nn.Linear keeps it), so q[b][n] = sum_i x[b][i] W[n][i].

    x_prev [B, h] and w_q [N, h] are 16-bit bits; returns [B, N] fp64.  The
    products and sums are exact-to-fp64 (numpy matmul as the one step).
    """
    x = widen(x_prev, kind)
    w = widen(w_q, kind)
    if x.ndim != 2 or w.ndim != 2 or x.shape[1] != w.shape[1]:
        raise ValueError("approx_query: x_prev [B, h] and w_q [N, h] expected")
    return x @ w.T


def kv_recompute(x, w_k, w_v, *, l, rows=None, kind=BF16, nthreads=0):
    """KVPR partial recompute in fp64: rows of X[:, 0:l] . W_K and . W_V.

    x [b, s, h] (16-bit bits); w_k, w_v [h, h].  rows: flat indices bi*l + t, or
    None for all b*l rows.  Returns (k [nrows, h], v [nrows, h]).
    """
    x = _u16(x); w_k = _u16(w_k); w_v = _u16(w_v)
    b, s, h = x.shape
    r = None if rows is None else _i32(rows)
    nrows = b * l if r is None else int(r.size)
    ko = np.zeros((nrows, h), np.float64)
    vo = np.zeros((nrows, h), np.float64)
    rc = _load().orc_kv_recompute(b, l, h, kind, _ptr(x), s * h, _ptr(w_k), _ptr(w_v), _ptr(r),
                                  nrows, _ptr(ko), _ptr(vo), nthreads)
    if rc != 0:
        raise ValueError("orc_kv_recompute: bad arguments")
    return ko, vo


def kvpr_cost(b, l, s_prime, h, p):
    """KVPR cost model (section A2): (bytes of X[0:l], bytes of KV[l:s'], FLOPs)."""
    mx, mkv, nf = ctypes.c_double(), ctypes.c_double(), ctypes.c_double()
    _load().orc_kvpr_cost(float(b), float(l), float(s_prime), float(h), float(p),
                          ctypes.byref(mx), ctypes.byref(mkv), ctypes.byref(nf))
    return mx.value, mkv.value, nf.value


def kvpr_time(b, l, s_prime, h, p, v_com, v_gpu):
    """KVPR section A2 layer time t(l) = M_X/v_com + max(N/v_gpu, M_KV/v_com)."""
    return _load().orc_kvpr_time(float(b), float(l), float(s_prime), float(h), float(p),
                                 float(v_com), float(v_gpu))


def kvpr_best_split(b, s_prime, l_max, h, p, v_com, v_gpu):
    """(l, t) of least t(l) over every integer l in [0, l_max], tried one by one."""
    t = ctypes.c_double()
    l = _load().orc_kvpr_best_split(float(b), int(s_prime), int(l_max), float(h), float(p),
                                    float(v_com), float(v_gpu), ctypes.byref(t))
    return l, t.value


def prefetch_missed(pool_k, pool_v, idx, idx_len, miss_list, buf_k, buf_v, buf_len,
                    head_map=None):
    """CLO miss-driven prefetch (CLO page, section 3: the heads the lookup of
    layer l misses are fetched during layer l-1, Figure 9; Figure 7: an update
    writes the new KV rows straight to their final place in the cache buffer).

    pool_k, pool_v [B, S, Hkv, D] (the offloaded full KV); idx [B, Hkv, max_k]
    and idx_len [B*Hkv] (each pair's selected token rows); miss_list: pairs
    b*Hkv + g; buf_k, buf_v [B, Hkv, buf_cap, D] and buf_len [B*Hkv] (the cache
    buffer before the update); head_map [Hkv] or None (slot >= 0: persistent
    head, never fetched).  For every listed buffer head:
        n = min(idx_len, max_k, buf_cap);  buf[b, g, i] = pool[b, idx[b, g, i], g]  (i < n);
        buf_len[b*Hkv + g] = n.
    Returns updated copies (buf_k, buf_v, buf_len); everything else is left as
    it was.  A listed pair outside the batch, or an index outside [0, S),
    raises ValueError.  Pinned by: a selection of every token reproduces the
    whole head; attention over the updated buffer equals the pinned gather
    attention over the same indices; the result ignores the list's order.
    """
    pool_k = np.asarray(pool_k); pool_v = np.asarray(pool_v)
    B, S, Hkv, D = pool_k.shape
    idx = np.asarray(idx, np.int32)
    idx_len = np.asarray(idx_len, np.int32).reshape(-1)
    max_k, buf_cap = idx.shape[2], np.asarray(buf_k).shape[2]
    bk = np.array(buf_k, copy=True); bv = np.array(buf_v, copy=True)
    bl = np.array(buf_len, np.int32, copy=True).reshape(-1)
    for p in np.asarray(miss_list, np.int64).reshape(-1):
        if p < 0 or p >= B * Hkv:
            raise ValueError(f"prefetch_missed: pair {p} outside the batch")
        b, g = divmod(int(p), Hkv)
        if head_map is not None and head_map[g] >= 0:
            continue
        n = max(0, min(int(idx_len[p]), max_k, buf_cap))
        rows = idx[b, g, :n]
        if np.any((rows < 0) | (rows >= S)):
            raise ValueError(f"prefetch_missed: index outside [0, {S}) for pair {p}")
        bk[b, g, :n] = pool_k[b, rows, g]
        bv[b, g, :n] = pool_v[b, rows, g]
        bl[p] = n
    return bk, bv, bl

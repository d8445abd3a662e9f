"""C-ABI checks that need no GPU: every declared symbol is exported, and every
validation error returns its status before any HIP call (fake device pointers
are never dereferenced on the host)."""
import ctypes
import os
import re

import numpy as np
import torch
import pytest

import long_kv_caches_amd as K
from long_kv_caches_amd import _lib
import oracle

HEADER = os.path.join(os.path.dirname(os.path.dirname(__file__)), "include", "kvdec.h")
FAKE = ctypes.c_void_p(0x10000)  # never dereferenced: validation fails first


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(kvdec_[a-z_0-9]+)\s*\(", text)))


def test_every_declared_symbol_is_exported():
    names = _declared()
    assert len(names) >= 10
    for n in names:
        assert hasattr(_lib.lib, n), n
    assert set(names) == set(_lib.EXPORTED)
    assert _lib.lib.kvdec_abi_version() == 11


def test_status_strings():
    assert K.status_string(0) == "KVDEC_OK"
    assert K.status_string(3) == "KVDEC_ERR_WORKSPACE"


def _desc(**kw):
    base = dict(batch=2, num_q_heads=8, num_kv_heads=2, dtype=0, layout=K.KVDEC_RAGGED,
                max_seqlen=100, kv_rows=200)
    base.update(kw)
    return K.attn_desc(**base)


def _decode(desc, ws=None, ws_bytes=0, **ptrs):
    p = dict(q=FAKE, k=FAKE, v=FAKE, seqlens=FAKE, cu=FAKE, bt=FAKE, out=FAKE, lse=None)
    p.update(ptrs)
    return _lib.lib.kvdec_decode_attn(ctypes.byref(desc) if desc is not None else None, p["q"],
                                      p["k"], p["v"], p["seqlens"], p["cu"], p["bt"], p["out"],
                                      p["lse"], ws, ws_bytes, None)


@pytest.mark.parametrize("kw,status,needle", [
    (dict(head_dim=64), K._lib.KVDEC_ERR_UNSUPPORTED, "head_dim"),
    (dict(num_q_heads=7), K._lib.KVDEC_ERR_INVALID, "num_q_heads"),
    (dict(num_q_heads=32, num_kv_heads=2), K._lib.KVDEC_ERR_UNSUPPORTED, "per KV head"),
    (dict(dtype=7), K._lib.KVDEC_ERR_UNSUPPORTED, "dtype"),
    (dict(layout=9), K._lib.KVDEC_ERR_INVALID, "layout"),
    (dict(batch=-1), K._lib.KVDEC_ERR_INVALID, "batch"),
    (dict(split_tokens=100), K._lib.KVDEC_ERR_INVALID, "split_tokens"),
    (dict(max_seqlen=-5), K._lib.KVDEC_ERR_INVALID, "max_seqlen"),
    (dict(layout=K.KVDEC_PAGED, page_size=8, max_pages_per_seq=20), K._lib.KVDEC_ERR_UNSUPPORTED,
     "page_size"),
    (dict(layout=K.KVDEC_PAGED, page_size=16, max_pages_per_seq=2), K._lib.KVDEC_ERR_INVALID,
     "max_pages_per_seq"),
    (dict(layout=K.KVDEC_PAGED, page_size=16, max_pages_per_seq=8, kv_rows=0),
     K._lib.KVDEC_ERR_INVALID, "kv_rows"),
    (dict(softmax_scale=float("inf")), K._lib.KVDEC_ERR_INVALID, "softmax_scale"),
])
def test_decode_desc_validation(kw, status, needle):
    d = _desc(**kw)
    assert _decode(d) == status
    assert needle in K.last_error()
    with pytest.raises(K.KvdecError):
        K.kvdec_decode_attn_workspace(d)


def test_decode_pointer_and_workspace_validation():
    assert _decode(None) == K._lib.KVDEC_ERR_INVALID
    assert _decode(_desc(), q=None) == K._lib.KVDEC_ERR_INVALID
    assert _decode(_desc(), cu=None) == K._lib.KVDEC_ERR_INVALID
    assert "cu_seqlens" in K.last_error()
    pd = _desc(layout=K.KVDEC_PAGED, page_size=16, max_pages_per_seq=8, kv_rows=10)
    assert _decode(pd, bt=None) == K._lib.KVDEC_ERR_INVALID
    # a long split problem needs a workspace
    big = _desc(batch=4, max_seqlen=40000, kv_rows=160000)
    need = K.kvdec_decode_attn_workspace(big)
    assert need > 0
    assert _decode(big, ws=None, ws_bytes=0) == K._lib.KVDEC_ERR_WORKSPACE
    assert _decode(big, ws=FAKE, ws_bytes=need - 1) == K._lib.KVDEC_ERR_WORKSPACE
    assert str(need) in K.last_error()
    assert _decode(big, ws=ctypes.c_void_p(0x10008), ws_bytes=need) == K._lib.KVDEC_ERR_WORKSPACE
    assert "16-byte aligned" in K.last_error()
    # empty batch is a no-op success
    assert _decode(_desc(batch=0)) == K._lib.KVDEC_OK


def test_workspace_sizes():
    # fixed chunks covering each sequence in one item need no partials
    small = _desc(max_seqlen=100, split_tokens=128)
    assert K.kvdec_decode_attn_workspace(small) == 0
    # the balanced schedule always keeps its per-unit column table and partial slots
    assert K.kvdec_decode_attn_workspace(_desc(max_seqlen=100)) > 0
    d = _desc(batch=16, num_q_heads=32, num_kv_heads=8, max_seqlen=32768, kv_rows=393216,
              split_tokens=512)
    items = 16 * 8 * (32768 // 512)
    up = lambda x: (x + 255) // 256 * 256
    assert K.kvdec_decode_attn_workspace(d) == up(items * 4 * 128 * 4) + up(items * 4 * 2 * 4)


def test_hybrid_validation():
    h = K.hybrid_desc(batch=1, num_q_heads=8, num_kv_heads=2, dtype=0, num_pers_slots=-1,
                      pers_cap=10, buf_cap=10)
    n = ctypes.c_size_t()
    assert _lib.lib.kvdec_sparse_hybrid_attn_workspace(ctypes.byref(h), ctypes.byref(n)) == 1
    h.num_pers_slots = 1
    rc = _lib.lib.kvdec_sparse_hybrid_attn(ctypes.byref(h), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
                                           FAKE, None, FAKE, None, None, 0, None)
    assert rc == K._lib.KVDEC_ERR_INVALID and "head_map" in K.last_error()


def test_lookup_validation():
    L = _lib.lib.kvdec_headcache_lookup
    args = [FAKE] * 5
    assert L(2, 8, 3, 128, 0, *args, None, None, None, None, None) == K._lib.KVDEC_ERR_INVALID
    assert L(2, 8, 2, 64, 0, *args, None, None, None, None, None) == K._lib.KVDEC_ERR_UNSUPPORTED
    assert L(2, 64, 2, 128, 0, *args, None, None, None, None, None) == K._lib.KVDEC_ERR_UNSUPPORTED
    assert L(2, 8, 2, 128, 0, *args, None, None, FAKE, None, None) == K._lib.KVDEC_ERR_INVALID
    assert "miss_list" in K.last_error()
    assert L(0, 8, 2, 128, 0, None, None, None, None, None, None, None, None, None, None) == 0


def test_lookup_ahead_validation():
    A = _lib.lib.kvdec_headcache_lookup_ahead
    lk = [FAKE] * 5  # q_approx, labels, weights, tau, hit
    # the lookup rules apply first
    assert A(2, 8, 3, 128, 4096, 0, FAKE, FAKE, *lk, None, None, None, None, None) == 1
    # h: a multiple of 8 in [8, 8192]
    assert A(2, 8, 2, 128, 4100, 0, FAKE, FAKE, *lk, None, None, None, None, None) == 2
    assert A(2, 8, 2, 128, 8200, 0, FAKE, FAKE, *lk, None, None, None, None, None) == 2
    assert A(2, 8, 2, 128, 0, 0, FAKE, FAKE, *lk, None, None, None, None, None) == 2
    assert A(2, 8, 2, 128, 4096, 0, None, FAKE, *lk, None, None, None, None, None) == 1
    assert "x_prev" in K.last_error()
    misaligned = ctypes.c_void_p(FAKE.value + 2)
    assert A(2, 8, 2, 128, 4096, 0, FAKE, misaligned, *lk, None, None, None, None, None) == 1
    assert "aligned" in K.last_error()
    assert A(0, 8, 2, 128, 4096, 0, None, None, None, None, None, None, None, None, None, None,
             None, None) == 0


def test_recompute_validation():
    R = _lib.lib.kvdec_kv_recompute
    assert R(2, 4, 5000, 40, 128, FAKE, 4 * 5000, FAKE, FAKE, 0, FAKE, FAKE, 8 * 5000, None) == 1
    assert R(2, 4, 5120, 40, 64, FAKE, 4 * 5120, FAKE, FAKE, 0, FAKE, FAKE, 8 * 5120, None) == 2
    assert R(2, 4, 384, 3, 128, FAKE, 4 * 384, FAKE, FAKE, 0, FAKE, FAKE, 8 * 384, None) == 2
    assert R(2, 4, 5120, 40, 128, FAKE, 3 * 5120, FAKE, FAKE, 0, FAKE, FAKE, 8 * 5120, None) == 1
    assert R(2, 4, 5120, 40, 128, FAKE, 4 * 5120, FAKE, FAKE, 2, FAKE, FAKE, 8 * 5120, None) == 1
    assert "w_layout" in K.last_error()
    assert R(2, 0, 5120, 40, 128, None, 0, None, None, 1, None, None, 0, None) == 0


def test_thresholds_host_helper_matches_oracle_bitwise():
    s = np.concatenate([[0.0, 1.0, 0.5], np.random.default_rng(0).beta(0.5, 2, 200)]).astype(np.float32)
    for eta, n in ((0.8, 3.0), (0.5, 1.0), (-1.0, 3.0), (0.95, 7.0)):
        ours = K.kvdec_headcache_thresholds(s, eta, n).numpy()
        ref = oracle.thresholds(s.astype(np.float64), eta, n).astype(np.float32)
        assert np.array_equal(ours, ref)
    with pytest.raises(K.KvdecError):
        K.kvdec_headcache_thresholds([1.5])
    with pytest.raises(K.KvdecError):
        K.kvdec_headcache_thresholds([0.5], eta=1.5)


def test_kernel_timing_without_launches():
    """Timing can be switched on and read with nothing launched (no GPU needed)."""
    K.kvdec_kernel_timing(True)
    assert K.kvdec_kernel_timing_read() == (0.0, 0)
    K.kvdec_kernel_timing(False)


def test_null_kv_only_without_rows():
    """k / v may be NULL only when no K/V row can be read."""
    assert _decode(_desc(kv_rows=100), k=None, v=None) == K._lib.KVDEC_ERR_INVALID
    assert "k and v" in K.last_error()
    assert _decode(_desc(layout=K.KVDEC_DENSE, max_seqlen=16), k=None) == K._lib.KVDEC_ERR_INVALID


def test_kvpr_split_matches_the_oracle_scan():
    """The closed-form split point equals the oracle's try-every-l scan."""
    rng = np.random.default_rng(5)
    cases = [(32, 1024, 1024, 5120, 2, 50e9, 1e15), (32, 1024, 256, 5120, 2, 50e9, 1e15),
             (1, 1, 1, 256, 2, 1e9, 1e9), (4, 0, 0, 512, 2, 1e9, 1e12)]
    for _ in range(300):
        s = int(rng.integers(0, 3000))
        cases.append((int(rng.integers(1, 64)), s, int(rng.integers(0, s + 1)), int(rng.integers(1, 9000)),
                      int(rng.choice([1, 2, 4])), float(10 ** rng.uniform(8, 12)), float(10 ** rng.uniform(11, 16))))
    for b, s, lmax, h, p, vc, vg in cases:
        l, t = K.kvdec_kvpr_split(b, s, lmax, h, p, vc, vg)
        lo, to = oracle.kvpr_best_split(b, s, lmax, h, p, vc, vg)
        assert abs(t - to) <= 1e-12 * max(to, 1e-30), (b, s, lmax, h, p, vc, vg)
        # equal times: the oracle keeps the smallest l, so l may only differ on an exact tie
        assert l == lo or oracle.kvpr_time(b, l, s, h, p, vc, vg) == to


def test_kvpr_split_and_load_validation():
    with pytest.raises(K.KvdecError):
        K.kvdec_kvpr_split(1, 10, 11, 256, 2, 1e9, 1e12)  # l_max > s'
    with pytest.raises(K.KvdecError):
        K.kvdec_kvpr_split(1, 10, 5, 256, 2, 0.0, 1e12)
    L = _lib.lib.kvdec_kvpr_load_layer
    S1, S2 = ctypes.c_void_p(0x10), ctypes.c_void_p(0x20)
    args = (FAKE, 4 * 512, FAKE, FAKE, FAKE, 8 * 512, FAKE, FAKE, 0, FAKE, FAKE, 8 * 512)
    assert L(2, 4, 8, 512, 4, 128, *args, S1, S1) == K._lib.KVDEC_ERR_INVALID  # same stream
    assert "differ" in K.last_error()
    assert L(2, 9, 8, 512, 4, 128, *args, S1, S2) == K._lib.KVDEC_ERR_INVALID  # l > s'
    assert L(2, 4, 8, 512, 4, 128, *args[:5], 7 * 512, *args[6:], S1, S2) == K._lib.KVDEC_ERR_INVALID
    assert "s_prime" in K.last_error()


def test_e4m3_kv_format_validation():
    D = K.attn_desc(batch=2, num_q_heads=8, num_kv_heads=2, dtype=torch.float16,
                    layout=K.KVDEC_DENSE, max_seqlen=64)
    n = ctypes.c_size_t()
    W = _lib.lib.kvdec_decode_attn_workspace
    D.kv_format = 7
    assert W(ctypes.byref(D), ctypes.byref(n)) == K._lib.KVDEC_ERR_UNSUPPORTED
    D.kv_format = K.KVDEC_KV_E4M3
    for ks, vs in ((0.0, 1.0), (1.0, -1.0), (float("nan"), 1.0), (1.0, float("inf"))):
        D.k_scale, D.v_scale = ks, vs
        assert W(ctypes.byref(D), ctypes.byref(n)) == K._lib.KVDEC_ERR_INVALID
        assert "scale" in K.last_error()
    D.k_scale, D.v_scale = 0.01, 0.02
    assert W(ctypes.byref(D), ctypes.byref(n)) == 0


def test_descriptor_layout_matches_the_header(tmp_path):
    """The ctypes descriptors have the C structs' size and field offsets."""
    import shutil
    import subprocess
    if shutil.which("gcc") is None or not os.path.isdir("/opt/rocm/include"):
        pytest.skip("gcc or the ROCm headers are not available")
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    fields = [f for f, _ in _lib.AttnDesc._fields_]
    src = tmp_path / "layout.c"
    lines = ['#include <stddef.h>', '#include <stdio.h>', '#include "kvdec.h"', "int main(void) {",
             'printf("%zu %zu\\n", sizeof(kvdec_attn_desc), sizeof(kvdec_hybrid_desc));']
    lines += [f'printf("%zu\\n", offsetof(kvdec_attn_desc, {f}));' for f in fields]
    lines += ["return 0; }"]
    src.write_text("\n".join(lines))
    exe = tmp_path / "layout"
    subprocess.check_call(["gcc", "-D__HIP_PLATFORM_AMD__", "-I", os.path.join(root, "include"),
                           "-I", "/opt/rocm/include", str(src), "-o", str(exe)])
    out = subprocess.check_output([str(exe)]).decode().split()
    assert int(out[0]) == ctypes.sizeof(_lib.AttnDesc)
    assert int(out[1]) == ctypes.sizeof(_lib.HybridDesc)
    for f, off in zip(fields, out[2:]):
        assert int(off) == getattr(_lib.AttnDesc, f).offset, f


def test_gather_and_topk_validation():
    n = ctypes.c_size_t()
    gd = K.gather_desc(batch=2, num_q_heads=8, num_kv_heads=2, dtype=torch.float16, max_seqlen=100,
                       max_k=10)
    assert _lib.lib.kvdec_gather_attn_workspace(ctypes.byref(gd), ctypes.byref(n)) == 0
    gd.max_k = -1
    assert _lib.lib.kvdec_gather_attn_workspace(ctypes.byref(gd), ctypes.byref(n)) == 1
    gd.max_k = 10
    gd.base.max_seqlen = 1 << 23  # S * Hkv * 256 B > 2^31
    assert _lib.lib.kvdec_gather_attn_workspace(ctypes.byref(gd), ctypes.byref(n)) == 2
    gd.base.max_seqlen = 100
    G = _lib.lib.kvdec_gather_attn
    assert G(ctypes.byref(gd), FAKE, FAKE, FAKE, None, FAKE, FAKE, None, None, 0, None) == 1
    assert "idx" in K.last_error()
    td = K.topk_desc(batch=2, num_q_heads=8, num_kv_heads=2, dtype=torch.float16, max_seqlen=100,
                     top_k=10)
    assert _lib.lib.kvdec_topk_select_workspace(ctypes.byref(td), ctypes.byref(n)) == 0
    # per pair: a score row of S rounded up to 4 floats, then three merged digit
    # histograms (2048 + 2048 + 1024 words), 8 words of state, and per
    # 16384-token chunk a 1024-bin histogram and 4 more words
    assert n.value == 2 * 2 * (100 * 4 + (5120 + 8 + 1 * 1028) * 4)  # S = 100: one chunk
    td.max_seqlen = 40001
    assert _lib.lib.kvdec_topk_select_workspace(ctypes.byref(td), ctypes.byref(n)) == 0
    assert n.value == 2 * 2 * (40004 * 4 + (5120 + 8 + 3 * 1028) * 4)  # three chunks
    td.max_seqlen = 100
    T = _lib.lib.kvdec_topk_select
    assert T(ctypes.byref(td), FAKE, FAKE, None, FAKE, FAKE, None, 0, None) == 3  # workspace
    td.max_seqlen = 300000
    assert _lib.lib.kvdec_topk_select_workspace(ctypes.byref(td), ctypes.byref(n)) == 2
    td.max_seqlen, td.top_k = 100, -1
    assert _lib.lib.kvdec_topk_select_workspace(ctypes.byref(td), ctypes.byref(n)) == 1


@pytest.mark.parametrize("src,nbytes,sink,needle", [
    (None, 1024, FAKE, "non-NULL"),
    (FAKE, 1024, None, "non-NULL"),
    (FAKE, 0, FAKE, "multiple of 16"),
    (FAKE, 1000, FAKE, "multiple of 16"),
    (ctypes.c_void_p(0x10008), 1024, FAKE, "aligned"),
])
def test_stream_read_validation(src, nbytes, sink, needle):
    st = _lib.lib.kvdec_stream_read(src, nbytes, sink, None)
    assert st == K._lib.KVDEC_ERR_INVALID
    assert needle in K.last_error()


def test_noalloc_rejects_calls_beyond_its_scratch():
    # Fixed 64-token chunks of a 2^20-token bound: 8 pairs x 16384 chunks x
    # 8 heads of partials, far above the library's scratch.  The call must say
    # so before any HIP call (the fake pointers are never touched).
    d = _desc(batch=1, num_q_heads=64, num_kv_heads=8, max_seqlen=1 << 20, kv_rows=16,
              split_tokens=64)
    need = K.kvdec_decode_attn_workspace(d)
    assert need > _lib.NOALLOC_SCRATCH_BYTES
    st = _lib.lib.kvdec_decode_attn_noalloc(ctypes.byref(d), FAKE, FAKE, FAKE, None, FAKE, None,
                                            FAKE, None, None)
    assert st == _lib.KVDEC_ERR_WORKSPACE
    assert "scratch" in K.last_error() and str(need) in K.last_error()
    # descriptor errors come first, as in kvdec_decode_attn
    bad = _desc(head_dim=64)
    st = _lib.lib.kvdec_decode_attn_noalloc(ctypes.byref(bad), FAKE, FAKE, FAKE, None, FAKE, None,
                                            FAKE, None, None)
    assert st == _lib.KVDEC_ERR_UNSUPPORTED
    # an empty batch is a no-op
    empty = _desc(batch=0)
    assert _lib.lib.kvdec_decode_attn_noalloc(ctypes.byref(empty), None, None, None, None, None,
                                              None, None, None, None) == _lib.KVDEC_OK


def test_check_mode_follows_the_environment(monkeypatch):
    monkeypatch.delenv("KVDEC_CHECK", raising=False)
    assert not K.check_enabled()
    monkeypatch.setenv("KVDEC_CHECK", "1")
    assert K.check_enabled()
    monkeypatch.setenv("KVDEC_CHECK", "0")
    assert not K.check_enabled()

"""GPU checks of the KVDEC_CHECK=1 debug mode: malformed device metadata is
rejected with KVDEC_ERR_INVALID before any launch (outputs keep their
sentinel values), and well-formed calls give the same bits as with the mode
off.  Every malformed value here is one the kernels also clamp, so no case
could make a kernel read out of bounds even if its check were missing."""
import numpy as np
import pytest
import torch

import kvgen
import long_kv_caches_amd as K
from long_kv_caches_amd import _lib
from gpu_util import bits, dev, say

pytestmark = pytest.mark.gpu


@pytest.fixture
def check_on(monkeypatch):
    monkeypatch.setenv("KVDEC_CHECK", "1")
    assert K.check_enabled()


def _rejects(fn, out, needle):
    before = bits(out).copy() if out.dtype != torch.int32 else out.cpu().numpy().copy()
    with pytest.raises(K.KvdecError) as e:
        fn()
    torch.cuda.synchronize()
    assert e.value.status == _lib.KVDEC_ERR_INVALID, str(e.value)
    assert "KVDEC_CHECK" in str(e.value) and needle in str(e.value), str(e.value)
    after = bits(out) if out.dtype != torch.int32 else out.cpu().numpy()
    assert np.array_equal(before, after)  # nothing ran
    say(f"  rejected: {str(e.value)[:110]}")


def _ragged_call(d, cu_host, max_seqlen=None, kv_rows=None):
    B, Hq, Hkv = d["B"], d["Hq"], d["Hkv"]
    q, k, v = dev(d["q"]), dev(d["k"]), dev(d["v"])
    cu = torch.from_numpy(np.asarray(cu_host, np.int32)).cuda()
    desc = K.attn_desc(batch=B, num_q_heads=Hq, num_kv_heads=Hkv, dtype=torch.float16,
                       layout=K.KVDEC_RAGGED,
                       max_seqlen=max_seqlen or int(np.diff(d["cu_seqlens"]).max()),
                       softmax_scale=d["scale"], kv_rows=kv_rows or d["k"].shape[0])
    ws = K.alloc_workspace(K.kvdec_decode_attn_workspace(desc))
    out = torch.full((B, Hq, 128), 3.0, dtype=torch.float16, device="cuda")
    return out, lambda: K.kvdec_decode_attn(desc, q, k, v, None, cu, None, out, None, ws)


def test_valid_calls_give_the_same_bits_with_checks_on(monkeypatch):
    d = kvgen.ragged_llama(seed=41, lens=[300, 0, 1000, 17], Hq=32, Hkv=8)
    monkeypatch.delenv("KVDEC_CHECK", raising=False)
    out0, run0 = _ragged_call(d, d["cu_seqlens"])
    run0()
    monkeypatch.setenv("KVDEC_CHECK", "1")
    out1, run1 = _ragged_call(d, d["cu_seqlens"])
    run1()
    torch.cuda.synchronize()
    assert np.array_equal(bits(out0), bits(out1))


def test_decode_ragged_rejections(check_on):
    d = kvgen.ragged_llama(seed=42, lens=[100, 200, 50], Hq=8, Hkv=2)
    cu = d["cu_seqlens"]
    say("[check] ragged metadata")
    out, run = _ragged_call(d, [1, cu[1], cu[2], cu[3]])
    _rejects(run, out, "cu_seqlens[0]")
    out, run = _ragged_call(d, [0, cu[2], cu[1], cu[3]], max_seqlen=400)
    _rejects(run, out, "decreases")
    out, run = _ragged_call(d, cu, max_seqlen=150)
    _rejects(run, out, "max_seqlen")
    out, run = _ragged_call(d, [0, cu[1], cu[2], cu[3] + 5], max_seqlen=300)
    _rejects(run, out, "kv_rows")


def test_decode_dense_and_paged_rejections(check_on):
    say("[check] dense seqlens and paged block table")
    d = kvgen.dense_small(seed=43, B=2, Hq=8, Hkv=2, S=64)
    q, k, v = dev(d["q"]), dev(d["k"]), dev(d["v"])
    desc = K.attn_desc(batch=2, num_q_heads=8, num_kv_heads=2, dtype=torch.float16,
                       layout=K.KVDEC_DENSE, max_seqlen=64, softmax_scale=d["scale"])
    ws = K.alloc_workspace(K.kvdec_decode_attn_workspace(desc))
    out = torch.full((2, 8, 128), 3.0, dtype=torch.float16, device="cuda")
    for bad in ([65, 10], [10, -1]):
        sl = torch.tensor(bad, dtype=torch.int32, device="cuda")
        _rejects(lambda: K.kvdec_decode_attn(desc, q, k, v, sl, None, None, out, None, ws), out,
                 "seqlens")
    p = kvgen.paged_mha(seed=44, B=3, H=4, median=40, lo=20, hi=90, max_pages=8)
    q, k, v = dev(p["q"]), dev(p["k"]), dev(p["v"])
    P = p["k"].shape[0]
    desc = K.attn_desc(batch=3, num_q_heads=4, num_kv_heads=4, dtype=torch.float16,
                       layout=K.KVDEC_PAGED, max_seqlen=int(p["seqlens"].max()),
                       softmax_scale=p["scale"], page_size=16, max_pages_per_seq=8, kv_rows=P)
    ws = K.alloc_workspace(K.kvdec_decode_attn_workspace(desc))
    out = torch.full((3, 4, 128), 3.0, dtype=torch.float16, device="cuda")
    sl = torch.from_numpy(p["seqlens"]).cuda()
    for bad in (P, -1):
        bt = p["block_table"].copy()
        bt[1, 0] = bad  # a used page of sequence 1
        btd = torch.from_numpy(bt).cuda()
        _rejects(lambda: K.kvdec_decode_attn(desc, q, k, v, sl, None, btd, out, None, ws), out,
                 "block_table[1][0]")
    # entries past a sequence's last page are never read and not checked
    bt = p["block_table"].copy()
    bt[0, 7] = P + 100
    K.kvdec_decode_attn(desc, q, k, v, sl, None, torch.from_numpy(bt).cuda(), out, None, ws)
    torch.cuda.synchronize()


def test_hybrid_rejections(check_on):
    say("[check] hybrid head map and lengths")
    B, Hq, Hkv, cap = 2, 8, 4, 32
    rng = np.random.default_rng(45)
    q = dev(rng.standard_normal((B, Hq, 128)).astype(np.float16))
    pk = dev(rng.standard_normal((B, 1, cap, 128)).astype(np.float16))
    bk = dev(rng.standard_normal((B, Hkv, cap, 128)).astype(np.float16))
    desc = K.hybrid_desc(batch=B, num_q_heads=Hq, num_kv_heads=Hkv, dtype=torch.float16,
                         num_pers_slots=1, pers_cap=cap, buf_cap=cap)
    ws = K.alloc_workspace(K.kvdec_sparse_hybrid_attn_workspace(desc))
    out = torch.full((B, Hq, 128), 3.0, dtype=torch.float16, device="cuda")
    i32 = lambda a: torch.tensor(a, dtype=torch.int32, device="cuda")
    good = dict(hm=[0, -1, -1, -1], pl=[cap, 5], bl=[1, 2, 3, 4, 5, 6, 7, 8])
    cases = [(dict(hm=[1, -1, -1, -1]), "head_map[0]"), (dict(hm=[0, -2, -1, -1]), "head_map[1]"),
             (dict(pl=[cap + 1, 5]), "pers_len[0]"), (dict(bl=[1, 2, 3, 4, 5, cap + 1, 7, 8]), "buf_len[5]"),
             (dict(bl=[1, -3, 3, 4, 5, 6, 7, 8]), "buf_len[1]")]
    for change, needle in cases:
        a = dict(good, **change)
        _rejects(lambda: K.kvdec_sparse_hybrid_attn(desc, q, pk, pk, i32(a["pl"]), bk, bk,
                                                    i32(a["bl"]), i32(a["hm"]), out, None, ws),
                 out, needle)
    # a persistent head's buf_len is not read, so it is not checked
    bl = list(good["bl"])
    bl[0] = cap + 50
    K.kvdec_sparse_hybrid_attn(desc, q, pk, pk, i32(good["pl"]), bk, bk, i32(bl), i32(good["hm"]),
                               out, None, ws)
    torch.cuda.synchronize()


def test_gather_and_topk_rejections(check_on):
    say("[check] gather indices and top-k lengths")
    B, Hq, Hkv, S, mk = 2, 8, 2, 100, 10
    rng = np.random.default_rng(46)
    q = dev(rng.standard_normal((B, Hq, 128)).astype(np.float16))
    k = dev(rng.standard_normal((B, S, Hkv, 128)).astype(np.float16))
    gd = K.gather_desc(batch=B, num_q_heads=Hq, num_kv_heads=Hkv, dtype=torch.float16,
                       max_seqlen=S, max_k=mk)
    ws = K.alloc_workspace(K.kvdec_gather_attn_workspace(gd))
    out = torch.full((B, Hq, 128), 3.0, dtype=torch.float16, device="cuda")
    idx = np.tile(np.arange(mk, dtype=np.int32), (B, Hkv, 1))
    n = np.full(B * Hkv, mk, np.int32)
    for what, needle in (("len", "idx_len[2]"), ("hi", "idx[1][4]"), ("lo", "idx[3][0]")):
        i2, n2 = idx.copy(), n.copy()
        if what == "len":
            n2[2] = mk + 1
        elif what == "hi":
            i2[0, 1, 4] = S
        else:
            i2[1, 1, 0] = -1
        _rejects(lambda: K.kvdec_gather_attn(gd, q, k, k, torch.from_numpy(i2).cuda(),
                                             torch.from_numpy(n2).cuda(), out, None, ws),
                 out, needle)
    td = K.topk_desc(batch=B, num_q_heads=Hq, num_kv_heads=Hkv, dtype=torch.float16, max_seqlen=S,
                     top_k=mk)
    tws = K.alloc_workspace(K.kvdec_topk_select_workspace(td))
    oidx = torch.full((B, Hkv, mk), -5, dtype=torch.int32, device="cuda")
    olen = torch.full((B * Hkv,), -5, dtype=torch.int32, device="cuda")
    sl = torch.tensor([S, S + 1], dtype=torch.int32, device="cuda")
    _rejects(lambda: K.kvdec_topk_select(td, q, k, sl, oidx, olen, tws), olen, "seqlens[1]")


def test_prefetch_rejections(check_on):
    say("[check] prefetch miss list and selections")
    d = kvgen.clo_prefetch(seed=47, B=2, S=256, frac=0.1)
    B, S, Hkv, D = d["pool_k"].shape
    top_k, hm = d["top_k"], d["head_map"]
    buf = int(np.argmax(hm < 0))  # a buffer head
    desc = K.prefetch_desc(batch=B, num_kv_heads=Hkv, elem_bytes=2, max_seqlen=S,
                           pool_strides=(S * Hkv * D, Hkv * D, D), max_k=top_k, buf_cap=top_k)
    pool = torch.from_numpy(d["pool_k"]).pin_memory()
    bk = torch.full((B, Hkv, top_k, D), 3.0, dtype=torch.float16, device="cuda")
    bl = torch.full((B * Hkv,), -7, dtype=torch.int32, device="cuda")
    hmd = torch.from_numpy(hm).cuda()
    i32 = lambda a: torch.tensor(a, dtype=torch.int32, device="cuda")

    def call(ml, mc, idx, n):
        return lambda: K.kvdec_headcache_prefetch(desc, i32(ml), i32([mc]), hmd,
                                                  torch.from_numpy(idx).cuda(),
                                                  torch.from_numpy(n).cuda(), pool, pool, bk, bk, bl)

    full = list(range(B * Hkv))
    idx, n = d["idx"], d["idx_len"]
    _rejects(call(full, B * Hkv + 1, idx, n), bk, "miss_count")
    _rejects(call([0, B * Hkv] + full[2:], 2, idx, n), bk, "miss_list[1]")
    n2 = n.copy()
    n2[buf] = top_k + 1
    _rejects(call(full, B * Hkv, idx, n2), bk, f"idx_len[{buf}]")
    i2 = idx.copy()
    i2[0, buf, 3] = S
    _rejects(call(full, B * Hkv, i2, n), bk, f"idx[{buf}][3]")
    # a persistent head's selection is never read, so it is not checked
    pers = int(np.argmax(hm >= 0))
    i3 = idx.copy()
    i3[0, pers, 0] = S + 9
    call([pers], 1, i3, n)()
    torch.cuda.synchronize()

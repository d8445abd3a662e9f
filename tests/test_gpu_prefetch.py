"""GPU checks of the miss-driven prefetch and the host-mapped flags.

The prefetch's buffer contents must equal, bit for bit, the oracle's gather
driven by the oracle's miss list (near-tie groups, flagged as in the lookup
tests, follow the GPU's decision).  Every flag a GPU wait depends on is raised
by the test itself, before the wait or from a host thread started before it
and joined in `finally`; the one case where it is never raised uses a short
time limit, so the kernel gives up and exits normally.
"""
import threading
import time

import numpy as np
import pytest
import torch

import kvgen
import long_kv_caches_amd as K
from long_kv_caches_amd import _lib
import oracle
from gpu_util import bits, check_close, check_lse, dev, host_f64, say

pytestmark = pytest.mark.gpu
FLAG_BAND = 1e-5


def _pinned(a):
    return torch.from_numpy(np.ascontiguousarray(a)).pin_memory()


def _poisoned_buffers(B, Hkv, cap, u8=False):
    shape = (B, Hkv, cap, 128)
    if u8:
        bk = torch.full(shape, 0x55, dtype=torch.uint8, device="cuda")
    else:
        bk = torch.full(shape, 1000.0, dtype=torch.float16, device="cuda")
    return bk, bk.clone(), torch.full((B * Hkv,), -7, dtype=torch.int32, device="cuda")


def _desc(d, u8=False):
    B, S, Hkv, D = d["pool_k"].shape
    return K.prefetch_desc(batch=B, num_kv_heads=Hkv, elem_bytes=1 if u8 else 2, max_seqlen=S,
                           pool_strides=(S * Hkv * D, Hkv * D, D), max_k=d["top_k"],
                           buf_cap=d["top_k"])


def _host(t):
    a = t.cpu().numpy()
    return a.view(np.uint16) if a.dtype == np.float16 else a


def _expected(d, miss_list, bk0, bv0, bl0, head_map):
    return oracle.prefetch_missed(d["pool_k"], d["pool_v"], d["idx"], d["idx_len"], miss_list,
                                  bk0, bv0, bl0, head_map=head_map)


def _check_buffers(got, exp, what):
    bk, bv, bl = got
    ek, ev, el = exp
    assert np.array_equal(bl.cpu().numpy(), el), f"{what}: buf_len"
    ek = ek.view(np.uint16) if ek.dtype == np.float16 else ek
    ev = ev.view(np.uint16) if ev.dtype == np.float16 else ev
    assert np.array_equal(_host(bk), ek), f"{what}: buf_k"
    assert np.array_equal(_host(bv), ev), f"{what}: buf_v"


@pytest.mark.parametrize("model", ["llama3-8b", "qwen2.5-14b"])
def test_lookup_then_prefetch_then_hybrid_attention(model):
    # The CLO step on one GPU: lookup (fused label update) -> miss list ->
    # the GPU pulls the missed buffer heads' selected rows from pinned host
    # memory -> hybrid attention over persistent heads and the updated buffer.
    d = kvgen.clo_prefetch(seed=31, model=model, B=3, S=4096, frac=0.1)
    B, S, Hkv, D = d["pool_k"].shape
    Hq, top_k, hm = d["Hq"], d["top_k"], d["head_map"]
    say(f"[prefetch] {model} B={B} S={S} top_k={top_k}")
    tau = np.full(Hkv, 0.87, np.float32)  # cosines ~0.80-0.95: a mix of hits and misses
    r = oracle.headcache_lookup(d["q"], d["labels"], d["weights"], tau, num_kv_heads=Hkv)
    flagged = np.abs(r["agg"] - tau[None, :]) < FLAG_BAND
    assert 0 < r["miss_count"] < B * Hkv

    q, labels = dev(d["q"]), dev(d["labels"])
    w = torch.from_numpy(d["weights"]).cuda()
    taud = torch.from_numpy(tau).cuda()
    hit = torch.empty(B * Hkv, dtype=torch.uint8, device="cuda")
    ml = torch.full((B * Hkv,), -1, dtype=torch.int32, device="cuda")
    mc = torch.zeros(1, dtype=torch.int32, device="cuda")
    pool_k, pool_v = _pinned(d["pool_k"]), _pinned(d["pool_v"])
    idx = torch.from_numpy(d["idx"]).cuda()
    idx_len = torch.from_numpy(d["idx_len"]).cuda()
    hmd = torch.from_numpy(hm).cuda()
    bk, bv, bl = _poisoned_buffers(B, Hkv, top_k)
    bk0, bv0, bl0 = _host(bk).view(np.float16), _host(bv).view(np.float16), bl.cpu().numpy()
    K.kvdec_headcache_lookup(q, labels, w, taud, hit, None, None, ml, mc)
    K.kvdec_headcache_prefetch(_desc(d), ml, mc, hmd, idx, idx_len, pool_k, pool_v, bk, bv, bl)
    torch.cuda.synchronize()

    gh = hit.cpu().numpy().reshape(B, Hkv)
    assert np.all((gh == r["hit"]) | flagged)
    gpu_list = ml.cpu().numpy()[:int(mc.item())]
    assert list(gpu_list) == [p for p in range(B * Hkv) if gh.reshape(-1)[p] == 0]
    if not flagged.any():
        assert np.array_equal(gpu_list, r["miss_list"])
    exp = _expected(d, gpu_list, bk0, bv0, bl0, hm)
    _check_buffers((bk, bv, bl), exp, model)
    fetched = [p for p in gpu_list if hm[p % Hkv] < 0]
    assert fetched, "no buffer head missed"

    # hybrid attention over the persistent heads' full KV and the updated buffer
    n_slots = int((hm >= 0).sum())
    pers_k = np.zeros((B, n_slots, S, D), np.float16)
    pers_v = np.zeros_like(pers_k)
    for g in range(Hkv):
        if hm[g] >= 0:
            pers_k[:, hm[g]] = d["pool_k"][:, :, g]
            pers_v[:, hm[g]] = d["pool_v"][:, :, g]
    # buffer heads that were not fetched hold poison: give them an empty length
    ek, ev, el = exp
    el = el.copy()
    el[el < 0] = 0
    bl.copy_(torch.from_numpy(el))
    desc = K.hybrid_desc(batch=B, num_q_heads=Hq, num_kv_heads=Hkv, dtype=torch.float16,
                         softmax_scale=d["scale"], num_pers_slots=n_slots, pers_cap=S,
                         buf_cap=top_k)
    ws = K.alloc_workspace(K.kvdec_sparse_hybrid_attn_workspace(desc))
    out = torch.empty((B, Hq, D), dtype=torch.float16, device="cuda")
    lse = torch.empty((B, Hq), dtype=torch.float32, device="cuda")
    pl = torch.full((B,), S, dtype=torch.int32, device="cuda")
    K.kvdec_sparse_hybrid_attn(desc, q, dev(pers_k), dev(pers_v), pl, bk, bv, bl, hmd, out, lse, ws)
    torch.cuda.synchronize()
    ro, rl = oracle.hybrid_attn(d["q"], pers_k, pers_v, np.full(B, S, np.int32), ek, ev, el, hm,
                                scale=d["scale"])
    check_close(host_f64(out), ro, f"{model} hybrid after prefetch")
    check_lse(lse.cpu().numpy(), rl, f"{model} hybrid lse")


def test_prefetch_of_e4m3_rows_and_clamped_metadata():
    # One-byte rows (e4m3 codes); a miss list holding entries outside the
    # batch and a persistent head (skipped); a selection longer than max_k
    # (clamped) and indices outside [0, S) (clamped to the first / last row).
    d = kvgen.clo_prefetch(seed=32, B=2, S=1000, frac=0.1, elem="u8")
    B, S, Hkv, D = d["pool_k"].shape
    top_k, hm = d["top_k"], d["head_map"]
    say(f"[prefetch] e4m3 rows B={B} S={S} top_k={top_k}")
    idx = d["idx"].copy()
    idx[0, 2, 5], idx[1, 4, 0] = -9, S + 17
    idx_len = d["idx_len"].copy()
    idx_len[2] = top_k + 50
    listed = [2, B * Hkv + 3, 12, -1, 1 * Hkv + 4, int(np.argmax(hm >= 0))]
    ml = torch.tensor(listed + [0] * (B * Hkv - len(listed)), dtype=torch.int32, device="cuda")
    mc = torch.tensor([len(listed)], dtype=torch.int32, device="cuda")
    bk, bv, bl = _poisoned_buffers(B, Hkv, top_k, u8=True)
    bk0, bv0, bl0 = _host(bk), _host(bv), bl.cpu().numpy()
    K.kvdec_headcache_prefetch(_desc(d, u8=True), ml, mc, torch.from_numpy(hm).cuda(),
                               torch.from_numpy(idx).cuda(), torch.from_numpy(idx_len).cuda(),
                               _pinned(d["pool_k"]), _pinned(d["pool_v"]), bk, bv, bl)
    torch.cuda.synchronize()
    # the documented clamping, applied before the oracle's gather
    idx_c = np.clip(idx, 0, S - 1)
    len_c = np.minimum(idx_len, top_k)
    valid = [p for p in listed if 0 <= p < B * Hkv]
    exp = oracle.prefetch_missed(d["pool_k"], d["pool_v"], idx_c, len_c, valid, bk0, bv0, bl0,
                                 head_map=hm)
    _check_buffers((bk, bv, bl), exp, "e4m3 rows")


def test_prefetch_waits_for_the_host_flag_and_sees_the_host_writes():
    # The pool starts as zeros; a host thread writes the real rows into the
    # pinned pool and only then raises the flag.  The GPU's copy, enqueued
    # before the thread writes anything, must see the real rows.
    d = kvgen.clo_prefetch(seed=33, B=2, S=2048, frac=0.1)
    B, S, Hkv, D = d["pool_k"].shape
    top_k = d["top_k"]
    say("[prefetch] waits for a host flag raised by a host thread after ~50 ms")
    pool_k = _pinned(np.zeros_like(d["pool_k"]))
    pool_v = _pinned(np.zeros_like(d["pool_v"]))
    flag = K.HostFlag()
    status = torch.full((1,), -1, dtype=torch.int32, device="cuda")
    all_pairs = torch.arange(B * Hkv, dtype=torch.int32, device="cuda")
    mc = torch.tensor([B * Hkv], dtype=torch.int32, device="cuda")
    bk, bv, bl = _poisoned_buffers(B, Hkv, top_k)
    bk0, bv0, bl0 = _host(bk).view(np.float16), _host(bv).view(np.float16), bl.cpu().numpy()
    idx = torch.from_numpy(d["idx"]).cuda()
    idx_len = torch.from_numpy(d["idx_len"]).cuda()
    # a first copy reads the zero pool, so lines of it may sit in the L2
    # caches when the host rewrites it: the flagged copy must not see them
    K.kvdec_headcache_prefetch(_desc(d), all_pairs, mc, None, idx, idx_len, pool_k, pool_v,
                               bk, bv, bl)
    torch.cuda.synchronize()
    assert not _host(bk)[:, :, : top_k].any()
    bk.fill_(1000.0)
    bv.fill_(1000.0)
    bl.fill_(-7)
    torch.cuda.synchronize()

    def host_transfer():
        time.sleep(0.05)
        pool_k.numpy()[...] = d["pool_k"]
        pool_v.numpy()[...] = d["pool_v"]
        flag.value = 3

    th = threading.Thread(target=host_transfer)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    try:
        th.start()
        e0.record()
        K.kvdec_headcache_prefetch(_desc(d), all_pairs, mc, None, idx, idx_len, pool_k, pool_v,
                                   bk, bv, bl, ready_flag=flag, ready_value=3, timeout_us=1000000,
                                   status=status)
        e1.record()
        torch.cuda.synchronize()
    finally:
        th.join()
    assert int(status.item()) == 0
    waited_ms = e0.elapsed_time(e1)
    say(f"  GPU-side wait + copy: {waited_ms:.1f} ms")
    assert waited_ms > 10.0  # the copy did not run before the host raised the flag
    exp = _expected(d, np.arange(B * Hkv), bk0, bv0, bl0, None)
    _check_buffers((bk, bv, bl), exp, "after the host flag")
    flag.close()


def test_wait_gives_up_when_the_flag_is_never_raised():
    # The host never raises the flag; the wait's 2 ms limit ends it, status
    # reads 1, nothing is copied and later work on the stream still runs.
    d = kvgen.clo_prefetch(seed=34, B=1, S=512, frac=0.1)
    B, S, Hkv, D = d["pool_k"].shape
    say("[prefetch] a flag the host never raises, 2 ms limit")
    flag = K.HostFlag()
    status = torch.full((1,), -1, dtype=torch.int32, device="cuda")
    ml = torch.arange(B * Hkv, dtype=torch.int32, device="cuda")
    mc = torch.tensor([B * Hkv], dtype=torch.int32, device="cuda")
    bk, bv, bl = _poisoned_buffers(B, Hkv, d["top_k"])
    before = (_host(bk).copy(), _host(bv).copy(), bl.cpu().numpy().copy())
    after = torch.zeros(1, device="cuda")
    K.kvdec_headcache_prefetch(_desc(d), ml, mc, None, torch.from_numpy(d["idx"]).cuda(),
                               torch.from_numpy(d["idx_len"]).cuda(), _pinned(d["pool_k"]),
                               _pinned(d["pool_v"]), bk, bv, bl, ready_flag=flag, ready_value=1,
                               timeout_us=2000, status=status)
    after += 1.0  # work queued after the wait runs once it has given up
    torch.cuda.synchronize()
    assert int(status.item()) == 1
    assert after.item() == 1.0
    assert np.array_equal(_host(bk), before[0]) and np.array_equal(_host(bv), before[1])
    assert np.array_equal(bl.cpu().numpy(), before[2])
    flag.close()


def test_flag_wait_and_signal():
    flag = K.HostFlag()
    status = torch.full((1,), -1, dtype=torch.int32, device="cuda")
    try:
        # raised before the wait: no waiting at all; sequence numbers compare
        # modulo 2^32, so 2 reaches a target of 0xFFFFFFFF
        flag.value = 2
        say("[flags] wait on a flag already raised")
        K.kvdec_flag_wait(flag, 0xFFFFFFFF, 1000000, status)
        torch.cuda.synchronize()
        assert int(status.item()) == 0
        # raised by a host thread during the wait
        say("[flags] wait on a flag a host thread raises after ~30 ms")
        th = threading.Thread(target=lambda: (time.sleep(0.03), setattr(flag, "value", 9)))
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        try:
            th.start()
            e0.record()
            K.kvdec_flag_wait(flag, 9, 1000000, status)
            e1.record()
            torch.cuda.synchronize()
        finally:
            th.join()
        assert int(status.item()) == 0
        assert e0.elapsed_time(e1) > 10.0
        # GPU -> host: the host polls the flag instead of synchronising
        say("[flags] signal after a kernel, polled from the host")
        x = torch.zeros(1 << 20, device="cuda")
        torch.cuda.synchronize()
        x += 5.0
        K.kvdec_flag_signal(flag, 21)
        deadline = time.time() + 10.0
        while flag.value != 21 and time.time() < deadline:
            time.sleep(0.0005)
        assert flag.value == 21
        torch.cuda.synchronize()
        assert float(x[-1].item()) == 5.0
    finally:
        torch.cuda.synchronize()
        flag.close()


def test_prefetch_refuses_pageable_or_short_pools():
    # The device miss count is 0, so no pool row would be read even if a check
    # let the call through.
    d = kvgen.clo_prefetch(seed=35, B=1, S=256, frac=0.1)
    B, S, Hkv, D = d["pool_k"].shape
    ml = torch.zeros(B * Hkv, dtype=torch.int32, device="cuda")
    mc = torch.zeros(1, dtype=torch.int32, device="cuda")
    bk, bv, bl = _poisoned_buffers(B, Hkv, d["top_k"])
    idx = torch.from_numpy(d["idx"]).cuda()
    n = torch.from_numpy(d["idx_len"]).cuda()
    pageable = torch.from_numpy(d["pool_k"].copy())
    pinned = _pinned(d["pool_k"])
    say("[prefetch] pageable pool is refused")
    with pytest.raises(K.KvdecError) as e:
        K.kvdec_headcache_prefetch(_desc(d), ml, mc, None, idx, n, pageable, pinned, bk, bv, bl)
    assert e.value.status == _lib.KVDEC_ERR_INVALID and "pool_k" in str(e.value)
    say("[prefetch] a pool shorter than the descriptor is refused")
    short = _pinned(d["pool_k"][:, : S // 2])
    with pytest.raises(K.KvdecError) as e:
        K.kvdec_headcache_prefetch(_desc(d), ml, mc, None, idx, n, pinned, short, bk, bv, bl)
    assert e.value.status == _lib.KVDEC_ERR_INVALID and "pool_v" in str(e.value)
    torch.cuda.synchronize()
    # a valid call with an empty miss list touches nothing
    before = _host(bk).copy()
    K.kvdec_headcache_prefetch(_desc(d), ml, mc, None, idx, n, pinned, pinned, bk, bv, bl)
    torch.cuda.synchronize()
    assert np.array_equal(_host(bk), before) and np.all(bl.cpu().numpy() == -7)

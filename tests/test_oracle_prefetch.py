"""Pins of the oracle's miss-driven prefetch (CLO page, section 3, Figures 7
and 9: the missed heads' selected KV rows go straight to their final place in
the cache buffer).  Each test ties it to something other than its own loop:
the whole head when every token is selected, the independently pinned gather
attention over the same indices, and invariances of the definition."""
import numpy as np
import pytest

import kvgen
import oracle


def _setup(seed=0, B=2, S=64, frac=0.25, model="llama3-8b"):
    d = kvgen.clo_prefetch(seed=seed, model=model, B=B, S=S, frac=frac)
    B, Hkv, D, top_k = d["B"], d["Hkv"], d["D"], d["top_k"]
    rng = np.random.default_rng(seed)
    buf_k = rng.standard_normal((B, Hkv, top_k, D)).astype(np.float16)
    buf_v = rng.standard_normal((B, Hkv, top_k, D)).astype(np.float16)
    buf_len = rng.integers(0, top_k + 1, B * Hkv).astype(np.int32)
    return d, buf_k, buf_v, buf_len


def test_selecting_every_token_reproduces_the_whole_head():
    d, _, _, _ = _setup(S=40)
    B, S, Hkv, D = d["pool_k"].shape
    idx = np.broadcast_to(np.arange(S, dtype=np.int32), (B, Hkv, S)).copy()
    n = np.full(B * Hkv, S, np.int32)
    bk0 = np.zeros((B, Hkv, S, D), np.float16)
    listed = [0, 3, B * Hkv - 1]
    bk, bv, bl = oracle.prefetch_missed(d["pool_k"], d["pool_v"], idx, n, listed, bk0, bk0,
                                        np.zeros(B * Hkv, np.int32))
    for p in range(B * Hkv):
        b, g = divmod(p, Hkv)
        if p in listed:
            assert np.array_equal(bk[b, g], d["pool_k"][b, :, g])
            assert np.array_equal(bv[b, g], d["pool_v"][b, :, g])
            assert bl[p] == S
        else:
            assert not bk[b, g].any() and not bv[b, g].any() and bl[p] == 0


def test_attention_over_the_prefetched_buffer_equals_gather_attention():
    # Every pair missed: the hybrid attention over the updated buffer (all
    # heads on the buffer) must equal the pinned gather attention over the
    # same indices into the full cache, bit for bit (same rows, same order).
    d, bk0, bv0, bl0 = _setup(seed=1, S=96, frac=0.3)
    B, S, Hkv, D = d["pool_k"].shape
    bk, bv, bl = oracle.prefetch_missed(d["pool_k"], d["pool_v"], d["idx"], d["idx_len"],
                                        np.arange(B * Hkv), bk0, bv0, bl0)
    assert np.array_equal(bl, d["idx_len"])
    pk = np.zeros((B, 1, 1, D), np.float16)
    o_h, l_h = oracle.hybrid_attn(d["q"], pk, pk, np.zeros(B, np.int32), bk, bv, bl,
                                  np.full(Hkv, -1, np.int32), scale=d["scale"])
    o_g, l_g = oracle.gather_attn(d["q"], d["pool_k"], d["pool_v"], d["idx"], d["idx_len"],
                                  num_kv_heads=Hkv, scale=d["scale"])
    assert np.array_equal(o_h, o_g) and np.array_equal(l_h, l_g)


def test_order_persistent_heads_and_untouched_rows():
    d, bk0, bv0, bl0 = _setup(seed=2, S=80)
    B, S, Hkv, D = d["pool_k"].shape
    hm = d["head_map"]
    idx_len = d["idx_len"].copy()
    idx_len[1] = 3  # a shorter selection: rows 3.. of that buffer keep their old contents
    listed = np.array([5, 1, 12, 0, 9, 3], np.int64)
    r1 = oracle.prefetch_missed(d["pool_k"], d["pool_v"], d["idx"], idx_len, listed, bk0, bv0, bl0,
                                head_map=hm)
    r2 = oracle.prefetch_missed(d["pool_k"], d["pool_v"], d["idx"], idx_len, listed[::-1], bk0,
                                bv0, bl0, head_map=hm)
    for a, b in zip(r1, r2):
        assert np.array_equal(a, b)
    bk, bv, bl = r1
    for p in range(B * Hkv):
        b, g = divmod(p, Hkv)
        fetched = p in listed and hm[g] < 0
        if not fetched:
            assert np.array_equal(bk[b, g], bk0[b, g]) and bl[p] == bl0[p]
            continue
        n = int(idx_len[p])
        assert bl[p] == n
        for i in range(n):  # element by element against the pool
            t = int(d["idx"][b, g, i])
            assert np.array_equal(bk[b, g, i], d["pool_k"][b, t, g])
            assert np.array_equal(bv[b, g, i], d["pool_v"][b, t, g])
        assert np.array_equal(bk[b, g, n:], bk0[b, g, n:])
    assert any(hm[p % Hkv] >= 0 for p in listed)  # a persistent head was listed and skipped


@pytest.mark.parametrize("bad", ["pair", "index"])
def test_out_of_range_inputs_are_rejected(bad):
    d, bk0, bv0, bl0 = _setup(seed=3, S=32)
    B, S, Hkv, D = d["pool_k"].shape
    idx = d["idx"].copy()
    listed = [0]
    if bad == "pair":
        listed = [B * Hkv]
    else:
        idx[0, 0, 0] = S
    with pytest.raises(ValueError):
        oracle.prefetch_missed(d["pool_k"], d["pool_v"], idx, d["idx_len"], listed, bk0, bv0, bl0)

"""Pins of the oracle's index-gather sparse attention and exact top-k
selection (CLO page: top-k sparse attention; Eq. 6, the ranking of q.k over
the keys does not depend on |q|), against brute force, the pinned dense
attention and constructed cases."""
import numpy as np

import kvgen
import oracle


def _small(seed=0, B=2, S=90, Hq=8, Hkv=2, lens=(90, 37)):
    d = kvgen.clo_gather(seed=seed, B=B, S=S, lens=lens)
    rng = np.random.default_rng(seed)
    # a smaller head count than the models': draw fresh arrays of that shape
    q = rng.standard_normal((B, Hq, 128)).astype(np.float16)
    k = rng.standard_normal((B, S, Hkv, 128)).astype(np.float16)
    v = rng.standard_normal((B, S, Hkv, 128)).astype(np.float16)
    return dict(d, q=q, k=k, v=v, Hq=Hq, Hkv=Hkv)


def test_gather_of_every_token_equals_dense_attention():
    d = _small()
    lens = d["seqlens"]
    idx = np.full((2, 2, 90), -1, np.int32)
    for b in range(2):
        idx[b, :, :lens[b]] = np.arange(lens[b])
    n = np.repeat(lens, 2).astype(np.int32)
    o1, l1 = oracle.gather_attn(d["q"], d["k"], d["v"], idx, n, num_kv_heads=2, scale=0.1)
    o2, l2 = oracle.decode_attn(d["q"], d["k"], d["v"], num_kv_heads=2, layout=oracle.DENSE,
                                scale=0.1, seqlens=lens)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)


def test_gather_equals_dense_attention_on_the_compacted_rows():
    d = _small(seed=1)
    idx, n = kvgen.random_indices(5, 2, 2, d["seqlens"], 20)
    o1, l1 = oracle.gather_attn(d["q"], d["k"], d["v"], idx, n, num_kv_heads=2, scale=0.1)
    for b in range(2):
        for g in range(2):
            rows = idx[b, g, :n[b * 2 + g]]
            kc = d["k"][b:b + 1, rows][:, :, g:g + 1]
            vc = d["v"][b:b + 1, rows][:, :, g:g + 1]
            o2, l2 = oracle.decode_attn(d["q"][b:b + 1, 4 * g:4 * g + 4], kc, vc, num_kv_heads=1,
                                        layout=oracle.DENSE, scale=0.1)
            assert np.array_equal(o1[b, 4 * g:4 * g + 4], o2[0]) and np.array_equal(l1[b, 4 * g:4 * g + 4], l2[0])


def test_gather_does_not_depend_on_index_order():
    d = _small(seed=2)
    idx, n = kvgen.random_indices(6, 2, 2, d["seqlens"], 25)
    rev = idx.copy()
    for b in range(2):
        for g in range(2):
            m = n[b * 2 + g]
            rev[b, g, :m] = idx[b, g, :m][::-1]
    o1, l1 = oracle.gather_attn(d["q"], d["k"], d["v"], idx, n, num_kv_heads=2, scale=0.1)
    o2, l2 = oracle.gather_attn(d["q"], d["k"], d["v"], rev, n, num_kv_heads=2, scale=0.1)
    np.testing.assert_allclose(o1, o2, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(l1, l2, rtol=1e-14)


def test_topk_scores_and_selection_brute_force():
    rng = np.random.default_rng(3)
    B, S, Hq, Hkv, D = 2, 12, 4, 2, 128
    q = rng.integers(-3, 4, (B, Hq, D)).astype(np.float16)
    k = rng.integers(-3, 4, (B, S, Hkv, D)).astype(np.float16)
    lens = np.array([12, 7], np.int32)
    s, m = oracle.topk_scores(q, k, num_kv_heads=Hkv, seqlens=lens)
    for b in range(B):
        for g in range(Hkv):
            for t in range(S):
                acc = 0
                mag = 0
                if t < lens[b]:
                    for j in range(2 * g, 2 * g + 2):
                        for dd in range(D):
                            acc += int(q[b, j, dd]) * int(k[b, t, g, dd])
                            mag += abs(int(q[b, j, dd]) * int(k[b, t, g, dd]))
                assert s[b, g, t] == acc and m[b, g, t] == mag
            want = sorted(range(lens[b]), key=lambda t: (-s[b, g, t], t))[:5]
            idx, n = oracle.topk_select(q, k, 5, num_kv_heads=Hkv, seqlens=lens)
            assert n[b * Hkv + g] == 5
            assert list(idx[b, g, :5]) == sorted(want)


def test_topk_edge_counts_and_ties():
    d = _small(seed=4, lens=(90, 0))
    idx, n = oracle.topk_select(d["q"], d["k"], 200, num_kv_heads=2, seqlens=d["seqlens"])
    assert list(n) == [90, 90, 0, 0]
    assert np.array_equal(idx[0, 0, :90], np.arange(90))
    # equal keys score equally: the smaller token indices win
    k = d["k"].copy()
    k[0, :, 0] = k[0, 10, 0]
    idx, n = oracle.topk_select(d["q"], k, 7, num_kv_heads=2, seqlens=d["seqlens"])
    assert list(idx[0, 0, :7]) == list(range(7))


def test_topk_set_is_invariant_to_the_query_norm():
    # Eq. 6: scaling the group's queries by a common positive factor (a power
    # of two, exact in fp16) scales every score alike and keeps the set
    d = _small(seed=5)
    idx1, n1 = oracle.topk_select(d["q"], d["k"], 9, num_kv_heads=2, seqlens=d["seqlens"])
    for c in (8.0, 0.25):
        q2 = (d["q"].astype(np.float64) * c).astype(np.float16)
        idx2, n2 = oracle.topk_select(q2, d["k"], 9, num_kv_heads=2, seqlens=d["seqlens"])
        assert np.array_equal(idx1, idx2) and np.array_equal(n1, n2)
    # one query head per KV head (MHA): each head's own norm is free
    q1 = d["q"][:, :2].copy()
    a, _ = oracle.topk_select(q1, d["k"], 9, num_kv_heads=2, seqlens=d["seqlens"])
    q1[:, 1] = (q1[:, 1].astype(np.float64) * 16).astype(np.float16)
    b_, _ = oracle.topk_select(q1, d["k"], 9, num_kv_heads=2, seqlens=d["seqlens"])
    assert np.array_equal(a, b_)

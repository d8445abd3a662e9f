"""Pins of the fp64 attention oracle against facts fixed by the mathematics.

The oracle computes softmax(q K^T * scale) V per query token (KVPR page, A3 MHA
equation).  Each test below checks it against something other than itself:
closed forms, invariants, a library routine (torch fp64 SDPA), or a brute-force
evaluation of a different formulation on tiny inputs.
"""
import math

import numpy as np
import pytest
import torch

import kvgen
import oracle

F16 = np.float16


def _widen(a):
    return np.asarray(a, np.float16).astype(np.float64)


def test_widen_f16_all_patterns():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ours = oracle.widen(bits, oracle.F16)
    ref = bits.view(np.float16).astype(np.float64)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert np.array_equal(ours[~nan], ref[~nan])


def test_widen_bf16_all_patterns():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ours = oracle.widen(bits, oracle.BF16)
    with np.errstate(invalid="ignore"):
        ref = (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert np.array_equal(ours[~nan], ref[~nan])


def _dense(q, k, v, scale=1.0, seqlens=None):
    Hkv = k.shape[2]
    return oracle.decode_attn(q, k, v, num_kv_heads=Hkv, layout=oracle.DENSE, scale=scale,
                              seqlens=seqlens)


def test_single_key_returns_v():
    rng = np.random.default_rng(1)
    q = rng.standard_normal((3, 4, 128)).astype(F16)
    k = rng.standard_normal((3, 1, 2, 128)).astype(F16)
    v = rng.standard_normal((3, 1, 2, 128)).astype(F16)
    out, lse = _dense(q, k, v, scale=0.125)
    for j in range(4):
        assert np.array_equal(out[:, j], _widen(v[:, 0, j // 2]))
    # lse of one key is its score
    s = 0.125 * np.einsum("bjd,bjd->bj", _widen(q), _widen(k[:, 0]).repeat(2, axis=1))
    np.testing.assert_allclose(lse, s, rtol=1e-13, atol=1e-13)


def test_identical_keys_give_mean_of_values():
    rng = np.random.default_rng(2)
    S = 37
    q = rng.standard_normal((1, 2, 128)).astype(F16)
    krow = rng.standard_normal((1, 1, 1, 128)).astype(F16)
    k = np.repeat(krow, S, axis=1)
    v = rng.standard_normal((1, S, 1, 128)).astype(F16)
    out, lse = _dense(q, k, v, scale=0.3)
    mean = _widen(v[0, :, 0]).mean(axis=0)
    np.testing.assert_allclose(out[0, 0], mean, rtol=0, atol=1e-14)
    np.testing.assert_allclose(out[0, 1], mean, rtol=0, atol=1e-14)
    # lse = s + ln S
    s = 0.3 * float(_widen(q[0, 0]) @ _widen(krow[0, 0, 0]))
    assert abs(lse[0, 0] - (s + math.log(S))) < 1e-12


def test_zero_query_gives_uniform_weights():
    rng = np.random.default_rng(3)
    q = np.zeros((1, 1, 128), F16)
    k = rng.standard_normal((1, 50, 1, 128)).astype(F16)
    v = rng.standard_normal((1, 50, 1, 128)).astype(F16)
    out, lse = _dense(q, k, v)
    np.testing.assert_allclose(out[0, 0], _widen(v[0, :, 0]).mean(axis=0), atol=1e-14)
    assert abs(lse[0, 0] - math.log(50)) < 1e-13


def test_two_keys_logistic_closed_form():
    # q = a e0, k_i = c_i e0 -> s_i = scale a c_i; softmax of two is a logistic.
    D = 128
    a, c1, c2, scale = 1.5, 2.0, -0.75, 0.5
    q = np.zeros((1, 1, D), F16); q[0, 0, 0] = a
    k = np.zeros((1, 2, 1, D), F16); k[0, 0, 0, 0] = c1; k[0, 1, 0, 0] = c2
    rng = np.random.default_rng(4)
    v = rng.standard_normal((1, 2, 1, D)).astype(F16)
    out, lse = _dense(q, k, v, scale)
    s1, s2 = scale * a * c1, scale * a * c2
    w1 = 1.0 / (1.0 + math.exp(s2 - s1))
    ref = w1 * _widen(v[0, 0, 0]) + (1 - w1) * _widen(v[0, 1, 0])
    np.testing.assert_allclose(out[0, 0], ref, rtol=1e-14, atol=1e-15)
    assert abs(lse[0, 0] - (max(s1, s2) + math.log1p(math.exp(-abs(s1 - s2))))) < 1e-14


def test_weights_sum_to_one_all_ones_values():
    rng = np.random.default_rng(5)
    q = (rng.standard_normal((2, 4, 128)) * 3).astype(F16)
    k = rng.standard_normal((2, 300, 2, 128)).astype(F16)
    v = np.ones((2, 300, 2, 128), F16)
    out, _ = _dense(q, k, v)
    np.testing.assert_allclose(out, 1.0, rtol=0, atol=1e-12)


def test_shift_invariance():
    # K_t <- K_t + u moves every score of a query by the same amount.
    rng = np.random.default_rng(6)
    q = (rng.integers(-8, 9, (1, 2, 128)) / 8).astype(F16)
    k = (rng.integers(-16, 17, (1, 64, 1, 128)) / 8).astype(F16)
    u = (rng.integers(-16, 17, (128,)) / 8).astype(F16)
    v = rng.standard_normal((1, 64, 1, 128)).astype(F16)
    k2 = (k.astype(np.float64) + u.astype(np.float64)).astype(F16)
    assert np.array_equal(k2.astype(np.float64), k.astype(np.float64) + u.astype(np.float64))
    o1, _ = _dense(q, k, v, 0.1)
    o2, _ = _dense(q, k2, v, 0.1)
    np.testing.assert_allclose(o2, o1, rtol=1e-12, atol=1e-14)


def test_token_permutation_invariance():
    d = kvgen.dense_small(seed=7, S=200)
    perm = np.random.default_rng(8).permutation(200)
    o1, l1 = _dense(d["q"], d["k"], d["v"], d["scale"])
    o2, l2 = _dense(d["q"], d["k"][:, perm], d["v"][:, perm], d["scale"])
    np.testing.assert_allclose(o2, o1, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(l2, l1, rtol=1e-13)


def test_gqa_equals_mha_with_repeated_kv():
    d = kvgen.dense_small(seed=9, B=2, Hq=8, Hkv=2, S=100)
    o_gqa, l_gqa = _dense(d["q"], d["k"], d["v"], d["scale"])
    k_rep = np.repeat(d["k"], 4, axis=2)
    v_rep = np.repeat(d["v"], 4, axis=2)
    o_mha, l_mha = _dense(d["q"], k_rep, v_rep, d["scale"])
    assert np.array_equal(o_gqa, o_mha) and np.array_equal(l_gqa, l_mha)
    # Hkv = 1 (MQA) against MHA with the single KV head repeated
    k1, v1 = d["k"][:, :, :1], d["v"][:, :, :1]
    o_mqa, _ = _dense(d["q"], k1, v1, d["scale"])
    o_rep, _ = _dense(d["q"], np.repeat(k1, 8, axis=2), np.repeat(v1, 8, axis=2), d["scale"])
    assert np.array_equal(o_mqa, o_rep)


def _sdpa_fp64(q, k_rows, v_rows, scale):
    """torch scaled_dot_product_attention in fp64 on the CPU for one sequence.
    q [Hq, D]; k_rows, v_rows [n, Hkv, D]."""
    Hq, Hkv = q.shape[0], k_rows.shape[1]
    qt = torch.from_numpy(_widen(q))[:, None, :]                       # [Hq, 1, D]
    kt = torch.from_numpy(_widen(k_rows)).permute(1, 0, 2)              # [Hkv, n, D]
    vt = torch.from_numpy(_widen(v_rows)).permute(1, 0, 2)
    kt = kt.repeat_interleave(Hq // Hkv, dim=0).contiguous()
    vt = vt.repeat_interleave(Hq // Hkv, dim=0).contiguous()
    o = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, scale=scale)
    s = torch.matmul(qt, kt.transpose(1, 2).contiguous()) * scale
    return o[:, 0, :].numpy(), torch.logsumexp(s[:, 0, :], dim=-1).numpy()


def test_ragged_against_torch_sdpa():
    d = kvgen.ragged_llama(seed=10, B=4, lo=1, hi=700, Hq=8, Hkv=2)
    out, lse = oracle.decode_attn(d["q"], d["k"], d["v"], num_kv_heads=2, layout=oracle.RAGGED,
                                  scale=d["scale"], cu_seqlens=d["cu_seqlens"])
    cu = d["cu_seqlens"]
    for b in range(d["B"]):
        ref_o, ref_l = _sdpa_fp64(d["q"][b], d["k"][cu[b]:cu[b + 1]], d["v"][cu[b]:cu[b + 1]],
                                  d["scale"])
        np.testing.assert_allclose(out[b], ref_o, rtol=1e-11, atol=1e-13)
        np.testing.assert_allclose(lse[b], ref_l, rtol=1e-12, atol=1e-12)


def test_paged_and_dense_equal_ragged_exactly():
    d = kvgen.ragged_llama(seed=11, B=5, lo=1, hi=300, Hq=8, Hkv=2)
    o_r, l_r = oracle.decode_attn(d["q"], d["k"], d["v"], num_kv_heads=2, layout=oracle.RAGGED,
                                  scale=d["scale"], cu_seqlens=d["cu_seqlens"])
    p = kvgen.ragged_to_paged(d, seed=3)
    o_p, l_p = oracle.decode_attn(p["q"], p["k"], p["v"], num_kv_heads=2, layout=oracle.PAGED,
                                  scale=d["scale"], seqlens=p["seqlens"],
                                  block_table=p["block_table"])
    dd = kvgen.ragged_to_dense(d)
    o_d, l_d = oracle.decode_attn(dd["q"], dd["k"], dd["v"], num_kv_heads=2, layout=oracle.DENSE,
                                  scale=d["scale"], seqlens=dd["seqlens"])
    assert np.array_equal(o_r, o_p) and np.array_equal(l_r, l_p)
    assert np.array_equal(o_r, o_d) and np.array_equal(l_r, l_d)


def test_paged_generator_against_sdpa():
    d = kvgen.paged_mha(seed=12, B=6, H=4, median=40, lo=1, hi=120, max_pages=8)
    out, lse = oracle.decode_attn(d["q"], d["k"], d["v"], num_kv_heads=4, layout=oracle.PAGED,
                                  scale=d["scale"], seqlens=d["seqlens"],
                                  block_table=d["block_table"])
    r = kvgen.paged_to_ragged(d)
    cu = r["cu_seqlens"]
    for b in range(d["B"]):
        ref_o, ref_l = _sdpa_fp64(d["q"][b], r["k"][cu[b]:cu[b + 1]], r["v"][cu[b]:cu[b + 1]],
                                  d["scale"])
        np.testing.assert_allclose(out[b], ref_o, rtol=1e-11, atol=1e-13)
        np.testing.assert_allclose(lse[b], ref_l, rtol=1e-12, atol=1e-12)
    assert np.all(np.isfinite(out))  # poison tail slots never read


def test_empty_sequence():
    d = kvgen.ragged_llama(seed=13, lens=[5, 0, 3], Hq=4, Hkv=2)
    out, lse = oracle.decode_attn(d["q"], d["k"], d["v"], num_kv_heads=2, layout=oracle.RAGGED,
                                  scale=d["scale"], cu_seqlens=d["cu_seqlens"])
    assert np.all(out[1] == 0.0) and np.all(np.isneginf(lse[1]))
    assert np.all(np.isfinite(lse[[0, 2]]))


def test_brute_force_tiny_without_max_subtraction():
    # Different formulation: direct exp(s) / sum exp(s), Python floats, no max shift.
    rng = np.random.default_rng(14)
    B, Hq, Hkv, D, S = 2, 4, 2, 8, 6
    q = rng.standard_normal((B, Hq, D)).astype(F16)
    k = rng.standard_normal((B, S, Hkv, D)).astype(F16)
    v = rng.standard_normal((B, S, Hkv, D)).astype(F16)
    lens = np.array([6, 4], np.int32)
    out, lse = _dense(q, k, v, 0.7, seqlens=lens)
    for b in range(B):
        for j in range(Hq):
            g = j // (Hq // Hkv)
            e = []
            for t in range(int(lens[b])):
                s = 0.0
                for dd in range(D):
                    s += float(q[b, j, dd]) * float(k[b, t, g, dd])
                e.append(math.exp(0.7 * s))
            z = sum(e)
            for dd in range(D):
                ref = sum(e[t] * float(v[b, t, g, dd]) for t in range(int(lens[b]))) / z
                assert abs(out[b, j, dd] - ref) < 1e-12
            assert abs(lse[b, j] - math.log(z)) < 1e-12


def test_split_merge_identity_any_partition_any_order():
    # Combining (o_c, m_c, l_c) of disjoint row ranges with weights exp(m_c - M)
    # reproduces the unsplit attention, for any cut points and merge order.
    d = kvgen.dense_small(seed=15, S=500)
    D, Hkv = 128, 2
    rows_all = np.arange(500) * Hkv + 1  # KV head 1 rows of the dense [1, S, Hkv, D] array
    q = d["q"][0, 5]
    o_full, m_full, l_full = oracle.attend_rows(q, d["k"], d["v"], rows_all, d["scale"])
    ref = o_full / l_full
    rng = np.random.default_rng(16)
    for _ in range(5):
        cuts = np.sort(rng.choice(np.arange(1, 500), size=rng.integers(1, 9), replace=False))
        parts = np.split(rows_all, cuts)
        res = [oracle.attend_rows(q, d["k"], d["v"], p, d["scale"]) for p in parts]
        order = rng.permutation(len(res))
        M = max(r[1] for r in res)
        num = np.zeros(D); den = 0.0
        for i in order:
            o, m, l = res[i]
            w = math.exp(m - M)
            num += w * o
            den += w * l
        np.testing.assert_allclose(num / den, ref, rtol=1e-12, atol=1e-15)
        assert abs((M + math.log(den)) - (m_full + math.log(l_full))) < 1e-12

"""Pins of the oracle's e4m3 KV path (CLO page, open questions: FP8 KV caches).

The e4m3 decoder is checked against torch's float8_e4m3fn conversion and the
format's defining values; the fp8-KV attention is tied to the already pinned
16-bit attention: e4m3 values (times power-of-two scales) are exact in fp16,
so both must give the same numbers bit for bit.
"""
import math

import numpy as np
import pytest
import torch

import kvgen
import oracle


def test_e4m3_decode_matches_torch_on_every_code():
    codes = np.arange(256, dtype=np.uint8)
    ours = oracle.widen_e4m3(codes)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    assert np.array_equal(np.isnan(ours), np.isnan(ref))
    assert np.array_equal(np.isnan(ours), np.isin(codes, [0x7F, 0xFF]))
    ok = ~np.isnan(ref)
    assert np.array_equal(ours[ok], ref[ok])
    assert np.array_equal(np.signbit(ours[ok]), np.signbit(ref[ok]))


def test_e4m3_defining_values():
    v = oracle.widen_e4m3(np.array([0x7E, 0x01, 0x07, 0x08, 0x38, 0xB8, 0x77, 0x00, 0x80, 0x3F],
                                   np.uint8))
    assert v[0] == 448.0 and v[1] == 2.0 ** -9 and v[2] == 7 * 2.0 ** -9 and v[3] == 2.0 ** -6
    assert v[4] == 1.0 and v[5] == -1.0 and v[6] == 240.0
    assert v[7] == 0.0 and not np.signbit(v[7]) and v[8] == 0.0 and np.signbit(v[8])
    assert v[9] == 1.875


def _random_codes(rng, shape):
    c = rng.integers(0, 256, size=shape).astype(np.uint8)
    c[(c & 0x7F) == 0x7F] = 0x38  # no NaN codes in a cache
    return c


@pytest.mark.parametrize("k_scale,v_scale", [(1.0, 1.0), (2.0 ** -3, 4.0)])
def test_fp8_attention_equals_16bit_attention_on_the_same_values(k_scale, v_scale):
    rng = np.random.default_rng(0)
    B, S, Hq, Hkv, D = 2, 37, 8, 2, 128
    k8 = _random_codes(rng, (B, S, Hkv, D))
    v8 = _random_codes(rng, (B, S, Hkv, D))
    q = rng.standard_normal((B, Hq, D)).astype(np.float16)
    # e4m3 values times these scales are exact in fp16
    k16 = (oracle.widen_e4m3(k8) * k_scale).astype(np.float16)
    v16 = (oracle.widen_e4m3(v8) * v_scale).astype(np.float16)
    assert np.array_equal(k16.astype(np.float64), oracle.widen_e4m3(k8) * k_scale)
    for seqlens in (None, np.array([37, 5], np.int32)):
        o8, l8 = oracle.decode_attn(q, k8, v8, num_kv_heads=Hkv, layout=oracle.DENSE, scale=0.05,
                                    seqlens=seqlens, k_scale=k_scale, v_scale=v_scale)
        o16, l16 = oracle.decode_attn(q, k16, v16, num_kv_heads=Hkv, layout=oracle.DENSE,
                                      scale=0.05, seqlens=seqlens)
        assert np.array_equal(o8, o16) and np.array_equal(l8, l16)


def test_k_scale_acts_through_the_scores_and_v_scale_scales_the_output():
    rng = np.random.default_rng(1)
    B, S, Hq, Hkv, D = 1, 50, 4, 1, 128
    k8, v8 = _random_codes(rng, (B, S, Hkv, D)), _random_codes(rng, (B, S, Hkv, D))
    q = rng.standard_normal((B, Hq, D)).astype(np.float16)
    a = dict(num_kv_heads=Hkv, layout=oracle.DENSE)
    o1, l1 = oracle.decode_attn(q, k8, v8, scale=0.01, k_scale=0.37, v_scale=1.0, **a)
    o2, l2 = oracle.decode_attn(q, k8, v8, scale=0.01 * 0.37, k_scale=1.0, v_scale=1.0, **a)
    np.testing.assert_allclose(o1, o2, rtol=1e-12, atol=1e-15)
    np.testing.assert_allclose(l1, l2, rtol=1e-12)
    o3, l3 = oracle.decode_attn(q, k8, v8, scale=0.01, k_scale=0.37, v_scale=0.125, **a)
    assert np.array_equal(o3, o1 * 0.125) and np.array_equal(l3, l1)


def test_fp8_hybrid_all_persistent_equals_dense():
    rng = np.random.default_rng(2)
    B, S, Hq, Hkv, D = 2, 40, 8, 2, 128
    k8, v8 = _random_codes(rng, (B, Hkv, S, D)), _random_codes(rng, (B, Hkv, S, D))
    q = rng.standard_normal((B, Hq, D)).astype(np.float16)
    lens = np.array([40, 17], np.int32)
    o_h, l_h = oracle.hybrid_attn(q, k8, v8, lens, k8[:, :, :1], v8[:, :, :1],
                                  np.zeros(B * Hkv, np.int32), np.arange(Hkv, dtype=np.int32),
                                  scale=0.09, k_scale=0.5, v_scale=2.0)
    # the same rows in the dense [B, S, Hkv, D] layout
    o_d, l_d = oracle.decode_attn(q, np.ascontiguousarray(k8.transpose(0, 2, 1, 3)),
                                  np.ascontiguousarray(v8.transpose(0, 2, 1, 3)), num_kv_heads=Hkv,
                                  layout=oracle.DENSE, scale=0.09, seqlens=lens, k_scale=0.5,
                                  v_scale=2.0)
    assert np.array_equal(o_h, o_d) and np.array_equal(l_h, l_d)


def test_generator_codes_round_to_nearest():
    # kvgen's e4m3 cast: each code is a nearest e4m3 value of x / scale
    x = np.random.default_rng(3).standard_normal(20000).astype(np.float16)
    s = kvgen.e4m3_scale(x)
    assert s == np.float32(np.abs(x.astype(np.float32)).max() / 448.0)
    c = kvgen.to_e4m3(x, s)
    vals = oracle.widen_e4m3(c)
    grid = np.unique(oracle.widen_e4m3(np.arange(256, dtype=np.uint8)))
    grid = grid[~np.isnan(grid)]
    t = x.astype(np.float32) / s
    nearest = np.abs(t[:, None].astype(np.float64) - grid[None, :]).min(axis=1)
    assert np.all(np.abs(t - vals) <= nearest + 1e-12)
    assert np.abs(vals).max() == 448.0


def test_fp8_hybrid_mixed_head_map_equals_16bit_hybrid():
    # Both branches with e4m3 codes: the 16-bit hybrid (pinned on its own) over
    # the same values, bit for bit.  Slots differ from head indices and every
    # (b, g) buffer has its own length.
    rng = np.random.default_rng(4)
    B, Hq, Hkv, D, P, pcap, bcap = 2, 8, 4, 128, 2, 30, 12
    pk8, pv8 = _random_codes(rng, (B, P, pcap, D)), _random_codes(rng, (B, P, pcap, D))
    bk8, bv8 = _random_codes(rng, (B, Hkv, bcap, D)), _random_codes(rng, (B, Hkv, bcap, D))
    q = rng.standard_normal((B, Hq, D)).astype(np.float16)
    head_map = np.array([-1, 1, -1, 0], np.int32)
    pers_len = np.array([30, 7], np.int32)
    buf_len = np.array([0, 3, 12, 5, 9, 1, 11, 2], np.int32)
    ks, vs = 0.25, 2.0
    w16 = lambda c, s: (oracle.widen_e4m3(c) * s).astype(np.float16)
    o8, l8 = oracle.hybrid_attn(q, pk8, pv8, pers_len, bk8, bv8, buf_len, head_map, scale=0.07,
                                k_scale=ks, v_scale=vs)
    o16, l16 = oracle.hybrid_attn(q, w16(pk8, ks), w16(pv8, vs), pers_len, w16(bk8, ks),
                                  w16(bv8, vs), buf_len, head_map, scale=0.07)
    assert np.array_equal(o8, o16) and np.array_equal(l8, l16)

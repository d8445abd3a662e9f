"""Pins of the fp64 hybrid-attention oracle (CLO page, section 7: the hybrid
kernel reads the persistent cache and the compacted cache buffer in place).

For KV head g the oracle reads persistent slot head_map[g] (rows
0..pers_len[b]-1) when head_map[g] >= 0, else the cache buffer of head g
(rows 0..buf_len[b*Hkv+g]-1).  Every test here drives one of the two branches
with shapes where a wrong index (b and g swapped in buf_len, a slot taken as g,
a base offset without buf_cap or pers_cap) reads a different row set and so a
different result: closed forms through the buffer branch, torch fp64 SDPA
over the rows each head should read, and the pinned dense oracle.
"""
import math

import numpy as np
import pytest
import torch

import oracle

F16 = np.float16
D = 128


def _widen(a):
    return np.asarray(a, np.float16).astype(np.float64)


def _sdpa_fp64(q_heads, k_rows, v_rows, scale):
    """torch fp64 SDPA of G query heads over one KV head's rows.
    q_heads [G, D]; k_rows, v_rows [n, D].  Returns (out [G, D], lse [G])."""
    qt = torch.from_numpy(_widen(q_heads))[:, None, :]
    kt = torch.from_numpy(_widen(k_rows))[None].expand(q_heads.shape[0], -1, -1).contiguous()
    vt = torch.from_numpy(_widen(v_rows))[None].expand(q_heads.shape[0], -1, -1).contiguous()
    o = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, scale=scale)
    s = torch.matmul(qt, kt.transpose(1, 2).contiguous()) * scale
    return o[:, 0, :].numpy(), torch.logsumexp(s[:, 0, :], dim=-1).numpy()


def _inputs(seed, B, Hq, Hkv, P_slots, pers_cap, buf_cap, poison=True):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((B, Hq, D)).astype(F16)
    pk = rng.standard_normal((B, P_slots, pers_cap, D)).astype(F16)
    pv = rng.standard_normal((B, P_slots, pers_cap, D)).astype(F16)
    bk = rng.standard_normal((B, Hkv, buf_cap, D)).astype(F16)
    bv = rng.standard_normal((B, Hkv, buf_cap, D)).astype(F16)
    return rng, q, pk, pv, bk, bv


def _poison_tails(pk, pv, pers_len, bk, bv, buf_len):
    """Rows past each length hold 1000.0: a read past the end shows in the output."""
    B, P_slots = pk.shape[:2]
    Hkv = bk.shape[1]
    for b in range(B):
        pk[b, :, pers_len[b]:] = 1000.0
        pv[b, :, pers_len[b]:] = 1000.0
        for g in range(Hkv):
            n = buf_len[b * Hkv + g]
            bk[b, g, n:] = 1000.0
            bv[b, g, n:] = 1000.0


def _hybrid(q, pk, pv, pers_len, bk, bv, buf_len, head_map, scale):
    return oracle.hybrid_attn(q, pk, pv, np.asarray(pers_len, np.int32), bk, bv,
                              np.asarray(buf_len, np.int32), np.asarray(head_map, np.int32),
                              scale=scale)


def test_buffer_branch_single_key_returns_v():
    # len 1 through the buffer branch: weight 1 exactly, so out = v bit for bit
    # in fp64, and lse = the single score.  Each (b, g) has its own buffer row.
    B, Hq, Hkv, cap = 3, 8, 4, 5
    _, q, pk, pv, bk, bv = _inputs(1, B, Hq, Hkv, 1, 7, cap)
    buf_len = np.ones(B * Hkv, np.int32)
    out, lse = _hybrid(q, pk, pv, [7] * B, bk, bv, buf_len, [-1] * Hkv, 0.25)
    G = Hq // Hkv
    for b in range(B):
        for j in range(Hq):
            g = j // G
            assert np.array_equal(out[b, j], _widen(bv[b, g, 0]))
            s = 0.25 * float(_widen(q[b, j]) @ _widen(bk[b, g, 0]))
            assert abs(lse[b, j] - s) < 1e-12


def test_buffer_branch_identical_keys_give_mean_of_values():
    # Identical keys make every weight 1/n: out = mean of the first n V rows of
    # that (b, g) buffer, lse = s + ln n, with n different for every (b, g).
    B, Hq, Hkv, cap = 2, 6, 3, 40
    rng, q, pk, pv, bk, bv = _inputs(2, B, Hq, Hkv, 1, 9, cap)
    buf_len = rng.permutation(np.arange(5, 5 + 5 * B * Hkv, 5))[:B * Hkv].astype(np.int32)
    assert len(set(buf_len.tolist())) == B * Hkv and buf_len.max() <= cap
    for b in range(B):
        for g in range(Hkv):
            bk[b, g] = bk[b, g, 0]
    _poison_tails(pk, pv, [9] * B, bk, bv, buf_len)
    out, lse = _hybrid(q, pk, pv, [9] * B, bk, bv, buf_len, [-1] * Hkv, 0.3)
    G = Hq // Hkv
    for b in range(B):
        for j in range(Hq):
            g = j // G
            n = int(buf_len[b * Hkv + g])
            np.testing.assert_allclose(out[b, j], _widen(bv[b, g, :n]).mean(axis=0),
                                       rtol=0, atol=1e-14)
            s = 0.3 * float(_widen(q[b, j]) @ _widen(bk[b, g, 0]))
            assert abs(lse[b, j] - (s + math.log(n))) < 1e-12


def test_all_buffer_heads_equal_dense_over_each_buffer():
    # Every head on the buffer, buf_len distinct for every (b, g) and spanning
    # 0 and buf_cap; tails poisoned.  Each (b, g) must equal the pinned DENSE
    # oracle over exactly that buffer's first buf_len rows, bit for bit.
    B, Hq, Hkv, cap = 3, 8, 4, 23
    rng, q, pk, pv, bk, bv = _inputs(3, B, Hq, Hkv, 1, 11, cap)
    lens = np.concatenate([[0, cap], rng.choice(np.arange(1, cap), B * Hkv - 2, replace=False)])
    buf_len = rng.permutation(lens).astype(np.int32)
    assert len(set(buf_len.tolist())) == B * Hkv
    _poison_tails(pk, pv, [11] * B, bk, bv, buf_len)
    scale = 1.0 / math.sqrt(D)
    out, lse = _hybrid(q, pk, pv, [11] * B, bk, bv, buf_len, [-1] * Hkv, scale)
    G = Hq // Hkv
    for b in range(B):
        for g in range(Hkv):
            n = int(buf_len[b * Hkv + g])
            k1 = bk[b, g][None, :, None, :]
            v1 = bv[b, g][None, :, None, :]
            qs = q[b, g * G:(g + 1) * G][None]
            o_d, l_d = oracle.decode_attn(qs, k1, v1, num_kv_heads=1, layout=oracle.DENSE,
                                          scale=scale, seqlens=np.array([n], np.int32))
            assert np.array_equal(out[b, g * G:(g + 1) * G], o_d[0]), (b, g, n)
            assert np.array_equal(lse[b, g * G:(g + 1) * G], l_d[0]), (b, g, n)
            if n == 0:
                assert np.all(o_d[0] == 0.0) and np.all(np.isneginf(l_d[0]))
    assert np.all(np.isfinite(out))  # no poisoned row was read


def test_full_buffer_in_token_order_equals_dense_over_all_rows():
    # A buffer that holds all S rows in order (the selection keeps every token)
    # gives DENSE attention over the full cache.
    B, Hq, Hkv, S = 2, 8, 2, 50
    rng = np.random.default_rng(4)
    q = rng.standard_normal((B, Hq, D)).astype(F16)
    kf = rng.standard_normal((B, S, Hkv, D)).astype(F16)
    vf = rng.standard_normal((B, S, Hkv, D)).astype(F16)
    bk = np.ascontiguousarray(kf.transpose(0, 2, 1, 3))
    bv = np.ascontiguousarray(vf.transpose(0, 2, 1, 3))
    pk = np.zeros((B, 1, 1, D), F16)
    out, lse = _hybrid(q, pk, pk, [0] * B, bk, bv, np.full(B * Hkv, S), [-1] * Hkv, 0.1)
    o_d, l_d = oracle.decode_attn(q, kf, vf, num_kv_heads=Hkv, layout=oracle.DENSE, scale=0.1)
    assert np.array_equal(out, o_d) and np.array_equal(lse, l_d)


def test_mixed_head_map_against_sdpa_per_head():
    # head_map mixes both branches, and the persistent slots are not the head
    # index: head 0 -> slot 1, head 2 -> slot 0, heads 1 and 3 -> their buffers.
    # pers_len differs per sequence and buf_len per (b, g).  Each head is
    # checked against torch fp64 SDPA over the rows it must read.
    B, Hq, Hkv, P_slots, pcap, bcap = 3, 12, 4, 2, 31, 17
    rng, q, pk, pv, bk, bv = _inputs(5, B, Hq, Hkv, P_slots, pcap, bcap)
    head_map = np.array([1, -1, 0, -1], np.int32)
    pers_len = np.array([31, 4, 19], np.int32)
    buf_len = rng.permutation(np.arange(2, 2 + B * Hkv)).astype(np.int32)
    _poison_tails(pk, pv, pers_len, bk, bv, buf_len)
    scale = 0.125
    out, lse = _hybrid(q, pk, pv, pers_len, bk, bv, buf_len, head_map, scale)
    G = Hq // Hkv
    for b in range(B):
        for g in range(Hkv):
            if head_map[g] >= 0:
                n = int(pers_len[b])
                kr, vr = pk[b, head_map[g], :n], pv[b, head_map[g], :n]
            else:
                n = int(buf_len[b * Hkv + g])
                kr, vr = bk[b, g, :n], bv[b, g, :n]
            ref_o, ref_l = _sdpa_fp64(q[b, g * G:(g + 1) * G], kr, vr, scale)
            np.testing.assert_allclose(out[b, g * G:(g + 1) * G], ref_o, rtol=1e-11, atol=1e-13)
            np.testing.assert_allclose(lse[b, g * G:(g + 1) * G], ref_l, rtol=1e-12, atol=1e-12)


def test_all_persistent_equals_dense():
    # Every head persistent with slot = head: DENSE over the slot arrays.
    B, Hq, Hkv, S = 2, 8, 4, 33
    rng = np.random.default_rng(6)
    q = rng.standard_normal((B, Hq, D)).astype(F16)
    pk = rng.standard_normal((B, Hkv, S, D)).astype(F16)
    pv = rng.standard_normal((B, Hkv, S, D)).astype(F16)
    lens = np.array([33, 20], np.int32)
    bk = np.zeros((B, Hkv, 1, D), F16)
    out, lse = _hybrid(q, pk, pv, lens, bk, bk, np.zeros(B * Hkv), np.arange(Hkv), 0.2)
    kd = np.ascontiguousarray(pk.transpose(0, 2, 1, 3))
    vd = np.ascontiguousarray(pv.transpose(0, 2, 1, 3))
    o_d, l_d = oracle.decode_attn(q, kd, vd, num_kv_heads=Hkv, layout=oracle.DENSE, scale=0.2,
                                  seqlens=lens)
    assert np.array_equal(out, o_d) and np.array_equal(lse, l_d)


@pytest.mark.parametrize("bad", ["slot", "pers_len", "buf_len", "negative"])
def test_out_of_range_metadata_is_rejected(bad):
    B, Hq, Hkv = 1, 4, 2
    _, q, pk, pv, bk, bv = _inputs(7, B, Hq, Hkv, 1, 8, 8)
    head_map, pers_len, buf_len = [0, -1], [8], [0, 8]
    if bad == "slot":
        head_map = [1, -1]          # only one slot exists
    elif bad == "pers_len":
        pers_len = [9]              # above pers_cap
    elif bad == "buf_len":
        buf_len = [0, 9]            # above buf_cap
    else:
        buf_len = [0, -1]
    with pytest.raises(ValueError):
        _hybrid(q, pk, pv, pers_len, bk, bv, buf_len, head_map, 1.0)

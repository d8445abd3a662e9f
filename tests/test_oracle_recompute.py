"""Pins of the fp64 KVPR recompute oracle (KVPR page, section A2) against unit
vectors, zero input, numpy's fp64 matmul and the printed Table 1 sizes."""
import os

import numpy as np
import pytest

import kvgen
import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "kvpr_table1_kv_sizes.txt")


def _bf16(a):
    return kvgen.f32_to_bf16_bits(np.asarray(a, np.float32))


def _f64(bits):
    return kvgen.bf16_bits_to_f32(bits).astype(np.float64)


def test_unit_vector_rows_select_weight_rows_exactly():
    rng = np.random.default_rng(0)
    b, l, h = 2, 5, 64
    x = np.zeros((b, l, h), np.float32)
    idx = rng.integers(0, h, size=(b, l))
    for bi in range(b):
        for t in range(l):
            x[bi, t, idx[bi, t]] = 1.0
    wk = _bf16(rng.standard_normal((h, h)) * 0.02)
    wv = _bf16(rng.standard_normal((h, h)) * 0.02)
    k, v = oracle.kv_recompute(_bf16(x), wk, wv, l=l)
    for bi in range(b):
        for t in range(l):
            assert np.array_equal(k[bi * l + t], _f64(wk[idx[bi, t]]))
            assert np.array_equal(v[bi * l + t], _f64(wv[idx[bi, t]]))


def test_zero_input_gives_zero():
    rng = np.random.default_rng(1)
    x = np.zeros((1, 4, 32), np.uint16)
    w = _bf16(rng.standard_normal((32, 32)))
    k, v = oracle.kv_recompute(x, w, w, l=4)
    assert np.all(k == 0) and np.all(v == 0)


def test_matches_numpy_matmul_and_row_subset():
    d = kvgen.kvpr_layer(seed=2, b=3, h=256, H=2, s=40, l=17)
    k, v = oracle.kv_recompute(d["x"], d["w_k"], d["w_v"], l=d["l"])
    X = _f64(d["x"]).reshape(-1, d["h"])
    np.testing.assert_allclose(k, X @ _f64(d["w_k"]), rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(v, X @ _f64(d["w_v"]), rtol=1e-12, atol=1e-13)
    rows = np.array([0, 16, 17, 50], np.int32)
    ks, vs = oracle.kv_recompute(d["x"], d["w_k"], d["w_v"], l=d["l"], rows=rows)
    assert np.array_equal(ks, k[rows]) and np.array_equal(vs, v[rows])


def test_split_point_uses_only_first_l_rows():
    # x has s rows per batch but only rows [0, l) enter the recompute
    rng = np.random.default_rng(3)
    b, s, l, h = 2, 9, 4, 32
    x = _bf16(rng.standard_normal((b, s, h)))
    w = _bf16(rng.standard_normal((h, h)))
    k, _ = oracle.kv_recompute(x, w, w, l=l)
    ref = _f64(x)[:, :l].reshape(-1, h) @ _f64(w)
    np.testing.assert_allclose(k, ref, rtol=1e-12, atol=1e-12)


def test_kvpr_table1_kv_sizes():
    for model, hdim, mib in (line.split() for line in open(GOLDEN) if not line.startswith("#")):
        _, m_kv, _ = oracle.kvpr_cost(32, 0, 1024, int(hdim), 2)
        assert m_kv == int(mib) * 2 ** 20, model


def test_kvpr_cost_closed_forms():
    m_x, m_kv, n = oracle.kvpr_cost(32, 256, 1024, 5120, 2)
    assert m_x == 32 * 256 * 5120 * 2
    assert m_kv == 2 * 32 * (1024 - 256) * 5120 * 2
    assert n == 4 * 32 * 256 * 5120 ** 2  # = 2 (b l) h (2 h): two h x h products


def test_kvpr_time_is_the_section_a2_formula_at_its_ends():
    """At l = 0 nothing is recomputed: t = M_KV(0) / v_com, the whole cache over
    PCIe.  At l = s' nothing but X crosses: t = M_X(s') / v_com + N(s') / v_gpu."""
    b, s, h, p, vc, vg = 32, 1024, 5120, 2, 50e9, 1e15
    assert oracle.kvpr_time(b, 0, s, h, p, vc, vg) == 2 * b * s * h * p / vc
    assert np.isclose(oracle.kvpr_time(b, s, s, h, p, vc, vg),
                      b * s * h * p / vc + 4 * b * s * h * h / vg, rtol=1e-15)


@pytest.mark.parametrize("vc,vg", [(50e9, 1e15), (25e9, 3e14), (1e12, 1e14), (8e9, 2.5e15)])
def test_kvpr_best_split_at_the_crossing(vc, vg):
    """t(l) = a l + max(c l, d (s' - l)) with a = d / 2: it falls while the
    transfer of the rows left dominates and rises after, so the scan's l must
    be one of the two integers around l_c = d s' / (c + d) (clamped)."""
    b, s, h, p = 32, 1024, 5120, 2
    c = 4 * b * h * h / vg
    d = 2 * b * h * p / vc
    lc = d * s / (c + d)
    for l_max in (s, 300, 0):
        l, t = oracle.kvpr_best_split(b, s, l_max, h, p, vc, vg)
        cands = sorted({min(max(int(np.floor(lc)), 0), l_max), min(max(int(np.ceil(lc)), 0), l_max)})
        best = min(cands, key=lambda x: (oracle.kvpr_time(b, x, s, h, p, vc, vg), x))
        assert l == best, (l, cands)
        assert t == oracle.kvpr_time(b, l, s, h, p, vc, vg)


def test_kvpr_best_split_limits():
    """Free compute recomputes every row it may; free transfer recomputes none."""
    b, s, h, p = 4, 500, 1024, 2
    assert oracle.kvpr_best_split(b, s, s, h, p, 1e9, 1e30)[0] == s
    assert oracle.kvpr_best_split(b, s, 123, h, p, 1e9, 1e30)[0] == 123
    assert oracle.kvpr_best_split(b, s, s, h, p, 1e30, 1e9)[0] == 0

"""Pins of the fp64 KVPR recompute oracle (KVPR page, section A2) against unit
vectors, zero input, numpy's fp64 matmul and the printed Table 1 sizes."""
import os

import numpy as np

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

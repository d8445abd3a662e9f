"""Pins of the fp64 head-wise cache oracle (CLO page, Eqs. 7-10 and the
lookup/update rule of sections 2-3) against printed values, identities,
a library cosine and brute force."""
import math
import os

import numpy as np
import pytest
from scipy.spatial.distance import cosine as scipy_cosine_distance

import kvgen
import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "clo_threshold_boundary.txt")


def _rows(path):
    with open(path) as f:
        return [line.split() for line in f if line.strip() and not line.startswith("#")]


def test_threshold_boundary_values_printed_on_page():
    for s, eta, n, tau in _rows(GOLDEN):
        got = oracle.thresholds([float(s)], float(eta), float(n))[0]
        assert abs(got - float(tau)) < 1e-15, (s, got, tau)


def test_threshold_identity_and_monotonicity():
    # lambda theta* + (1 - lambda) pi = pi - lambda (pi - arccos eta), and
    # pi - arccos(eta) = arccos(-eta), so tau = -cos(s^n arccos(-eta)).
    s = np.linspace(0, 1, 1001)
    for eta in (0.8, 0.5, 0.0, -0.3):
        for n in (1.0, 3.0, 5.0):
            tau = oracle.thresholds(s, eta, n)
            alt = -np.cos(s ** n * np.arccos(-eta))
            np.testing.assert_allclose(tau, alt, rtol=0, atol=1e-14)
            assert np.all(np.diff(tau) >= -1e-15)
            assert tau[0] == -1.0 and abs(tau[-1] - eta) < 1e-15


def test_threshold_special_cases():
    s = np.random.default_rng(0).uniform(0, 1, 50)
    np.testing.assert_allclose(oracle.thresholds(s, -1.0, 3.0), -1.0, atol=1e-15)
    big = oracle.thresholds(np.minimum(s, 0.9), 0.8, 400.0)
    np.testing.assert_allclose(big, -1.0, atol=1e-12)


def _lookup(q, lab, w, tau, Hkv):
    return oracle.headcache_lookup(q, lab, w, tau, num_kv_heads=Hkv)


def test_cosines_match_scipy():
    d = kvgen.clo_queries(seed=1, model="qwen2.5-14b", B=3)
    tau = np.full(d["Hkv"], -1.0, np.float32)
    r = _lookup(d["q"], d["labels"], d["weights"], tau, d["Hkv"])
    for b in range(d["B"]):
        for j in range(d["Hq"]):
            ref = 1.0 - scipy_cosine_distance(d["q"][b, j].astype(np.float64),
                                              d["labels"][b, j].astype(np.float64))
            assert abs(r["cos"][b, j] - ref) < 1e-14


def test_equal_cosines_aggregate_to_that_cosine():
    # Eq. 10 rule 2 (CLO page, section 4, check 3): all cosines equal -> a = c.
    rng = np.random.default_rng(2)
    B, Hq, Hkv, D = 2, 8, 2, 128
    qrow = rng.standard_normal(D).astype(np.float16)
    lrow = rng.standard_normal(D).astype(np.float16)
    q = np.broadcast_to(qrow, (B, Hq, D)).copy()
    lab = np.broadcast_to(lrow, (B, Hq, D)).copy()
    w = rng.uniform(0.01, 1, Hq).astype(np.float32)
    r = _lookup(q, lab, w, np.zeros(Hkv, np.float32), Hkv)
    c = r["cos"][0, 0]
    assert np.all(r["cos"] == c)
    np.testing.assert_allclose(r["agg"], c, rtol=0, atol=1e-15)


def test_one_hot_weight_selects_single_head():
    d = kvgen.clo_queries(seed=3, B=2)
    G = d["Hq"] // d["Hkv"]
    w = np.zeros(d["Hq"], np.float32)
    w[2::G] = 1.0  # third head of every group
    r = _lookup(d["q"], d["labels"], w, np.zeros(d["Hkv"], np.float32), d["Hkv"])
    np.testing.assert_allclose(r["agg"], r["cos"][:, 2::G], rtol=0, atol=1e-15)


def test_query_equal_label_hits_and_opposite_misses():
    rng = np.random.default_rng(4)
    B, Hq, Hkv, D = 2, 8, 4, 128
    lab = rng.standard_normal((B, Hq, D)).astype(np.float16)
    w = rng.uniform(0.1, 1, Hq).astype(np.float32)
    tau = np.full(Hkv, 0.8, np.float32)
    r = _lookup(lab.copy(), lab, w, tau, Hkv)
    assert np.all(r["hit"] == 1) and r["miss_count"] == 0
    np.testing.assert_allclose(r["cos"], 1.0, atol=1e-15)
    assert np.array_equal(r["labels"], lab.view(np.uint16))
    neg = -lab
    r2 = _lookup(neg, lab, w, np.full(Hkv, -0.999, np.float32), Hkv)
    assert np.all(r2["hit"] == 0)
    np.testing.assert_allclose(r2["cos"], -1.0, atol=1e-15)
    assert np.array_equal(r2["labels"], neg.view(np.uint16))  # whole head replaced
    assert list(r2["miss_list"]) == list(range(B * Hkv))


def test_power_of_two_scaling_leaves_decisions_unchanged():
    # Eq. 6 of the CLO page: the cosine does not depend on the norm of q.
    d = kvgen.clo_queries(seed=5, B=4)
    tau = np.linspace(0.6, 0.95, d["Hkv"]).astype(np.float32)
    r1 = _lookup(d["q"], d["labels"], d["weights"], tau, d["Hkv"])
    for e in (1, 4, 8):  # stays in the normal fp16 range, so the scaling is exact
        q2 = (d["q"].astype(np.float64) * 2.0 ** e).astype(np.float16)
        assert np.array_equal(q2.astype(np.float64), d["q"].astype(np.float64) * 2.0 ** e)
        r2 = _lookup(q2, d["labels"], d["weights"], tau, d["Hkv"])
        assert np.array_equal(r1["hit"], r2["hit"])
        assert np.array_equal(r1["cos"], r2["cos"])


def test_second_lookup_with_same_query_hits_everywhere():
    d = kvgen.clo_queries(seed=6, B=4)
    tau = np.full(d["Hkv"], 0.95, np.float32)
    r1 = _lookup(d["q"], d["labels"], d["weights"], tau, d["Hkv"])
    assert r1["miss_count"] > 0
    r2 = _lookup(d["q"], r1["labels"].view(np.float16), d["weights"], tau, d["Hkv"])
    missed = r1["hit"] == 0
    assert np.all(r2["hit"][missed] == 1)
    assert np.all(r2["hit"][~missed] == r1["hit"][~missed])


def test_zero_norm_group_misses():
    d = kvgen.clo_queries(seed=7, B=2)
    lab = d["labels"].copy()
    lab[1, 0] = 0  # empty label in group 0 of batch 1
    r = _lookup(d["q"], lab, d["weights"], np.full(d["Hkv"], -1.0, np.float32), d["Hkv"])
    assert r["hit"][1, 0] == 0 and r["hit"].sum() == d["B"] * d["Hkv"] - 1
    assert list(r["miss_list"]) == [1 * d["Hkv"] + 0]


def test_brute_force_tiny():
    rng = np.random.default_rng(8)
    B, Hq, Hkv, D = 3, 6, 2, 8
    q = rng.standard_normal((B, Hq, D)).astype(np.float16)
    lab = rng.standard_normal((B, Hq, D)).astype(np.float16)
    w = rng.uniform(0, 1, Hq).astype(np.float32)
    tau = np.array([-0.1, 0.2], np.float32)
    r = _lookup(q, lab, w, tau, Hkv)
    G = Hq // Hkv
    new_lab = lab.copy()
    misses = []
    for b in range(B):
        for g in range(Hkv):
            num = den = 0.0
            for jj in range(G):
                j = g * G + jj
                qv = [float(x) for x in q[b, j]]
                lv = [float(x) for x in lab[b, j]]
                c = sum(a * c for a, c in zip(qv, lv)) / (
                    math.sqrt(sum(a * a for a in qv)) * math.sqrt(sum(c * c for c in lv)))
                num += float(w[j]) * c
                den += float(w[j])
            a = num / den
            assert abs(r["agg"][b, g] - a) < 1e-13
            hit = a >= float(tau[g])
            assert r["hit"][b, g] == hit
            if not hit:
                new_lab[b, g * G:(g + 1) * G] = q[b, g * G:(g + 1) * G]
                misses.append(b * Hkv + g)
    assert np.array_equal(r["labels"], new_lab.view(np.uint16))
    assert list(r["miss_list"]) == misses


def test_generated_cosine_band():
    # The query construction targets label/query cosines of about 0.80-0.95.
    d = kvgen.clo_queries(seed=0, B=64)
    r = _lookup(d["q"], d["labels"], d["weights"], np.full(d["Hkv"], -1.0, np.float32),
                d["Hkv"])
    c = r["cos"].ravel()
    # noise scale 2.96 gives 0.9 / sqrt(0.81 + 0.01 * 2.96^2) = 0.95, 6.75 gives 0.80;
    # finite D = 128 spreads each draw by about +-0.02 around that.
    assert 0.77 < np.percentile(c, 5) and np.percentile(c, 95) < 0.955
    assert 0.85 < np.median(c) < 0.91


# ---------------------------------------------------------------------------
# One-layer-ahead approximate query q_approx = x_{l-1} W_Q^l (CLO page,
# section 3, decoding flow, Figure 9), W_Q stored output index first.
# ---------------------------------------------------------------------------

def test_approx_query_basis_rows_pick_weight_columns():
    # x = e_i gives q[n] = W[n][i] exactly; a transposed operand would give W[i][n]
    rng = np.random.default_rng(11)
    h, N = 24, 40
    w = rng.standard_normal((N, h)).astype(np.float16)
    x = np.eye(h, dtype=np.float16)[[0, 5, 23]]
    q = oracle.approx_query(x, w)
    assert np.array_equal(q, w[:, [0, 5, 23]].T.astype(np.float64))


def test_approx_query_brute_force_tiny():
    rng = np.random.default_rng(12)
    B, h, N = 3, 8, 6
    x = rng.integers(-8, 9, (B, h)).astype(np.float16)
    w = rng.integers(-8, 9, (N, h)).astype(np.float16)
    q = oracle.approx_query(x, w)
    for b in range(B):
        for n in range(N):
            acc = 0
            for i in range(h):
                acc += int(x[b, i]) * int(w[n, i])
            assert q[b, n] == acc


def test_approx_query_matches_the_c_recompute_loop():
    # the independently written X . W loop, fed W_Q's transpose (input index first)
    d = kvgen.clo_ahead(seed=13, model="llama3-8b", B=3, h=256, Hq=2, Hkv=1)
    q = oracle.approx_query(d["x_prev"], d["w_q"])
    wt = np.ascontiguousarray(d["w_q"].T)
    k, _ = oracle.kv_recompute(d["x_prev"][:, None, :], wt, wt, l=1, kind=oracle.F16)
    np.testing.assert_allclose(q, k, rtol=0, atol=1e-12)


def test_approx_query_bf16_widening():
    # bf16 bit patterns of small integers multiply exactly
    x = kvgen.f32_to_bf16_bits(np.array([[1, 2, -3, 4, 0, 0, 0, 1]], np.float32))
    w = kvgen.f32_to_bf16_bits(np.array([[1, 1, 1, 1, 1, 1, 1, 1],
                                         [0, 0, 2, 0, 0, 0, 0, 64]], np.float32))
    assert oracle.approx_query(x, w, kind=oracle.BF16).tolist() == [[5.0, 58.0]]


def test_clo_ahead_drift_sets_cosines():
    # x_label = x + s n with x, n independent N(0, I): the cosine of the two
    # projections is close to 1 / sqrt(1 + s^2) (checked on the oracle's fp64
    # projections; spread about 1 / sqrt(h))
    d = kvgen.clo_ahead(seed=14, model="llama3-8b", B=8, h=2048, Hq=8, Hkv=2)
    qa = oracle.approx_query(d["x_prev"], d["w_q"])
    ql = oracle.approx_query(d["x_label"], d["w_q"])
    cos = (qa * ql).sum(1) / np.linalg.norm(qa, axis=1) / np.linalg.norm(ql, axis=1)
    expect = 1.0 / np.sqrt(1.0 + d["drift"].astype(np.float64) ** 2)
    assert np.all(np.abs(cos - expect) < 0.06), (cos, expect)


def _bits(values, kind):
    """16-bit patterns of values exactly representable in fp16 and bf16."""
    v = np.asarray(values, np.float64)
    if kind == oracle.F16:
        out = v.astype(np.float16)
        assert np.array_equal(out.astype(np.float64), v)
        return out.view(np.uint16)
    f = v.astype(np.float32)
    assert np.array_equal(f.astype(np.float64), v)
    u = f.view(np.uint32)
    assert np.all(u & 0xFFFF == 0)
    return (u >> 16).astype(np.uint16)


@pytest.mark.parametrize("kind", [oracle.F16, oracle.BF16])
@pytest.mark.parametrize("case", ["cos_one", "cos_half", "eq10_mix"])
def test_aggregate_equal_to_tau_is_a_hit(kind, case):
    # CLO page, section 2: a head hits when its cosine reaches tau (>=).  The
    # inputs make the fp64 aggregate exactly a float32 value:
    #   cos_one : q = label = 2 e0 -> c = 4 / (2 * 2) = 1
    #   cos_half: q = e0, label = e0 + e1 + e2 + e3 -> c = 1 / (1 * 2) = 1/2
    #   eq10_mix: heads with c = 1/2 and c = 1, weights 1/4 and 3/4 ->
    #             a = (1/8 + 3/4) / 1 = 7/8 (Eq. 10)
    # tau = a must hit, the next float32 above a must miss, the one below hit.
    D = 128
    e = np.eye(D)
    half_q, half_l = e[0], e[0] + e[1] + e[2] + e[3]
    if case == "cos_one":
        qv, lv, w, a = [2 * e[0]], [2 * e[0]], [1.0], 1.0
    elif case == "cos_half":
        qv, lv, w, a = [half_q], [half_l], [0.5], 0.5
    else:
        qv, lv, w, a = [half_q, 2 * e[0]], [half_l, 2 * e[0]], [0.25, 0.75], 0.875
    G = len(qv)
    q = _bits(np.array(qv)[None], kind)
    lab = _bits(np.array(lv)[None], kind)
    w = np.array(w, np.float32)
    a32 = np.float32(a)
    assert float(a32) == a
    for tau, want in ((a32, 1), (np.nextafter(a32, np.float32(2)), 0),
                      (np.nextafter(a32, np.float32(-2)), 1)):
        r = oracle.headcache_lookup(q, lab, w, np.array([tau], np.float32), num_kv_heads=1,
                                    kind=kind)
        assert r["agg"][0, 0] == a
        assert r["hit"][0, 0] == want, (case, float(tau))
        assert r["miss_count"] == 1 - want
        # a miss replaces every label of the group with q; a hit keeps them
        assert np.array_equal(r["labels"], q if want == 0 else lab)
        assert G == r["cos"].shape[1]

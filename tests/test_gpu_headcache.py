"""GPU parity of kvdec_headcache_lookup (fused cosine lookup + label update).

Decisions, labels and the miss list must be bit-exact with the fp64 oracle,
except groups whose oracle aggregate lies within 1e-5 of tau: those are
flagged, and their labels are checked against the GPU's own decision.
Cosines and aggregates (fp32) must be within 1e-5 of the oracle.
"""
import numpy as np
import pytest
import torch

import kvgen
import long_kv_caches_amd as K
import oracle
from gpu_util import bits, dev, say

pytestmark = pytest.mark.gpu
FLAG_BAND = 1e-5


def lookup_on_gpu(q, labels, w, tau, Hkv, bf16=False):
    B, Hq, D = q.shape
    qd, ld = dev(q, bf16), dev(labels, bf16)
    wt = torch.from_numpy(np.asarray(w, np.float32)).cuda()
    tt = torch.from_numpy(np.asarray(tau, np.float32)).cuda()
    hit = torch.full((B * Hkv,), 7, dtype=torch.uint8, device="cuda")
    agg = torch.empty(B * Hkv, dtype=torch.float32, device="cuda")
    cos = torch.empty(B * Hq, dtype=torch.float32, device="cuda")
    ml = torch.full((B * Hkv,), -1, dtype=torch.int32, device="cuda")
    mc = torch.full((1,), -1, dtype=torch.int32, device="cuda")
    K.kvdec_headcache_lookup(qd, ld, wt, tt, hit, agg, cos, ml, mc)
    torch.cuda.synchronize()
    n = int(mc.item())
    return dict(hit=hit.cpu().numpy().reshape(B, Hkv), agg=agg.cpu().numpy().reshape(B, Hkv),
                cos=cos.cpu().numpy().reshape(B, Hq), labels=bits(ld), miss_count=n,
                miss_list=ml.cpu().numpy()[:n])


def compare(q, labels, w, tau, Hkv, what, bf16=False):
    say(f"[lookup] {what}")
    g = lookup_on_gpu(q, labels, w, tau, Hkv, bf16)
    r = oracle.headcache_lookup(q, labels, w, tau, num_kv_heads=Hkv,
                                kind=oracle.BF16 if bf16 else oracle.F16)
    B, Hq, D = q.shape
    G = Hq // Hkv
    flagged = np.abs(r["agg"] - np.asarray(tau, np.float32)[None, :]) < FLAG_BAND
    agree = g["hit"] == r["hit"]
    assert np.all(agree | flagged), f"{(~(agree | flagged)).sum()} unflagged decision mismatches"
    assert np.all(np.isin(g["hit"], [0, 1]))
    np.testing.assert_allclose(g["cos"], r["cos"], rtol=0, atol=1e-5)
    np.testing.assert_allclose(g["agg"], r["agg"], rtol=0, atol=1e-5)
    # labels follow the GPU's decision, bit for bit
    q_bits = np.asarray(q).view(np.uint16)
    exp = np.asarray(labels).view(np.uint16).copy()
    for b in range(B):
        for h in range(Hkv):
            if g["hit"][b, h] == 0:
                exp[b, h * G:(h + 1) * G] = q_bits[b, h * G:(h + 1) * G]
    assert np.array_equal(g["labels"], exp)
    misses = [b * Hkv + h for b in range(B) for h in range(Hkv) if g["hit"][b, h] == 0]
    assert g["miss_count"] == len(misses) and list(g["miss_list"]) == misses
    say(f"  hits {int(g['hit'].sum())}/{B * Hkv}, flagged {int(flagged.sum())}")
    return g, r


def _taus(s, Hkv, eta=0.8, n=3.0):
    sg = kvgen.group_importance(s, Hkv).astype(np.float32)
    return K.kvdec_headcache_thresholds(sg, eta, n).numpy()


@pytest.mark.parametrize("model", ["llama3-8b", "qwen2.5-14b"])
def test_clo_config(model):
    d = kvgen.clo_queries(seed=0, model=model, B=4)
    compare(d["q"], d["labels"], d["weights"], _taus(d["s"], d["Hkv"]), d["Hkv"], model)


def test_strict_thresholds_mixed_decisions():
    # every importance 1 -> tau = eta = 0.8, cosines spread over [0.7, 0.95]
    d = kvgen.clo_queries(seed=1, model="llama3-8b", B=64)
    tau = _taus(np.ones(d["Hq"]), d["Hkv"])
    assert np.allclose(tau, 0.8, atol=1e-7)
    g, r = compare(d["q"], d["labels"], d["weights"], tau, d["Hkv"], "tau=0.8, B=64")
    assert 0 < g["hit"].sum() < g["hit"].size


def test_near_ties_are_flagged_not_failed():
    d = kvgen.clo_queries(seed=2, model="qwen2.5-14b", B=32)
    r = oracle.headcache_lookup(d["q"], d["labels"], d["weights"], np.zeros(8, np.float32),
                                num_kv_heads=8)
    # thresholds placed exactly at (fp32 of) some aggregates
    tau = r["agg"][0].astype(np.float32)
    compare(d["q"], d["labels"], d["weights"], tau, 8, "near ties")


def test_many_groups_multi_block_path():
    d = kvgen.clo_queries(seed=3, model="llama3-8b", B=4096)
    tau = np.linspace(0.75, 0.95, 8).astype(np.float32)
    compare(d["q"], d["labels"], d["weights"], tau, 8, "B=4096 (multi-workgroup + compaction)")


def test_second_call_hits_everything_it_replaced():
    d = kvgen.clo_queries(seed=4, model="llama3-8b", B=16)
    tau = np.full(8, 0.9, np.float32)
    g1 = lookup_on_gpu(d["q"], d["labels"], d["weights"], tau, 8)
    assert g1["miss_count"] > 0
    g2 = lookup_on_gpu(d["q"], g1["labels"].view(np.float16), d["weights"], tau, 8)
    assert np.all(g2["hit"][g1["hit"] == 0] == 1)


def test_zero_norm_label_misses_and_scale_invariance():
    d = kvgen.clo_queries(seed=5, model="llama3-8b", B=8)
    lab = d["labels"].copy()
    lab[3, 4:8] = 0
    tau = np.full(8, -1.0, np.float32)
    g, _ = compare(d["q"], lab, d["weights"], tau, 8, "zero-norm label")
    assert g["hit"][3, 1] == 0 and g["hit"].sum() == 8 * 8 - 1
    tau = np.linspace(0.7, 0.95, 8).astype(np.float32)
    g1 = lookup_on_gpu(d["q"], d["labels"], d["weights"], tau, 8)
    q2 = (d["q"].astype(np.float64) * 16).astype(np.float16)
    g2 = lookup_on_gpu(q2, d["labels"], d["weights"], tau, 8)
    assert np.array_equal(g1["hit"], g2["hit"]) and np.array_equal(g1["cos"], g2["cos"])


def test_bf16_inputs():
    d = kvgen.clo_queries(seed=6, model="qwen2.5-14b", B=8)
    from gpu_util import to_bf16_bits
    compare(to_bf16_bits(d["q"]), to_bf16_bits(d["labels"]), d["weights"],
            np.linspace(0.7, 0.95, 8).astype(np.float32), 8, "bf16", bf16=True)


# ---------------------------------------------------------------------------
# kvdec_headcache_lookup_ahead: q_approx = x_prev . W_Q^T, then the lookup on it.
#
# The kernel sums in fp32 and rounds once; the oracle sums in fp64 and the test
# rounds that once to the same 16-bit type.  The two q_approx differ only where
# the exact value sits within the fp32 sum's error of a rounding midpoint, and
# then by one unit in the last place plus at most that error.  A cosine
# moves by at most |dq| / |q| when its query moves by dq (the gradient of
# q.l / (|q| |l|) in q has norm sin(angle) / |q|), so per query head the
# cosine tolerance is 1e-5 (the fp32 lookup's) plus |q_gpu - q_ref| / (0.99 |q_ref|),
# and a group's aggregate (a weighted mean) gets the largest of its heads'.
# Decisions are compared outside that band, as in the lookup tests.
# ---------------------------------------------------------------------------

def ahead_on_gpu(d, labels, tau, bf16=False):
    B, Hq, Hkv, D = d["B"], d["Hq"], d["Hkv"], d["D"]
    x, w = dev(d["x_prev"], bf16), dev(d["w_q"], bf16)
    qa = torch.full((B, Hq, D), 7.0, dtype=x.dtype, device="cuda")
    ld = dev(labels, bf16)
    wt = torch.from_numpy(np.asarray(d["weights"], np.float32)).cuda()
    tt = torch.from_numpy(np.asarray(tau, np.float32)).cuda()
    hit = torch.full((B * Hkv,), 7, dtype=torch.uint8, device="cuda")
    agg = torch.empty(B * Hkv, dtype=torch.float32, device="cuda")
    cos = torch.empty(B * Hq, dtype=torch.float32, device="cuda")
    ml = torch.full((B * Hkv,), -1, dtype=torch.int32, device="cuda")
    mc = torch.full((1,), -1, dtype=torch.int32, device="cuda")
    K.kvdec_headcache_lookup_ahead(x, w, qa, ld, wt, tt, hit, agg, cos, ml, mc)
    torch.cuda.synchronize()
    n = int(mc.item())
    return dict(q=bits(qa), hit=hit.cpu().numpy().reshape(B, Hkv),
                agg=agg.cpu().numpy().reshape(B, Hkv), cos=cos.cpu().numpy().reshape(B, Hq),
                labels=bits(ld), miss_count=n, miss_list=ml.cpu().numpy()[:n])


def _round16(a, bf16):
    return kvgen.f32_to_bf16_bits(a.astype(np.float32)) if bf16 else a.astype(np.float16).view(np.uint16)


def compare_ahead(d, labels, tau, what, bf16=False):
    from gpu_util import check_close
    say(f"[lookup-ahead] {what}")
    kind = oracle.BF16 if bf16 else oracle.F16
    B, Hq, Hkv, D = d["B"], d["Hq"], d["Hkv"], d["D"]
    G = Hq // Hkv
    g = ahead_on_gpu(d, labels, tau, bf16)
    q_exact = oracle.approx_query(d["x_prev"], d["w_q"], kind=kind)        # [B, Hq*D] fp64
    check_close(oracle.widen(g["q"], kind).reshape(B, -1), q_exact, "q_approx", bf16_out=bf16)
    q_ref = _round16(q_exact, bf16).reshape(B, Hq, D)
    qg = oracle.widen(g["q"], kind)
    qr = oracle.widen(q_ref, kind)
    # the kernel's fp32 sum is within h * 2^-24 * sum_i |x_i w_ni| of the exact
    # one (any summation order), so its 16-bit rounding is within that plus
    # one unit in the last place of the oracle's rounding
    sabs = (np.abs(oracle.widen(d["x_prev"], kind)) @ np.abs(oracle.widen(d["w_q"], kind)).T).reshape(qr.shape)
    allowed = _ulp16(np.maximum(np.abs(qr), np.abs(qg)), bf16) + d["h"] * 2.0 ** -24 * sabs
    assert np.all(np.abs(qg - qr) <= allowed), "q_approx beyond the fp32-sum bound plus one unit"
    say(f"  q_approx elements that differ from the oracle's rounding: {int((g['q'] != q_ref).sum())} "
        f"of {q_ref.size}")
    r = oracle.headcache_lookup(q_ref, labels, d["weights"], tau, num_kv_heads=Hkv, kind=kind)
    nq = np.linalg.norm(qr, axis=-1)
    dq = np.linalg.norm(qg - qr, axis=-1)
    tol_cos = 1e-5 + np.where(nq > 0, dq / (0.99 * np.where(nq > 0, nq, 1.0)), 0.0)
    tol_agg = 1e-5 + (tol_cos - 1e-5).reshape(B, Hkv, G).max(axis=2)
    assert np.all(np.abs(g["cos"] - r["cos"]) <= tol_cos)
    assert np.all(np.abs(g["agg"] - r["agg"]) <= tol_agg)
    flagged = np.abs(r["agg"] - np.asarray(tau, np.float32)[None, :]) < tol_agg
    agree = g["hit"] == r["hit"]
    assert np.all(agree | flagged), f"{(~(agree | flagged)).sum()} unflagged decision mismatches"
    # missed groups take the kernel's own q_approx as their labels, bit for bit
    exp = _u16(labels).copy()
    for b in range(B):
        for h in range(Hkv):
            if g["hit"][b, h] == 0:
                exp[b, h * G:(h + 1) * G] = g["q"][b, h * G:(h + 1) * G]
    assert np.array_equal(g["labels"], exp)
    misses = [b * Hkv + h for b in range(B) for h in range(Hkv) if g["hit"][b, h] == 0]
    assert g["miss_count"] == len(misses) and list(g["miss_list"]) == misses
    say(f"  hits {int(g['hit'].sum())}/{B * Hkv}, flagged {int(flagged.sum())}")
    return g, r


def _ulp16(v, bf16):
    """Spacing of the 16-bit grid at each (representable) value of v."""
    if not bf16:
        return np.spacing(np.abs(v).astype(np.float16)).astype(np.float64)
    a = np.abs(v)
    e = np.floor(np.log2(np.where(a > 0, a, 1.0)))
    return np.where(a >= 2.0 ** -126, 2.0 ** (e - 7), 2.0 ** -133)


def _u16(a):
    a = np.ascontiguousarray(a)
    return a.view(np.uint16) if a.dtype == np.float16 else a


def _ahead_labels(d, bf16=False):
    kind = oracle.BF16 if bf16 else oracle.F16
    ql = oracle.approx_query(d["x_label"], d["w_q"], kind=kind)
    lab = _round16(ql, bf16).reshape(d["B"], d["Hq"], d["D"])
    return lab if bf16 else lab.view(np.float16)


@pytest.mark.parametrize("model", ["llama3-8b", "qwen2.5-14b"])
@pytest.mark.parametrize("B", [1, 4, 7])
def test_lookup_ahead_clo_config(model, B):
    # B = 7: one full group of four batch rows and a ragged group of three
    d = kvgen.clo_ahead(seed=20 + B, model=model, B=B)
    tau = np.full(d["Hkv"], 0.85, np.float32)
    compare_ahead(d, _ahead_labels(d), tau, f"{model} B={B} h={d['h']}")


@pytest.mark.parametrize("h,Hq,Hkv", [(8, 12, 4), (1000, 12, 4), (8192, 12, 4), (64, 160, 16),
                                       (256, 1, 1), (128, 32, 2)])
def test_lookup_ahead_shapes(h, Hq, Hkv):
    # h = 8: one 16-byte piece per row, most waves' slices empty; 1000: slices
    # of unequal piece counts; 8192: the largest h, two pieces per lane;
    # Hq = 160: N = 20480 rows, more than 64 per CU (the per-workgroup cap);
    # Hq = 1: N = 128, one row per workgroup; Hq = 32 on 2 KV heads: G = 16,
    # the largest group
    d = kvgen.clo_ahead(seed=30, model="llama3-8b", B=5, h=h, Hq=Hq, Hkv=Hkv)
    compare_ahead(d, _ahead_labels(d), np.linspace(0.7, 0.95, Hkv).astype(np.float32),
                  f"h={h} Hq={Hq} Hkv={Hkv}")


def test_lookup_ahead_many_groups_and_importance_thresholds():
    # importances near 1 with n = 1 put the Eq. 7-9 thresholds in [0.5, 0.8],
    # where the drifted labels' cosines fall, so decisions are mixed
    d = kvgen.clo_ahead(seed=31, model="llama3-8b", B=160, h=1024)
    sg = np.linspace(0.85, 1.0, d["Hkv"]).astype(np.float32)
    tau = K.kvdec_headcache_thresholds(sg, d["eta"], 1.0).numpy()
    g, _ = compare_ahead(d, _ahead_labels(d), tau, "B=160, Eqs. 7-9 thresholds")
    assert 0 < g["hit"].sum() < g["hit"].size


def test_lookup_ahead_bf16():
    d = kvgen.clo_ahead(seed=32, model="qwen2.5-14b", B=6, out_dtype=np.uint16)
    compare_ahead(d, _ahead_labels(d, bf16=True), np.full(8, 0.85, np.float32), "bf16", bf16=True)


def test_lookup_ahead_replaced_labels_hit_next_time():
    d = kvgen.clo_ahead(seed=33, model="llama3-8b", B=4)
    tau = np.full(8, 0.95, np.float32)
    g1 = ahead_on_gpu(d, _ahead_labels(d), tau)
    assert g1["miss_count"] > 0
    g2 = ahead_on_gpu(d, g1["labels"].view(np.float16), tau)
    assert np.all(g2["hit"][g1["hit"] == 0] == 1)
    assert np.array_equal(g1["q"], g2["q"])

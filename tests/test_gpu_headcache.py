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

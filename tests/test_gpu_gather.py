"""GPU parity of index-gather sparse attention (kvdec_gather_attn) and the
exact top-k selection (kvdec_topk_select) against the fp64 oracle.

Gather attention takes its indices from the test (seeded random selections,
or the oracle's own top-k), so both sides attend to the same rows; the
tolerances are those of the other attention paths.

The selection decides a set from fp32 scores.  The GPU's score of token t
is (sum_j q_j) . K_t in fp32; any fp32 evaluation of this sum of G * 128 exact
products differs from the exact value by at most (G * 128 + G) * 2^-24 *
sum |q_jd K_td| (the oracle returns that sum of magnitudes), so a token may
trade places with another only if their exact scores lie within the sum of
their two bands.  The count, the order (ascending) and everything outside
such trades must match the oracle exactly.
"""
import numpy as np
import pytest
import torch

import kvgen
import long_kv_caches_amd as K
import oracle
from gpu_util import check_close, check_lse, dev, host_f64, say, to_bf16_bits

pytestmark = pytest.mark.gpu


def gather_on_gpu(d, idx, n, split=0, fp8=False, bf16=False):
    B, Hq, Hkv, S = d["B"], d["Hq"], d["Hkv"], d["S"]
    fmt = dict(kv_format=K.KVDEC_KV_E4M3, k_scale=d["k_scale"], v_scale=d["v_scale"]) if fp8 else {}
    dt = torch.bfloat16 if bf16 else torch.float16
    c = (lambda x: dev(to_bf16_bits(x), True)) if bf16 else dev
    desc = K.gather_desc(batch=B, num_q_heads=Hq, num_kv_heads=Hkv, dtype=dt, max_seqlen=S,
                         softmax_scale=d["scale"], split_tokens=split, max_k=idx.shape[2], **fmt)
    ws = K.alloc_workspace(K.kvdec_gather_attn_workspace(desc))
    out = torch.empty((B, Hq, 128), dtype=dt, device="cuda")
    lse = torch.empty((B, Hq), dtype=torch.float32, device="cuda")
    i32 = lambda a: torch.from_numpy(np.ascontiguousarray(a, np.int32)).cuda()
    K.kvdec_gather_attn(desc, c(d["q"]), c(d["k"]), c(d["v"]), i32(idx), i32(n), out, lse, ws)
    torch.cuda.synchronize()
    return host_f64(out), lse.cpu().numpy()


def _model_small(model, seed, S=3000, lens=(3000, 1234, 0, 17)):
    return kvgen.clo_gather(seed=seed, model=model, B=len(lens), S=S, lens=lens)


@pytest.mark.parametrize("model", ["llama3-8b", "qwen2.5-14b"])
@pytest.mark.parametrize("split", [0, 128])
def test_gather_random_indices(model, split):
    d = _model_small(model, 60)
    idx, n = kvgen.random_indices(61, d["B"], d["Hkv"], d["seqlens"], 300)
    say(f"[gather] {model} random indices split={split}")
    go, gl = gather_on_gpu(d, idx, n, split)
    ro, rl = oracle.gather_attn(d["q"], d["k"], d["v"], idx, n, num_kv_heads=d["Hkv"], scale=d["scale"])
    check_close(go, ro, "gather")
    check_lse(gl, rl, "gather lse")


def test_gather_bf16():
    d = _model_small("llama3-8b", 75)
    idx, n = kvgen.random_indices(76, d["B"], d["Hkv"], d["seqlens"], 300)
    c = to_bf16_bits
    ro, rl = oracle.gather_attn(c(d["q"]), c(d["k"]), c(d["v"]), idx, n, num_kv_heads=8, scale=d["scale"],
                                kind=oracle.BF16)
    for split in (0, 128):
        say(f"[gather] bf16 split={split}")
        go, gl = gather_on_gpu(d, idx, n, split=split, bf16=True)
        check_close(go, ro, f"gather bf16 split={split}", bf16_out=True)
        check_lse(gl, rl, "gather bf16 lse")


def test_gather_unsorted_and_repeated_indices():
    d = _model_small("llama3-8b", 62, lens=(3000, 500))
    idx, n = kvgen.random_indices(63, d["B"], d["Hkv"], d["seqlens"], 200)
    rng = np.random.default_rng(64)
    for b in range(d["B"]):
        for g in range(d["Hkv"]):
            m = n[b * d["Hkv"] + g]
            idx[b, g, :m] = rng.permutation(idx[b, g, :m])
            idx[b, g, 5] = idx[b, g, 3]  # a row listed twice counts twice
    say("[gather] unsorted, repeated")
    go, gl = gather_on_gpu(d, idx, n)
    ro, rl = oracle.gather_attn(d["q"], d["k"], d["v"], idx, n, num_kv_heads=d["Hkv"], scale=d["scale"])
    check_close(go, ro, "gather unsorted")
    check_lse(gl, rl, "gather unsorted lse")


@pytest.mark.parametrize("split", [0, 128])
def test_gather_e4m3(split):
    d = kvgen.fp8_kv(_model_small("llama3-8b", 65))
    idx, n = kvgen.random_indices(66, d["B"], d["Hkv"], d["seqlens"], 300)
    say(f"[gather] e4m3 split={split}")
    go, gl = gather_on_gpu(d, idx, n, split, fp8=True)
    # the same rows compacted per (sequence, KV head): the hybrid oracle's cache buffer
    B, Hkv, kk = d["B"], d["Hkv"], idx.shape[2]
    bk = np.zeros((B, Hkv, kk, 128), np.uint8)
    bv = np.zeros_like(bk)
    for b in range(B):
        for g in range(Hkv):
            m = n[b * Hkv + g]
            bk[b, g, :m] = d["k"][b, idx[b, g, :m], g]
            bv[b, g, :m] = d["v"][b, idx[b, g, :m], g]
    ro, rl = oracle.hybrid_attn(d["q"], bk[:, :1], bv[:, :1], np.zeros(B, np.int32), bk, bv, n,
                                np.full(Hkv, -1, np.int32), scale=d["scale"], k_scale=d["k_scale"],
                                v_scale=d["v_scale"])
    check_close(go, ro, "gather e4m3")
    check_lse(gl, rl, "gather e4m3 lse")


def topk_on_gpu(d, top_k, null_seqlens=False, dirty_workspace=False, bf16=False):
    B, Hq, Hkv, S = d["B"], d["Hq"], d["Hkv"], d["S"]
    desc = K.topk_desc(batch=B, num_q_heads=Hq, num_kv_heads=Hkv,
                       dtype=torch.bfloat16 if bf16 else torch.float16, max_seqlen=S, top_k=top_k)
    conv = to_bf16_bits if bf16 else (lambda x: x)
    ws = K.alloc_workspace(K.kvdec_topk_select_workspace(desc))
    if dirty_workspace:
        ws.fill_(255)  # the selection must not depend on what the workspace held
    idx = torch.full((B, Hkv, max(top_k, 1)), -7, dtype=torch.int32, device="cuda")
    n = torch.full((B * Hkv,), -7, dtype=torch.int32, device="cuda")
    sl = None if null_seqlens else torch.from_numpy(np.asarray(d["seqlens"], np.int32)).cuda()
    K.kvdec_topk_select(desc, dev(conv(d["q"]), bf16), dev(conv(d["k"]), bf16), sl, idx, n, ws)
    torch.cuda.synchronize()
    return idx.cpu().numpy(), n.cpu().numpy()


def check_topk(d, top_k, what, pairs=None, bf16=False, **gpu_kw):
    say(f"[topk] {what} top_k={top_k} bf16={bf16}")
    gi, gn = topk_on_gpu(d, top_k, bf16=bf16, **gpu_kw)
    q, k = (to_bf16_bits(d["q"]), to_bf16_bits(d["k"])) if bf16 else (d["q"], d["k"])
    kind = oracle.BF16 if bf16 else oracle.F16
    sl = np.asarray(d["seqlens"])
    if pairs is not None:  # check a sample of (b, g) pairs (the oracle on those sequences only)
        bs = sorted({p // d["Hkv"] for p in pairs})
    else:
        bs = list(range(d["B"]))
    s, m = oracle.topk_scores(q[bs], k[bs], num_kv_heads=d["Hkv"], seqlens=sl[bs], kind=kind)
    oi, on = oracle.topk_select(q[bs], k[bs], top_k, num_kv_heads=d["Hkv"], seqlens=sl[bs], kind=kind)
    G = d["Hq"] // d["Hkv"]
    swaps = 0
    for bi, b in enumerate(bs):
        for g in range(d["Hkv"]):
            if pairs is not None and b * d["Hkv"] + g not in pairs:
                continue
            want = on[bi * d["Hkv"] + g]
            got = gn[b * d["Hkv"] + g]
            assert got == want == min(top_k, sl[b]), (b, g, got, want)
            sel = gi[b, g, :got]
            assert np.all(np.diff(sel) > 0) and (got == 0 or (sel[0] >= 0 and sel[-1] < sl[b]))
            ref = oi[bi, g, :want]
            extra, missing = np.setdiff1d(sel, ref), np.setdiff1d(ref, sel)
            if extra.size:
                band = 2.0 ** -24 * (G * 128 + G) * m[bi, g]
                sc = s[bi, g]
                assert np.max(sc[missing] - band[missing]) <= np.min(sc[extra] + band[extra]), (b, g)
                swaps += extra.size
    say(f"  traded places within the fp32 band: {swaps}")
    return gi, gn


@pytest.mark.parametrize("model", ["llama3-8b", "qwen2.5-14b"])
def test_topk_small(model):
    d = _model_small(model, 67)
    for top_k in (0, 1, 300, 1234, 5000):
        check_topk(d, top_k, f"{model} S=3000")


def test_topk_rows_not_a_multiple_of_four():
    # score rows padded to 4 floats; lengths ending inside a 16-byte group
    d = _model_small("llama3-8b", 70, S=3001, lens=(3001, 2999, 5, 1))
    for top_k in (1, 3, 777):
        check_topk(d, top_k, "S=3001")


@pytest.mark.parametrize("Hq,Hkv", [(4, 1), (6, 2), (15, 5), (64, 64), (65, 65)])
def test_topk_head_layouts(Hq, Hkv):
    # the score pass walks (token, head) pieces in memory order, four pieces
    # per load: one or two KV heads (several tokens per load), a head count
    # that is no power of two, the largest count whose query sums fit its
    # LDS table, and one more (one KV head at a time)
    d = kvgen.dense_small(seed=71 + Hkv, B=3, Hq=Hq, Hkv=Hkv, S=777, seqlens=[777, 500, 3])
    for top_k in (1, 100, 600):
        check_topk(d, top_k, f"Hq={Hq} Hkv={Hkv} S=777")


@pytest.mark.parametrize("Hq,Hkv,S,lens", [(32, 8, 17000, (17000, 12345)), (65, 65, 777, (777, 300))])
def test_topk_bf16(Hq, Hkv, S, lens):
    # bf16 K and q: the whole-row score pass over two selection chunks, and
    # the one-head-at-a-time pass (more than 64 KV heads)
    d = kvgen.dense_small(seed=74 + Hkv, B=2, Hq=Hq, Hkv=Hkv, S=S, seqlens=list(lens))
    for top_k in (1, 250, 3000):
        check_topk(d, top_k, f"bf16 Hq={Hq} Hkv={Hkv} S={S}", bf16=True)


def test_topk_ties_go_to_smaller_tokens():
    d = _model_small("llama3-8b", 68, lens=(3000, 2000))
    d["k"][0, :, 3] = d["k"][0, 77, 3]  # every row of head 3 equal: all scores tie
    gi, gn = check_topk(d, 50, "ties")
    assert np.array_equal(gi[0, 3, :50], np.arange(50))


def test_topk_chunks_and_ties_across_chunk_boundaries():
    # 40000 rows: the selection splits each pair into 16384-token chunks.
    # Sequence 0, head 3: every row equal, so all scores tie and the smallest
    # tokens are kept, across the first chunk boundary.  Head 5: rows
    # 16000..17999 equal and scoring above every other row (8 * the sign of the
    # group's query sum), a tie band across the same boundary.
    d = _model_small("llama3-8b", 72, S=40000, lens=(40000, 33000))
    d["k"][0, :, 3] = d["k"][0, 77, 3]
    qsum = np.asarray(d["q"][0, 20:24], np.float64).sum(axis=0)
    d["k"][0, 16000:18000, 5] = 8.0 * np.where(qsum >= 0, 1.0, -1.0)
    gi, gn = check_topk(d, 1500, "S=40000 tie band")
    assert np.array_equal(gi[0, 5, :1500], np.arange(16000, 17500))
    gi, gn = check_topk(d, 20000, "S=40000 all tie")
    assert np.array_equal(gi[0, 3, :20000], np.arange(20000))
    assert np.isin(np.arange(16000, 18000), gi[0, 5, :20000]).all()  # the band is inside
    gi, gn = check_topk(d, 40000, "S=40000 keep all")
    assert np.array_equal(gi[0, 0, :40000], np.arange(40000))
    assert np.array_equal(gi[1, 7, :33000], np.arange(33000))


def test_topk_null_seqlens_and_dirty_workspace():
    # seqlens NULL: every sequence has all S rows (two selection chunks); the
    # workspace holds all-ones bytes before the call (it needs no initialisation)
    d = _model_small("llama3-8b", 73, S=20000, lens=(20000, 20000))
    for top_k in (1, 2500, 19999):
        check_topk(d, top_k, "S=20000 seqlens NULL", null_seqlens=True, dirty_workspace=True)


def test_topk_no_rows():
    # max_seqlen 0: only the counts are written; q, k, idx and the workspace may be NULL
    desc = K.topk_desc(batch=3, num_q_heads=8, num_kv_heads=2, dtype=torch.float16, max_seqlen=0,
                       top_k=5)
    n = torch.full((6,), -7, dtype=torch.int32, device="cuda")
    K.kvdec_topk_select(desc, None, None, None, None, n, None)
    torch.cuda.synchronize()
    assert n.cpu().numpy().tolist() == [0] * 6


def test_topk_then_gather_end_to_end():
    d = _model_small("llama3-8b", 69, S=5000, lens=(5000, 4000, 300, 0))
    top_k = 500
    gi, gn = topk_on_gpu(d, top_k)
    oi, on = oracle.topk_select(d["q"], d["k"], top_k, num_kv_heads=d["Hkv"], seqlens=d["seqlens"])
    same = all(np.array_equal(gi[b, g, :gn[b * 8 + g]], oi[b, g, :on[b * 8 + g]])
               for b in range(d["B"]) for g in range(8))
    assert same, "selections differ (a near-tie at the boundary): not expected for this seed"
    go, gl = gather_on_gpu(d, oi, on)
    ro, rl = oracle.gather_attn(d["q"], d["k"], d["v"], oi, on, num_kv_heads=8, scale=d["scale"])
    check_close(go, ro, "top-k + gather")
    check_lse(gl, rl, "top-k + gather lse")


def test_clo_full_size_sampled():
    """The CLO 128K shapes (Llama3-8B heads, batch 4, 10% kept): top-k on all
    pairs with five of them checked, and gather attention over the oracle's
    selection of sequence 1 checked in full."""
    d = kvgen.clo_gather(seed=0)
    check_topk(d, d["top_k"], "Llama3-8B 128K", pairs={0, 7, 9, 20, 31})
    idx, n = oracle.topk_select(d["q"][1:2], d["k"][1:2], d["top_k"], num_kv_heads=8,
                                seqlens=d["seqlens"][1:2])
    full_idx = np.zeros((4, 8, d["top_k"]), np.int32)
    full_n = np.zeros(32, np.int32)
    full_idx[1], full_n[8:16] = idx[0], n
    go, gl = gather_on_gpu(d, full_idx, full_n)
    ro, rl = oracle.gather_attn(d["q"][1:2], d["k"][1:2], d["v"][1:2], idx, n, num_kv_heads=8,
                                scale=d["scale"])
    check_close(go[1:2], ro, "gather 128K (sequence 1)")
    check_lse(gl[1:2], rl, "gather 128K lse (sequence 1)")


def test_topk_maximum_length_all_sixteen_chunks():
    # S = 262144, the longest sequence the selection takes: 16 chunks of 16384
    # tokens, every count row of the threshold scan in use.  Head 0: rows
    # 245000..246999 equal and scoring above every other row, a tie band
    # across the chunk 14 / 15 boundary (token 245760), so the smallest 1500
    # of them are kept.  Then every row (keep-all) and every row but one.
    S = 262144
    d = kvgen.dense_small(seed=78, B=1, Hq=4, Hkv=2, S=S, seqlens=[S])
    qsum = np.asarray(d["q"][0, 0:2], np.float64).sum(axis=0)
    d["k"][0, 245000:247000, 0] = 8.0 * np.where(qsum >= 0, 1.0, -1.0)
    gi, gn = check_topk(d, 1500, "S=262144 tie band across chunks 14/15")
    assert np.array_equal(gi[0, 0, :1500], np.arange(245000, 246500))
    gi, gn = check_topk(d, S, "S=262144 keep all")
    assert np.array_equal(gi[0, 0, :S], np.arange(S)) and np.array_equal(gi[0, 1, :S], np.arange(S))
    gi, gn = check_topk(d, S - 1, "S=262144 all but one")
    assert gn.tolist() == [S - 1, S - 1]

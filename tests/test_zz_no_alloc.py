"""GPU checks of kvdec_decode_attn_noalloc, the workspace-free decode entry
point: its results equal kvdec_decode_attn's (with a caller workspace) bit for
bit, and the fp64 oracle's to the usual tolerance, over consecutive calls that
reuse the library's scratch with different and smaller shapes."""
import numpy as np
import pytest
import torch

import kvgen
import long_kv_caches_amd as K
from long_kv_caches_amd import _lib
import oracle
from gpu_util import bits, check_close, check_lse, dev, host_f64, say

pytestmark = pytest.mark.gpu


def _desc_and_args(d, split_tokens=0, max_seqlen=None):
    B, Hq, Hkv = d["B"], d["Hq"], d["Hkv"]
    q, k, v = dev(d["q"]), dev(d["k"]), dev(d["v"])
    seqlens = cu = None
    if d["layout"] == "ragged":
        cu = torch.from_numpy(np.asarray(d["cu_seqlens"], np.int32)).cuda()
        ms = int(np.diff(d["cu_seqlens"]).max())
        desc = K.attn_desc(batch=B, num_q_heads=Hq, num_kv_heads=Hkv, dtype=torch.float16,
                           layout=K.KVDEC_RAGGED, max_seqlen=max_seqlen or ms,
                           softmax_scale=d["scale"], split_tokens=split_tokens,
                           kv_rows=d["k"].shape[0])
    else:
        if d.get("seqlens") is not None:
            seqlens = torch.from_numpy(np.asarray(d["seqlens"], np.int32)).cuda()
        desc = K.attn_desc(batch=B, num_q_heads=Hq, num_kv_heads=Hkv, dtype=torch.float16,
                           layout=K.KVDEC_DENSE, max_seqlen=d["S"], softmax_scale=d["scale"],
                           split_tokens=split_tokens)
    return desc, (q, k, v, seqlens, cu)


def _both(d, what, split_tokens=0, max_seqlen=None):
    """Runs the workspace call, then the workspace-free call; checks they agree
    bit for bit and that the latter matches the oracle."""
    desc, (q, k, v, seqlens, cu) = _desc_and_args(d, split_tokens, max_seqlen)
    B, Hq = d["B"], d["Hq"]
    need = K.kvdec_decode_attn_workspace(desc)
    say(f"[noalloc] {what}: workspace {need} B of {K.NOALLOC_SCRATCH_BYTES}")
    assert need <= K.NOALLOC_SCRATCH_BYTES
    ws = K.alloc_workspace(need)
    out_ws = torch.empty((B, Hq, 128), dtype=torch.float16, device="cuda")
    lse_ws = torch.empty((B, Hq), dtype=torch.float32, device="cuda")
    K.kvdec_decode_attn(desc, q, k, v, seqlens, cu, None, out_ws, lse_ws, ws)
    out = torch.full((B, Hq, 128), float("nan"), dtype=torch.float16, device="cuda")
    lse = torch.full((B, Hq), float("nan"), dtype=torch.float32, device="cuda")
    K.kvdec_decode_attn_noalloc(desc, q, k, v, seqlens, cu, None, out, lse)
    torch.cuda.synchronize()
    assert np.array_equal(bits(out), bits(out_ws)), what
    assert np.array_equal(lse.cpu().numpy().view(np.uint32), lse_ws.cpu().numpy().view(np.uint32))
    layout = oracle.RAGGED if d["layout"] == "ragged" else oracle.DENSE
    ref_o, ref_l = oracle.decode_attn(d["q"], d["k"], d["v"], num_kv_heads=d["Hkv"], layout=layout,
                                      scale=d["scale"], seqlens=d.get("seqlens"),
                                      cu_seqlens=d.get("cu_seqlens"))
    check_close(host_f64(out), ref_o, what)
    check_lse(lse.cpu().numpy(), ref_l, what + " lse")
    return need


def test_noalloc_equals_workspace_call_on_consecutive_calls():
    # 1: the balanced schedule on a ragged Llama3-8B-shaped batch (G = 4)
    d1 = kvgen.ragged_llama(seed=21, B=16, lo=2048, hi=6000)
    n1 = _both(d1, "ragged 16 x [2048, 6000] 32q/8kv")
    # 2: a smaller dense call with other group size and lengths, reusing the
    #    same scratch with stale partials of call 1 in it
    d2 = kvgen.dense_small(seed=22, B=2, Hq=8, Hkv=2, S=300, seqlens=[300, 77])
    n2 = _both(d2, "dense 2 x 300 8q/2kv")
    assert 0 < n2 < n1
    # 3: fixed chunks, smaller still
    d3 = kvgen.ragged_llama(seed=23, lens=[1, 64, 129, 0, 700], Hq=8, Hkv=8)
    _both(d3, "ragged chunks of 64", split_tokens=64)


def test_noalloc_near_the_scratch_limit():
    # 64-token chunks over a 128000-token bound and 32 KV heads: 64000 partial
    # slots, just under the scratch size.  The real length is short: chunks
    # past it do no work and the merge reads only the chunks it covers.
    d = kvgen.ragged_llama(seed=24, lens=[1000], Hq=32, Hkv=32)
    need = _both(d, "ragged chunks, 128000-token bound", split_tokens=64, max_seqlen=128000)
    assert need > K.NOALLOC_SCRATCH_BYTES * 0.95


def test_noalloc_rejects_beyond_the_scratch_and_launches_nothing():
    d = kvgen.ragged_llama(seed=25, lens=[100], Hq=32, Hkv=32)
    desc, (q, k, v, _, cu) = _desc_and_args(d, split_tokens=64, max_seqlen=1 << 20)
    assert K.kvdec_decode_attn_workspace(desc) > K.NOALLOC_SCRATCH_BYTES
    out = torch.full((1, 32, 128), 7.0, dtype=torch.float16, device="cuda")
    with pytest.raises(K.KvdecError) as e:
        K.kvdec_decode_attn_noalloc(desc, q, k, v, None, cu, None, out, None)
    assert e.value.status == _lib.KVDEC_ERR_WORKSPACE
    torch.cuda.synchronize()
    assert torch.all(out == 7.0)


def test_noalloc_replays_under_graph_capture():
    # The call this entry point is for: captured once in a graph, replayed
    # with new queries written between replays by ordinary eager work; every
    # replay must equal the workspace call on the same inputs, bit for bit.
    d = kvgen.ragged_llama(seed=26, B=8, lo=1000, hi=3000)
    desc, (q, k, v, _, cu) = _desc_and_args(d)
    B, Hq = d["B"], d["Hq"]
    out = torch.empty((B, Hq, 128), dtype=torch.float16, device="cuda")
    lse = torch.empty((B, Hq), dtype=torch.float32, device="cuda")
    say("[noalloc] graph capture, 3 replays")
    K.kvdec_decode_attn_noalloc(desc, q, k, v, None, cu, None, out, lse)  # first use: set-up
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        K.kvdec_decode_attn_noalloc(desc, q, k, v, None, cu, None, out, lse)
    torch.cuda.synchronize()
    ws = K.alloc_workspace(K.kvdec_decode_attn_workspace(desc))
    ref = torch.empty_like(out)
    ref_lse = torch.empty_like(lse)
    gen = torch.Generator(device="cuda").manual_seed(27)
    for rep in range(3):
        q.copy_(torch.randn(q.shape, generator=gen, device="cuda").to(torch.float16))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        K.kvdec_decode_attn(desc, q, k, v, None, cu, None, ref, ref_lse, ws)
        torch.cuda.synchronize()
        assert np.array_equal(bits(out), bits(ref)), rep
        assert np.array_equal(lse.cpu().numpy().view(np.uint32), ref_lse.cpu().numpy().view(np.uint32))

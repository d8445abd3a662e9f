"""GPU parity of kvdec_sparse_hybrid_attn (CLO cache buffer + persistent cache)."""
import numpy as np
import pytest
import torch

import kvgen
import long_kv_caches_amd as K
import oracle
from gpu_util import bits, check_close, check_lse, decode_on_gpu, dev, host_f64, say, to_bf16_bits

pytestmark = pytest.mark.gpu


def hybrid_on_gpu(d, split_tokens=0, head_map=None, bf16=False):
    hm = d["head_map"] if head_map is None else head_map
    B, Hq, Hkv = d["B"], d["Hq"], d["Hkv"]
    fp8 = d["pers_k"].dtype == np.uint8
    fmt = dict(kv_format=K.KVDEC_KV_E4M3, k_scale=d["k_scale"], v_scale=d["v_scale"]) if fp8 else {}
    dt = torch.bfloat16 if bf16 else torch.float16
    c = (lambda x: dev(to_bf16_bits(x), True)) if bf16 else dev
    desc = K.hybrid_desc(batch=B, num_q_heads=Hq, num_kv_heads=Hkv, dtype=dt,
                         softmax_scale=d["scale"], split_tokens=split_tokens,
                         num_pers_slots=d["pers_k"].shape[1], pers_cap=d["pers_k"].shape[2],
                         buf_cap=d["buf_k"].shape[2], **fmt)
    ws = K.alloc_workspace(K.kvdec_sparse_hybrid_attn_workspace(desc))
    out = torch.empty((B, Hq, 128), dtype=dt, device="cuda")
    lse = torch.empty((B, Hq), dtype=torch.float32, device="cuda")
    i32 = lambda a: torch.from_numpy(np.asarray(a, np.int32)).cuda()
    K.kvdec_sparse_hybrid_attn(desc, c(d["q"]), c(d["pers_k"]), c(d["pers_v"]),
                               i32(d["pers_len"]), c(d["buf_k"]), c(d["buf_v"]),
                               i32(d["buf_len"]), i32(hm), out, lse, ws)
    torch.cuda.synchronize()
    return out, lse.cpu().numpy()


def hybrid_oracle(d, head_map=None, bf16=False):
    hm = d["head_map"] if head_map is None else head_map
    c = to_bf16_bits if bf16 else (lambda x: x)
    return oracle.hybrid_attn(c(d["q"]), c(d["pers_k"]), c(d["pers_v"]), d["pers_len"], c(d["buf_k"]),
                              c(d["buf_v"]), d["buf_len"], hm, scale=d["scale"],
                              kind=oracle.BF16 if bf16 else oracle.F16,
                              k_scale=d.get("k_scale"), v_scale=d.get("v_scale"))


@pytest.mark.parametrize("model", ["llama3-8b", "qwen2.5-14b"])
def test_hybrid_reduced_context(model):
    d = kvgen.clo_hybrid(seed=1, model=model, B=4, S=4096)
    say(f"[hybrid] {model} S=4096")
    for split in (0, 128):
        out, lse = hybrid_on_gpu(d, split)
        ro, rl = hybrid_oracle(d)
        check_close(host_f64(out), ro, f"hybrid {model} split={split}")
        check_lse(lse, rl)


def test_hybrid_bf16():
    # bf16 q, K and V (the output is bf16), at G = 4 (Llama3-8B heads) and
    # G = 5 (Qwen2.5-14B heads), both on the matrix-core tile path
    for model in ("llama3-8b", "qwen2.5-14b"):
        d = kvgen.clo_hybrid(seed=6, model=model, B=2, S=4096)
        ro, rl = hybrid_oracle(d, bf16=True)
        for split in (0, 128):
            say(f"[hybrid] bf16 {model} split={split}")
            out, lse = hybrid_on_gpu(d, split, bf16=True)
            check_close(host_f64(out), ro, f"hybrid bf16 {model} split={split}", bf16_out=True)
            check_lse(lse, rl)


def _dense_view(kf, vf, d, rows=None):
    """[B, Hkv, S, D] full KV -> dense decode workload [B, S, Hkv, D]."""
    k = np.ascontiguousarray(kf.transpose(0, 2, 1, 3))
    v = np.ascontiguousarray(vf.transpose(0, 2, 1, 3))
    return dict(layout="dense", B=d["B"], Hq=d["Hq"], Hkv=d["Hkv"], D=128, S=k.shape[1], q=d["q"],
                k=k, v=v, seqlens=None, scale=d["scale"])


def test_hybrid_heads_bitwise_equal_decode_on_same_rows():
    d = kvgen.clo_hybrid(seed=2, B=2, S=2048)
    G = d["Hq"] // d["Hkv"]
    say("[hybrid] per-head bit identity with kvdec_decode_attn")
    out_h, _ = hybrid_on_gpu(d, split_tokens=128)
    hb = bits(out_h)
    # persistent heads: dense decode over the full KV
    out_full, _ = decode_on_gpu(_dense_view(d["k_full"], d["v_full"], d), split_tokens=128)
    fb = bits(out_full)
    # buffer heads: dense decode over the compacted buffers
    out_buf, _ = decode_on_gpu(_dense_view(d["buf_k"], d["buf_v"], d), split_tokens=128)
    bb = bits(out_buf)
    for g in range(d["Hkv"]):
        js = slice(g * G, (g + 1) * G)
        ref = fb if d["head_map"][g] >= 0 else bb
        assert np.array_equal(hb[:, js], ref[:, js]), g


def test_all_persistent_equals_dense_oracle():
    d = kvgen.clo_hybrid(seed=3, B=2, S=1024, n_pers=8)
    assert np.all(d["head_map"] >= 0)
    say("[hybrid] all heads persistent")
    out, _ = hybrid_on_gpu(d, split_tokens=64)
    ro, _ = oracle.decode_attn(_dense_view(d["k_full"], d["v_full"], d)["q"],
                               _dense_view(d["k_full"], d["v_full"], d)["k"],
                               _dense_view(d["k_full"], d["v_full"], d)["v"], num_kv_heads=8,
                               layout=oracle.DENSE, scale=d["scale"])
    check_close(host_f64(out), ro, "all persistent")


def test_hybrid_full_size_128k():
    for model in ("llama3-8b", "qwen2.5-14b"):
        d = kvgen.clo_hybrid(seed=0, model=model)
        say(f"[hybrid] {model} 128K full size")
        out, lse = hybrid_on_gpu(d)
        ro, rl = hybrid_oracle(d)
        check_close(host_f64(out), ro, f"hybrid {model} 128K")
        check_lse(lse, rl)
        del d


@pytest.mark.parametrize("split", [0, 128])
def test_uneven_and_empty_lengths(split):
    """Persistent and buffer lengths that differ per sequence and per head,
    including empty ones and single rows (the oracle takes the same lengths)."""
    d = kvgen.clo_hybrid(seed=5, B=3, S=3000, frac=0.3)
    Hkv = d["Hkv"]
    d["pers_len"] = np.array([3000, 1, 0], np.int32)
    bl = d["buf_len"].reshape(3, Hkv).copy()
    buf_heads = np.nonzero(d["head_map"] < 0)[0]
    cap = d["buf_k"].shape[2]
    pattern = [0, 1, 17, cap, cap - 5, 255]
    for b in range(3):
        for i, g in enumerate(buf_heads):
            bl[b, g] = min(cap, pattern[(i + 2 * b) % len(pattern)])
    d["buf_len"] = bl.reshape(-1)
    say(f"[hybrid] uneven lengths split={split}")
    out, lse = hybrid_on_gpu(d, split)
    ro, rl = hybrid_oracle(d)
    check_close(host_f64(out), ro, f"hybrid uneven lengths split={split}")
    check_lse(lse, rl)

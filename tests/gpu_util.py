"""Helpers for the GPU parity tests: host arrays -> device tensors, calls through
the C ABI, and the tolerance checks.

Tolerances (floating-point outputs of fp16/bf16 kernels with fp32
accumulation, compared with the fp64 oracle on the same 16-bit inputs):
  * fp16 outputs: max-abs error <= 4e-3 and relative L2 error <= 1e-3 over the
    tensor;
  * bf16 outputs: the same budget on top of the error that rounding the exact
    result to bf16 already has (bf16 keeps 8 significant bits, so that rounding
    alone is about 1.1e-3 relative L2 on these outputs);
  * lse (fp32 output): |error| <= 2e-4 + 1e-5 |lse|.  The kernel's scores carry
    fp32 rounding of 128-term dot products (about 1e-6 relative) and the
    log-sum-exp an fp32 sum over up to 1e5 terms (about 1e-5 relative).
"""
import sys

import numpy as np
import torch

import kvgen
import long_kv_caches_amd as K

MAX_ABS = 4e-3
REL_L2 = 1e-3


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def dev(a, bf16=False):
    """numpy -> cuda tensor.  float16 stays fp16; uint16 with bf16=True is bf16
    bits; uint8 (e4m3 codes) stays uint8."""
    t = torch.from_numpy(np.ascontiguousarray(a))
    if a.dtype == np.uint16:
        t = t.view(torch.int16).view(torch.bfloat16 if bf16 else torch.float16)
    return t.cuda()


def host_f64(t):
    """cuda fp16 / bf16 tensor -> float64 numpy."""
    if t.dtype == torch.bfloat16:
        return t.float().cpu().numpy().astype(np.float64)
    return t.cpu().numpy().astype(np.float64)


def bits(t):
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def to_bf16_bits(a_f16):
    return kvgen.f32_to_bf16_bits(np.asarray(a_f16, np.float32))


def check_close(got, ref, what="", max_abs=MAX_ABS, rel_l2=REL_L2, bf16_out=False):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    if bf16_out:
        rounded = kvgen.bf16_bits_to_f32(kvgen.f32_to_bf16_bits(ref.astype(np.float32)))
        rerr = rounded.astype(np.float64) - ref
        max_abs += float(np.abs(rerr).max()) if rerr.size else 0.0
        nref = float(np.linalg.norm(ref))
        rel_l2 += float(np.linalg.norm(rerr) / nref) if nref > 0 else 0.0
    assert got.shape == ref.shape, (got.shape, ref.shape)
    err = np.abs(got - ref)
    mae = float(err.max()) if err.size else 0.0
    den = float(np.linalg.norm(ref))
    rl2 = float(np.linalg.norm(got - ref) / den) if den > 0 else float(np.linalg.norm(got - ref))
    say(f"  {what}: max_abs={mae:.3e} rel_l2={rl2:.3e}")
    assert mae <= max_abs, f"{what}: max abs error {mae} > {max_abs}"
    assert rl2 <= rel_l2, f"{what}: relative L2 error {rl2} > {rel_l2}"


def check_lse(got, ref, what="lse"):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    inf = np.isneginf(ref)
    assert np.array_equal(np.isneginf(got), inf), f"{what}: -inf positions differ"
    tol = 2e-4 + 1e-5 * np.abs(ref[~inf])
    bad = np.abs(got[~inf] - ref[~inf]) > tol
    assert not bad.any(), f"{what}: {bad.sum()} values off, worst {np.abs(got[~inf]-ref[~inf]).max()}"


LAYOUTS = {"dense": K.KVDEC_DENSE, "ragged": K.KVDEC_RAGGED, "paged": K.KVDEC_PAGED}


def decode_on_gpu(d, split_tokens=0, bf16=False, want_lse=True, repeat=1, dev_inputs=None):
    """Runs kvdec_decode_attn on a kvgen workload dict.  Returns (out, lse) as a
    cuda tensor and a numpy array; with repeat > 1 returns a list of outs."""
    layout = LAYOUTS[d["layout"]]
    B, Hq, Hkv = d["B"], d["Hq"], d["Hkv"]
    fp8 = d["k"].dtype == np.uint8  # e4m3 codes with d["k_scale"], d["v_scale"]
    if dev_inputs is None:
        conv = to_bf16_bits if bf16 else (lambda x: x)
        kv = (lambda x: x) if fp8 else conv
        dev_inputs = dict(q=dev(conv(d["q"]), bf16), k=dev(kv(d["k"]), bf16),
                          v=dev(kv(d["v"]), bf16))
    q, k, v = dev_inputs["q"], dev_inputs["k"], dev_inputs["v"]
    seqlens = cu = bt = None
    kv_rows, page, max_pages = 0, 0, 0
    if layout == K.KVDEC_DENSE:
        max_seqlen = d["S"]
        if d.get("seqlens") is not None:
            seqlens = torch.from_numpy(np.asarray(d["seqlens"], np.int32)).cuda()
    elif layout == K.KVDEC_RAGGED:
        cu = torch.from_numpy(np.asarray(d["cu_seqlens"], np.int32)).cuda()
        max_seqlen = int(np.diff(d["cu_seqlens"]).max()) if B else 0
        kv_rows = d["k"].shape[0]
    else:
        seqlens = torch.from_numpy(np.asarray(d["seqlens"], np.int32)).cuda()
        bt = torch.from_numpy(d["block_table"]).cuda()
        max_seqlen = int(np.max(d["seqlens"])) if B else 0
        kv_rows, page, max_pages = d["k"].shape[0], d["page"], d["block_table"].shape[1]
    fmt = dict(kv_format=K.KVDEC_KV_E4M3, k_scale=d["k_scale"], v_scale=d["v_scale"]) if fp8 else {}
    desc = K.attn_desc(batch=B, num_q_heads=Hq, num_kv_heads=Hkv, dtype=q.dtype, layout=layout,
                       max_seqlen=max_seqlen, softmax_scale=d["scale"], page_size=page,
                       max_pages_per_seq=max_pages, split_tokens=split_tokens, kv_rows=kv_rows,
                       **fmt)
    ws = K.alloc_workspace(K.kvdec_decode_attn_workspace(desc))
    lse = torch.empty((B, Hq), dtype=torch.float32, device="cuda") if want_lse else None
    outs = []
    for _ in range(repeat):
        out = torch.empty((B, Hq, 128), dtype=q.dtype, device="cuda")
        K.kvdec_decode_attn(desc, q, k, v, seqlens, cu, bt, out, lse, ws)
        outs.append(out)
    torch.cuda.synchronize()
    if repeat > 1:
        return outs, (lse.cpu().numpy() if want_lse else None)
    return outs[0], (lse.cpu().numpy() if want_lse else None)

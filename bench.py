"""Benchmark of the decode-attention hot path on one MI355X.

Workload: one Llama3-8B-shaped decode layer (32 query heads on 8 KV heads,
head_dim 128), batch 16, context lengths uniform in [16384, 32768], ragged fp16
KV with per-channel LogNormal(0, 0.5) K outlier scales (seeded synthetic
data).  One step = one kvdec_decode_attn call over the whole batch: work
split, Q load, K stream + MFMA scores, online softmax, V stream + P.V, the
in-workgroup merge and the split-K merge into the fp16 output and lse.

Prints ONE JSON line.  `value` is achieved HBM throughput (algorithmic bytes /
time per step, TB/s) with inputs resident in HBM; `roofline` prices the same
bytes against the 8 TB/s HBM3E peak; `cpu_baseline` times the fp64 CPU oracle
on the same workload.

Usage: python bench.py [--gpus 1] [--steps 50] [--warmup 10] [--split-tokens N]
                       [--calibrate-copy] [--no-cpu-baseline]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "decode_attn_llama3_8b_32k_traffic.json")
KERNEL_SOURCES = ["long_kv_caches_amd/csrc/decode_attn.hip", "long_kv_caches_amd/csrc/device_common.h",
                  "long_kv_caches_amd/csrc/internal.h", "long_kv_caches_amd/csrc/api.cpp"]


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def measured_traffic(per_launch_algorithmic):
    """HBM bytes per launch from the committed counter summary, if it was taken
    on the current kernel sources; else None."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("kernel_source_hash") != kernel_source_hash():
        return None
    return t.get("hbm_bytes_per_launch")


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--split-tokens", type=int, default=0)
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="also run a 1 GiB device copy (counter calibration under rocprofv3)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py: this build runs on one GPU only (no multi-GPU path); use --gpus 1",
              file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import kvgen
    import long_kv_caches_amd as K

    d = kvgen.ragged_llama(seed=args.seed)
    B, Hq, Hkv, D = d["B"], d["Hq"], d["Hkv"], d["D"]
    lens = np.diff(d["cu_seqlens"]).astype(np.int64)
    T = int(lens.sum())
    dev = torch.device("cuda:0")
    q = torch.from_numpy(d["q"]).to(dev)
    k = torch.from_numpy(d["k"]).to(dev)
    v = torch.from_numpy(d["v"]).to(dev)
    cu = torch.from_numpy(d["cu_seqlens"]).to(dev)
    max_seqlen = int(lens.max())
    desc = K.attn_desc(batch=B, num_q_heads=Hq, num_kv_heads=Hkv, dtype=torch.float16,
                       layout=K.KVDEC_RAGGED, max_seqlen=max_seqlen, softmax_scale=d["scale"],
                       split_tokens=args.split_tokens, kv_rows=T)
    ws = K.alloc_workspace(K.kvdec_decode_attn_workspace(desc), device=dev)
    out = torch.empty((B, Hq, D), dtype=torch.float16, device=dev)
    lse = torch.empty((B, Hq), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream(dev)

    # algorithmic bytes of one step: attended K and V rows, q, out, lse, cu_seqlens
    kv_bytes = T * Hkv * D * 2 * 2
    step_bytes = kv_bytes + B * Hq * D * 2 * 2 + B * Hq * 4 + (B + 1) * 4
    token_heads = T * Hkv

    def step():
        K.kvdec_decode_attn(desc, q, k, v, None, cu, None, out, lse, ws, stream=stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    K.kvdec_kernel_timing(True)  # HIP events around each split-kernel launch, on `stream`
    t0.record(stream)
    for _ in range(args.steps):
        step()
    t1.record(stream)
    torch.cuda.synchronize()
    kern_ms_total, kern_launches = K.kvdec_kernel_timing_read()
    K.kvdec_kernel_timing(False)
    ms = t0.elapsed_time(t1) / args.steps
    sec = ms / 1e3
    kern_sec = kern_ms_total / max(kern_launches, 1) / 1e3

    if args.calibrate_copy:
        src = torch.ones(1 << 29, dtype=torch.float16, device=dev)  # 1 GiB
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()

    achieved_gbs = step_bytes / sec / 1e9
    # roofline of the dominant kernel (the split kernel: it streams all of K
    # and V); its algorithmic bytes per launch are the step's bytes
    kern_gbs = step_bytes / kern_sec / 1e9
    traffic = measured_traffic(step_bytes)
    result = {
        "metric": "decode-attn achieved HBM TB/s (% of peak) + KV tokens·heads/s, Llama3-8B 32K",
        "value": round(achieved_gbs / 1e3, 4),
        "unit": "TB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16",
        "data": "synthetic (seeded; shapes and distributions of the Llama3-8B 32K decode workload)",
        "config": {
            "workload": "llama3-8b-32k-ragged-decode-attention",
            "batch": B, "num_q_heads": Hq, "num_kv_heads": Hkv, "head_dim": D,
            "context_lengths": "uniform [16384, 32768]", "total_tokens": T,
            "layout": "ragged", "split_tokens": args.split_tokens or "auto",
        },
        "pct_of_hbm_peak": round(100.0 * achieved_gbs / HBM_PEAK_GBS, 2),
        "kv_token_heads_per_s": round(token_heads / sec, 1),
        "roofline": {
            "bound": "hbm",
            "kernel": "decode_balanced_kernel" if args.split_tokens == 0 else "decode_chunk_kernel",
            "achieved": round(kern_gbs, 1),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(kern_gbs / HBM_PEAK_GBS, 4),
            "traffic": traffic,
            "kernel_us": round(kern_sec * 1e6, 2),
            "launches_timed": kern_launches,
        },
    }

    if not args.no_cpu_baseline:
        import oracle
        reps, times = 3, []
        for _ in range(reps):
            c0 = time.perf_counter()
            oracle.decode_attn(d["q"], d["k"], d["v"], num_kv_heads=Hkv, layout=oracle.RAGGED,
                               scale=d["scale"], cu_seqlens=d["cu_seqlens"])
            times.append(time.perf_counter() - c0)
        cs = sorted(times)[reps // 2]
        result["cpu_baseline"] = {
            "value": round(step_bytes / cs / 1e12, 6),
            "unit": "TB/s",
            "cores": oracle.max_threads(),
            "kind": "oracle",
            "sample": f"the full workload (all {B} sequences, {T} tokens), median of {reps} runs, "
                      f"{cs:.2f} s each",
        }
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()

"""Benchmark of the decode-attention hot path on one MI355X.

Workload: one Llama3-8B-shaped decode layer (32 query heads on 8 KV heads,
head_dim 128), batch 16, context lengths uniform in [16384, 32768], ragged fp16
KV with per-channel LogNormal(0, 0.5) K outlier scales (seeded synthetic
data).  One step = one kvdec_decode_attn call over the whole batch: work
split, Q load, K stream + dot2 scores, online softmax, V stream + P.V, the
in-workgroup merge and the split-K merge into the fp16 output and lse.

Prints ONE JSON line.  `value` is achieved HBM throughput (algorithmic bytes /
time per step, TB/s) with inputs resident in HBM; `roofline` prices the same
bytes against the 8 TB/s HBM3E peak (and, as `frac_of_stream_read`, against
`stream_read`: the HBM read rate of the library's streaming-read reference
kernel on the same box); `isolated_call` times single calls with L2 and the
MALL flushed before each (p10 / p50 / p90); `cpu_baseline` times the fp64 CPU
oracle on the same workload.

Other workloads (one JSON line each, same fields): --workload llama2-7b-paged
(batch-1024 paged MHA), clo-llama3-8b-128k / clo-qwen2.5-14b-128k (CLO hybrid
attention, plus the fused head-cache lookup's latency), kvpr-opt13b (partial
K/V recompute TFLOP/s against the bf16 MFMA peak, plus attention over the
merged cache).

Usage: python bench.py [--gpus 1] [--steps 50] [--warmup 10] [--workload W]
                       [--split-tokens N] [--calibrate-copy] [--no-cpu-baseline]
                       [--no-stream-read]
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
_CSRC = "long_kv_caches_amd/csrc/"
DECODE_SOURCES = [_CSRC + f for f in ("decode_attn.hip", "device_common.h", "internal.h", "api.cpp")]
RECOMPUTE_SOURCES = [_CSRC + f for f in ("kv_recompute.hip", "device_common.h", "internal.h", "api.cpp")]

# Counter summaries in profiles/, per workload: the file, the main kernel it
# covers (a substring of the kernel's name in rocprofv3's output) and the
# sources that kernel is built from.  `bench.py --summarize-pmc DIR` writes
# them from rocprofv3 counter runs of this script (the commands are in each
# file); a summary counts only while those sources hash to what it records.
COUNTERS = {
    "llama3-8b-32k": ("decode_attn_llama3_8b_32k_traffic.json", "decode_balanced_kernel<", DECODE_SOURCES),
    "llama3-8b-32k-fp8": ("decode_attn_llama3_8b_32k_e4m3_traffic.json", "decode_balanced_kernel<",
                          DECODE_SOURCES),
    "llama2-7b-paged": ("decode_attn_llama2_7b_paged_b1024_traffic.json", "decode_balanced_kernel<",
                        DECODE_SOURCES),
    "clo-llama3-8b-128k": ("clo_hybrid_attn_llama3_8b_128k_traffic.json", "decode_balanced_kernel<",
                           DECODE_SOURCES),
    "clo-qwen2.5-14b-128k": ("clo_hybrid_attn_qwen2_5_14b_128k_traffic.json", "decode_balanced_kernel<",
                             DECODE_SOURCES),
    "clo-gather-llama3-8b-128k": ("gather_attn_llama3_8b_128k_traffic.json", "decode_balanced_kernel<",
                                  DECODE_SOURCES),
    "kvpr-opt13b": ("kv_recompute_opt13b_counters.json", "kv_recompute_kernel_wide<1>", RECOMPUTE_SOURCES),
    "kvpr-opt13b-attention": ("decode_attn_opt13b_merged_cache_traffic.json", "decode_balanced_kernel<",
                              DECODE_SOURCES),
}
# Kernel-trace summaries in profiles/, per workload (`--summarize-trace DIR`).
TRACES = {
    "llama3-8b-32k": ("decode_attn_llama3_8b_32k_kernel_trace.txt",
                      "Llama3-8B 32K ragged decode attention (16 sequences, 32 query / 8 KV heads, fp16)"),
    "llama3-8b-32k-fp8": ("decode_attn_llama3_8b_32k_e4m3_kernel_trace.txt",
                          "Llama3-8B 32K ragged decode attention over e4m3 K/V"),
    "llama2-7b-paged": ("decode_attn_llama2_7b_paged_b1024_kernel_trace.txt",
                        "Llama-2-7B paged decode attention, batch 1024, 16-token pages"),
    "clo-llama3-8b-128k": ("clo_hybrid_attn_and_lookup_llama3_8b_128k_kernel_trace.txt",
                           "CLO hybrid attention, head-cache lookup (and one layer ahead) and the "
                           "miss-driven prefetch, Llama3-8B 128K batch 4"),
    "clo-qwen2.5-14b-128k": ("clo_hybrid_attn_and_lookup_qwen2_5_14b_128k_kernel_trace.txt",
                             "CLO hybrid attention, head-cache lookup (and one layer ahead) and the "
                             "miss-driven prefetch, Qwen2.5-14B 128K batch 4"),
    "clo-gather-llama3-8b-128k": ("gather_attn_and_topk_llama3_8b_128k_kernel_trace.txt",
                                  "index-gather attention over the exact top-10% rows and the top-k "
                                  "selection, Llama3-8B heads, 128K cache, batch 8"),
    "kvpr-opt13b": ("kv_recompute_and_attn_opt13b_kernel_trace.txt",
                    "KVPR partial K/V recompute GEMM (b=32, l=256, h=5120 -> 0.859 TFLOP) and attention "
                    "over the merged 1024-token cache, OPT-13B layer"),
    "kvpr-overlap": ("kvpr_overlapped_layer_load_opt13b_kernel_trace.txt",
                     "KVPR layer load: X[0:l] and K/V[l:s') over PCIe overlapped with the recompute, "
                     "OPT-13B layer"),
}


def trace_command(workload):
    return (f"rocprofv3 --kernel-trace --stats -f csv -d <out>/TRACE -o run -- python3 <repo>/bench.py "
            f"--workload {workload} --no-cpu-baseline > <out>/TRACE/bench.json")


def summarize_trace(workload, out_dir):
    """Writes profiles/<trace file> from the rocprofv3 kernel-trace run in
    out_dir/TRACE (trace_command): the kernels by total time, and the bench
    line of the same run."""
    import csv
    import glob
    d = os.path.join(out_dir, "TRACE")
    stats = glob.glob(os.path.join(d, "**", "*kernel_stats.csv"), recursive=True)
    if not stats:
        raise SystemExit(f"summarize-trace: no kernel_stats.csv under {d}")
    with open(stats[0]) as f:
        rows = list(csv.DictReader(f))
    rows.sort(key=lambda r: -float(r["TotalDurationNs"]))
    name, what = TRACES[workload]
    lines = [f"rocprofv3 kernel-trace summary: {what}.", "",
             "Command (repository root on the GPU box; cd /tmp && export TMPDIR=/tmp first):",
             "  " + trace_command(workload),
             "  (bench.py: 200 ms device-copy prewarm, then per timed call: warmup steps, 50 timed steps, "
             "50 more with per-launch kernel events)", "",
             f"{'kernel':<66}{'calls':>7}{'avg us':>10}{'min us':>10}{'max us':>10}{'% time':>8}"]
    for r in rows[:14]:
        k = r["Name"].replace("void kvdec::(anonymous namespace)::", "").replace("void kvdec::", "")
        k = k.replace("kvdec::(anonymous namespace)::", "").replace("kvdec::", "")
        k = k.split("(")[0] if not k.startswith("void at::") else k[:64]
        lines.append(f"{k[:64]:<66}{int(r['Calls']):>7}{float(r['AverageNs']) / 1e3:>10.2f}"
                     f"{float(r['MinNs']) / 1e3:>10.2f}{float(r['MaxNs']) / 1e3:>10.2f}"
                     f"{float(r['Percentage']):>8.2f}")
    try:
        with open(os.path.join(d, "bench.json")) as f:
            b = json.loads(f.read().strip().splitlines()[-1])
        lines += ["", "The bench line of the same run (under the profiler):",
                  f"  value {b['value']} {b['unit']}, ms_per_step {b['ms_per_step']}",
                  "  roofline: " + json.dumps(b["roofline"])]
        for extra in ("attention", "lookup", "lookup_ahead", "prefetch", "topk_select", "by_split_point"):
            if extra in b:
                lines.append(f"  {extra}: " + json.dumps(b[extra]))
    except (OSError, ValueError, IndexError, KeyError):
        pass
    with open(os.path.join(ROOT, "profiles", name), "w") as f:
        f.write("\n".join(lines) + "\n")
    print(json.dumps({"summaries": [name]}))


PMC_GROUPS = {"FETCH_SIZE": ["FETCH_SIZE"], "WRITE_SIZE": ["WRITE_SIZE"],
              "MFMA": ["SQ_VALU_MFMA_BUSY_CYCLES", "GRBM_GUI_ACTIVE", "SQ_INSTS_VALU_MFMA_MOPS_BF16",
                       "SQ_BUSY_CYCLES"],
              "LDS": ["SQ_LDS_BANK_CONFLICT", "SQ_LDS_IDX_ACTIVE", "SQ_INSTS_LDS", "GRBM_GUI_ACTIVE"]}


def pmc_command(workload, group):
    """The rocprofv3 counter run of one group (each group a run of its own,
    the program straight after --), from the repository root on the GPU machine."""
    return (f"rocprofv3 --pmc {' '.join(PMC_GROUPS[group])} -f csv -d <out>/{group} -o run -- "
            f"python3 <repo>/bench.py --workload {workload} --no-cpu-baseline --no-stream-read "
            f"--steps 10 --warmup 3 --prewarm-ms 0 --calibrate-copy > <out>/{group}/bench.json")


def summarize_pmc(workload, out_dir):
    """Writes the counter summaries of `workload` into profiles/ from the
    rocprofv3 runs in out_dir/<group>/ (pmc_command).  FETCH_SIZE and
    WRITE_SIZE (KiB per dispatch) are scaled by what the same counters read
    for the calibration run's 1 GiB device copies (__amd_rocclr_copyBuffer),
    and compared with the algorithmic bytes the bench line reports."""
    import csv
    import glob
    from collections import defaultdict

    def group(name):
        files = glob.glob(os.path.join(out_dir, name, "**", "*counter_collection.csv"), recursive=True)
        if not files:
            return None, None
        per = defaultdict(lambda: defaultdict(list))  # kernel -> counter -> [(value, grid, ns)]
        with open(files[0]) as f:
            for r in csv.DictReader(f):
                per[r["Kernel_Name"]][r["Counter_Name"]].append(
                    (float(r["Counter_Value"]), int(r["Grid_Size"]),
                     int(r["End_Timestamp"]) - int(r["Start_Timestamp"])))
        bench_line = None
        try:
            with open(os.path.join(out_dir, name, "bench.json")) as f:
                bench_line = json.loads(f.read().strip().splitlines()[-1])
        except (OSError, ValueError, IndexError):
            pass
        agents = glob.glob(os.path.join(out_dir, name, "**", "*agent_info.csv"), recursive=True)
        gpu = {}
        if agents:
            with open(agents[0]) as f:
                for r in csv.DictReader(f):
                    if r.get("Agent_Type") == "GPU":
                        gpu = r
        return per, (bench_line, gpu)

    def mean_of(per, match, counter, exclude=()):
        vals = [v for k, cs in per.items() if match in k and not any(e in k for e in exclude)
                for v in cs.get(counter, [])]
        return (sum(v[0] for v in vals) / len(vals), len(vals), sum(v[2] for v in vals) / len(vals)) if vals else None

    def calibration(per, counter, nbytes):
        # the calibration copies (nbytes each) read the most: other copies
        # through the same copy kernel (a prewarm) are 4 times smaller
        vals = [v[0] for k, cs in per.items() if "copyBuffer" in k for v in cs.get(counter, [])]
        top = max(vals)
        sel = [v for v in vals if v >= 0.75 * top]
        return nbytes / (sum(sel) / len(sel) * 1024.0)

    fetch, fmeta = group("FETCH_SIZE")
    write, _ = group("WRITE_SIZE")
    targets = [workload] + (["kvpr-opt13b-attention"] if workload == "kvpr-opt13b" else [])
    written = []
    for tw in targets:
        name, match, sources = COUNTERS[tw]
        bench_line = fmeta[0] if fmeta else None
        out = {"kernel": match.rstrip("<"), "workload": tw, "kernel_source_hash": source_hash(sources),
               "commands": [pmc_command(workload, g) for g in PMC_GROUPS
                            if os.path.isdir(os.path.join(out_dir, g))]}
        if fetch is not None and write is not None:
            if not bench_line or "calibration_copy_bytes" not in bench_line:
                raise SystemExit("summarize-pmc: the counter runs need --calibrate-copy")
            cb = int(bench_line["calibration_copy_bytes"])
            ff, fw = calibration(fetch, "FETCH_SIZE", cb), calibration(write, "WRITE_SIZE", cb)
            fk, nf, _ = mean_of(fetch, match, "FETCH_SIZE")
            wk, nw, _ = mean_of(write, match, "WRITE_SIZE")
            hbm = int(round((fk * ff + wk * fw) * 1024))
            out.update({"fetch_kib_per_dispatch": round(fk, 1), "write_kib_per_dispatch": round(wk, 1),
                        "dispatches": nf,
                        "copy_calibration": {"fetch_factor": round(ff, 4), "write_factor": round(fw, 4),
                                             "copy_bytes": cb,
                                             "note": "device-to-device copies of copy_bytes "
                                                     "(__amd_rocclr_copyBuffer) read by the same counters "
                                                     "in the same process"},
                        "hbm_bytes_per_launch": hbm})
            algo = None
            if bench_line:
                if tw == "kvpr-opt13b":
                    algo = bench_line["roofline"].get("bytes_per_launch")
                elif tw == "kvpr-opt13b-attention":
                    algo = bench_line.get("attention", {}).get("bytes")
                else:
                    algo = bench_line["roofline"].get("bytes_per_launch")
            if algo:
                out["algorithmic_bytes_per_launch"] = int(algo)
                out["traffic_over_algorithmic"] = round(hbm / algo, 4)
            if "decode_balanced_kernel" in match:
                mf = mean_of(fetch, "decode_balanced_merge_kernel<", "FETCH_SIZE")
                mw = mean_of(write, "decode_balanced_merge_kernel<", "WRITE_SIZE")
                if mf and mw:
                    out["merge_kernel_fetch_kib"] = round(mf[0], 1)
                    out["merge_kernel_write_kib"] = round(mw[0], 1)
        if tw == "kvpr-opt13b":
            mfma, mmeta = group("MFMA")
            if mfma is not None:
                gpu = mmeta[1]
                xcc = int(gpu.get("Num_Xcc", 8) or 8)
                simds = int(gpu.get("Simd_Count", 0) or 0) or 4 * int(gpu.get("Cu_Count", 256))
                busy, n, ns = mean_of(mfma, match, "SQ_VALU_MFMA_BUSY_CYCLES")
                grbm, _, _ = mean_of(mfma, match, "GRBM_GUI_ACTIVE")
                mops, _, _ = mean_of(mfma, match, "SQ_INSTS_VALU_MFMA_MOPS_BF16")
                sqb, _, _ = mean_of(mfma, match, "SQ_BUSY_CYCLES")
                active = grbm / xcc  # GRBM_GUI_ACTIVE is summed over the XCDs
                out["mfma"] = {"sq_valu_mfma_busy_cycles": busy, "grbm_gui_active": grbm,
                               "sq_insts_valu_mfma_mops_bf16": mops, "sq_busy_cycles": sqb,
                               "xcds": xcc, "simds": simds, "dispatches": n,
                               "kernel_ns_under_counters": round(ns, 1),
                               "bf16_flop_per_launch": mops * 512,
                               "busy_frac": round(busy / simds / active, 4),
                               "implied_clock_ghz": round(active / ns, 3),
                               "note": "busy_frac = SQ_VALU_MFMA_BUSY_CYCLES / (SIMDs x GRBM_GUI_ACTIVE per "
                                       "XCD); the clock is GRBM_GUI_ACTIVE per XCD over the dispatch's time"}
                vend = [k for k in mfma if k.startswith("Cijk_")]
                if vend:
                    vb, vn, vns = mean_of(mfma, vend[0], "SQ_VALU_MFMA_BUSY_CYCLES")
                    vg, _, _ = mean_of(mfma, vend[0], "GRBM_GUI_ACTIVE")
                    out["vendor_gemm_mfma"] = {
                        "kernel": vend[0][:120], "dispatches": vn,
                        "busy_frac": round(vb / simds / (vg / xcc), 4),
                        "implied_clock_ghz": round(vg / xcc / vns, 3),
                        "kernel_ns_under_counters": round(vns, 1)}
            lds, _ = group("LDS")
            if lds is not None:
                for variant in ("kv_recompute_kernel_wide<1>", "kv_recompute_kernel_wide<0>"):
                    conf = mean_of(lds, variant, "SQ_LDS_BANK_CONFLICT")
                    act = mean_of(lds, variant, "SQ_LDS_IDX_ACTIVE")
                    if conf and act:
                        out.setdefault("lds", {})[variant] = {
                            "sq_lds_bank_conflict": conf[0], "sq_lds_idx_active": act[0],
                            "conflict_frac_of_active": round(conf[0] / act[0], 4)}
        with open(os.path.join(ROOT, "profiles", name), "w") as f:
            json.dump(out, f, indent=1)
            f.write("\n")
        written.append(name)
    print(json.dumps({"summaries": written}))


def source_hash(sources) -> str:
    h = hashlib.sha256()
    for rel in sources:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def counter_summary(workload):
    """The workload's counter summary from profiles/, if it was taken on the
    current sources of its kernel; else None."""
    name, _, sources = COUNTERS[workload]
    try:
        with open(os.path.join(ROOT, "profiles", name)) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    return t if t.get("kernel_source_hash") == source_hash(sources) else None


def measured_traffic(workload):
    """HBM bytes per launch of the workload's main kernel, from its counter summary."""
    t = counter_summary(workload)
    return None if t is None else t.get("hbm_bytes_per_launch")


WORKLOADS = ("llama3-8b-32k", "llama2-7b-paged", "clo-llama3-8b-128k", "clo-qwen2.5-14b-128k",
             "kvpr-opt13b", "kvpr-overlap", "llama3-8b-32k-fp8", "clo-gather-llama3-8b-128k")


def prewarm(torch, dev, ms):
    """Device copies for about `ms` milliseconds before the warmup steps.  GPU
    clocks are not locked on the boxes this runs on; they ramp up under load,
    and the first ~10 ms of work run measurably slower."""
    if ms <= 0:
        return
    buf = torch.empty(1 << 27, dtype=torch.float16, device=dev)  # 256 MiB
    dst = torch.empty_like(buf)
    t0 = time.perf_counter()
    while (time.perf_counter() - t0) * 1e3 < ms:
        for _ in range(8):
            dst.copy_(buf)
        torch.cuda.synchronize()
    del buf, dst


def time_steps(step, steps, warmup, stream, K, torch, prewarm_ms=0.0):
    """(ms per step, mean main-kernel us, launches timed).

    Two back-to-back timed passes of `steps` steps each, after the warmup:
    the first, bracketed by events on `stream` only, gives ms per step; the
    second records HIP events around every main-kernel launch on the stream it
    is launched on and gives that kernel's mean duration.  The per-launch
    events are kept out of the first pass because on these GPUs they add
    about 5 us to a 250 us decode step (measured: 245-247 us per step without
    them, 250-258 with them)."""
    prewarm(torch, torch.device("cuda:0"), prewarm_ms)
    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    t0.record(stream)
    for _ in range(steps):
        step()
    t1.record(stream)
    torch.cuda.synchronize()
    ms = t0.elapsed_time(t1) / steps
    K.kvdec_kernel_timing(True)  # HIP events around each main-kernel launch, on `stream`
    for _ in range(steps):
        step()
    torch.cuda.synchronize()
    kern_ms_total, launches = K.kvdec_kernel_timing_read()
    K.kvdec_kernel_timing(False)
    return ms, kern_ms_total * 1e3 / max(launches, 1), launches


def isolated_calls(step, stream, torch, dev, amount, unit, reps=50, flush_bytes=1 << 30):
    """Per-call times with the caches cold: before each call (outside its event
    pair) a 1 GiB buffer is written on the same stream, which evicts L2 and the
    256 MB MALL.  Returns p10 / p50 / p90 in us and the rate at the median
    (`amount` per call in `unit`: bytes -> TB/s, FLOPs -> TFLOP/s)."""
    import numpy as np
    flush = torch.empty(flush_bytes // 4, dtype=torch.int32, device=dev)
    times = []
    for r in range(reps):
        flush.fill_(r)
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        step()
        e1.record(stream)
        torch.cuda.synchronize()
        times.append(e0.elapsed_time(e1) * 1e3)
    del flush
    p10, p50, p90 = (float(x) for x in np.percentile(times, [10, 50, 90]))
    rate = amount / (p50 * 1e-6) / 1e12
    return {"reps": reps, "flush_bytes_before_each": flush_bytes, "us_p10": round(p10, 2),
            "us_p50": round(p50, 2), "us_p90": round(p90, 2),
            ("tbs_at_p50" if unit == "bytes" else "tflops_at_p50"): round(rate, 4)}


def stream_read_reference(K, torch, dev, stream, nbytes=2 << 30, reps=20):
    """The library's streaming-read reference kernel over a 2 GiB buffer (larger
    than L2 and the MALL): the HBM read rate one kernel reaches on this machine,
    by its kernel events."""
    buf = torch.ones(nbytes // 2, dtype=torch.float16, device=dev)
    sink = torch.zeros(1, dtype=torch.int32, device=dev)
    for _ in range(3):
        K.kvdec_stream_read(buf, sink, stream=stream)
    torch.cuda.synchronize()
    K.kvdec_kernel_timing(True)
    for _ in range(reps):
        K.kvdec_stream_read(buf, sink, stream=stream)
    torch.cuda.synchronize()
    ms, n = K.kvdec_kernel_timing_read()
    K.kvdec_kernel_timing(False)
    del buf
    return {"kernel": "stream_read_kernel", "bytes": nbytes, "launches": n,
            "tbs": round(nbytes / (ms / max(n, 1) * 1e-3) / 1e12, 4)}


def cpu_model() -> str:
    """The host CPU's model name (from /proc/cpuinfo), for the CPU baseline."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def oracle_seconds(fn, reps=3):
    times = []
    for _ in range(reps):
        c0 = time.perf_counter()
        fn()
        times.append(time.perf_counter() - c0)
    return sorted(times)[reps // 2]


def hbm_roofline(kernel, nbytes, kern_us, traffic=None):
    gbs = nbytes / (kern_us * 1e-6) / 1e9
    return {"bound": "hbm", "kernel": kernel, "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS,
            "unit": "GB/s", "frac": round(gbs / HBM_PEAK_GBS, 4), "traffic": traffic,
            "kernel_us": round(kern_us, 2), "bytes_per_launch": int(nbytes)}


def common(args, workload, metric, unit, value, ms, dtype, data, config, higher=True):
    return {"metric": metric, "value": value, "unit": unit, "n_gpus": 1, "steps": args.steps,
            "warmup": args.warmup, "ms_per_step": round(ms, 4), "higher_is_better": higher,
            "scaling": "weak", "vs_baseline": None, "dtype": dtype, "data": data,
            "config": dict({"workload": workload}, **config), "prewarm_ms": args.prewarm_ms}


def single_thread_oracle(d, np, oracle, seed):
    """The oracle on one thread: the small dense config (1 sequence of 1024
    tokens, 8 query / 2 KV heads) and a seeded 1/16 subset of the headline batch
    (one of its 16 sequences).  Median of 3 runs each."""
    import kvgen
    out = {}
    c1 = kvgen.dense_small(seed=0)
    b1 = c1["S"] * c1["Hkv"] * c1["D"] * 4 + c1["Hq"] * c1["D"] * 4
    t1 = oracle_seconds(lambda: oracle.decode_attn(c1["q"], c1["k"], c1["v"], num_kv_heads=c1["Hkv"],
                                                   layout=oracle.DENSE, scale=c1["scale"], nthreads=1))
    out["dense_1x1024_8q2kv"] = {"seconds": round(t1, 6), "gbs": round(b1 / t1 / 1e9, 3)}
    i = int(np.random.default_rng(seed).integers(d["B"]))
    cu = d["cu_seqlens"]
    lo, hi = int(cu[i]), int(cu[i + 1])
    Hkv, D, Hq = d["Hkv"], d["D"], d["Hq"]
    b2 = (hi - lo) * Hkv * D * 4 + Hq * D * 4
    t2 = oracle_seconds(lambda: oracle.decode_attn(d["q"][i:i + 1], d["k"][lo:hi], d["v"][lo:hi], num_kv_heads=Hkv,
                                                   layout=oracle.RAGGED, scale=d["scale"],
                                                   cu_seqlens=np.array([0, hi - lo], np.int32), nthreads=1))
    out["headline_sequence_subset"] = {"sequence": i, "tokens": hi - lo, "seconds": round(t2, 4),
                                       "gbs": round(b2 / t2 / 1e9, 3)}
    return out


def bench_llama3(args, K, np, torch, dev, stream, fp8=False):
    import kvgen
    d = kvgen.ragged_llama(seed=args.seed)
    if fp8:  # e4m3 K/V codes with per-tensor scales
        d = kvgen.fp8_kv(d)
    kv_bytes = 1 if fp8 else 2
    B, Hq, Hkv, D = d["B"], d["Hq"], d["Hkv"], d["D"]
    lens = np.diff(d["cu_seqlens"]).astype(np.int64)
    T = int(lens.sum())
    q = torch.from_numpy(d["q"]).to(dev)
    k = torch.from_numpy(d["k"]).to(dev)
    v = torch.from_numpy(d["v"]).to(dev)
    cu = torch.from_numpy(d["cu_seqlens"]).to(dev)
    fmt = dict(kv_format=K.KVDEC_KV_E4M3, k_scale=d["k_scale"], v_scale=d["v_scale"]) if fp8 else {}
    desc = K.attn_desc(batch=B, num_q_heads=Hq, num_kv_heads=Hkv, dtype=torch.float16,
                       layout=K.KVDEC_RAGGED, max_seqlen=int(lens.max()), softmax_scale=d["scale"],
                       split_tokens=args.split_tokens, kv_rows=T, **fmt)
    ws = K.alloc_workspace(K.kvdec_decode_attn_workspace(desc), device=dev)
    out = torch.empty((B, Hq, D), dtype=torch.float16, device=dev)
    lse = torch.empty((B, Hq), dtype=torch.float32, device=dev)
    # algorithmic bytes of one step: attended K and V rows, q, out, lse, cu_seqlens
    step_bytes = T * Hkv * D * kv_bytes * 2 + B * Hq * D * 2 * 2 + B * Hq * 4 + (B + 1) * 4

    def step():
        K.kvdec_decode_attn(desc, q, k, v, None, cu, None, out, lse, ws, stream=stream)

    ms, kern_us, launches = time_steps(step, args.steps, args.warmup, stream, K, torch, args.prewarm_ms)
    gbs = step_bytes / (ms * 1e-3) / 1e9
    config = {"batch": B, "num_q_heads": Hq, "num_kv_heads": Hkv, "head_dim": D,
              "context_lengths": "uniform [16384, 32768]", "total_tokens": T, "layout": "ragged",
              "split_tokens": args.split_tokens or "auto"}
    if fp8:
        config.update(kv_format="e4m3 (per-tensor scales)", k_scale=d["k_scale"], v_scale=d["v_scale"])
        r = common(args, "llama3-8b-32k-ragged-decode-attention-e4m3-kv",
                   "decode-attn over e4m3 K/V: achieved HBM TB/s (% of peak) + KV tokens·heads/s, Llama3-8B 32K",
                   "TB/s", round(gbs / 1e3, 4), ms, "f16 q/out, e4m3 K/V, fp32 accumulate",
                   "synthetic (seeded; the Llama3-8B 32K decode workload, K/V cast to e4m3 with amax scales)",
                   config)
    else:
        r = common(args, "llama3-8b-32k-ragged-decode-attention",
                   "decode-attn achieved HBM TB/s (% of peak) + KV tokens·heads/s, Llama3-8B 32K",
                   "TB/s", round(gbs / 1e3, 4), ms, "f16",
                   "synthetic (seeded; shapes and distributions of the Llama3-8B 32K decode workload)",
                   config)
    r["pct_of_hbm_peak"] = round(100.0 * gbs / HBM_PEAK_GBS, 2)
    r["kv_token_heads_per_s"] = round(T * Hkv / (ms * 1e-3), 1)
    r["roofline"] = hbm_roofline("decode_balanced_kernel" if args.split_tokens == 0 else "decode_chunk_kernel",
                                 step_bytes, kern_us,
                                 measured_traffic("llama3-8b-32k-fp8" if fp8 else "llama3-8b-32k"))
    r["roofline"]["launches_timed"] = launches
    r["isolated_call"] = isolated_calls(step, stream, torch, dev, step_bytes, "bytes")
    if not args.no_cpu_baseline:
        import oracle
        if fp8:  # a bounded sample: the first 4 sequences
            n = 4
            cu4 = d["cu_seqlens"][:n + 1]
            sub_bytes = int(cu4[-1]) * Hkv * D * kv_bytes * 2 + n * Hq * D * 4
            cs = oracle_seconds(lambda: oracle.decode_attn(
                d["q"][:n], d["k"][:cu4[-1]], d["v"][:cu4[-1]], num_kv_heads=Hkv, layout=oracle.RAGGED,
                scale=d["scale"], cu_seqlens=cu4, k_scale=d["k_scale"], v_scale=d["v_scale"]))
            sample = f"the first {n} of {B} sequences ({int(cu4[-1])} tokens), median of 3 runs, {cs:.2f} s each"
        else:
            sub_bytes = step_bytes
            cs = oracle_seconds(lambda: oracle.decode_attn(d["q"], d["k"], d["v"], num_kv_heads=Hkv,
                                                           layout=oracle.RAGGED, scale=d["scale"],
                                                           cu_seqlens=d["cu_seqlens"]))
            sample = f"the full workload (all {B} sequences, {T} tokens), median of 3 runs, {cs:.2f} s each"
        r["cpu_baseline"] = {"value": round(sub_bytes / cs / 1e12, 6), "unit": "TB/s",
                             "cores": oracle.max_threads(), "cpu_model": cpu_model(), "kind": "oracle", "sample": sample}
        r["cpu_baseline"]["gpu_speedup"] = round(r["value"] / r["cpu_baseline"]["value"], 1)
        if not fp8:
            r["cpu_baseline"]["single_thread"] = single_thread_oracle(d, np, oracle, args.seed)
    return r


def bench_paged(args, K, np, torch, dev, stream):
    import kvgen
    d = kvgen.paged_mha(seed=args.seed)
    B, H, D, page = d["B"], d["Hq"], d["D"], d["page"]
    lens = d["seqlens"].astype(np.int64)
    T = int(lens.sum())
    q = torch.from_numpy(d["q"]).to(dev)
    k = torch.from_numpy(d["k"]).to(dev)
    v = torch.from_numpy(d["v"]).to(dev)
    bt = torch.from_numpy(d["block_table"]).to(dev)
    sl = torch.from_numpy(d["seqlens"]).to(dev)
    P = d["k"].shape[0]
    desc = K.attn_desc(batch=B, num_q_heads=H, num_kv_heads=H, dtype=torch.float16,
                       layout=K.KVDEC_PAGED, max_seqlen=int(lens.max()), softmax_scale=d["scale"],
                       page_size=page, max_pages_per_seq=d["max_pages"],
                       split_tokens=args.split_tokens, kv_rows=P)
    ws = K.alloc_workspace(K.kvdec_decode_attn_workspace(desc), device=dev)
    out = torch.empty((B, H, D), dtype=torch.float16, device=dev)
    lse = torch.empty((B, H), dtype=torch.float32, device=dev)
    used_pages = int(((lens + page - 1) // page).sum())
    step_bytes = T * H * D * 4 + B * H * D * 4 + B * H * 4 + B * 4 + used_pages * 4

    def step():
        K.kvdec_decode_attn(desc, q, k, v, sl, None, bt, out, lse, ws, stream=stream)

    ms, kern_us, launches = time_steps(step, args.steps, args.warmup, stream, K, torch, args.prewarm_ms)
    gbs = step_bytes / (ms * 1e-3) / 1e9
    r = common(args, "llama2-7b-paged-decode-attention",
               "paged decode-attn achieved HBM TB/s (% of peak), Llama-2-7B MHA batch 1024", "TB/s",
               round(gbs / 1e3, 4), ms, "f16",
               "synthetic (seeded; LogNormal(ln 1024, 1.0) lengths clipped to [128, 4096], shuffled page pool)",
               {"batch": B, "num_q_heads": H, "num_kv_heads": H, "head_dim": D, "page_size": page,
                "total_tokens": T, "pool_pages": P, "layout": "paged",
                "split_tokens": args.split_tokens or "auto"})
    r["pct_of_hbm_peak"] = round(100.0 * gbs / HBM_PEAK_GBS, 2)
    r["kv_token_heads_per_s"] = round(T * H / (ms * 1e-3), 1)
    r["roofline"] = hbm_roofline("decode_balanced_kernel" if args.split_tokens == 0 else "decode_chunk_kernel",
                                 step_bytes, kern_us, measured_traffic("llama2-7b-paged"))
    r["roofline"]["launches_timed"] = launches
    r["isolated_call"] = isolated_calls(step, stream, torch, dev, step_bytes, "bytes", reps=20)
    if not args.no_cpu_baseline:
        import oracle
        n = 64  # a bounded sample: the first 64 sequences
        sub_bytes = int(lens[:n].sum()) * H * D * 4 + n * H * D * 4
        cs = oracle_seconds(lambda: oracle.decode_attn(d["q"][:n], d["k"], d["v"], num_kv_heads=H,
                                                       layout=oracle.PAGED, scale=d["scale"],
                                                       seqlens=d["seqlens"][:n],
                                                       block_table=d["block_table"][:n], page_size=page))
        r["cpu_baseline"] = {"value": round(sub_bytes / cs / 1e12, 6), "unit": "TB/s",
                             "cores": oracle.max_threads(), "cpu_model": cpu_model(), "kind": "oracle",
                             "sample": f"the first {n} of {B} sequences ({int(lens[:n].sum())} tokens), "
                                       f"median of 3 runs, {cs:.2f} s each"}
    return r


def bench_clo(args, K, np, torch, dev, stream, model):
    import kvgen
    d = kvgen.clo_hybrid(seed=args.seed, model=model)
    B, Hq, Hkv, D = d["B"], d["Hq"], d["Hkv"], d["D"]
    G = Hq // Hkv
    to = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev)
    q, pk, pv, bk, bv = (to(d[n]) for n in ("q", "pers_k", "pers_v", "buf_k", "buf_v"))
    pl, blen, hm = to(d["pers_len"]), to(d["buf_len"]), to(d["head_map"])
    desc = K.hybrid_desc(batch=B, num_q_heads=Hq, num_kv_heads=Hkv, dtype=torch.float16,
                         softmax_scale=d["scale"], split_tokens=args.split_tokens,
                         num_pers_slots=d["pers_k"].shape[1], pers_cap=d["pers_k"].shape[2],
                         buf_cap=d["buf_k"].shape[2])
    ws = K.alloc_workspace(K.kvdec_sparse_hybrid_attn_workspace(desc), device=dev)
    out = torch.empty((B, Hq, D), dtype=torch.float16, device=dev)
    lse = torch.empty((B, Hq), dtype=torch.float32, device=dev)
    hmn = d["head_map"]
    rows = sum(int(d["pers_len"][b]) if hmn[g] >= 0 else int(d["buf_len"][b * Hkv + g])
               for b in range(B) for g in range(Hkv))
    step_bytes = rows * D * 4 + B * Hq * D * 4 + B * Hq * 4 + (B + B * Hkv + Hkv) * 4

    def step():
        K.kvdec_sparse_hybrid_attn(desc, q, pk, pv, pl, bk, bv, blen, hm, out, lse, ws, stream=stream)

    ms, kern_us, launches = time_steps(step, args.steps, args.warmup, stream, K, torch, args.prewarm_ms)
    gbs = step_bytes / (ms * 1e-3) / 1e9
    name = {"llama3-8b": "Llama3-8B", "qwen2.5-14b": "Qwen2.5-14B"}[model]
    r = common(args, f"clo-{model}-128k-hybrid-attention",
               f"CLO hybrid (buffer + persistent) attn achieved HBM TB/s, {name} 128K batch 4", "TB/s",
               round(gbs / 1e3, 4), ms, "f16",
               "synthetic (seeded; 2 persistent KV heads with all 131072 rows, 10% of rows per buffer head)",
               {"batch": B, "num_q_heads": Hq, "num_kv_heads": Hkv, "head_dim": D, "context": d["S"],
                "persistent_heads": int((hmn >= 0).sum()), "buffer_rows": d["ksel"],
                "split_tokens": args.split_tokens or "auto"})
    r["pct_of_hbm_peak"] = round(100.0 * gbs / HBM_PEAK_GBS, 2)
    r["kv_token_heads_per_s"] = round(rows / (ms * 1e-3), 1)
    r["roofline"] = hbm_roofline("decode_balanced_kernel" if args.split_tokens == 0 else "decode_chunk_kernel",
                                 step_bytes, kern_us, measured_traffic(args.workload))
    r["roofline"]["launches_timed"] = launches
    r["isolated_call"] = isolated_calls(step, stream, torch, dev, step_bytes, "bytes")

    # the fused head-cache lookup on the same queries (launch-bound at this size)
    tau = K.kvdec_headcache_thresholds(kvgen.group_importance(d["s"], Hkv).astype(np.float32),
                                       d["eta"], d["n_exp"]).to(dev)
    labels = to(d["labels"])
    w = to(d["weights"])
    hit = torch.empty(B * Hkv, dtype=torch.uint8, device=dev)
    ml = torch.empty(B * Hkv, dtype=torch.int32, device=dev)
    mc = torch.empty(1, dtype=torch.int32, device=dev)

    def lookup():
        K.kvdec_headcache_lookup(q, labels, w, tau, hit, None, None, ml, mc, stream=stream)

    lookup()  # decides against the generated labels; later calls see the updated labels
    torch.cuda.synchronize()
    misses_first = int(mc.item())
    lms, lkern_us, _ = time_steps(lookup, args.steps, args.warmup, stream, K, torch)
    lbytes = B * Hq * D * 2 * 2 + Hq * 4 + Hkv * 4 + B * Hkv * 1 + 4
    events_note = ("kernel_us from HIP events stamped from the kernel's dispatch; for a kernel of a few us, "
                   "issued one call at a time, they include the dispatch latency (the rocprofv3 kernel "
                   "traces give the kernel's own duration)")
    r["lookup"] = {"us_per_call": round(lms * 1e3, 2), "kernel_us": round(lkern_us, 2),
                   "bytes": lbytes, "misses_on_first_call": misses_first, "groups": B * Hkv,
                   "achieved_gbs": round(lbytes / (lkern_us * 1e-6) / 1e9, 1), "note": events_note}
    # the same lookup one layer ahead: q_approx = x_{l-1} W_Q^l (GEMV over the
    # next layer's W_Q), then the lookup on it
    a = kvgen.clo_ahead(seed=args.seed, model=model, B=B)
    x_prev = to(a["x_prev"])
    # one W_Q per layer, 12 layers in turn (more bytes than the 256 MB last-level
    # cache holds), so each call reads its W_Q from HBM as a layer would
    w_layers = [to(a["w_q"]) for _ in range(12)]
    q_approx = torch.empty((B, Hq, D), dtype=torch.float16, device=dev)
    labels2 = to(d["labels"])
    layer = [0]

    def ahead():
        wq = w_layers[layer[0] % len(w_layers)]
        layer[0] += 1
        K.kvdec_headcache_lookup_ahead(x_prev, wq, q_approx, labels2, w, tau, hit, None, None, ml, mc,
                                       stream=stream)

    ams, akern_us, alaunches = time_steps(ahead, args.steps, args.warmup, stream, K, torch)
    proj_us = akern_us * alaunches / args.steps - lkern_us  # per call, both kernels less the lookup's
    pbytes = a["w_q"].nbytes + a["x_prev"].nbytes + B * Hq * D * 2
    r["lookup_ahead"] = {"us_per_call": round(ams * 1e3, 2), "hidden": a["h"], "w_q_layers_cycled": len(w_layers),
                         "w_q_bytes": a["w_q"].nbytes, "projection_kernel_us": round(proj_us, 2),
                         "projection_achieved_gbs": round(pbytes / (proj_us * 1e-6) / 1e9, 1),
                         "projection_frac_of_hbm_peak": round(pbytes / (proj_us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
                         "note": events_note}
    r["prefetch"] = bench_prefetch(args, K, np, torch, dev, stream, d)
    if not args.no_cpu_baseline:
        import oracle
        sub_rows = sum(int(d["pers_len"][0]) if hmn[g] >= 0 else int(d["buf_len"][g]) for g in range(Hkv))
        sub_bytes = sub_rows * D * 4 + Hq * D * 4
        cs = oracle_seconds(lambda: oracle.hybrid_attn(d["q"][:1], d["pers_k"][:1], d["pers_v"][:1],
                                                       d["pers_len"][:1], d["buf_k"][:1], d["buf_v"][:1],
                                                       d["buf_len"][:Hkv], hmn, scale=d["scale"]))
        r["cpu_baseline"] = {"value": round(sub_bytes / cs / 1e12, 6), "unit": "TB/s",
                             "cores": oracle.max_threads(), "cpu_model": cpu_model(), "kind": "oracle",
                             "sample": f"batch element 0 of {B} ({sub_rows} KV rows), median of 3 runs, "
                                       f"{cs:.2f} s each"}
    return r


def bench_prefetch(args, K, np, torch, dev, stream, d):
    """The miss-driven prefetch at the CLO shapes: every buffer head of every
    sequence missed, so each of the B * 6 buffer heads pulls its 10% selection
    (13107 rows of K and of V) from the full KV in pinned host memory over
    PCIe.  Its rate is set beside a pinned host-to-device copy of the same
    number of contiguous bytes, and the call is timed again behind an
    already-raised host flag (the GPU-centric wait's cost)."""
    B, Hkv, S, D = d["k_full"].shape
    ksel, hm = d["ksel"], d["head_map"]
    pool_k = torch.from_numpy(d["k_full"]).pin_memory()  # [B, Hkv, S, D]
    pool_v = torch.from_numpy(d["v_full"]).pin_memory()
    idx = np.zeros((B, Hkv, ksel), np.int32)
    idx_len = np.zeros(B * Hkv, np.int32)
    for (b, g), sel in d["selection"].items():
        idx[b, g] = sel
        idx_len[b * Hkv + g] = sel.size
    miss = [b * Hkv + g for b in range(B) for g in range(Hkv) if hm[g] < 0]
    to = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev)
    ml, mc = to(np.array(miss, np.int32)), to(np.array([len(miss)], np.int32))
    idx_d, len_d, hm_d = to(idx), to(idx_len), to(hm)
    desc = K.prefetch_desc(batch=B, num_kv_heads=Hkv, elem_bytes=2, max_seqlen=S,
                           pool_strides=(Hkv * S * D, D, S * D), max_k=ksel, buf_cap=ksel)
    bk = torch.empty((B, Hkv, ksel, D), dtype=torch.float16, device=dev)
    bv = torch.empty_like(bk)
    bl = torch.zeros(B * Hkv, dtype=torch.int32, device=dev)
    flag = K.HostFlag()
    flag.value = 1
    status = torch.zeros(1, dtype=torch.int32, device=dev)

    def pf():
        K.kvdec_headcache_prefetch(desc, ml, mc, hm_d, idx_d, len_d, pool_k, pool_v, bk, bv, bl,
                                   stream=stream)

    def pf_flag():
        K.kvdec_headcache_prefetch(desc, ml, mc, hm_d, idx_d, len_d, pool_k, pool_v, bk, bv, bl,
                                   ready_flag=flag, ready_value=1, timeout_us=1000000,
                                   status=status, stream=stream)

    nbytes = len(miss) * ksel * D * 2 * 2
    src = torch.empty(nbytes, dtype=torch.uint8).pin_memory()
    dst = torch.empty(nbytes, dtype=torch.uint8, device=dev)

    def h2d():
        dst.copy_(src, non_blocking=True)

    def timed(fn, reps=10):
        for _ in range(2):
            fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(reps):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / reps

    ms = timed(pf)
    ms_flag = timed(pf_flag)
    ms_h2d = timed(h2d)
    buf_heads = torch.from_numpy(hm < 0).to(dev)
    same = bool(torch.equal(bk[:, buf_heads], to(d["buf_k"])[:, buf_heads]) and
                torch.equal(bv[:, buf_heads], to(d["buf_v"])[:, buf_heads]) and
                int(status.item()) == 0)
    flag.close()
    del pool_k, pool_v, src, dst
    return {"missed_buffer_heads": len(miss), "rows_per_head": ksel, "bytes": nbytes,
            "ms_per_call": round(ms, 4), "gbs": round(nbytes / (ms * 1e-3) / 1e9, 2),
            "ms_per_call_behind_raised_flag": round(ms_flag, 4),
            "pinned_h2d_copy_gbs": round(nbytes / (ms_h2d * 1e-3) / 1e9, 2),
            "frac_of_pinned_h2d": round(ms_h2d / ms, 4),
            "buffer_equals_generated_selection": same,
            "note": "the GPU reads each selected 256-byte row of the pinned host pool itself "
                    "(no host gather); pinned_h2d_copy_gbs is one contiguous DMA copy of the "
                    "same bytes"}


def bench_gather(args, K, np, torch, dev, stream):
    """Index-gather sparse attention over a full 128K cache: the exact top-k
    selection (10% per KV head) and the attention over the selected rows.
    Batch 8, so that the selected rows (about 430 MB) do not fit in the 256 MB
    MALL from one step to the next (at batch 4, 215 MB, steps ran 13% faster
    than single calls with the caches flushed)."""
    import kvgen
    d = kvgen.clo_gather(seed=args.seed, B=8)
    B, Hq, Hkv, D, S, top_k = d["B"], d["Hq"], d["Hkv"], d["D"], d["S"], d["top_k"]
    to = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev)
    q, k, v, sl = to(d["q"]), to(d["k"]), to(d["v"]), to(d["seqlens"])
    td = K.topk_desc(batch=B, num_q_heads=Hq, num_kv_heads=Hkv, dtype=torch.float16, max_seqlen=S,
                     top_k=top_k)
    tws = K.alloc_workspace(K.kvdec_topk_select_workspace(td), device=dev)
    idx = torch.empty((B, Hkv, top_k), dtype=torch.int32, device=dev)
    n = torch.empty(B * Hkv, dtype=torch.int32, device=dev)
    gd = K.gather_desc(batch=B, num_q_heads=Hq, num_kv_heads=Hkv, dtype=torch.float16, max_seqlen=S,
                       softmax_scale=d["scale"], split_tokens=args.split_tokens, max_k=top_k)
    gws = K.alloc_workspace(K.kvdec_gather_attn_workspace(gd), device=dev)
    out = torch.empty((B, Hq, D), dtype=torch.float16, device=dev)
    lse = torch.empty((B, Hq), dtype=torch.float32, device=dev)
    K.kvdec_topk_select(td, q, k, sl, idx, n, tws, stream=stream)
    torch.cuda.synchronize()
    rows = int(n.sum().item())
    step_bytes = rows * D * 2 * 2 + rows * 4 + B * Hq * D * 4 + B * Hq * 4 + B * Hkv * 4

    def step():
        K.kvdec_gather_attn(gd, q, k, v, idx, n, out, lse, gws, stream=stream)

    ms, kern_us, launches = time_steps(step, args.steps, args.warmup, stream, K, torch, args.prewarm_ms)
    gbs = step_bytes / (ms * 1e-3) / 1e9
    r = common(args, "clo-gather-llama3-8b-128k-sparse-attention",
               "index-gather sparse attn achieved HBM TB/s (top-10% rows of a full 128K cache), Llama3-8B batch 8",
               "TB/s", round(gbs / 1e3, 4), ms, "f16",
               "synthetic (seeded; full dense cache, lengths uniform in [64K, 128K], selection = exact top-k of the summed group scores)",
               {"batch": B, "num_q_heads": Hq, "num_kv_heads": Hkv, "head_dim": D, "cache_rows": S,
                "top_k": top_k, "selected_rows": rows, "split_tokens": args.split_tokens or "auto"})
    r["pct_of_hbm_peak"] = round(100.0 * gbs / HBM_PEAK_GBS, 2)
    r["kv_token_heads_per_s"] = round(rows / (ms * 1e-3), 1)
    r["roofline"] = hbm_roofline("decode_balanced_kernel" if args.split_tokens == 0 else "decode_chunk_kernel",
                                 step_bytes, kern_us, measured_traffic("clo-gather-llama3-8b-128k"))
    r["roofline"]["launches_timed"] = launches
    r["isolated_call"] = isolated_calls(step, stream, torch, dev, step_bytes, "bytes")

    def select():
        K.kvdec_topk_select(td, q, k, sl, idx, n, tws, stream=stream)

    sms, skern_us, slaunches = time_steps(select, args.steps, args.warmup, stream, K, torch)
    tokens = int(d["seqlens"].sum())
    score_bytes = tokens * Hkv * D * 2 + tokens * Hkv * 4
    r["topk_select"] = {"us_per_call": round(sms * 1e3, 2),
                        "kernels": "topk_score_rows_kernel + topk_radix_kernel<0..2> + topk_final_kernel + topk_write_kernel",
                        "kernel_us_per_call": round(skern_us * slaunches / max(args.steps, 1), 2),
                        "score_pass_bytes": score_bytes,
                        "score_pass_gbs_over_call": round(score_bytes / (sms * 1e-3) / 1e9, 1)}
    if not args.no_cpu_baseline:
        import oracle
        # a bounded sample: sequence 0 over the GPU selection's shape (the oracle's own top-k)
        oi, on = oracle.topk_select(d["q"][:1], d["k"][:1], top_k, num_kv_heads=Hkv, seqlens=d["seqlens"][:1])
        sub_rows = int(on.sum())
        sub_bytes = sub_rows * D * 4 + Hq * D * 4
        cs = oracle_seconds(lambda: oracle.gather_attn(d["q"][:1], d["k"][:1], d["v"][:1], oi, on,
                                                       num_kv_heads=Hkv, scale=d["scale"]))
        r["cpu_baseline"] = {"value": round(sub_bytes / cs / 1e12, 6), "unit": "TB/s",
                             "cores": oracle.max_threads(), "cpu_model": cpu_model(), "kind": "oracle",
                             "sample": f"sequence 0 of {B} ({sub_rows} selected rows), median of 3 runs, {cs:.2f} s each"}
    return r


def bench_kvpr(args, K, np, torch, dev, stream):
    import kvgen
    d = kvgen.kvpr_layer(seed=args.seed)
    b, h, H, D, s, l = d["b"], d["h"], d["H"], d["D"], d["s"], d["l"]
    to = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev)
    x = to(d["x"]).view(torch.bfloat16)
    # W as a model stores its projection weights (nn.Linear: [out, in]); the
    # [in, out] layout is timed too and reported beside it
    wk_io = to(d["w_k"]).view(torch.bfloat16)
    wv_io = to(d["w_v"]).view(torch.bfloat16)
    wk = wk_io.t().contiguous()
    wv = wv_io.t().contiguous()
    kc, vc, q = to(d["k_cache"]), to(d["v_cache"]), to(d["q"])
    flops = 4.0 * b * l * h * h

    def step():
        K.kvdec_kv_recompute(x, wk, wv, kc, vc, l, K.KVDEC_W_OUT_IN, stream=stream)

    def step_io():
        K.kvdec_kv_recompute(x, wk_io, wv_io, kc, vc, l, K.KVDEC_W_IN_OUT, stream=stream)

    ms, kern_us, launches = time_steps(step, args.steps, args.warmup, stream, K, torch, args.prewarm_ms)
    tflops = flops / (ms * 1e-3) / 1e12
    kern_tflops = flops / (kern_us * 1e-6) / 1e12
    r = common(args, "kvpr-opt13b-partial-recompute",
               "KVPR partial K/V recompute TFLOP/s (% of bf16 MFMA peak), OPT-13B b=32 l=256", "TFLOP/s",
               round(tflops, 2), ms, "bf16",
               "synthetic (seeded; X ~ N(0,1), W ~ N(0, 1/h), bf16)",
               {"batch": b, "hidden": h, "num_heads": H, "head_dim": D, "split_point": l,
                "context": s, "flops_per_step": flops, "w_layout": "out_in (nn.Linear)"})
    # algorithmic bytes of one call: X, W_K and W_V read, the K/V rows written
    rbytes = b * l * h * 2 + 2 * h * h * 2 + 2 * b * l * h * 2
    c = counter_summary("kvpr-opt13b")
    r["roofline"] = {"bound": "mfma", "kernel": "kv_recompute_kernel_wide", "achieved": round(kern_tflops, 2),
                     "peak": 2500.0, "unit": "TFLOP/s", "frac": round(kern_tflops / 2500.0, 4),
                     "traffic": c.get("hbm_bytes_per_launch") if c else None, "bytes_per_launch": rbytes,
                     "kernel_us": round(kern_us, 2), "launches_timed": launches}
    if c and "mfma" in c:
        m = c["mfma"]
        peak_at_clock = m["simds"] * 1024 * m["implied_clock_ghz"] * 1e9 / 1e12  # bf16: 1024 flop/clk/SIMD
        r["roofline"]["counters"] = {
            "mfma_busy_frac": m["busy_frac"], "implied_clock_ghz": m["implied_clock_ghz"],
            "mfma_peak_at_that_clock_tflops": round(peak_at_clock, 1),
            "source": "profiles/" + COUNTERS["kvpr-opt13b"][0]}
        if "vendor_gemm_mfma" in c:
            r["roofline"]["counters"]["vendor_gemm_mfma_busy_frac"] = c["vendor_gemm_mfma"]["busy_frac"]
            r["roofline"]["counters"]["vendor_gemm_implied_clock_ghz"] = c["vendor_gemm_mfma"]["implied_clock_ghz"]
        if "lds" in c:
            r["roofline"]["counters"]["lds_bank_conflict_frac"] = {
                k: v["conflict_frac_of_active"] for k, v in c["lds"].items()}
    r["isolated_call"] = isolated_calls(step, stream, torch, dev, flops, "flops", reps=20)
    # the vendor GEMM on the same product, in the same run: hipBLASLt through
    # torch.matmul, X [b*l, h] times [W_K | W_V] [h, 2h], contiguous, bf16 out
    xm = x.reshape(b * l, h)
    wcat = torch.cat([wk_io, wv_io], dim=1).contiguous()
    vout = torch.empty((b * l, 2 * h), dtype=torch.bfloat16, device=dev)
    for _ in range(args.warmup):
        torch.matmul(xm, wcat, out=vout)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(args.steps):
        torch.matmul(xm, wcat, out=vout)
    e1.record(stream)
    torch.cuda.synchronize()
    vms = e0.elapsed_time(e1) / args.steps
    r["vendor_gemm"] = {"library": "hipBLASLt (torch.matmul), bf16 output, same inputs",
                        "us_per_call": round(vms * 1e3, 2),
                        "tflops": round(flops / (vms * 1e-3) / 1e12, 2)}
    del vout, wcat
    io_ms, io_kern_us, _ = time_steps(step_io, args.steps, args.warmup, stream, K, torch)
    r["w_in_out"] = {"ms_per_step": round(io_ms, 4), "tflops": round(flops / (io_ms * 1e-3) / 1e12, 2),
                     "kernel_us": round(io_kern_us, 2),
                     "kernel_frac_of_mfma_peak": round(flops / (io_kern_us * 1e-6) / 1e12 / 2500.0, 4)}
    # attention over the merged cache [0, s') (dense MHA)
    desc = K.attn_desc(batch=b, num_q_heads=H, num_kv_heads=H, dtype=torch.float16,
                       layout=K.KVDEC_DENSE, max_seqlen=s, softmax_scale=d["scale"])
    ws = K.alloc_workspace(K.kvdec_decode_attn_workspace(desc), device=dev)
    out = torch.empty((b, H, D), dtype=torch.float16, device=dev)
    lse = torch.empty((b, H), dtype=torch.float32, device=dev)

    def attn():
        K.kvdec_decode_attn(desc, q, kc, vc, None, None, None, out, lse, ws, stream=stream)

    ams, akern_us, _ = time_steps(attn, args.steps, args.warmup, stream, K, torch)
    abytes = b * s * H * D * 4 + b * H * D * 4 + b * H * 4
    r["attention"] = {"us_per_call": round(ams * 1e3, 2), "kernel_us": round(akern_us, 2),
                      "bytes": abytes, "tbs": round(abytes / (ams * 1e-3) / 1e12, 4),
                      "kernel_frac_of_hbm_peak": round(abytes / (akern_us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
                      "traffic": measured_traffic("kvpr-opt13b-attention")}
    if not args.no_cpu_baseline:
        import oracle
        rows = np.arange(0, b * l, (b * l) // 16, dtype=np.int32)  # 16 of the b*l rows
        cs = oracle_seconds(lambda: oracle.kv_recompute(d["x"], d["w_k"], d["w_v"], l=l, rows=rows))
        r["cpu_baseline"] = {"value": round(4.0 * rows.size * h * h / cs / 1e12, 6), "unit": "TFLOP/s",
                             "cores": oracle.max_threads(), "cpu_model": cpu_model(), "kind": "oracle",
                             "sample": f"{rows.size} of the {b * l} recomputed rows (both K and V), "
                                       f"median of 3 runs, {cs:.2f} s each"}
    return r


def bench_kvpr_overlap(args, K, np, torch, dev, stream):
    """One OPT-13B layer load with partial recompute: X[0:l] and K/V[l:s') cross
    PCIe from pinned host memory on a copy stream while the GPU recomputes
    K/V[0:l].  v_com (pinned host-to-device rate) and v_gpu (recompute rate)
    are measured here, l comes from kvdec_kvpr_split, and the load is timed at
    that l, at l = 0 (transfer only), at the 256 of the recompute config and at
    l = s' (recompute only)."""
    import kvgen
    b, h, H, D, s = 32, 5120, 40, 128, 1024
    d = kvgen.kvpr_layer(seed=args.seed, b=b, h=h, H=H, s=s, l=s)     # activations of all s' rows
    kv = kvgen.kvpr_layer(seed=args.seed + 1, b=b, h=h, H=H, s=s, l=0)  # a full host cache
    x_host = torch.from_numpy(d["x"].view(np.int16)).pin_memory()
    k_host = torch.from_numpy(kv["k_cache"]).pin_memory()
    v_host = torch.from_numpy(kv["v_cache"]).pin_memory()
    wk = torch.from_numpy(np.ascontiguousarray(d["w_k"].T).view(np.int16)).to(dev).view(torch.bfloat16)
    wv = torch.from_numpy(np.ascontiguousarray(d["w_v"].T).view(np.int16)).to(dev).view(torch.bfloat16)
    kc = torch.empty((b, s, H, D), dtype=torch.float16, device=dev)
    vc = torch.empty_like(kc)
    x_dev = torch.empty((b, s, h), dtype=torch.bfloat16, device=dev)
    copy_stream = torch.cuda.Stream(dev)
    prewarm(torch, dev, args.prewarm_ms)

    def timed(fn, reps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        for _ in range(2):
            fn()
        torch.cuda.synchronize()
        e0.record(stream)
        copy_stream.wait_event(e0)  # both streams start at e0
        for _ in range(reps):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / reps / 1e3  # seconds

    # v_com: the K and V rows of the whole cache from pinned memory, on the copy stream
    kv_bytes = 2 * b * s * h * 2

    def h2d():
        with torch.cuda.stream(copy_stream):
            kc.copy_(k_host.view_as(kc), non_blocking=True)
            vc.copy_(v_host.view_as(vc), non_blocking=True)
        stream.wait_stream(copy_stream)
    v_com = kv_bytes / timed(h2d, 5)
    # v_gpu: the recompute at the recompute config's split point
    x_dev_l = torch.empty((b, 256, h), dtype=torch.bfloat16, device=dev)
    x_dev_l.copy_(torch.from_numpy(d["x"][:, :256].copy().view(np.int16)).view(torch.bfloat16).to(dev))
    v_gpu = 4.0 * b * 256 * h * h / timed(
        lambda: K.kvdec_kv_recompute(x_dev_l, wk, wv, kc, vc, 256, K.KVDEC_W_OUT_IN, stream=stream), 10)
    l_best, t_model = K.kvdec_kvpr_split(b, s, s, h, 2, v_com, v_gpu)

    def load(l):
        def one():
            # layers one after another (the row-wise, latency schedule): this
            # layer's copies wait for the work already queued on the compute
            # stream, which also frees x_dev and the cache for them
            ev = torch.cuda.Event()
            ev.record(stream)
            copy_stream.wait_event(ev)
            K.kvdec_kvpr_load_layer(x_host, x_dev, k_host, v_host, wk, wv, kc, vc, l, s,
                                    K.KVDEC_W_OUT_IN, compute_stream=stream, copy_stream=copy_stream)
        return one
    reps = max(3, min(args.steps, 20))
    rows = {}
    def model(l):  # the section A2 layer time with the measured rates
        return b * l * h * 2 / v_com + max(4.0 * b * l * h * h / v_gpu, 2.0 * b * (s - l) * h * 2 / v_com)
    for l in sorted({0, 256, l_best, s}):
        rows[str(l)] = {"ms": round(timed(load(l), reps) * 1e3, 4), "model_ms": round(model(l) * 1e3, 4)}
    t_best = rows[str(l_best)]["ms"]
    r = common(args, "kvpr-opt13b-overlapped-layer-load",
               "KVPR layer load with partial recompute: ms per layer (X[0:l] + K/V[l:s') over PCIe, "
               "K/V[0:l] recomputed), OPT-13B b=32 s'=1024", "ms", t_best, t_best, "bf16",
               "synthetic (seeded; pinned host activations and K/V, W as nn.Linear stores it)",
               {"batch": b, "hidden": h, "num_heads": H, "head_dim": D, "context": s,
                "split_point": l_best, "w_layout": "out_in (nn.Linear)"}, higher=False)
    r["steps"] = reps
    r["v_com_gbs"] = round(v_com / 1e9, 2)
    r["v_gpu_tflops"] = round(v_gpu / 1e12, 1)
    r["model_ms_at_split"] = round(t_model * 1e3, 4)
    r["by_split_point"] = rows
    r["speedup_vs_transfer_only"] = round(rows["0"]["ms"] / t_best, 3)
    r["roofline"] = {"bound": "pcie", "kernel": "kvdec_kvpr_load_layer (copies + kv_recompute_kernel_wide)",
                     "achieved": round((b * l_best * h * 2 + 2 * b * (s - l_best) * h * 2) / (t_best * 1e-3) / 1e9, 2),
                     "peak": round(v_com / 1e9, 2), "unit": "GB/s", "frac": None, "traffic": None,
                     "note": "bytes that crossed PCIe per ms of layer load, against the measured "
                             "pinned host-to-device rate; the model time at the split is model_ms_at_split"}
    r["roofline"]["frac"] = round(r["roofline"]["achieved"] / r["roofline"]["peak"], 4)
    return r


def calibrate_copy(torch, dev):
    """Three 1 GiB device-to-device copies: what HBM counters read for a
    copy of known size, in the same process as the kernels they scale."""
    src = torch.ones(1 << 29, dtype=torch.float16, device=dev)  # 1 GiB
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    return src.numel() * src.element_size()


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--workload", choices=WORKLOADS, default=WORKLOADS[0])
    ap.add_argument("--split-tokens", type=int, default=0)
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="also run a 1 GiB device copy (counter calibration under rocprofv3)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-stream-read", action="store_true",
                    help="skip the streaming-read reference (HBM read rate of one kernel on this box)")
    ap.add_argument("--prewarm-ms", type=float, default=200.0,
                    help="device copies before the warmup steps, to bring the unlocked clocks up")
    ap.add_argument("--summarize-pmc", metavar="DIR",
                    help="write the workload's counter summaries into profiles/ from the rocprofv3 "
                         "counter runs in DIR/<group>/ (no GPU needed)")
    ap.add_argument("--summarize-trace", metavar="DIR",
                    help="write the workload's kernel-trace summary into profiles/ from the rocprofv3 "
                         "run in DIR/TRACE (no GPU needed)")
    args = ap.parse_args()
    if args.summarize_pmc or args.summarize_trace:
        if args.summarize_pmc:
            summarize_pmc(args.workload, args.summarize_pmc)
        if args.summarize_trace:
            summarize_trace(args.workload, args.summarize_trace)
        return

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py: this build runs on one GPU only (no multi-GPU path); use --gpus 1",
              file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import long_kv_caches_amd as K

    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream(dev)
    if args.workload == "llama3-8b-32k":
        r = bench_llama3(args, K, np, torch, dev, stream)
    elif args.workload == "clo-gather-llama3-8b-128k":
        r = bench_gather(args, K, np, torch, dev, stream)
    elif args.workload == "llama3-8b-32k-fp8":
        r = bench_llama3(args, K, np, torch, dev, stream, fp8=True)
    elif args.workload == "llama2-7b-paged":
        r = bench_paged(args, K, np, torch, dev, stream)
    elif args.workload.startswith("clo-"):
        r = bench_clo(args, K, np, torch, dev, stream, args.workload[4:-5])
    elif args.workload == "kvpr-overlap":
        r = bench_kvpr_overlap(args, K, np, torch, dev, stream)
    else:
        r = bench_kvpr(args, K, np, torch, dev, stream)
    if args.calibrate_copy:
        r["calibration_copy_bytes"] = calibrate_copy(torch, dev)
    if r["roofline"]["bound"] == "hbm" and not args.no_stream_read:
        ref = stream_read_reference(K, torch, dev, stream)
        r["stream_read"] = ref
        r["roofline"]["frac_of_stream_read"] = round(r["roofline"]["achieved"] / (ref["tbs"] * 1e3), 4)
    print(json.dumps(r), flush=True)


if __name__ == "__main__":
    main()

"""A seeded sweep of decode-attention configurations against the fp64 oracle.

Each case draws, from its own seed: the layout (dense with lengths, ragged,
paged with 16- or 32-token pages), the K/V format (fp16, bf16, or e4m3 codes
with fp16 or bf16 queries), the number of KV heads (1, 2, 4, 8) and query
heads per KV head (1 to 8, so both the vector and the matrix-core tile paths),
the batch (1 to 6 sequences) and each sequence's length (empty, one token,
tile edges, or up to 2500 tokens), and the schedule (the persistent default
or fixed chunks of 64 to 320 tokens).  The case is printed before it runs.
A second sweep draws batches large enough for a full persistent grid, where
the columns are placed by XCD (1, 8 or 32 KV heads, fp16 or bf16).  The
tolerances are those of every other parity test (tests/gpu_util.py).
"""
import numpy as np
import pytest

import kvgen
import oracle
from gpu_util import check_close, check_lse, decode_on_gpu, host_f64, say, to_bf16_bits
from test_gpu_decode import ORC_LAYOUT

pytestmark = pytest.mark.gpu

N_CASES = 80
EDGE_LENGTHS = [0, 1, 15, 16, 17, 63, 64, 65]


def draw_case(i):
    rng = np.random.default_rng(20_000 + i)
    layout = str(rng.choice(["dense", "ragged", "paged"]))
    fmt = str(rng.choice(["f16", "bf16", "e4m3", "e4m3-bf16"]))
    hkv = int(rng.choice([1, 2, 4, 8]))
    g = int(rng.integers(1, 9))
    b = int(rng.integers(1, 7))
    lens = rng.integers(1, 2501, size=b)
    for j in range(b):  # about a third of the sequences take an edge length
        if rng.random() < 0.35:
            lens[j] = int(rng.choice(EDGE_LENGTHS))
    if lens.max() == 0:
        lens[0] = int(rng.integers(1, 200))
    split = int(rng.choice([0, 0, 0, 64, 128, 320]))
    page = int(rng.choice([16, 32]))
    return dict(layout=layout, fmt=fmt, hkv=hkv, g=g, lens=[int(x) for x in lens], split=split,
                page=page, seed=30_000 + i)


def build(c):
    d = kvgen.ragged_llama(seed=c["seed"], lens=c["lens"], Hq=c["g"] * c["hkv"], Hkv=c["hkv"])
    if c["layout"] == "dense":
        d = kvgen.ragged_to_dense(d)
    elif c["layout"] == "paged":
        d = kvgen.ragged_to_paged(d, seed=c["seed"] + 1, page=c["page"])
    if c["fmt"].startswith("e4m3"):
        d = kvgen.fp8_kv(d)
    return d


def reference(d, bf16):
    conv = to_bf16_bits if bf16 else (lambda x: x)
    fp8 = d["k"].dtype == np.uint8
    kv = (lambda x: x) if fp8 else conv
    extra = dict(k_scale=d["k_scale"], v_scale=d["v_scale"]) if fp8 else {}
    return oracle.decode_attn(conv(d["q"]), kv(d["k"]), kv(d["v"]), num_kv_heads=d["Hkv"],
                              layout=ORC_LAYOUT[d["layout"]], scale=d["scale"],
                              kind=oracle.BF16 if bf16 else oracle.F16, seqlens=d.get("seqlens"),
                              cu_seqlens=d.get("cu_seqlens"), block_table=d.get("block_table"),
                              **extra)


@pytest.mark.parametrize("i", range(N_CASES))
def test_decode_sweep(i):
    c = draw_case(i)
    say(f"[sweep {i}] {c}")
    d = build(c)
    bf16 = c["fmt"] in ("bf16", "e4m3-bf16")
    out, lse = decode_on_gpu(d, split_tokens=c["split"], bf16=bf16)
    ref_o, ref_l = reference(d, bf16)
    check_close(host_f64(out), ref_o, f"sweep {i}", bf16_out=bf16)
    check_lse(lse, ref_l, f"sweep {i} lse")


# ---------------------------------------------------------------------------
# CLO hybrid attention: persistent slots and cache-buffer heads
# ---------------------------------------------------------------------------

N_HYBRID = 40


def draw_hybrid(i):
    rng = np.random.default_rng(40_000 + i)
    fmt = str(rng.choice(["f16", "bf16", "e4m3"]))
    hkv = int(rng.choice([2, 4, 8]))
    g = int(rng.integers(1, 9))
    b = int(rng.integers(1, 6))
    slots = int(rng.integers(1 if fmt == "e4m3" else 0, min(3, hkv) + 1))
    pers_cap = int(rng.integers(1, 3001)) if slots else 0
    buf_cap = int(rng.integers(1, 1501))
    head_map = np.full(hkv, -1, np.int32)
    if slots:
        head_map[rng.choice(hkv, size=slots, replace=False)] = np.arange(slots, dtype=np.int32)
    pick = lambda cap, n: [int(x) if rng.random() > 0.3 else int(rng.choice([0, 1, 16, 17, cap]))
                           for x in rng.integers(0, cap + 1, size=n)]
    pers_len = [min(x, pers_cap) for x in pick(pers_cap, b)] if slots else [0] * b
    buf_len = [min(x, buf_cap) for x in pick(buf_cap, b * hkv)]
    split = int(rng.choice([0, 0, 64, 128]))
    return dict(fmt=fmt, hkv=hkv, g=g, b=b, slots=slots, pers_cap=pers_cap, buf_cap=buf_cap,
                head_map=head_map.tolist(), pers_len=pers_len, buf_len=buf_len, split=split,
                seed=50_000 + i)


def build_hybrid(c):
    dr = kvgen.Draws(c["seed"])
    b, hkv = c["b"], c["hkv"]
    d = dict(B=b, Hq=c["g"] * hkv, Hkv=hkv, D=128, scale=1.0 / np.sqrt(128.0),
             q=dr.normal((b, c["g"] * hkv, 128)),
             pers_k=dr.normal((b, c["slots"], c["pers_cap"], 128)),
             pers_v=dr.normal((b, c["slots"], c["pers_cap"], 128)),
             buf_k=dr.normal((b, hkv, c["buf_cap"], 128)),
             buf_v=dr.normal((b, hkv, c["buf_cap"], 128)),
             pers_len=np.asarray(c["pers_len"], np.int32), buf_len=np.asarray(c["buf_len"], np.int32),
             head_map=np.asarray(c["head_map"], np.int32))
    return kvgen.fp8_hybrid(d) if c["fmt"] == "e4m3" else d


@pytest.mark.parametrize("i", range(N_HYBRID))
def test_hybrid_sweep(i):
    from test_gpu_hybrid import hybrid_on_gpu, hybrid_oracle
    c = draw_hybrid(i)
    say(f"[hybrid sweep {i}] { {k: v for k, v in c.items() if k not in ('pers_len', 'buf_len')} }")
    d = build_hybrid(c)
    bf16 = c["fmt"] == "bf16"
    out, lse = hybrid_on_gpu(d, c["split"], bf16=bf16)
    ro, rl = hybrid_oracle(d, bf16=bf16)
    check_close(host_f64(out), ro, f"hybrid sweep {i}", bf16_out=bf16)
    check_lse(lse, rl, f"hybrid sweep {i} lse")


# ---------------------------------------------------------------------------
# Index-gather attention over a dense cache
# ---------------------------------------------------------------------------

N_GATHER = 24


@pytest.mark.parametrize("i", range(N_GATHER))
def test_gather_sweep(i):
    from test_gpu_gather import gather_on_gpu
    rng = np.random.default_rng(60_000 + i)
    hkv = int(rng.choice([1, 2, 4, 8]))
    g = int(rng.integers(1, 9))
    b = int(rng.integers(1, 6))
    s = int(rng.integers(17, 4001))
    lens = [int(x) if rng.random() > 0.25 else int(rng.choice([0, 1, s])) for x in
            rng.integers(1, s + 1, size=b)]
    top_k = int(rng.integers(1, min(s, 600) + 1))
    split = int(rng.choice([0, 0, 64, 128]))
    bf16 = bool(rng.random() < 0.3)
    say(f"[gather sweep {i}] hkv={hkv} g={g} lens={lens} S={s} top_k={top_k} split={split} "
        f"bf16={bf16}")
    d = kvgen.dense_small(seed=70_000 + i, B=b, Hq=g * hkv, Hkv=hkv, S=s)
    idx, n = kvgen.random_indices(80_000 + i, b, hkv, lens, top_k)
    conv = to_bf16_bits if bf16 else (lambda x: x)
    go, gl = gather_on_gpu(d, idx, n, split=split, bf16=bf16)
    ro, rl = oracle.gather_attn(conv(d["q"]), conv(d["k"]), conv(d["v"]), idx, n, num_kv_heads=hkv,
                                scale=d["scale"], kind=oracle.BF16 if bf16 else oracle.F16)
    check_close(go, ro, f"gather sweep {i}", bf16_out=bf16)
    check_lse(gl, rl, f"gather sweep {i} lse")


# ---------------------------------------------------------------------------
# Grids of one or two workgroups per CU whose columns are placed by XCD
# ---------------------------------------------------------------------------

N_XCD = 24


def draw_xcd_case(i):
    """Batches with enough tiles that the default plan fills a full grid
    (est. tiles >= 32 per persistent workgroup): 1, 8 or 32 KV heads (a column
    of one wave, two or eight workgroups), fp16 or bf16, any layout."""
    rng = np.random.default_rng(90_000 + i)
    hkv = int(rng.choice([1, 8, 32]))
    g = int(rng.integers(1, 9 if hkv < 32 else 3))
    bf16 = bool(rng.random() < 0.3)
    b = int(rng.integers(2, 6))
    need = (16384 if bf16 else 8192) * 16 // (b * hkv)  # tokens of the longest sequence
    top = int(need + rng.integers(0, need // 4 + 1))
    lens = [top] + [int(x) if rng.random() > 0.3 else int(rng.choice([0, 1, 17, top]))
                    for x in rng.integers(0, top + 1, size=b - 1)]
    layout = str(rng.choice(["ragged", "dense", "paged"]))
    return dict(hkv=hkv, g=g, bf16=bf16, lens=lens, layout=layout, seed=91_000 + i)


@pytest.mark.parametrize("i", range(N_XCD))
def test_xcd_columns_sweep(i):
    c = draw_xcd_case(i)
    say(f"[xcd sweep {i}] {c}")
    d = kvgen.ragged_llama(seed=c["seed"], lens=c["lens"], Hq=c["g"] * c["hkv"], Hkv=c["hkv"])
    if c["layout"] == "dense":
        d = kvgen.ragged_to_dense(d)
    elif c["layout"] == "paged":
        d = kvgen.ragged_to_paged(d, seed=c["seed"] + 1)
    out, lse = decode_on_gpu(d, split_tokens=0, bf16=c["bf16"])
    ref_o, ref_l = reference(d, c["bf16"])
    check_close(host_f64(out), ref_o, f"xcd sweep {i}", bf16_out=c["bf16"])
    check_lse(lse, ref_l, f"xcd sweep {i} lse")

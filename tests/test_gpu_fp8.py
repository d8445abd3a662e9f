"""GPU parity of decode attention over e4m3 K/V (kv_format = KVDEC_KV_E4M3)
against the fp64 oracle on the same codes and scales.

The oracle decodes the codes exactly, so the tolerances are those of the
16-bit path (fp32 accumulation, one rounding of the output; the matrix-core
path used from three query heads per KV head on also rounds each softmax
weight to fp16 once, about 2^-11 relative, well inside them).  A single key
returns v_scale * V exactly, which checks the kernel's decoding of every code.
"""
import numpy as np
import pytest
import torch

import kvgen
import oracle
from gpu_util import check_close, check_lse, decode_on_gpu, host_f64, say, to_bf16_bits
from test_gpu_decode import ORC_LAYOUT
from test_gpu_hybrid import hybrid_on_gpu, hybrid_oracle

pytestmark = pytest.mark.gpu


def oracle_fp8(d, bf16=False):
    conv = to_bf16_bits if bf16 else (lambda x: x)
    return oracle.decode_attn(conv(d["q"]), d["k"], d["v"], num_kv_heads=d["Hkv"],
                              layout=ORC_LAYOUT[d["layout"]], scale=d["scale"],
                              kind=oracle.BF16 if bf16 else oracle.F16, seqlens=d.get("seqlens"),
                              cu_seqlens=d.get("cu_seqlens"), block_table=d.get("block_table"),
                              k_scale=d["k_scale"], v_scale=d["v_scale"])


def _parity(d, what, split_tokens=0, bf16=False):
    say(f"[fp8] {what} split={split_tokens} bf16={bf16}")
    out, lse = decode_on_gpu(d, split_tokens=split_tokens, bf16=bf16)
    ref_o, ref_l = oracle_fp8(d, bf16)
    check_close(host_f64(out), ref_o, what, bf16_out=bf16)
    check_lse(lse, ref_l, what + " lse")


@pytest.mark.parametrize("bf16", [False, True])
def test_single_key_decodes_every_code_exactly(bf16):
    # one token per sequence: out = v_scale * V for every query head; V holds
    # every non-NaN code, and v_scale = 2^-4 keeps every product exact
    d = kvgen.dense_small(seed=40, B=1, Hq=8, Hkv=2, S=1)
    codes = np.arange(256, dtype=np.uint8)
    codes[(codes & 0x7F) == 0x7F] = 0
    d = dict(d, k=np.full((1, 1, 2, 128), 0x38, np.uint8), v=codes.reshape(1, 1, 2, 128),
             k_scale=1.0, v_scale=2.0 ** -4)
    say(f"[fp8] single key, all codes, bf16={bf16}")
    out, _ = decode_on_gpu(d, bf16=bf16)
    exact = oracle.widen_e4m3(codes).reshape(2, 128) * 2.0 ** -4
    got = host_f64(out)
    # every value exactly (the sum starts at +0, so code 0x80 gives +0, not -0)
    for j in range(8):
        assert np.array_equal(got[0, j], exact[j // 4]), j


@pytest.mark.parametrize("split", [0, 64])
@pytest.mark.parametrize("bf16", [False, True])
def test_dense_small(split, bf16):
    d = kvgen.fp8_kv(kvgen.dense_small(seed=41))
    _parity(d, "dense 1x8/2x1024", split_tokens=split, bf16=bf16)


@pytest.mark.parametrize("split", [0, 128])
def test_ragged_tiles_tails_and_empty(split):
    lens = [0, 1, 15, 16, 17, 63, 64, 65, 127, 700, 1000, 0, 3001, 64 * 37 + 5]
    d = kvgen.fp8_kv(kvgen.ragged_llama(seed=42, lens=lens, Hq=32, Hkv=8))
    _parity(d, "ragged tails", split_tokens=split)


@pytest.mark.parametrize("hq,hkv", [(8, 8), (16, 8), (24, 8), (40, 8), (64, 8)])
def test_group_sizes(hq, hkv):
    d = kvgen.fp8_kv(kvgen.ragged_llama(seed=43, lens=[300, 2000, 45], Hq=hq, Hkv=hkv))
    _parity(d, f"G={hq // hkv}")


def test_paged():
    d = kvgen.fp8_kv(kvgen.ragged_to_paged(kvgen.ragged_llama(seed=44, lens=[31, 500, 33, 2900],
                                                              Hq=8, Hkv=8), seed=45, page=32))
    _parity(d, "paged page_size=32")
    _parity(d, "paged page_size=32", split_tokens=128)


def test_headline_shape_sampled():
    """Llama3-8B 32K ragged batch at full size, e4m3 K/V, default plan as the
    bench runs it; four sequences checked against the oracle."""
    d = kvgen.fp8_kv(kvgen.ragged_llama(seed=0))
    say(f"[fp8] Llama3-8B full size, k_scale={d['k_scale']:.4g} v_scale={d['v_scale']:.4g}")
    out, lse = decode_on_gpu(d)
    cu = d["cu_seqlens"]
    for b in (0, 5, 11, 15):
        sub = dict(d, B=1, q=d["q"][b:b + 1], k=d["k"][cu[b]:cu[b + 1]], v=d["v"][cu[b]:cu[b + 1]],
                   cu_seqlens=np.array([0, cu[b + 1] - cu[b]], np.int32))
        ref_o, ref_l = oracle_fp8(sub)
        check_close(host_f64(out)[b:b + 1], ref_o, f"full size, sequence {b}")
        check_lse(lse[b:b + 1], ref_l, f"full size lse, sequence {b}")


@pytest.mark.parametrize("split", [0, 128])
def test_hybrid(split):
    d = kvgen.fp8_hybrid(kvgen.clo_hybrid(seed=46, B=3, S=3000, frac=0.3))
    d["pers_len"] = np.array([3000, 17, 0], np.int32)
    say(f"[fp8] hybrid split={split}")
    out, lse = hybrid_on_gpu(d, split_tokens=split)
    ref_o, ref_l = hybrid_oracle(d)
    check_close(host_f64(out), ref_o, "hybrid e4m3")
    check_lse(lse, ref_l, "hybrid e4m3 lse")

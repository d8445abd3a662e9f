"""GPU parity of kvdec_decode_attn (dense, ragged, paged) against the fp64 oracle.

Every case is seeded; shapes span several 16-token tiles, several 64-token
waves of a work item, several work items per sequence and ragged tails.
"""
import numpy as np
import pytest
import torch

import kvgen
import oracle
from gpu_util import (bits, check_close, check_lse, decode_on_gpu, dev, host_f64, say,
                      to_bf16_bits)

pytestmark = pytest.mark.gpu

ORC_LAYOUT = {"dense": oracle.DENSE, "ragged": oracle.RAGGED, "paged": oracle.PAGED}


def oracle_ref(d, bf16=False):
    conv = to_bf16_bits if bf16 else (lambda x: x)
    return oracle.decode_attn(conv(d["q"]), conv(d["k"]), conv(d["v"]), num_kv_heads=d["Hkv"],
                              layout=ORC_LAYOUT[d["layout"]], scale=d["scale"],
                              kind=oracle.BF16 if bf16 else oracle.F16,
                              seqlens=d.get("seqlens"), cu_seqlens=d.get("cu_seqlens"),
                              block_table=d.get("block_table"))


def _parity(d, what, split_tokens=0, bf16=False):
    say(f"[decode] {what} split={split_tokens} bf16={bf16}")
    out, lse = decode_on_gpu(d, split_tokens=split_tokens, bf16=bf16)
    ref_o, ref_l = oracle_ref(d, bf16)
    check_close(host_f64(out), ref_o, what, bf16_out=bf16)
    check_lse(lse, ref_l, what + " lse")
    return out


def test_dense_small_config():
    d = kvgen.dense_small(seed=0)
    _parity(d, "dense 1x8/2x1024")
    _parity(d, "dense 1x8/2x1024", split_tokens=64)


@pytest.mark.parametrize("hq", [8, 16])  # G = 4 (VALU tile path), G = 8 (matrix-core tile path)
def test_single_key_returns_v_bit_exact(hq):
    G = hq // 2
    for layout in ("dense", "ragged"):
        d = kvgen.dense_small(seed=1, B=3, Hq=hq, Hkv=2, S=1)
        if layout == "ragged":
            d = dict(d, layout="ragged", k=d["k"].reshape(3, 2, 128), v=d["v"].reshape(3, 2, 128),
                     cu_seqlens=np.arange(4, dtype=np.int32), seqlens=np.ones(3, np.int32))
        say(f"[decode] single key {layout} G={G}")
        out, lse = decode_on_gpu(d)
        got = bits(out)
        v = d["v"].reshape(3, 2, 128).view(np.uint16)
        for j in range(hq):
            assert np.array_equal(got[:, j], v[:, j // G]), (layout, j)


@pytest.mark.parametrize("split", [0, 64, 128, 512])
def test_ragged_tiles_and_tails(split):
    lens = [1, 15, 16, 17, 63, 64, 65, 127, 700, 1000, 3001, 64 * 37 + 5]
    d = kvgen.ragged_llama(seed=2, lens=lens, Hq=32, Hkv=8)
    _parity(d, f"ragged lens={lens}", split_tokens=split)


@pytest.mark.parametrize("split", [0, 256])
def test_deterministic_repeats(split):
    d = kvgen.ragged_llama(seed=3, lens=[5000, 333, 4097], Hq=32, Hkv=8)
    say(f"[decode] determinism x3 split={split}")
    outs, _ = decode_on_gpu(d, split_tokens=split, repeat=3)
    b0 = bits(outs[0])
    for o in outs[1:]:
        assert np.array_equal(bits(o), b0)


@pytest.mark.parametrize("split", [0, 64])
def test_empty_sequences(split):
    d = kvgen.ragged_llama(seed=4, lens=[0, 5, 0, 300, 0], Hq=8, Hkv=2)
    out = _parity(d, "ragged with empty sequences", split_tokens=split)
    got = host_f64(out)
    assert np.all(got[[0, 2, 4]] == 0.0)


@pytest.mark.parametrize("split", [0, 256])
@pytest.mark.parametrize("hq,hkv", [(8, 8), (8, 4), (12, 4), (40, 8), (48, 8), (56, 8), (64, 8), (8, 1), (3, 1)])
def test_group_sizes(hq, hkv, split):
    d = kvgen.ragged_llama(seed=5, lens=[1, 77, 1500, 2049], Hq=hq, Hkv=hkv)
    _parity(d, f"G={hq // hkv}", split_tokens=split)


@pytest.mark.parametrize("split", [0, 128])
def test_dense_with_seqlens(split):
    d = kvgen.dense_small(seed=6, B=4, Hq=16, Hkv=4, S=2000, seqlens=[2000, 1, 999, 0])
    _parity(d, "dense with seqlens", split_tokens=split)


@pytest.mark.parametrize("split", [0, 256])
def test_bf16(split):
    d = kvgen.ragged_llama(seed=7, lens=[100, 2000, 4321], Hq=32, Hkv=8)
    _parity(d, "ragged bf16", split_tokens=split, bf16=True)


@pytest.mark.parametrize("split", [0, 256])
@pytest.mark.parametrize("hq", [24, 64])  # G = 3 and 8: the matrix-core tile path, P split hi + lo
def test_bf16_matrix_core_groups(hq, split):
    """bf16 K/V with G >= 3 take the matrix-core tile path with each softmax
    weight split into two bf16 parts; sequences of 1-5 tokens are where a
    single bf16 rounding of the weights would show."""
    d = kvgen.ragged_llama(seed=16, lens=[1, 2, 5, 300, 2049], Hq=hq, Hkv=8)
    _parity(d, f"ragged bf16 G={hq // 8}", split_tokens=split, bf16=True)


@pytest.mark.parametrize("lens", [[1], [17, 0, 3], [0, 0], [16] * 40])
def test_tiny_lines_default_plan(lens):
    """Fewer line tiles than persistent waves (columns capped at the line length,
    equal weights below two tiles per column) and all-empty batches."""
    d = kvgen.ragged_llama(seed=13, lens=lens, Hq=32, Hkv=8)
    out = _parity(d, f"tiny ragged lens={lens[:4]}{'...' if len(lens) > 4 else ''}", split_tokens=0)
    empty = [i for i, n in enumerate(lens) if n == 0]
    assert np.all(host_f64(out)[empty] == 0.0)


def test_paged_bitwise_equals_ragged():
    d = kvgen.ragged_llama(seed=8, lens=[16, 17, 1000, 2047, 5000], Hq=32, Hkv=8)
    p = kvgen.ragged_to_paged(d, seed=9)
    say("[decode] paged vs ragged bitwise")
    for split in (0, 64, 512):
        out_r, lse_r = decode_on_gpu(d, split_tokens=split)
        out_p, lse_p = decode_on_gpu(p, split_tokens=split)
        assert np.array_equal(bits(out_r), bits(out_p))
        assert np.array_equal(lse_r.view(np.uint32), lse_p.view(np.uint32))
    _parity(p, "paged (from ragged)", split_tokens=512)


def test_paged_mha_reduced_batch():
    d = kvgen.paged_mha(seed=10, B=96)
    _parity(d, "paged Llama-2-7B MHA, B=96")
    _parity(d, "paged Llama-2-7B MHA, B=96", split_tokens=256)  # 3072 heads: 8-row merge


def test_ragged_mha_columns_on_one_xcd():
    # 32 KV heads with enough tiles for a full one-workgroup-per-CU grid: each
    # column's eight workgroups run on one XCD, with odd XCDs' columns weighted
    d = kvgen.ragged_llama(seed=18, lens=[1000, 1777, 64, 2049, 900, 1, 1500, 1311], Hq=32, Hkv=32)
    _parity(d, "ragged MHA 8 sequences x 32 heads")


@pytest.mark.parametrize("hq", [8, 32, 64])  # G = 1, 4 (vector path) and 8 (matrix cores)
def test_ragged_gqa_columns_on_one_xcd(hq):
    # 8 KV heads with enough tiles for a full one-workgroup-per-CU grid: each
    # column's two workgroups run on one XCD, with odd XCDs' columns weighted
    d = kvgen.ragged_llama(seed=25, lens=[4100, 3000, 17, 2222], Hq=hq, Hkv=8)
    _parity(d, f"ragged 4 sequences x {hq}/8 heads")


@pytest.mark.parametrize("hq", [8, 32])
def test_bf16_columns_on_one_xcd_two_workgroups_per_cu(hq):
    # bf16 K/V with enough tiles for two workgroups per CU: XCD-local columns
    # with the first-round and odd-XCD weights together
    d = kvgen.ragged_llama(seed=27, lens=[8200, 5000, 17, 3000], Hq=hq, Hkv=8)
    _parity(d, f"ragged bf16 4 sequences x {hq}/8 heads", bf16=True)


@pytest.mark.parametrize("layout", ["ragged", "dense"])
def test_one_kv_head_columns_on_one_xcd(layout):
    # one KV head (a column per wave) with enough tiles for a full
    # one-workgroup-per-CU grid: wave i of block 8t + x runs column
    # 8 (4t + i) + x, with odd XCDs' columns weighted
    d = kvgen.ragged_llama(seed=26, lens=[32768, 20000, 1, 31000], Hq=4, Hkv=1)
    if layout == "dense":
        d = kvgen.ragged_to_dense(d)
    _parity(d, f"{layout} 4 sequences x 4/1 heads, up to 32K")


@pytest.mark.parametrize("hq,hkv,layout,bf16", [
    (40, 40, "dense", False),   # OPT-13B's 40 heads: 25 columns of 40 on 1024 waves
    (40, 40, "paged", False),
    (40, 40, "ragged", True),
    (24, 12, "ragged", False),
    (10, 5, "dense", False),
    (9, 3, "paged", False),     # G = 3, matrix-core tiles
])
def test_kv_heads_not_dividing_the_waves(hq, hkv, layout, bf16):
    # Hkv does not divide the persistent waves: W % Hkv of them run no column
    d = kvgen.ragged_llama(seed=22, lens=[700, 1, 0, 1333, 65, 2100], Hq=hq, Hkv=hkv)
    if layout == "dense":
        d = kvgen.ragged_to_dense(d)
    elif layout == "paged":
        d = kvgen.ragged_to_paged(d, seed=23)
    _parity(d, f"{layout} {hq}/{hkv} heads, 6 sequences", bf16=bf16)


def test_many_short_sequences_of_40_heads():
    rng = np.random.default_rng(24)
    lens = rng.integers(0, 40, size=1000).tolist()
    d = kvgen.ragged_llama(seed=24, lens=lens, Hq=40, Hkv=40)
    _parity(d, "ragged B=1000 x 40 heads, short sequences")


def test_merge_of_many_short_heads():
    # 260 x 32 = 8320 query heads: the merge folds 4 rows of partials per head
    d = kvgen.dense_small(seed=17, B=260, Hq=32, Hkv=16, S=256)
    _parity(d, "dense 260x32/16x256", split_tokens=64)
    _parity(d, "dense 260x32/16x256")


def test_page_size_32():
    d = kvgen.ragged_llama(seed=11, lens=[31, 32, 33, 900], Hq=8, Hkv=8)
    p = kvgen.ragged_to_paged(d, seed=12, page=32)
    _parity(p, "paged page_size=32", split_tokens=128)


@pytest.mark.parametrize("bf16", [False, True])
@pytest.mark.parametrize("split", [0, 128])
def test_paged_matrix_core_group(split, bf16):
    """16-bit K/V with G = 8 take the matrix-core tile path; the paged source
    addresses its tiles in bytes of the 16-bit elements."""
    d = kvgen.ragged_llama(seed=14, lens=[33, 700, 16, 2100], Hq=64, Hkv=8)
    p = kvgen.ragged_to_paged(d, seed=15, page=32)
    _parity(p, "paged G=8 page_size=32", split_tokens=split, bf16=bf16)


def test_headline_full_size():
    """Llama3-8B 32K ragged batch at full size, default plan (as the bench runs it)."""
    d = kvgen.ragged_llama(seed=0)
    _parity(d, "Llama3-8B ragged B=16 16K-32K (full)")


def test_paged_llama2_full_size_sampled():
    """Llama-2-7B paged MHA at full size (B = 1024, ~1.4M tokens, 24 GB of K/V),
    default plan as the bench runs it; 24 sequences checked against the oracle:
    the shortest, the longest and 22 drawn at random (seeded)."""
    d = kvgen.paged_mha(seed=0)
    lens = d["seqlens"]
    rng = np.random.default_rng(1234)
    pick = np.unique(np.concatenate([[int(np.argmin(lens)), int(np.argmax(lens))],
                                     rng.choice(d["B"], 22, replace=False)]))
    say(f"[decode] paged Llama-2-7B full size, B={d['B']}, tokens={int(lens.sum())}, "
        f"checking {pick.size} sequences")
    out, lse = decode_on_gpu(d)
    ref_o, ref_l = oracle.decode_attn(d["q"][pick], d["k"], d["v"], num_kv_heads=d["Hkv"],
                                      layout=oracle.PAGED, scale=d["scale"],
                                      seqlens=lens[pick], block_table=d["block_table"][pick])
    check_close(host_f64(out)[pick], ref_o, "paged full size (sampled sequences)")
    check_lse(lse[pick], ref_l, "paged full size lse (sampled)")


def test_many_sequences_fall_back_to_chunks():
    """More sequences than the balanced schedule keeps in LDS (4096): the
    default plan falls back to fixed chunks."""
    rng = np.random.default_rng(21)
    lens = rng.integers(0, 80, size=5000).tolist()
    d = kvgen.ragged_llama(seed=21, lens=lens, Hq=8, Hkv=2)
    _parity(d, "ragged B=5000 short sequences (default plan)", split_tokens=0)

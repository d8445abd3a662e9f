"""GPU parity of kvdec_kv_recompute (KVPR partial recompute, MFMA GEMM) and of
attention over the merged cache [0, s')."""
import numpy as np
import pytest
import torch

import kvgen
import long_kv_caches_amd as K
import oracle
from gpu_util import bits, check_close, decode_on_gpu, dev, host_f64, say

pytestmark = pytest.mark.gpu


LAYOUTS = [K.KVDEC_W_IN_OUT, K.KVDEC_W_OUT_IN]


def recompute_on_gpu(d, w_layout=K.KVDEC_W_IN_OUT):
    """The generated W is [in, out]; the [out, in] layout gets its transpose
    (the same matrix stored the other way, as nn.Linear stores it)."""
    conv = (lambda w: np.ascontiguousarray(w.T)) if w_layout == K.KVDEC_W_OUT_IN else (lambda w: w)
    x = dev(d["x"], bf16=True)
    wk = dev(conv(d["w_k"]), bf16=True)
    wv = dev(conv(d["w_v"]), bf16=True)
    kc = dev(d["k_cache"])
    vc = dev(d["v_cache"])
    K.kvdec_kv_recompute(x, wk, wv, kc, vc, d["l"], w_layout)
    torch.cuda.synchronize()
    return kc, vc


def _check_rows(d, kc, vc, rows=None):
    b, l, h = d["b"], d["l"], d["h"]
    ko, vo = oracle.kv_recompute(d["x"], d["w_k"], d["w_v"], l=l, rows=rows)
    kg = host_f64(kc).reshape(b, -1, h)[:, :l].reshape(b * l, h)
    vg = host_f64(vc).reshape(b, -1, h)[:, :l].reshape(b * l, h)
    if rows is not None:
        kg, vg = kg[rows], vg[rows]
    check_close(kg, ko, "K rows")
    check_close(vg, vo, "V rows")
    # rows [l, s') untouched, bit for bit
    s = d["k_cache"].shape[1]
    assert np.array_equal(bits(kc)[:, l:], d["k_cache"][:, l:].view(np.uint16))
    assert np.array_equal(bits(vc)[:, l:], d["v_cache"][:, l:].view(np.uint16))


@pytest.mark.parametrize("w_layout", LAYOUTS)
@pytest.mark.parametrize("b,l,h,H", [(3, 17, 256, 2), (2, 150, 512, 4), (1, 1, 256, 2),
                                     (4, 128, 1024, 8)])
def test_small_shapes(b, l, h, H, w_layout):
    d = kvgen.kvpr_layer(seed=1, b=b, h=h, H=H, s=l + 40, l=l)
    say(f"[recompute] b={b} l={l} h={h} w_layout={w_layout}")
    kc, vc = recompute_on_gpu(d, w_layout)
    _check_rows(d, kc, vc)


@pytest.mark.parametrize("w_layout", LAYOUTS)
def test_unit_vector_rows_bit_exact(w_layout):
    rng = np.random.default_rng(2)
    d = kvgen.kvpr_layer(seed=2, b=2, h=512, H=4, s=40, l=33)
    idx = rng.integers(0, 512, size=(2, 33))
    x = np.zeros((2, 33, 512), np.float32)
    for i in range(2):
        for t in range(33):
            x[i, t, idx[i, t]] = 1.0
    d["x"] = kvgen.f32_to_bf16_bits(x)
    say(f"[recompute] unit-vector rows w_layout={w_layout}")
    kc, vc = recompute_on_gpu(d, w_layout)
    kg = bits(kc).reshape(2, 40, 512)
    vg = bits(vc).reshape(2, 40, 512)
    wk16 = kvgen.bf16_bits_to_f32(d["w_k"]).astype(np.float16).view(np.uint16)
    wv16 = kvgen.bf16_bits_to_f32(d["w_v"]).astype(np.float16).view(np.uint16)
    for i in range(2):
        for t in range(33):
            assert np.array_equal(kg[i, t], wk16[idx[i, t]])
            assert np.array_equal(vg[i, t], wv16[idx[i, t]])


@pytest.mark.parametrize("w_layout", LAYOUTS)
def test_opt13b_full_size_sampled_rows_then_attention(w_layout):
    d = kvgen.kvpr_layer(seed=0)
    say(f"[recompute] OPT-13B b=32 l=256 h=5120 (sampled rows) w_layout={w_layout}")
    kc, vc = recompute_on_gpu(d, w_layout)
    rows = np.sort(np.random.default_rng(3).choice(d["b"] * d["l"], 40, replace=False)).astype(np.int32)
    _check_rows(d, kc, vc, rows=rows)
    # attention over [0, s'): first with the GPU's own recomputed rows (isolates attention)
    w = dict(layout="dense", B=d["b"], Hq=d["H"], Hkv=d["H"], D=128, S=d["s"], q=d["q"],
             k=bits(kc).view(np.float16), v=bits(vc).view(np.float16), seqlens=None,
             scale=d["scale"])
    say("[recompute] attention over the merged cache")
    out, _ = decode_on_gpu(w, dev_inputs=dict(q=dev(d["q"]), k=kc, v=vc))
    ro, _ = oracle.decode_attn(w["q"], w["k"], w["v"], num_kv_heads=d["H"], layout=oracle.DENSE,
                               scale=d["scale"])
    check_close(host_f64(out), ro, "attention (GPU rows)")


@pytest.mark.parametrize("w_layout", LAYOUTS)
def test_wide_tiles_ragged_rows(w_layout):
    """b*l = 2100 rows and h = 4096 make a grid of 9 x 32 tiles of 256 x 256, the
    size at which [out, in] weights take the one-workgroup-per-CU kernel.  The
    last row tile holds 52 rows and two batch boundaries fall inside tiles."""
    d = kvgen.kvpr_layer(seed=8, b=3, h=4096, H=32, s=708, l=700)
    say(f"[recompute] b=3 l=700 h=4096 (256 x 256 tiles, ragged) w_layout={w_layout}")
    kc, vc = recompute_on_gpu(d, w_layout)
    edges = [0, 1, 255, 256, 699, 700, 1399, 1400, 2047, 2048, 2098, 2099]
    pick = np.random.default_rng(9).choice(2100, 24, replace=False)
    rows = np.unique(np.concatenate([edges, pick])).astype(np.int32)
    _check_rows(d, kc, vc, rows=rows)


@pytest.mark.parametrize("w_layout", LAYOUTS)
def test_wide_tiles_shortest_k(w_layout):
    """h = 256: four 64-wide K steps, so the loads two steps ahead clamp from
    the first step on; b*l = 32768 rows make exactly 256 tiles of 256 x 256."""
    d = kvgen.kvpr_layer(seed=17, b=4, h=256, H=2, s=8200, l=8192)
    say(f"[recompute] b=4 l=8192 h=256 (256 x 256 tiles, 4 K steps) w_layout={w_layout}")
    kc, vc = recompute_on_gpu(d, w_layout)
    edges = [0, 255, 256, 8191, 8192, 16383, 24576, 32767]
    pick = np.random.default_rng(18).choice(32768, 40, replace=False)
    rows = np.unique(np.concatenate([edges, pick])).astype(np.int32)
    _check_rows(d, kc, vc, rows=rows)


@pytest.mark.parametrize("w_layout", LAYOUTS)
def test_wide_tiles_beyond_one_round(w_layout):
    """b*l = 40000 rows and h = 256: 157 x 2 tiles of 256 x 256 (the last row
    tile holds 64 rows), more than one round of one workgroup per CU, with
    four K steps.  Two rows of every row tile are checked, all columns."""
    d = kvgen.kvpr_layer(seed=19, b=5, h=256, H=2, s=8008, l=8000)
    say(f"[recompute] b=5 l=8000 h=256 (314 tiles, 4 K steps) w_layout={w_layout}")
    kc, vc = recompute_on_gpu(d, w_layout)
    rng = np.random.default_rng(20)
    band = np.arange(0, 40000, 256)
    inside = np.concatenate([band + rng.integers(0, 256, band.size), band + 255])
    edges = [0, 7999, 8000, 39935, 39936, 39999]
    rows = np.unique(np.concatenate([edges, np.minimum(inside, 39999)])).astype(np.int32)
    _check_rows(d, kc, vc, rows=rows)


def test_end_to_end_against_fp64_recompute():
    d = kvgen.kvpr_layer(seed=4, b=2, h=1024, H=8, s=200, l=120)
    say("[recompute] end to end vs fp64 X.W")
    kc, vc = recompute_on_gpu(d)
    ko, vo = oracle.kv_recompute(d["x"], d["w_k"], d["w_v"], l=d["l"])
    kref = d["k_cache"].copy()
    vref = d["v_cache"].copy()
    kref[:, :d["l"]] = ko.reshape(2, d["l"], 8, 128).astype(np.float16)
    vref[:, :d["l"]] = vo.reshape(2, d["l"], 8, 128).astype(np.float16)
    w = dict(layout="dense", B=2, Hq=8, Hkv=8, D=128, S=200, q=d["q"], k=kref, v=vref,
             seqlens=None, scale=d["scale"])
    out, _ = decode_on_gpu(w, dev_inputs=dict(q=dev(d["q"]), k=kc, v=vc))
    ro, _ = oracle.decode_attn(d["q"], kref, vref, num_kv_heads=8, layout=oracle.DENSE,
                               scale=d["scale"])
    check_close(host_f64(out), ro, "end to end")


@pytest.mark.parametrize("w_layout", LAYOUTS)
@pytest.mark.parametrize("l", [0, 40, 96])
def test_kvpr_load_layer(l, w_layout):
    """Overlapped layer load: rows [0, l) recomputed from X copied in from
    pinned host memory, rows [l, s') copied bit for bit from the pinned host
    cache, rows from s' on left untouched; the staging buffer holds X[0:l]."""
    b, h, H, s_cap, s_prime = 2, 512, 4, 120, 96
    d = kvgen.kvpr_layer(seed=6, b=b, h=h, H=H, s=s_cap, l=s_prime)   # X: s' rows of activations
    kv = kvgen.kvpr_layer(seed=7, b=b, h=h, H=H, s=s_cap, l=0)        # host cache: every row drawn
    conv = (lambda w: np.ascontiguousarray(w.T)) if w_layout == K.KVDEC_W_OUT_IN else (lambda w: w)
    x_host = torch.from_numpy(d["x"].view(np.int16)).pin_memory()
    k_host = torch.from_numpy(kv["k_cache"]).pin_memory()
    v_host = torch.from_numpy(kv["v_cache"]).pin_memory()
    wk = dev(conv(d["w_k"]), bf16=True)
    wv = dev(conv(d["w_v"]), bf16=True)
    kc = torch.full((b, s_cap, H, 128), 1000.0, dtype=torch.float16, device="cuda")
    vc = torch.full((b, s_cap, H, 128), 1000.0, dtype=torch.float16, device="cuda")
    x_dev = torch.zeros((b, max(l, 1), h), dtype=torch.bfloat16, device="cuda")
    copy_stream = torch.cuda.Stream()
    say(f"[kvpr load] l={l} s'={s_prime} w_layout={w_layout}")
    K.kvdec_kvpr_load_layer(x_host, x_dev, k_host, v_host, wk, wv, kc, vc, l, s_prime, w_layout,
                            copy_stream=copy_stream)
    torch.cuda.synchronize()
    kb = bits(kc).reshape(b, s_cap, h)
    vb = bits(vc).reshape(b, s_cap, h)
    poison = np.float16(1000.0).view(np.uint16)
    assert np.all(kb[:, s_prime:] == poison) and np.all(vb[:, s_prime:] == poison)
    assert np.array_equal(kb[:, l:s_prime], kv["k_cache"].view(np.uint16).reshape(b, s_cap, h)[:, l:s_prime])
    assert np.array_equal(vb[:, l:s_prime], kv["v_cache"].view(np.uint16).reshape(b, s_cap, h)[:, l:s_prime])
    if l > 0:
        assert np.array_equal(bits(x_dev), d["x"][:, :l])
        ko, vo = oracle.kv_recompute(d["x"], d["w_k"], d["w_v"], l=l)
        check_close(host_f64(kc).reshape(b, s_cap, h)[:, :l].reshape(b * l, h), ko, "K rows [0, l)")
        check_close(host_f64(vc).reshape(b, s_cap, h)[:, :l].reshape(b * l, h), vo, "V rows [0, l)")

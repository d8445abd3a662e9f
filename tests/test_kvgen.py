"""Seeded input generators: determinism, shapes and the stated structure."""
import numpy as np

import kvgen


def test_deterministic_per_seed():
    a = kvgen.ragged_llama(seed=3, B=3, lo=10, hi=40)
    b = kvgen.ragged_llama(seed=3, B=3, lo=10, hi=40)
    c = kvgen.ragged_llama(seed=4, B=3, lo=10, hi=40)
    for key in ("q", "k", "v", "cu_seqlens"):
        assert np.array_equal(a[key], b[key])
    assert not np.array_equal(a["q"], c["q"])


def test_draws_independent_of_thread_count():
    n = 3 * kvgen.BLOCK + 1000
    a = kvgen.Draws(5).normal((n,))
    saved = kvgen._THREADS
    try:
        kvgen._THREADS = 1
        b = kvgen.Draws(5).normal((n,))
    finally:
        kvgen._THREADS = saved
    assert np.array_equal(a.view(np.uint16), b.view(np.uint16))
    # block 1 is stream (seed, 1) jumped once
    bg = np.random.PCG64(np.random.SeedSequence([5, 1])).jumped(1)
    ref = np.random.Generator(bg).standard_normal(kvgen.BLOCK, dtype=np.float32)
    assert np.array_equal(a[kvgen.BLOCK:2 * kvgen.BLOCK], ref.astype(np.float16))


def test_ragged_shapes_and_ranges():
    d = kvgen.ragged_llama(seed=0, B=16, lo=100, hi=200)
    assert d["k"].shape == (d["cu_seqlens"][-1], 8, 128)
    lens = np.diff(d["cu_seqlens"])
    assert lens.min() >= 100 and lens.max() <= 200
    assert d["q"].shape == (16, 32, 128)


def test_paged_structure():
    d = kvgen.paged_mha(seed=1, B=20, H=4, median=50, lo=3, hi=200, max_pages=16)
    lens, bt = d["seqlens"], d["block_table"]
    npg = (lens + 15) // 16
    used = np.concatenate([bt[b, :npg[b]] for b in range(20)])
    assert np.array_equal(np.sort(used), np.arange(d["k"].shape[0]))  # every page once
    for b in range(20):
        assert np.all(bt[b, npg[b]:] == -1)
        tail = lens[b] % 16
        if tail:
            assert np.all(d["k"][bt[b, npg[b] - 1], :, tail:] == kvgen.POISON_F16)


def test_lognormal_lengths_median_and_clip():
    rng = kvgen.Draws(0).ctl
    lens = kvgen.lognormal_lengths(rng, 20000)
    assert lens.min() >= 128 and lens.max() <= 4096
    assert 950 < np.median(lens) < 1100


def test_clo_hybrid_structure():
    d = kvgen.clo_hybrid(seed=2, B=2, S=640)
    hm = d["head_map"]
    assert (hm >= 0).sum() == 2 and sorted(hm[hm >= 0]) == [0, 1]
    sg = kvgen.group_importance(d["s"], d["Hkv"])
    assert set(np.flatnonzero(hm >= 0)) == set(np.argsort(-sg, kind="stable")[:2])
    assert d["ksel"] == 64
    for (b, g), idx in d["selection"].items():
        assert np.all(np.diff(idx) > 0)
        assert np.array_equal(d["buf_k"][b, g], d["k_full"][b, g, idx])


def test_bf16_rounding_is_nearest_even():
    x = np.array([1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -2.5, 3.0e-3], np.float32)
    bits = kvgen.f32_to_bf16_bits(x)
    back = kvgen.bf16_bits_to_f32(bits)
    assert back[0] == 1.0 and back[1] == 1.0            # tie -> even
    assert back[2] == 1.0 + 4 * 2 ** -8                  # tie -> even (up)
    assert back[3] == -2.5
    assert abs(back[4] - 3.0e-3) <= 2 ** -8 * 3.0e-3  # half an ulp (8-bit significand)

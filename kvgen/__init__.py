"""Seeded synthetic inputs shaped like the pages' workloads.

This module serves both sides of every parity check (the fp64 oracle and the
GPU library), so it holds none of the method's arithmetic: only seeded draws,
16-bit casts (round to nearest even) and layout packing.  Every workload draws
from a ``Draws(seed)`` source (numpy PCG64 streams, see its docstring) in the
order its docstring lists.  Normal draws are ``standard_normal(dtype=float32)``
then scaled and cast.

Workload shapes:
  * ``dense_small``  -- batch 1, 8 query heads on 2 KV heads, context 1024.
  * ``ragged_llama`` -- Llama3-8B decode layer (32 Qh / 8 KVh, D 128), batch 16,
    lengths uniform in [16384, 32768], K with per-channel LogNormal(0, 0.5)
    outlier scales, ragged packing with cu_seqlens.
  * ``paged_mha``    -- Llama-2-7B MHA layer (32 heads), batch 1024, LogNormal
    lengths (median 1024, sigma 1) clipped to [128, 4096], 16-token pages in a
    shuffled pool with a per-sequence block table.
  * ``clo_hybrid``   -- CLO head-wise cache at 128K (Llama3-8B 32/8 or
    Qwen2.5-14B 40/8), batch 4: labels, queries near their labels, Beta(0.5, 2)
    importances, 2 persistent heads, a 10% token selection per buffer head.
  * ``clo_ahead``    -- CLO one-layer-ahead lookup: hidden states x [B, h] of
    the previous layer, the next layer's W_Q [Hq*D, h] (nn.Linear layout), and
    hidden states of the step the labels came from (x plus a per-sequence drift).
  * ``clo_gather``   -- a full dense cache (Llama3-8B or Qwen2.5-14B heads,
    batch 4, 128K) for CLO-style top-k sparse attention gathered in place.
  * ``kvpr_layer``   -- KVPR OPT-13B layer: h 5120, 40 heads, batch 32,
    s' 1024, split l 256, bf16 X and W, fp16 resident cache rows.
"""
from __future__ import annotations

import concurrent.futures as cf
import math
import os

import numpy as np

D_HEAD = 128
BLOCK = 1 << 22  # values per independently seeded block of a large draw

POISON_F16 = np.float16(1000.0)

_THREADS = max(1, min(16, os.cpu_count() or 1))


class Draws:
    """Seeded source of every random value of one workload.

    Small draws (lengths, scales, importances, permutations) come, in order,
    from ``ctl`` = PCG64(SeedSequence([seed, 0])).  The k-th large array
    (k = 1, 2, ...) is drawn block by block: its block i of BLOCK values is
    ``standard_normal(float32)`` from PCG64(SeedSequence([seed, k])).jumped(i).
    Blocks are filled in parallel threads; the values do not depend on the
    thread count.
    """

    def __init__(self, seed: int):
        self.seed = int(seed)
        self.ctl = np.random.Generator(np.random.PCG64(np.random.SeedSequence([self.seed, 0])))
        self._k = 0

    def _next_bitgen(self):
        self._k += 1
        return np.random.PCG64(np.random.SeedSequence([self.seed, self._k]))

    def normal(self, shape, scale=None, out_dtype=np.float16, std=1.0):
        """Array of N(0,1) float32 draws, times ``std`` and an optional scale
        broadcast over the trailing dims, cast to ``out_dtype`` (float16, or
        uint16 meaning bfloat16 bit patterns); casts round to nearest even."""
        shape = tuple(int(s) for s in shape)
        n = int(np.prod(shape)) if shape else 1
        out = np.empty(n, out_dtype)
        sc_row = None
        if scale is not None:
            sc = np.asarray(scale, np.float32)
            sc_row = np.broadcast_to(sc, shape[len(shape) - sc.ndim:]).reshape(-1)
        base = self._next_bitgen()

        def fill(i):
            lo, hi = i * BLOCK, min(n, (i + 1) * BLOCK)
            g = np.random.Generator(base.jumped(i))
            blk = g.standard_normal(hi - lo, dtype=np.float32)
            if std != 1.0:
                blk *= np.float32(std)
            if sc_row is not None and BLOCK % sc_row.size == 0:
                blk = (blk.reshape(-1, sc_row.size) * sc_row[None, :]).reshape(-1)
            elif sc_row is not None:  # a period that straddles blocks (e.g. 40 x 128)
                blk = blk * sc_row[np.arange(lo, hi) % sc_row.size]
            out[lo:hi] = blk.astype(np.float16) if out_dtype == np.float16 else f32_to_bf16_bits(blk)

        nblk = (n + BLOCK - 1) // BLOCK
        if nblk <= 1:
            for i in range(nblk):
                fill(i)
        else:
            with cf.ThreadPoolExecutor(min(_THREADS, nblk)) as ex:
                list(ex.map(fill, range(nblk)))
        return out.reshape(shape)


def f32_to_bf16_bits(a):
    """float32 -> bfloat16 bit patterns, round to nearest even (finite inputs)."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    rounding = ((u >> 16) & 1) + np.uint32(0x7FFF)
    return ((u + rounding) >> 16).astype(np.uint16)


def bf16_bits_to_f32(bits):
    return (np.asarray(bits, np.uint16).astype(np.uint32) << 16).view(np.float32)


# ---------------------------------------------------------------------------
# Decode attention workloads
# ---------------------------------------------------------------------------

E4M3_MAX = 448.0


def e4m3_scale(x):
    """Per-tensor scale of an e4m3 KV cache: max |x| / 448 in fp32 (1 for an
    all-zero tensor), so the largest element maps to the largest code."""
    amax = 0.0
    flat = np.asarray(x).reshape(-1)
    for lo in range(0, flat.size, BLOCK):
        blk = flat[lo:lo + BLOCK].astype(np.float32)
        amax = max(amax, float(np.abs(blk).max()) if blk.size else 0.0)
    return np.float32(amax / E4M3_MAX) if amax > 0 else np.float32(1.0)


def to_e4m3(x, scale):
    """e4m3 ("fn") codes of x / scale: the quotient in fp32, clipped to +-448,
    then one round-to-nearest-even cast (torch's float8_e4m3fn)."""
    import torch
    flat = np.asarray(x).reshape(-1)
    out = np.empty(flat.size, np.uint8)
    inv = np.float32(scale)
    for lo in range(0, flat.size, BLOCK):
        blk = flat[lo:lo + BLOCK].astype(np.float32) / inv
        t = torch.from_numpy(np.clip(blk, -E4M3_MAX, E4M3_MAX)).to(torch.float8_e4m3fn)
        out[lo:lo + blk.size] = t.view(torch.uint8).numpy()
    return out.reshape(np.asarray(x).shape)


def fp8_kv(d, keys=("k", "v")):
    """A copy of workload d whose K/V arrays (``keys``, K first) are e4m3
    codes with per-tensor scales ``k_scale`` / ``v_scale`` (the arrays keep
    their layout; one byte per element)."""
    out = dict(d)
    kname, vname = keys
    ks, vs = e4m3_scale(d[kname]), e4m3_scale(d[vname])
    out[kname] = to_e4m3(d[kname], ks)
    out[vname] = to_e4m3(d[vname], vs)
    out["k_scale"], out["v_scale"] = float(ks), float(vs)
    return out


def fp8_hybrid(d):
    """A copy of a ``clo_hybrid`` workload with e4m3 persistent and buffer K/V:
    one K scale and one V scale shared by both sources (amax over the two)."""
    out = dict(d)
    ks = max(e4m3_scale(d["pers_k"]), e4m3_scale(d["buf_k"]))
    vs = max(e4m3_scale(d["pers_v"]), e4m3_scale(d["buf_v"]))
    for name, sc in (("pers_k", ks), ("buf_k", ks), ("pers_v", vs), ("buf_v", vs)):
        out[name] = to_e4m3(d[name], sc)
    out["k_scale"], out["v_scale"] = float(ks), float(vs)
    return out


def dense_small(seed=0, B=1, Hq=8, Hkv=2, S=1024, D=D_HEAD, seqlens=None):
    """Dense KV [B, S, Hkv, D].  Draw order: q, K, V (all N(0,1) -> fp16)."""
    dr = Draws(seed)
    q = dr.normal((B, Hq, D))
    k = dr.normal((B, S, Hkv, D))
    v = dr.normal((B, S, Hkv, D))
    return dict(layout="dense", B=B, Hq=Hq, Hkv=Hkv, D=D, S=S, q=q, k=k, v=v,
                seqlens=None if seqlens is None else np.asarray(seqlens, np.int32),
                scale=1.0 / math.sqrt(D))


def ragged_llama(seed=0, B=16, lo=16384, hi=32768, Hq=32, Hkv=8, D=D_HEAD, lens=None,
                 outlier_sigma=0.5):
    """Ragged KV [T, Hkv, D] + cu_seqlens.

    Draw order: lengths ~ U{lo..hi} (unless given); per-(KV head, channel) K
    outlier scale ~ LogNormal(0, outlier_sigma), shared by all tokens and
    sequences; K = N(0,1) * scale; V ~ N(0,1); q ~ N(0,1).
    """
    dr = Draws(seed)
    if lens is None:
        lens = dr.ctl.integers(lo, hi + 1, size=B)
    lens = np.asarray(lens, np.int64)
    B = int(lens.size)
    sigma = dr.ctl.lognormal(0.0, outlier_sigma, size=(Hkv, D)).astype(np.float32)
    T = int(lens.sum())
    k = dr.normal((T, Hkv, D), scale=sigma)
    v = dr.normal((T, Hkv, D))
    q = dr.normal((B, Hq, D))
    cu = np.zeros(B + 1, np.int32)
    cu[1:] = np.cumsum(lens)
    return dict(layout="ragged", B=B, Hq=Hq, Hkv=Hkv, D=D, q=q, k=k, v=v, cu_seqlens=cu,
                seqlens=lens.astype(np.int32), max_seqlen=int(lens.max()) if B else 0,
                scale=1.0 / math.sqrt(D))


def lognormal_lengths(rng, B, median=1024, sigma=1.0, lo=128, hi=4096):
    z = rng.standard_normal(B)
    return np.clip(np.rint(np.exp(math.log(median) + sigma * z)), lo, hi).astype(np.int64)


def paged_mha(seed=0, B=1024, H=32, Hkv=None, D=D_HEAD, page=16, max_pages=256, median=1024,
              sigma=1.0, lo=128, hi=4096, lens=None):
    """Paged KV pool [P, Hkv, page, D] + block_table [B, max_pages] (-1 padded).

    Draw order: lengths (LogNormal, median/sigma, clipped) unless given; page
    permutation of the P = sum ceil(len/page) pages; pool K; pool V; q.  Slots
    past the end of a sequence's last page hold the poison value 1000.0.
    """
    dr = Draws(seed)
    rng = dr.ctl
    Hkv = H if Hkv is None else Hkv
    if lens is None:
        lens = lognormal_lengths(rng, B, median, sigma, lo, hi)
    lens = np.asarray(lens, np.int64)
    B = int(lens.size)
    npg = (lens + page - 1) // page
    if int(npg.max(initial=0)) > max_pages:
        raise ValueError("a sequence needs more pages than max_pages")
    P = int(npg.sum())
    perm = rng.permutation(P).astype(np.int32)
    bt = np.full((B, max_pages), -1, np.int32)
    off = 0
    for b in range(B):
        bt[b, : npg[b]] = perm[off: off + npg[b]]
        off += int(npg[b])
    k = dr.normal((P, Hkv, page, D))
    v = dr.normal((P, Hkv, page, D))
    q = dr.normal((B, H, D))
    for b in range(B):
        tail = int(lens[b] % page)
        if tail and npg[b]:
            last = bt[b, npg[b] - 1]
            k[last, :, tail:, :] = POISON_F16
            v[last, :, tail:, :] = POISON_F16
    return dict(layout="paged", B=B, Hq=H, Hkv=Hkv, D=D, q=q, k=k, v=v, block_table=bt,
                seqlens=lens.astype(np.int32), page=page, max_pages=max_pages,
                max_seqlen=int(lens.max()) if B else 0, scale=1.0 / math.sqrt(D))


# --- layout packing helpers (no arithmetic) --------------------------------

def paged_to_ragged(d):
    """Gather a paged workload into the ragged layout (same logical tokens)."""
    page, bt, lens = d["page"], d["block_table"], d["seqlens"]
    parts_k, parts_v = [], []
    for b in range(d["B"]):
        n = int(lens[b])
        npg = (n + page - 1) // page
        pk = d["k"][bt[b, :npg]].transpose(0, 2, 1, 3).reshape(npg * page, d["Hkv"], d["D"])
        pv = d["v"][bt[b, :npg]].transpose(0, 2, 1, 3).reshape(npg * page, d["Hkv"], d["D"])
        parts_k.append(pk[:n]); parts_v.append(pv[:n])
    cu = np.zeros(d["B"] + 1, np.int32)
    cu[1:] = np.cumsum(lens)
    return dict(d, layout="ragged", k=np.ascontiguousarray(np.concatenate(parts_k)),
                v=np.ascontiguousarray(np.concatenate(parts_v)), cu_seqlens=cu)


def ragged_to_dense(d, S=None):
    """Scatter a ragged workload into dense [B, S, Hkv, D] (padding rows = poison)."""
    lens = d["seqlens"]
    S = int(lens.max()) if S is None else S
    shape = (d["B"], S, d["Hkv"], d["D"])
    k = np.full(shape, POISON_F16, np.float16)
    v = np.full(shape, POISON_F16, np.float16)
    cu = d["cu_seqlens"]
    for b in range(d["B"]):
        n = int(lens[b])
        k[b, :n] = d["k"][cu[b]: cu[b] + n]
        v[b, :n] = d["v"][cu[b]: cu[b] + n]
    return dict(d, layout="dense", k=k, v=v, S=S)


def ragged_to_paged(d, seed=0, page=16, max_pages=None):
    """Scatter a ragged workload into a shuffled page pool (draw: permutation)."""
    rng = Draws(seed).ctl
    lens = np.asarray(d["seqlens"], np.int64)
    npg = (lens + page - 1) // page
    max_pages = int(npg.max(initial=1)) if max_pages is None else max_pages
    P = int(npg.sum())
    perm = rng.permutation(P).astype(np.int32)
    bt = np.full((d["B"], max_pages), -1, np.int32)
    k = np.full((P, d["Hkv"], page, d["D"]), POISON_F16, np.float16)
    v = np.full_like(k, POISON_F16)
    off = 0
    cu = d["cu_seqlens"]
    for b in range(d["B"]):
        bt[b, : npg[b]] = perm[off: off + npg[b]]
        off += int(npg[b])
        for t0 in range(0, int(lens[b]), page):
            n = min(page, int(lens[b]) - t0)
            p = bt[b, t0 // page]
            k[p, :, :n] = d["k"][cu[b] + t0: cu[b] + t0 + n].transpose(1, 0, 2)
            v[p, :, :n] = d["v"][cu[b] + t0: cu[b] + t0 + n].transpose(1, 0, 2)
    return dict(d, layout="paged", k=k, v=v, block_table=bt, page=page, max_pages=max_pages)


# ---------------------------------------------------------------------------
# CLO head-wise cache workload
# ---------------------------------------------------------------------------

CLO_MODELS = {"llama3-8b": (32, 8), "qwen2.5-14b": (40, 8)}


def clo_queries(seed=0, model="llama3-8b", B=4, D=D_HEAD):
    """Labels, queries near them, and importances for the head-wise cache.

    Draw order: importance s_j ~ Beta(0.5, 2) per query head; labels ~ N(0, I);
    per-(b, j) noise scale ~ U[2.96, 6.75]; noise ~ N(0, I).  The query is
    0.9 * label + 0.1 * scale * noise, normalised to unit length, cast to fp16.
    The noise scale band puts the label/query cosines near 0.80-0.95.
    """
    Hq, Hkv = CLO_MODELS[model]
    rng = Draws(seed).ctl
    s = rng.beta(0.5, 2.0, size=Hq)
    lab32 = rng.standard_normal((B, Hq, D), dtype=np.float32)
    sig = rng.uniform(2.96, 6.75, size=(B, Hq)).astype(np.float32)
    noise = rng.standard_normal((B, Hq, D), dtype=np.float32)
    q32 = np.float32(0.9) * lab32 + np.float32(0.1) * sig[..., None] * noise
    q32 /= np.linalg.norm(q32, axis=-1, keepdims=True)
    return dict(model=model, B=B, Hq=Hq, Hkv=Hkv, D=D, s=s, weights=s.astype(np.float32),
                labels=lab32.astype(np.float16), q=q32.astype(np.float16), eta=0.8, n_exp=3.0)


def group_importance(s, Hkv):
    """Per-KV-head importance: the largest importance among its query heads."""
    s = np.asarray(s)
    return s.reshape(Hkv, -1).max(axis=1)


def persistent_heads(s, Hkv, n_pers=2):
    """Head map: the n_pers KV heads of largest group importance (ties -> lower
    index) get persistent slots 0.. in ascending head order; others -1."""
    sg = group_importance(s, Hkv)
    top = np.sort(np.argsort(-sg, kind="stable")[:n_pers])
    hm = np.full(Hkv, -1, np.int32)
    hm[top] = np.arange(len(top), dtype=np.int32)
    return hm


def clo_hybrid(seed=0, model="llama3-8b", B=4, S=131072, frac=0.1, n_pers=2, D=D_HEAD):
    """CLO cache buffer + persistent cache inputs.

    Draw order: the ``clo_queries`` draws (``Draws(seed)``); then, from
    ``Draws(seed + 1000003)``, full K and V [B, Hkv, S, D] ~ N(0,1) and, per
    (b, buffer head) in ascending order, a sorted random selection of
    round(frac * S) token indices without replacement (from its ``ctl``).
    Persistent heads copy their full KV into slot arrays; buffer heads copy the
    selected rows, compacted in ascending token order.
    """
    base = clo_queries(seed, model, B, D)
    Hq, Hkv = base["Hq"], base["Hkv"]
    dr = Draws(seed + 1_000_003)
    rng = dr.ctl
    kf = dr.normal((B, Hkv, S, D))
    vf = dr.normal((B, Hkv, S, D))
    hm = persistent_heads(base["s"], Hkv, n_pers)
    ksel = int(round(frac * S))
    P_slots = int((hm >= 0).sum())
    pers_k = np.zeros((B, max(P_slots, 1), S, D), np.float16)
    pers_v = np.zeros_like(pers_k)
    buf_k = np.zeros((B, Hkv, ksel, D), np.float16)
    buf_v = np.zeros_like(buf_k)
    buf_len = np.zeros(B * Hkv, np.int32)
    sel = {}
    for b in range(B):
        for g in range(Hkv):
            if hm[g] >= 0:
                pers_k[b, hm[g]] = kf[b, g]
                pers_v[b, hm[g]] = vf[b, g]
            else:
                idx = np.sort(rng.choice(S, size=ksel, replace=False))
                sel[(b, g)] = idx
                buf_k[b, g] = kf[b, g, idx]
                buf_v[b, g] = vf[b, g, idx]
                buf_len[b * Hkv + g] = ksel
    return dict(base, S=S, k_full=kf, v_full=vf, head_map=hm, pers_k=pers_k, pers_v=pers_v,
                pers_len=np.full(B, S, np.int32), buf_k=buf_k, buf_v=buf_v, buf_len=buf_len,
                selection=sel, ksel=ksel, scale=1.0 / math.sqrt(D))


CLO_HIDDEN = {"llama3-8b": 4096, "qwen2.5-14b": 5120}


def clo_ahead(seed=0, model="llama3-8b", B=4, h=None, Hq=None, Hkv=None, D=D_HEAD,
              drift=(0.1, 1.0), out_dtype=np.float16):
    """Inputs of the one-layer-ahead head-cache lookup.

    Draw order: the ``clo_queries`` importances (``Draws(seed).ctl``, first
    draw only); then from ``Draws(seed + 2000003)``: per-sequence drift scale
    ~ U[drift] (``ctl``), x_prev [B, h] ~ N(0,1), drift noise [B, h] ~ N(0,1),
    W_Q [Hq*D, h] ~ N(0, 1/h).  x_label = x_prev + scale_b * noise (fp32, cast
    once): the hidden state of the step whose query became the label, so the
    label/query cosines fall as the drift grows.  h, Hq, Hkv default to the
    model's; out_dtype float16, or uint16 for bfloat16 bits.
    """
    mq, mkv = CLO_MODELS[model]
    Hq = mq if Hq is None else Hq
    Hkv = mkv if Hkv is None else Hkv
    h = CLO_HIDDEN[model] if h is None else h
    s = Draws(seed).ctl.beta(0.5, 2.0, size=Hq)
    dr = Draws(seed + 2_000_003)
    scale = dr.ctl.uniform(drift[0], drift[1], size=B).astype(np.float32)
    x32 = dr.normal((B, h), out_dtype=np.float16).astype(np.float32)
    noise = dr.normal((B, h), out_dtype=np.float16).astype(np.float32)
    w = dr.normal((Hq * D, h), out_dtype=out_dtype, std=1.0 / math.sqrt(h))
    cast = (lambda a: a.astype(np.float16)) if out_dtype == np.float16 else f32_to_bf16_bits
    return dict(model=model, B=B, Hq=Hq, Hkv=Hkv, D=D, h=h, s=s, weights=s.astype(np.float32),
                x_prev=cast(x32), x_label=cast(x32 + scale[:, None] * noise), w_q=w,
                drift=scale, eta=0.8, n_exp=3.0)


def clo_gather(seed=0, model="llama3-8b", B=4, S=131072, frac=0.1, D=D_HEAD, lens=None):
    """A full GPU-resident cache for index-gather sparse attention.

    Draw order (``Draws(seed + 3000017)``): per-(KV head, channel) K outlier
    scale ~ LogNormal(0, 0.5) (``ctl``), lengths ~ U{S/2..S} unless given
    (``ctl``), q [B, Hq, D] ~ N(0,1), K = N(0,1) * scale, V ~ N(0,1), all in
    the dense layout [B, S, Hkv, D]; top_k = round(frac * S).
    """
    Hq, Hkv = CLO_MODELS[model]
    dr = Draws(seed + 3_000_017)
    sigma = dr.ctl.lognormal(0.0, 0.5, size=(Hkv, D)).astype(np.float32)
    if lens is None:
        lens = dr.ctl.integers(S // 2, S + 1, size=B)
    lens = np.asarray(lens, np.int32)
    q = dr.normal((B, Hq, D))
    k = dr.normal((B, S, Hkv, D), scale=sigma)
    v = dr.normal((B, S, Hkv, D))
    return dict(model=model, B=B, Hq=Hq, Hkv=Hkv, D=D, S=S, q=q, k=k, v=v, seqlens=lens,
                top_k=int(round(frac * S)), scale=1.0 / math.sqrt(D))


def random_indices(seed, B, Hkv, lens, top_k):
    """Sorted random token selections without replacement per (b, g):
    min(top_k, len_b) of [0, len_b), in the layout [B, Hkv, top_k] (-1 pad)."""
    rng = Draws(seed).ctl
    idx = np.full((B, Hkv, top_k), -1, np.int32)
    n = np.zeros(B * Hkv, np.int32)
    for b in range(B):
        for g in range(Hkv):
            m = min(top_k, int(lens[b]))
            idx[b, g, :m] = np.sort(rng.choice(int(lens[b]), size=m, replace=False))
            n[b * Hkv + g] = m
    return idx, n


def clo_prefetch(seed=0, model="llama3-8b", B=4, S=131072, frac=0.1, n_pers=2, D=D_HEAD,
                 elem="f16"):
    """Inputs of the miss-driven prefetch: the ``clo_queries`` draws; then,
    from ``Draws(seed + 4000037)``, the offloaded full KV in the dense layout
    [B, S, Hkv, D] ~ N(0,1) (K then V; fp16, or e4m3-like random byte codes
    with no NaN pattern when elem="u8"); the selections come from
    ``random_indices(seed + 5000011, ...)``: round(frac * S) sorted token rows
    per (b, g).  The head map puts the n_pers KV heads of largest importance
    on persistent slots."""
    base = clo_queries(seed, model, B, D)
    Hq, Hkv = base["Hq"], base["Hkv"]
    dr = Draws(seed + 4_000_037)
    if elem == "u8":
        codes = lambda: dr.ctl.integers(0, 0x7E, size=(B, S, Hkv, D), dtype=np.uint8) | (
            dr.ctl.integers(0, 2, size=(B, S, Hkv, D), dtype=np.uint8) << 7)
        pool_k, pool_v = codes(), codes()
    else:
        pool_k = dr.normal((B, S, Hkv, D))
        pool_v = dr.normal((B, S, Hkv, D))
    top_k = int(round(frac * S))
    idx, idx_len = random_indices(seed + 5_000_011, B, Hkv, np.full(B, S), top_k)
    return dict(base, S=S, pool_k=pool_k, pool_v=pool_v, idx=idx, idx_len=idx_len, top_k=top_k,
                head_map=persistent_heads(base["s"], Hkv, n_pers), scale=1.0 / math.sqrt(D))


# ---------------------------------------------------------------------------
# KVPR partial-recompute workload
# ---------------------------------------------------------------------------

def kvpr_layer(seed=0, b=32, h=5120, H=40, s=1024, l=256):
    """OPT-13B-shaped layer for partial recompute + attention.

    Draw order: X [b, l, h] ~ N(0,1) (bf16); W_K, W_V [h, h] ~ N(0, 1/h) (bf16);
    resident cache rows K[:, l:s], V[:, l:s] ~ N(0,1) (fp16); q [b, H, h/H] (fp16).
    Cache rows [0, l) start as the poison value 1000.0 (the recompute fills them).
    """
    D = h // H
    dr = Draws(seed)
    x = dr.normal((b, l, h), out_dtype=np.uint16)
    std = 1.0 / math.sqrt(h)
    wk = dr.normal((h, h), out_dtype=np.uint16, std=std)
    wv = dr.normal((h, h), out_dtype=np.uint16, std=std)
    kc = np.empty((b, s, H, D), np.float16)
    vc = np.empty((b, s, H, D), np.float16)
    kc[:, :l] = POISON_F16
    vc[:, :l] = POISON_F16
    kc[:, l:] = dr.normal((b, s - l, H, D))
    vc[:, l:] = dr.normal((b, s - l, H, D))
    q = dr.normal((b, H, D))
    return dict(b=b, h=h, H=H, D=D, s=s, l=l, x=x, w_k=wk, w_v=wv, k_cache=kc, v_cache=vc,
                q=q, scale=1.0 / math.sqrt(D))

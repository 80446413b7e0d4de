"""Workload descriptions and seeded synthetic inputs.

Plain data and random-number generation only: nothing here computes any part
of the attention.  Both the GPU library's binding and the CPU oracle read these
descriptions, each translating them into its own descriptor.

Pattern vocabulary (per grid dimension unless noted):

* ``na``      window of ``window[d]`` positions centred on the query and shifted
              inside the grid at the borders (neighbourhood attention);
              optional ``stride`` (groups sharing one window), ``shift`` (the
              groups' phase: they start at positions congruent to -shift),
              ``dilation`` and ``causal`` (per dimension: the window ends at
              the query and is cut at the start, e.g. causal in time for video).
* ``sa``      the same window cut at the grid borders instead of shifted
              (slide attention, zero padding).
* ``band``    1-D only: keys in [x - left, x + right] cut at the ends
              (bidirectional band; causal when right = 0).
* ``blocked`` non-overlapping windows of ``window[d]`` positions; optional
              ``shift[d]`` moves the window boundaries back (shifted windows).
* any 1-D pattern may add pi-Attention's online partner: ``skip`` (pi),
              ``skip_both`` (also x + pi), ``skip_mode`` ("union",
              "fixed_fusion", "separate") and ``skip_prior`` (alpha).
* ``sta``     sliding tile attention: tiles of ``tile[d]`` positions; the query's
              tile attends ``window_tiles[d]`` whole tiles shifted inside.

Orders: ``row_major``; ``tiled`` (tile by tile with tile extents ``tile``,
row-major inside); ``hilbert`` (2-D grid of any size along a Hilbert curve; the
pattern is then 1-D over the position along the curve).
"""
from __future__ import annotations

import math

# The five benchmark workloads.  Each gets its own seed (its index, 1-5).
CONFIGS = {
    "na2d_fp32": dict(
        name="na2d_fp32", B=1, H=1, D=32, dtype="fp32", grid=[8, 8], order="row_major",
        pattern=dict(kind="na", window=[3, 3]), seed=1,
        note="2-D neighbourhood attention, 8x8 grid, 3x3 window clamped at borders"),
    "na2d_bf16": dict(
        name="na2d_bf16", B=2, H=8, D=64, dtype="bf16", grid=[64, 64], order="row_major",
        pattern=dict(kind="na", window=[13, 13]), seed=2,
        note="2-D neighbourhood attention, 64x64 grid, 13x13 window clamped at borders"),
    "sta3d_bf16": dict(
        name="sta3d_bf16", B=1, H=24, D=128, dtype="bf16", grid=[30, 48, 80], order="tiled",
        tile=[6, 8, 8], pattern=dict(kind="sta", tile=[6, 8, 8], window_tiles=[3, 5, 7]),
        seed=3,
        note="3-D sliding tile attention, 30x48x80 grid, 6x8x8 tiles, 3x5x7-tile window"),
    "hilbert_band_bf16": dict(
        name="hilbert_band_bf16", B=4, H=12, D=64, dtype="bf16", grid=[128, 128],
        order="hilbert", pattern=dict(kind="band", left=256, right=256), seed=4,
        note="Hilbert slide attention, 128x128 grid, band radius 256 on the curve"),
    "causal1d_bf16": dict(
        name="causal1d_bf16", B=1, H=32, D=128, dtype="bf16", grid=[32768], order="row_major",
        pattern=dict(kind="band", left=4095, right=0), seed=5,
        note="1-D causal sliding window, 32768 tokens, 4096 keys including self"),
}

# The Hilbert page's kernel benchmarks ("Hilbert-Guided Sparse Local Attention",
# Tables 1-3): batch 16, 2 heads, head_dim 64, patterns formed on the curve.  A
# k x k window becomes k*k consecutive curve positions (HWA: non-overlapping
# windows; HSWA: the same windows shifted by half a window); a k x k slide or
# neighbourhood kernel becomes k*k positions around the query (HSA: band of
# radius (k*k - 1) / 2 cut at the ends; HNA: window of k*k shifted inside).
# 56 x 56 and 96 x 96 are not powers of two: they run on the generalised curve.
HILBERT_PAGE = {
    "hwa96_bf16": dict(
        name="hwa96_bf16", B=16, H=2, D=64, dtype="bf16", grid=[96, 96], order="hilbert",
        pattern=dict(kind="blocked", window=[64]), seed=11,
        note="Hilbert window attention, 96x96 input, 8x8 window (Table 1)"),
    "hswa96_bf16": dict(
        name="hswa96_bf16", B=16, H=2, D=64, dtype="bf16", grid=[96, 96], order="hilbert",
        pattern=dict(kind="blocked", window=[64], shift=[32]), seed=12,
        note="Hilbert shifted window attention, 96x96 input, 8x8 window shifted by 32"),
    "hwa128_bf16": dict(
        name="hwa128_bf16", B=16, H=2, D=64, dtype="bf16", grid=[128, 128], order="hilbert",
        pattern=dict(kind="blocked", window=[256]), seed=13,
        note="Hilbert window attention, 128x128 input, 16x16 window (Tables 1-2)"),
    "hsa56_bf16": dict(
        name="hsa56_bf16", B=16, H=2, D=64, dtype="bf16", grid=[56, 56], order="hilbert",
        pattern=dict(kind="band", left=24, right=24), seed=14,
        note="Hilbert slide attention, 56x56 input, 7x7 kernel (Table 3)"),
    "hna56_bf16": dict(
        name="hna56_bf16", B=16, H=2, D=64, dtype="bf16", grid=[56, 56], order="hilbert",
        pattern=dict(kind="na", window=[49]), seed=15,
        note="Hilbert neighbourhood attention, 56x56 input, 7x7 kernel (Table 3)"),
    "hsa96_bf16": dict(
        name="hsa96_bf16", B=16, H=2, D=64, dtype="bf16", grid=[96, 96], order="hilbert",
        pattern=dict(kind="band", left=24, right=24), seed=16,
        note="Hilbert slide attention, 96x96 input, 7x7 kernel (Table 3)"),
    "hna96_bf16": dict(
        name="hna96_bf16", B=16, H=2, D=64, dtype="bf16", grid=[96, 96], order="hilbert",
        pattern=dict(kind="na", window=[49]), seed=17,
        note="Hilbert neighbourhood attention, 96x96 input, 7x7 kernel (Table 3)"),
}

# Generalised neighbourhood attention beyond the five benchmark shapes
# ("Generalized Neighborhood Attention", abstract: sliding, strided and blocked
# windows in any number of dimensions).
GNA = {
    # the 64x64 13x13 neighbourhood workload with the token order cut into 8x8
    # patches: same neighbourhoods, fewer and denser tile pairs
    "na2d_tiled_bf16": dict(
        name="na2d_tiled_bf16", B=2, H=8, D=64, dtype="bf16", grid=[64, 64], order="tiled",
        tile=[8, 8], pattern=dict(kind="na", window=[13, 13]), seed=21,
        note="2-D neighbourhood attention, 64x64 grid, 13x13 window, 8x8 patch order"),
    # sliding tile attention on the 30x48x80 video grid made causal in time:
    # each chunk of 6 frames attends to itself and the chunk before it, and to
    # the 3x5 spatial tiles around its own (block-causal video attention)
    "sta3d_causal_t_bf16": dict(
        name="sta3d_causal_t_bf16", B=1, H=24, D=128, dtype="bf16", grid=[30, 48, 80],
        order="tiled", tile=[6, 8, 8],
        pattern=dict(kind="na", window=[12, 24, 40], stride=[6, 8, 8], causal=[1, 0, 0]),
        seed=22,
        note="3-D sliding tile attention causal in time, 30x48x80 grid, 6x8x8 tiles, "
             "2 chunks of 6 frames x 3x5 tiles"),
}

# pi-Attention ("pi-Attention: Online Efficient Sparse Transformers for
# Long-Context Modeling"): causal local window of k = 4 (Eq. 5: keys i-4 .. i)
# plus the online partner i - pi with pi = 16 (Eqs. 8-9), the page's defaults,
# at the Medium model's attention shape (16 heads of 64) over 8192 tokens.
_PI = dict(B=4, H=16, D=64, dtype="bf16", grid=[8192], order="row_major")
PI_ATTENTION = {
    "pi_union_bf16": dict(
        _PI, name="pi_union_bf16", seed=31,
        pattern=dict(kind="band", left=4, right=0, skip=16, skip_mode="union"),
        note="pi-Attention, one softmax over window u partner (Eq. 11), k=4, pi=16, 8192 tokens"),
    "pi_fusion_bf16": dict(
        _PI, name="pi_fusion_bf16", seed=32,
        pattern=dict(kind="band", left=4, right=0, skip=16, skip_mode="fixed_fusion",
                     skip_prior=0.5),
        note="pi-Attention fixed fusion (Eqs. 16-17), alpha=0.5, k=4, pi=16, 8192 tokens"),
    "pi_separate_bf16": dict(
        _PI, name="pi_separate_bf16", seed=33,
        pattern=dict(kind="band", left=4, right=0, skip=16, skip_mode="separate"),
        note="pi-Attention separate softmax (Eq. 15), k=4, pi=16, 8192 tokens"),
}

# Every named workload.
ALL = {**CONFIGS, **HILBERT_PAGE, **GNA, **PI_ATTENTION}

# The workload the benchmark times by default (the headline metric's config).
HEADLINE = "sta3d_bf16"


def num_tokens(w: dict) -> int:
    return int(math.prod(int(g) for g in w["grid"]))


def default_scale(w: dict) -> float:
    return 1.0 / math.sqrt(int(w["D"]))


def scaled(w: dict, **over) -> dict:
    """A copy of workload w with fields replaced (e.g. fewer heads)."""
    out = dict(w)
    out.update(over)
    return out


def make_qkv(w: dict, device="cpu", seed: int | None = None):
    """q, k, v ~ i.i.d. N(0, 1) of shape [B, H, N, D], drawn in that order in
    fp32 from one generator seeded with the workload's seed, then rounded to
    bf16 (round to nearest even) for bf16 workloads."""
    import torch

    g = torch.Generator(device=device)
    g.manual_seed(int(w["seed"] if seed is None else seed))
    shape = (int(w["B"]), int(w["H"]), num_tokens(w), int(w["D"]))
    out = []
    for _ in range(3):
        x = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
        if w["dtype"] == "bf16":
            x = x.to(torch.bfloat16)
        out.append(x)
    return tuple(out)


def make_dout(w: dict, device="cpu", seed: int | None = None):
    """The upstream gradient for the backward pass: i.i.d. N(0, 1) of shape
    [B, H, N, D] in fp32 from a generator seeded with 1000 + the workload's
    seed, rounded like q, k, v."""
    import torch

    g = torch.Generator(device=device)
    g.manual_seed(1000 + int(w["seed"] if seed is None else seed))
    shape = (int(w["B"]), int(w["H"]), num_tokens(w), int(w["D"]))
    x = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
    return x.to(torch.bfloat16) if w["dtype"] == "bf16" else x

"""Pins of the fp64 CPU oracle against facts fixed independently of it.

Each pin is chosen so that a plausible mistake in the oracle (a dropped term, a
wrong sign or index, a transposed operand, an off-by-one window) fails one of
them:

* the block sparsities printed on the Hilbert page (tests/golden),
* the Hilbert-curve defining properties (bijection, 4-neighbour steps, every
  aligned quadrant contiguous, fixed corners),
* brute-force set-builder forms of every 1-D rule on small axes,
* closed-form attended-pair counts,
* dense attention as a library routine when the window covers the grid,
* output = v and lse = scale q.k for a one-token window, rows summing to one.
"""
import json
import math
import os

import numpy as np
import pytest
from scipy.special import logsumexp, softmax

import oracle
from dimensional_sparse_local_amd import workloads as W


# ---------------------------------------------------------------------------
# Brute-force set builders written from the definitions (independent of the
# oracle's arithmetic: they search / filter instead of computing bounds).
# ---------------------------------------------------------------------------

def bf_window_clamp(L, w, x):
    """Of all windows of w consecutive positions inside [0, L), the one whose
    centre (start + w//2) is nearest x (neighbourhood attention)."""
    if w >= L:
        return list(range(L))
    best = min(range(0, L - w + 1), key=lambda s: abs(s + w // 2 - x))
    return list(range(best, best + w))


def bf_window_cut(L, left, right, x):
    """{j in [0, L) : -left <= j - x <= right} (Eq. 5 of the pi-Attention page
    generalised to unequal extents)."""
    return [j for j in range(L) if -left <= j - x <= right]


def bf_blocked(L, w, x):
    return [j for j in range(L) if j // w == x // w]


def bf_sta(L, tile, wt, x):
    """The wt consecutive tiles inside the axis whose middle tile is nearest the
    query's tile; all positions of those tiles."""
    T = -(-L // tile)
    if wt >= T:
        tiles = range(T)
    else:
        first = min(range(0, T - wt + 1), key=lambda s: abs(s + wt // 2 - x // tile))
        tiles = range(first, first + wt)
    return [j for j in range(L) if j // tile in tiles]


def bf_subgrid(L, dil, x, rule):
    """Dilation: run `rule(Lg, xl)` on the positions congruent to x mod dil."""
    sub = [j for j in range(L) if j % dil == x % dil]
    xl = sub.index(x)
    return [sub[t] for t in rule(len(sub), xl)]


def bf_grouped(L, stride, x, rule):
    """Stride: a group of `stride` positions uses its middle position's window."""
    leader = (x // stride) * stride + stride // 2
    return rule(L, leader)


# ---------------------------------------------------------------------------
# Hilbert curve
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("n", [1, 2, 4, 8, 16, 32, 128])
def test_hilbert_defining_properties(n):
    perm = oracle.hilbert(n)
    assert sorted(perm.tolist()) == list(range(n * n))           # bijection
    r, c = perm // n, perm % n
    steps = np.abs(np.diff(r)) + np.abs(np.diff(c))
    assert np.all(steps == 1)                                      # 4-neighbour steps
    assert (r[0], c[0]) == (0, 0) and (r[-1], c[-1]) == (0, n - 1)  # corners
    # every aligned 2^k x 2^k block is one contiguous, aligned run of the curve
    k = 1
    while k < n:
        blk = (r // k) * (n // k) + (c // k)
        runs = blk.reshape(-1, k * k)
        assert np.all(runs == runs[:, :1]), k
        k *= 2


# The classic Hilbert curve written out by hand ("Hilbert-Guided Sparse Local
# Attention", Methodology in Plain English: tokens are reordered along a
# Hilbert curve; the orientation is the reading that the curve starts at row 0,
# column 0 and ends at row 0, column n - 1, x = column, y = row).  On 4 x 4 the
# curve visits the 2 x 2 quadrants rows 0-1 / cols 0-1, rows 2-3 / cols 0-1,
# rows 2-3 / cols 2-3, rows 0-1 / cols 2-3 (a U), walking the first one along
# row 0 first and leaving the last one at row 0: perm[p] = row * 4 + col.
HILBERT_4X4 = [0, 1, 5, 4, 8, 12, 13, 9, 10, 14, 15, 11, 7, 6, 2, 3]


def test_hilbert_literal_4x4():
    assert oracle.hilbert(4).tolist() == HILBERT_4X4
    # the generalised curve reduces to the same literal order on this square
    assert oracle.hilbert_grid(4, 4).tolist() == HILBERT_4X4


def test_hilbert_literal_128_ends():
    # 128 x 128: the curve opens with (0,0), (1,0), (1,1), (0,1) (row, col):
    # a 2 x 2 block walked down, right, up, since an odd number of levels
    # (7) transposes the first block; it closes at row 0, column 127.
    perm = oracle.hilbert(128)
    assert perm[:4].tolist() == [0, 128, 129, 1]
    assert int(perm[-1]) == 127


def test_hilbert_invalid_side():
    with pytest.raises(ValueError):
        oracle.hilbert(96)


# The generalised curve (any rows x cols grid) is a reading: the pages name no
# curve for the 56x56 and 96x96 inputs of the Hilbert page's Tables 1 and 3.
# What pins it: it is the classic curve above on power-of-two squares, and on
# every grid it has the properties that make it a Hilbert-type order.

@pytest.mark.parametrize("n", [1, 2, 4, 8, 16, 32, 64, 128])
def test_hilbert_grid_reduces_to_classic(n):
    assert np.array_equal(oracle.hilbert_grid(n, n), oracle.hilbert(n))


def _four_neighbour_path_exists(rows, cols):
    """Parity argument: colour cell (r, c) by (r + c) % 2.  A 4-neighbour path
    alternates colours, so a path through all rows*cols cells from (0, 0) to
    (0, cols-1) needs the two ends to differ in colour when rows*cols is even
    (cols even) and to share the majority colour when it is odd (cols odd, rows
    odd).  With one column the path simply runs down."""
    return cols == 1 or cols % 2 == 0 or rows % 2 == 1


@pytest.mark.parametrize("rows", list(range(1, 21)) + [56, 96])
def test_hilbert_grid_properties(rows):
    for cols in list(range(1, 21)) + [56, 96]:
        perm = oracle.hilbert_grid(rows, cols)
        assert sorted(perm.tolist()) == list(range(rows * cols)), (rows, cols)   # bijection
        r, c = perm // cols, perm % cols
        dr, dc = np.abs(np.diff(r)), np.abs(np.diff(c))
        assert np.all(np.maximum(dr, dc) == 1), (rows, cols)    # every step to an adjacent cell
        diagonal = int(np.sum((dr == 1) & (dc == 1)))
        assert diagonal == (0 if _four_neighbour_path_exists(rows, cols) else 1), (rows, cols)
        assert (r[0], c[0]) == (0, 0)
        if cols >= 2:
            assert (r[-1], c[-1]) == (0, cols - 1), (rows, cols)


@pytest.mark.parametrize("rows,cols", [(96, 96), (56, 56), (100, 60), (30, 200), (97, 61)])
def test_hilbert_grid_locality(rows, cols):
    """Every run of L consecutive cells lies in a bounding box of at most 3L cells
    (the classic curve on 128 x 128 stays under 2L for these L)."""
    perm = oracle.hilbert_grid(rows, cols)
    r, c = perm // cols, perm % cols
    for L in (16, 49, 64):
        for s in range(0, rows * cols - L + 1, 3):
            rr, cc = r[s:s + L], c[s:s + L]
            assert (np.ptp(rr) + 1) * (np.ptp(cc) + 1) <= 3 * L, (rows, cols, L, s)


# ---------------------------------------------------------------------------
# 1-D rules against brute force
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("L", [1, 2, 5, 9, 16, 23])
def test_rule_na_clamp(L):
    for w in [1, 2, 3, 4, 5, 7, 30]:
        for x in range(L):
            got = oracle.rule_set(dict(kind="na", window=[w]), 0, L, x).tolist()
            assert got == bf_window_clamp(L, w, x), (L, w, x)
            if w <= L:
                assert len(got) == w and x in got


@pytest.mark.parametrize("L", [1, 2, 5, 9, 16, 23])
def test_rule_sa_cut(L):
    for w in [1, 2, 3, 4, 5, 7, 30]:
        for x in range(L):
            got = oracle.rule_set(dict(kind="sa", window=[w]), 0, L, x).tolist()
            assert got == bf_window_cut(L, w // 2, w - 1 - w // 2, x), (L, w, x)


@pytest.mark.parametrize("L", [1, 3, 10, 37])
def test_rule_band_eq5(L):
    for left, right in [(0, 0), (1, 1), (3, 0), (0, 2), (4, 4), (40, 40), (5, 2)]:
        for x in range(L):
            got = oracle.rule_set(dict(kind="band", left=left, right=right), 0, L, x).tolist()
            assert got == bf_window_cut(L, left, right, x)
    # Eq. 5 literally: causal {j : max(0, i-k) <= j <= i}; bidirectional |j-i| <= k
    k = 3
    for x in range(L):
        causal = oracle.rule_set(dict(kind="band", left=k, right=0), 0, L, x).tolist()
        assert causal == [j for j in range(L) if max(0, x - k) <= j <= x]
        bid = oracle.rule_set(dict(kind="band", left=k, right=k), 0, L, x).tolist()
        assert bid == [j for j in range(L) if abs(j - x) <= k]


@pytest.mark.parametrize("L", [1, 4, 10, 17])
def test_rule_blocked(L):
    for w in [1, 2, 3, 4, 8]:
        for x in range(L):
            got = oracle.rule_set(dict(kind="blocked", window=[w]), 0, L, x).tolist()
            assert got == bf_blocked(L, w, x)
            # blocked == window of w with stride w, cut at the ends
            strided = oracle.rule_set(dict(kind="sa", window=[w], stride=[w]), 0, L, x).tolist()
            assert strided == got, (L, w, x)


def bf_shifted_blocked(L, w, shift, x):
    """Windows [k*w - shift, (k+1)*w - shift) as a partition: same window index."""
    return [j for j in range(L) if (j + shift) // w == (x + shift) // w]


def cyclic_shift_windows(L, w, s):
    """Shifted windows built the way Swin builds them: roll the sequence back by s,
    cut windows of w, and mask pairs whose tokens came from different segments
    of the unrolled sequence (the wrapped tail).  Returns the key sets per
    query.  L must be a multiple of w."""
    rolled = [(p + s) % L for p in range(L)]          # rolled slot t holds token rolled[t]
    label = [0 if t < L - s else 1 for t in range(L)]  # wrapped tokens form their own segment
    keys = {x: [] for x in range(L)}
    for t in range(L):
        for u in range(L):
            if t // w == u // w and label[t] == label[u]:
                keys[rolled[t]].append(rolled[u])
    return {x: sorted(v) for x, v in keys.items()}


@pytest.mark.parametrize("L", [1, 4, 10, 17, 24])
def test_rule_shifted_blocked(L):
    for w in [1, 2, 3, 4, 8]:
        for shift in range(w):
            pat = dict(kind="blocked", window=[w], shift=[shift])
            for x in range(L):
                got = oracle.rule_set(pat, 0, L, x).tolist()
                assert got == bf_shifted_blocked(L, w, shift, x), (L, w, shift, x)
                # the same windows as a window of w with stride w and shifted groups
                strided = oracle.rule_set(dict(kind="sa", window=[w], stride=[w], shift=[shift]),
                                          0, L, x).tolist()
                assert strided == got, (L, w, shift, x)


@pytest.mark.parametrize("L,w", [(16, 4), (24, 8), (64, 16), (30, 6)])
def test_shifted_windows_equal_cyclic_shift_with_mask(L, w):
    """Shift s by roll-and-mask equals truncated windows whose boundaries sit at
    positions congruent to s (phase w - s); at s = w / 2 the two phases agree."""
    for s in range(1, w):
        ref = cyclic_shift_windows(L, w, s)
        pat = dict(kind="blocked", window=[w], shift=[w - s])
        for x in range(L):
            assert oracle.rule_set(pat, 0, L, x).tolist() == ref[x], (L, w, s, x)


@pytest.mark.parametrize("L,tile,wt", [(30, 6, 3), (48, 8, 5), (80, 8, 7), (10, 4, 1),
                                       (10, 4, 2), (12, 3, 5), (7, 2, 9)])
def test_rule_sta(L, tile, wt):
    for x in range(L):
        got = oracle.rule_set(dict(kind="sta", tile=[tile], window_tiles=[wt]), 0, L, x).tolist()
        assert got == bf_sta(L, tile, wt, x), (L, tile, wt, x)
        if L % tile == 0:
            # with whole tiles, STA == neighbourhood window of wt*tile positions
            # with stride = tile (the strided-window reading)
            na = oracle.rule_set(dict(kind="na", window=[wt * tile], stride=[tile]), 0, L,
                                 x).tolist()
            assert na == got, (L, tile, wt, x)


@pytest.mark.parametrize("L", [5, 12, 19])
def test_rule_stride_and_dilation(L):
    for w in [1, 3, 4, 5]:
        for s in [1, 2, 3, 4]:
            for dil in [1, 2, 3]:
                for kind in ["na", "sa"]:
                    pat = dict(kind=kind, window=[w], stride=[s], dilation=[dil])
                    if kind == "na":
                        base = lambda Lg, y: bf_window_clamp(Lg, w, y)
                    else:
                        base = lambda Lg, y: bf_window_cut(Lg, w // 2, w - 1 - w // 2, y)
                    for x in range(L):
                        got = oracle.rule_set(pat, 0, L, x).tolist()
                        want = bf_subgrid(
                            L, dil, x,
                            lambda Lg, xl: [t for t in bf_grouped(Lg, s, xl, base)
                                            if 0 <= t < Lg])
                        assert got == want, (kind, L, w, s, dil, x)


def bf_causal(L, w, stride, x):
    """Causal window of w positions as a filter: the keys j with
    0 <= last - j < w, where `last` is the final position of x's group of
    `stride` (block-causal: a chunk sees itself and the w - stride positions
    before it; stride 1 is Eq. 5 of the pi-Attention page with k = w - 1)."""
    last = (x // stride) * stride + stride - 1
    return [j for j in range(L) if 0 <= last - j < w]


@pytest.mark.parametrize("L", [1, 6, 13])
def test_rule_causal(L):
    for w in [1, 2, 3, 5, 8]:
        for s in range(1, w + 1):
            for x in range(L):
                got = oracle.rule_set(dict(kind="na", window=[w], stride=[s], causal=[1]), 0, L,
                                      x).tolist()
                assert got == bf_causal(L, w, s, x), (L, w, s, x)
                assert x in got  # every position sees itself
                if s == 1:
                    band = oracle.rule_set(dict(kind="band", left=w - 1, right=0), 0, L, x)
                    assert got == band.tolist()


def test_neighbors_nd_causal_in_time():
    """Video-style 3-D window: causal in time (first axis), neighbourhood in
    space, as the product of the per-axis sets."""
    wl = dict(grid=[6, 5, 7], pattern=dict(kind="na", window=[3, 3, 5], causal=[1, 0, 0]))
    for i in range(0, 210, 7):
        c0, c1, c2 = i // 35, (i // 7) % 5, i % 7
        want = sorted((a * 5 + b) * 7 + c
                      for a in bf_causal(6, 3, 1, c0)
                      for b in bf_window_clamp(5, 3, c1)
                      for c in bf_window_clamp(7, 5, c2))
        assert oracle.neighbors(wl, i).tolist() == want


def test_neighbors_nd_is_product():
    wl = dict(grid=[5, 6, 7], pattern=dict(kind="na", window=[3, 5, 3]))
    for i in [0, 17, 100, 209]:
        c0, c1, c2 = i // 42, (i // 7) % 6, i % 7
        want = sorted((a * 6 + b) * 7 + c
                      for a in bf_window_clamp(5, 3, c0)
                      for b in bf_window_clamp(6, 5, c1)
                      for c in bf_window_clamp(7, 3, c2))
        assert oracle.neighbors(wl, i).tolist() == want


def test_neighbors_hilbert_on_curve_positions():
    wl = dict(grid=[8, 8], order="hilbert", pattern=dict(kind="band", left=3, right=3))
    perm = oracle.hilbert(8)
    pos = np.argsort(perm)
    for i in range(64):
        want = sorted(int(perm[p]) for p in range(64) if abs(p - pos[i]) <= 3)
        assert oracle.neighbors(wl, i).tolist() == want


def test_tiled_order():
    wl = dict(grid=[4, 4, 6], order="tiled", tile=[2, 2, 3],
              pattern=dict(kind="sta", tile=[2, 2, 3], window_tiles=[1, 1, 1]))
    perm = oracle.order(wl)
    assert sorted(perm.tolist()) == list(range(96))
    # each run of 12 positions is one whole 2x2x3 tile, row-major inside
    for t in range(8):
        run = perm[t * 12:(t + 1) * 12]
        a, b, c = run // 24, (run // 6) % 4, run % 6
        assert len(set(zip(a // 2, b // 2, c // 3))) == 1
        assert np.all(np.diff(run) > 0)


# ---------------------------------------------------------------------------
# Closed-form attended-pair counts
# ---------------------------------------------------------------------------

def test_pairs_closed_forms():
    # NA with w <= L on every axis: every query sees prod(w) keys
    assert oracle.attended_pairs(dict(grid=[8, 8], pattern=dict(kind="na", window=[3, 3]))) \
        == 64 * 9
    assert oracle.attended_pairs(dict(grid=[64, 64], pattern=dict(kind="na", window=[13, 13]))) \
        == 4096 * 169
    # bidirectional band of radius r: n(2r+1) - r(r+1)
    for n, r in [(100, 7), (16384, 256), (9, 4)]:
        assert oracle.attended_pairs(dict(grid=[n], pattern=dict(kind="band", left=r, right=r))) \
            == n * (2 * r + 1) - r * (r + 1)
    # causal window of W keys including self: W(W+1)/2 + (N-W)W
    for n, wk in [(50, 8), (32768, 4096)]:
        assert oracle.attended_pairs(
            dict(grid=[n], pattern=dict(kind="band", left=wk - 1, right=0))) \
            == wk * (wk - 1) // 2 + wk + (n - wk) * wk


@pytest.mark.slow
def test_pairs_sta_headline():
    wl = W.CONFIGS["sta3d_bf16"]
    # every query attends 3*6 x 5*8 x 7*8 = 40320 keys = 35.00% of 115200
    assert oracle.attended_pairs(wl) == 115200 * 40320
    assert 40320 / 115200 == 0.35


# ---------------------------------------------------------------------------
# Tile classes: pages' tables, brute force, worked example
# ---------------------------------------------------------------------------

def test_page_block_sparsity(golden_dir):
    data = json.load(open(os.path.join(golden_dir, "hilbert_block_sparsity.json")))
    for case in data["cases"]:
        wl = dict(grid=case["grid"], order=case["order"], pattern=case["pattern"])
        cls, _ = oracle.tile_classes(wl, case["block"], case["block"])
        pct = 100.0 * float((cls == 0).sum()) / cls.size
        assert round(pct, 2) == case["empty_pct"], (case["label"], pct)


def _bf_classes(wl, qb, kb):
    n = oracle.num_tokens(wl)
    perm = oracle.order(wl)
    pos = np.argsort(perm)
    mask = np.zeros((n, n), dtype=bool)      # in sequence positions
    for i in range(n):
        for j in oracle.neighbors(wl, i):
            mask[pos[i], pos[j]] = True
    nq, nk = -(-n // qb), -(-n // kb)
    cls = np.zeros((nq, nk), dtype=np.uint8)
    for a in range(nq):
        for b in range(nk):
            blk = mask[a * qb:(a + 1) * qb, b * kb:(b + 1) * kb]
            cls[a, b] = 2 if blk.all() else (1 if blk.any() else 0)
    return cls


@pytest.mark.parametrize("wl,qb,kb", [
    (dict(grid=[8, 8], pattern=dict(kind="na", window=[3, 3])), 16, 16),
    (dict(grid=[7, 9], pattern=dict(kind="sa", window=[5, 3])), 8, 4),
    (dict(grid=[5, 4, 6], pattern=dict(kind="na", window=[3, 3, 5])), 12, 7),
    (dict(grid=[100], pattern=dict(kind="band", left=9, right=0)), 16, 8),
    (dict(grid=[16, 16], order="hilbert", pattern=dict(kind="band", left=7, right=7)), 16, 8),
    (dict(grid=[6, 8, 8], order="tiled", tile=[2, 4, 4],
          pattern=dict(kind="sta", tile=[2, 4, 4], window_tiles=[1, 1, 3])), 32, 16),
    (dict(grid=[6, 8, 8], order="tiled", tile=[2, 4, 4],
          pattern=dict(kind="sta", tile=[2, 4, 4], window_tiles=[1, 1, 3])), 24, 20),
])
def test_tile_classes_bruteforce(wl, qb, kb):
    cls, pairs = oracle.tile_classes(wl, qb, kb)
    assert np.array_equal(cls, _bf_classes(wl, qb, kb))
    assert pairs == oracle.attended_pairs(wl)


def test_worked_example(golden_dir):
    ex = json.load(open(os.path.join(golden_dir, "worked_example_4x4.json")))
    rep = ex["reproduced"]

    def counts(wl):
        c, _ = oracle.tile_classes(wl, 4, 4)
        return int((c == 0).sum()), int((c == 1).sum()), int((c == 2).sum())

    # slide half: reproduced exactly
    e0, p0, f0 = counts(dict(grid=[4, 4], pattern=dict(kind="na", window=[3, 3])))
    e1, p1, f1 = counts(dict(grid=[4, 4], order="hilbert", pattern=dict(kind="na", window=[9])))
    assert (e0, e1) == (rep["slide_empty_rowmajor"], rep["slide_empty_hilbert"])
    assert p0 / (p0 + f0) == rep["slide_partial_ratio_rowmajor"]
    assert p1 / (p1 + f1) == rep["slide_partial_ratio_hilbert"]
    # window half: the printed 0% -> 50% is not reachable; assert what the
    # definitions give (50% -> 75% empty)
    assert counts(dict(grid=[4, 4], pattern=dict(kind="blocked", window=[2, 2]))) == (8, 8, 0)
    assert counts(dict(grid=[4, 4], order="hilbert",
                       pattern=dict(kind="blocked", window=[4]))) == (12, 0, 4)


def test_config_tile_maps_small():
    # class counts at the kernel blocks for the two small 2-D configs
    c, p = oracle.tile_classes(W.CONFIGS["na2d_fp32"], 16, 16)
    assert [(c == k).sum() for k in range(3)] == [6, 10, 0] and p == 576
    c, p = oracle.tile_classes(W.CONFIGS["na2d_bf16"], 128, 64)
    assert [(c == k).sum() for k in range(3)] == [1606, 442, 0] and p == 692224


# ---------------------------------------------------------------------------
# Attention values
# ---------------------------------------------------------------------------

def _rand(shape, seed, bf16=False):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal(shape).astype(np.float32)
    if bf16:  # round to nearest even into bf16 bit patterns
        u = x.view(np.uint32).astype(np.uint64)
        u = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
        return u.astype(np.uint16)
    return x


def _as_f64(x):
    if x.dtype == np.uint16:
        return (x.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return x.astype(np.float64)


@pytest.mark.parametrize("bf16", [False, True])
def test_dense_special_case(bf16):
    """Window covering the whole grid == textbook softmax(QK^T scale) V
    ("pi-Attention", Eq. 1) computed with library routines."""
    B, H, D = 2, 3, 16
    wl = dict(grid=[5, 6], pattern=dict(kind="na", window=[5, 6]))
    N = 30
    q, k, v = (_rand((B, H, N, D), s, bf16) for s in (1, 2, 3))
    scale = 0.37
    out, lse = oracle.attention(wl, q, k, v, scale)
    qf, kf, vf = _as_f64(q), _as_f64(k), _as_f64(v)
    logits = np.matmul(qf, np.swapaxes(kf, -1, -2)) * scale
    ref = np.matmul(softmax(logits, axis=-1), vf)
    assert np.max(np.abs(out - ref)) < 1e-12
    assert np.max(np.abs(lse - logsumexp(logits, axis=-1))) < 1e-12
    # also as a band covering everything, and in Hilbert order
    out2, _ = oracle.attention(dict(grid=[30], pattern=dict(kind="band", left=40, right=40)),
                               q, k, v, scale)
    assert np.max(np.abs(out2 - ref)) < 1e-12


def test_one_token_window():
    B, H, D = 1, 2, 8
    wl = dict(grid=[4, 5], pattern=dict(kind="na", window=[1, 1]))
    q, k, v = (_rand((B, H, 20, D), s) for s in (4, 5, 6))
    out, lse = oracle.attention(wl, q, k, v, 0.5)
    assert np.array_equal(out, v.astype(np.float64))          # exact
    want = 0.5 * np.sum(q.astype(np.float64) * k.astype(np.float64), axis=-1)
    assert np.max(np.abs(lse - want)) < 1e-12


def test_rows_sum_to_one():
    wl = dict(grid=[6, 7], pattern=dict(kind="sa", window=[3, 5]))
    q, k = (_rand((1, 2, 42, 8), s) for s in (7, 8))
    v = np.ones((1, 2, 42, 8), dtype=np.float32)
    out, _ = oracle.attention(wl, q, k, v, 1.0)
    assert np.max(np.abs(out - 1.0)) < 1e-12


@pytest.mark.parametrize("wl", [
    dict(grid=[5, 7], pattern=dict(kind="na", window=[3, 5])),
    dict(grid=[6, 6], pattern=dict(kind="sa", window=[3, 3])),
    dict(grid=[40], pattern=dict(kind="band", left=7, right=0)),
    dict(grid=[4, 4, 4], order="tiled", tile=[2, 2, 2],
         pattern=dict(kind="sta", tile=[2, 2, 2], window_tiles=[1, 1, 1])),
    dict(grid=[8, 8], order="hilbert", pattern=dict(kind="band", left=5, right=5)),
    dict(grid=[9, 9], pattern=dict(kind="na", window=[3, 3], stride=[2, 1], dilation=[1, 2])),
])
def test_masked_dense_library(wl):
    """Masked dense attention with library softmax, mask from brute-force sets."""
    N = oracle.num_tokens(wl)
    q, k, v = (_rand((1, 2, N, 12), s) for s in (9, 10, 11))
    out, lse = oracle.attention(wl, q, k, v, 0.3)
    mask = np.zeros((N, N), dtype=bool)
    perm = oracle.order(wl)
    pos = np.argsort(perm)
    pat = wl["pattern"]
    grid = wl["grid"]
    for i in range(N):
        if wl.get("order") == "hilbert":
            keys = [perm[p] for p in range(N)
                    if -pat["left"] <= p - pos[i] <= pat["right"]]
        else:
            coords = np.unravel_index(i, grid)
            sets = []
            for d, L in enumerate(grid):
                x = int(coords[d])
                if pat["kind"] == "na":
                    s, dl, w = pat.get("stride", [1] * 3)[d], pat.get("dilation", [1] * 3)[d], \
                        pat["window"][d]
                    sets.append(bf_subgrid(L, dl, x, lambda Lg, xl: bf_grouped(
                        Lg, s, xl, lambda L2, y: bf_window_clamp(L2, w, min(y, L2 - 1)))))
                elif pat["kind"] == "sa":
                    w = pat["window"][d]
                    sets.append(bf_window_cut(L, w // 2, w - 1 - w // 2, x))
                elif pat["kind"] == "band":
                    sets.append(bf_window_cut(L, pat["left"], pat["right"], x))
                elif pat["kind"] == "sta":
                    sets.append(bf_sta(L, pat["tile"][d], pat["window_tiles"][d], x))
            keys = [int(np.ravel_multi_index(c, grid)) for c in np.array(
                np.meshgrid(*sets, indexing="ij")).reshape(len(grid), -1).T]
        mask[i, keys] = True
    logits = np.matmul(q.astype(np.float64), np.swapaxes(k.astype(np.float64), -1, -2)) * 0.3
    logits = np.where(mask, logits, -np.inf)
    ref = np.matmul(softmax(logits, axis=-1), v.astype(np.float64))
    assert np.max(np.abs(out - ref)) < 1e-12
    assert np.max(np.abs(lse - logsumexp(logits, axis=-1))) < 1e-12


def test_hilbert_direct_equals_permute_attend_unpermute():
    """Hilbert patterns evaluated directly on row-major data == gather into curve
    order, run the 1-D rule, scatter back."""
    wl = dict(grid=[16, 16], order="hilbert", pattern=dict(kind="band", left=9, right=9))
    q, k, v = (_rand((2, 1, 256, 8), s, bf16=True) for s in (12, 13, 14))
    out, lse = oracle.attention(wl, q, k, v, 0.25)
    perm = oracle.hilbert(16)
    seq = dict(grid=[256], pattern=dict(kind="band", left=9, right=9))
    o2, l2 = oracle.attention(seq, q[:, :, perm], k[:, :, perm], v[:, :, perm], 0.25)
    back = np.empty_like(o2)
    back[:, :, perm] = o2
    lback = np.empty_like(l2)
    lback[:, :, perm] = l2
    assert np.max(np.abs(out - back)) < 1e-13
    assert np.max(np.abs(lse - lback)) < 1e-13


def test_rows_subset_and_bf16_upcast():
    wl = dict(grid=[6, 6], pattern=dict(kind="na", window=[3, 3]))
    qb, kb, vb = (_rand((1, 2, 36, 8), s, bf16=True) for s in (15, 16, 17))
    full, lfull = oracle.attention(wl, qb, kb, vb, 0.5)
    rows = [35, 0, 17]
    part, lpart = oracle.attention(wl, qb, kb, vb, 0.5, rows=rows)
    assert np.array_equal(part, full[:, :, rows]) and np.array_equal(lpart, lfull[:, :, rows])
    # bf16 bits are read exactly: same as feeding their fp32 values
    f32 = [_as_f64(x).astype(np.float32) for x in (qb, kb, vb)]
    o2, _ = oracle.attention(wl, *f32, 0.5)
    assert np.array_equal(o2, full)


def test_torch_bf16_inputs_match_bits():
    torch = pytest.importorskip("torch")
    wl = W.scaled(W.CONFIGS["na2d_fp32"], dtype="bf16")
    q, k, v = W.make_qkv(wl)
    assert q.dtype == torch.bfloat16
    out, _ = oracle.attention(wl, q, k, v, 0.25, rows=[0, 63])
    f = [x.float().numpy() for x in (q, k, v)]
    o2, _ = oracle.attention(wl, *f, 0.25, rows=[0, 63])
    assert np.array_equal(out, o2)

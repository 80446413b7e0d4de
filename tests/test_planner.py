"""Host planner (through the C ABI, host-only plans) against the oracle.

Tile classes must match bit for bit; orders, pair counts and class counts
exactly.  No GPU is needed: plans are built with NA_PLAN_HOST_ONLY.
"""
import json
import os

import numpy as np
import pytest

import oracle
from dimensional_sparse_local_amd import na
from dimensional_sparse_local_amd import workloads as W

pytestmark = pytest.mark.skipif(not os.path.exists(na._LIB_PATH), reason="libna.so not built")


def _plan(wl, qb, kb, D=64, dtype="bf16"):
    wl = dict(wl)
    wl.setdefault("D", D)
    wl.setdefault("dtype", dtype)
    return na.Plan(wl, host_only=True, q_block=qb, kv_block=kb)


def _compare(wl, qb, kb):
    p = _plan(wl, qb, kb)
    want, pairs = oracle.tile_classes(wl, qb, kb)
    got = p.classes()
    assert got.shape == want.shape
    assert np.array_equal(got, want), "tile classes differ at %s" % (
        np.argwhere(got != want)[:5].tolist(),)
    st = p.stats
    assert st["attended_pairs"] == pairs
    assert (st["n_empty"], st["n_partial"], st["n_full"]) == tuple(
        int((want == c).sum()) for c in range(3))
    assert np.array_equal(p.order().astype(np.int64), oracle.order(wl))
    return p


@pytest.mark.parametrize("name", ["na2d_fp32", "na2d_bf16", "hilbert_band_bf16", "causal1d_bf16"])
def test_config_tile_maps(name):
    wl = W.CONFIGS[name]
    p = na.Plan(wl, host_only=True)           # library default blocks
    qb, kb = p.stats["q_block"], p.stats["kv_block"]
    _compare(wl, qb, kb)
    for qb2, kb2 in [(128, 64), (256, 64), (16, 16)]:
        if oracle.num_tokens(wl) <= 20000:
            _compare(wl, qb2, kb2)


@pytest.mark.slow
@pytest.mark.parametrize("qb", [128, 256])
def test_config_tile_map_sta(qb):
    wl = W.CONFIGS["sta3d_bf16"]
    p = _compare(wl, qb, 64)
    st = p.stats
    assert st["attended_pairs"] == 115200 * 40320
    if 384 % qb == 0:
        # query block divides the 6x8x8 tile: no partial tiles, 105 of 300
        # tiles attended by every query tile (35%)
        assert st["n_partial"] == 0
        assert st["n_full"] == (115200 // qb) * (105 * 384 // 64)
    else:
        # a query block straddling two tiles sees the union of their windows
        assert st["n_partial"] > 0


def test_config_class_counts():
    # counts of the benchmark workloads at 128-query, 64-key tiles
    expect = {"na2d_bf16": (1606, 442, 0, 692224),
              "hilbert_band_bf16": (31500, 504, 764, 8339200),
              "causal1d_bf16": (115232, 960, 14880, 125831168)}
    for name, (e, p_, f, pairs) in expect.items():
        st = na.Plan(W.CONFIGS[name], host_only=True, q_block=128, kv_block=64).stats
        assert (st["n_empty"], st["n_partial"], st["n_full"], st["attended_pairs"]) == \
            (e, p_, f, pairs), name


def test_page_tables_through_planner(golden_dir):
    data = json.load(open(os.path.join(golden_dir, "hilbert_block_sparsity.json")))
    for case in data["cases"]:
        wl = dict(grid=case["grid"], order=case["order"], pattern=case["pattern"])
        p = _compare(wl, case["block"], case["block"])
        pct = 100.0 * p.stats["n_empty"] / (p.stats["n_q_tiles"] * p.stats["n_kv_tiles"])
        assert round(pct, 2) == case["empty_pct"], case["label"]


@pytest.mark.parametrize("n", [1, 2, 4, 8, 16, 64, 128, 256])
def test_hilbert_order_matches_oracle(n):
    wl = dict(grid=[n, n], order="hilbert", pattern=dict(kind="band", left=1, right=1))
    p = _plan(wl, 16, 16)
    assert np.array_equal(p.order().astype(np.int64), oracle.hilbert(n))


def test_hilbert_order_literals():
    # the planner's curve against the hand-written classic order (4 x 4) and
    # the 128 x 128 curve's ends, the same literals the oracle is pinned to
    four = _plan(dict(grid=[4, 4], order="hilbert", pattern=dict(kind="band", left=1, right=1)), 16, 16)
    assert four.order().tolist() == [0, 1, 5, 4, 8, 12, 13, 9, 10, 14, 15, 11, 7, 6, 2, 3]
    big = _plan(dict(grid=[128, 128], order="hilbert", pattern=dict(kind="band", left=1, right=1)), 16, 16)
    perm = big.order()
    assert perm[:4].tolist() == [0, 128, 129, 1] and int(perm[-1]) == 127


def _random_workload(rng):
    kind = rng.choice(["na", "sa", "band", "blocked", "sta", "hilbert"])
    if kind == "band":
        n = int(rng.integers(1, 300))
        left, right = int(rng.integers(0, 40)), int(rng.integers(0, 40))
        return dict(grid=[n], pattern=dict(kind="band", left=left, right=right))
    if kind == "hilbert":
        if rng.random() < 0.3:
            grid = [int(2 ** rng.integers(1, 5))] * 2
        else:
            grid = [int(rng.integers(1, 14)), int(rng.integers(1, 14))]
        sub = rng.choice(["band", "blocked", "na"])
        if sub == "band":
            r = int(rng.integers(0, 20))
            pat = dict(kind="band", left=r, right=int(rng.integers(0, 20)))
        elif sub == "blocked":
            w = int(rng.integers(1, 20))
            pat = dict(kind="blocked", window=[w], shift=[int(rng.integers(0, w))])
        else:
            pat = dict(kind="na", window=[int(rng.integers(1, 30))])
        return dict(grid=grid, order="hilbert", pattern=pat)
    ndim = int(rng.integers(1, 4))
    grid = [int(rng.integers(1, 12)) for _ in range(ndim)]
    if kind == "sta":
        tile = [int(rng.integers(1, 4)) for _ in range(ndim)]
        grid = [t * int(rng.integers(1, 5)) for t in tile]
        wt = [int(rng.integers(1, 4)) for _ in range(ndim)]
        order = "tiled" if rng.random() < 0.7 else "row_major"
        return dict(grid=grid, order=order, tile=tile,
                    pattern=dict(kind="sta", tile=tile, window_tiles=wt))
    window = [int(rng.integers(1, g + 3)) for g in grid]
    pat = dict(kind=kind, window=window)
    if kind in ("na", "sa"):
        pat["stride"] = [int(rng.integers(1, min(3, w) + 1)) for w in window]
        pat["shift"] = [int(rng.integers(0, st)) for st in pat["stride"]]
        pat["dilation"] = [int(rng.integers(1, 3)) for _ in grid]
        pat["causal"] = [int(rng.random() < 0.3) for _ in grid]
    if kind == "blocked":
        pat["shift"] = [int(rng.integers(0, w)) for w in window]
    wl = dict(grid=grid, pattern=pat)
    if rng.random() < 0.3:
        wl["order"] = "tiled"
        wl["tile"] = [int(rng.integers(1, 4)) for _ in grid]
    return wl


def test_random_tiny_workloads():
    rng = np.random.default_rng(1234)
    for it in range(300):
        wl = _random_workload(rng)
        n = oracle.num_tokens(wl)
        qb = int(rng.integers(1, max(2, n // 2 + 2)))
        kb = int(rng.integers(1, max(2, n // 2 + 2)))
        try:
            _compare(wl, qb, kb)
        except AssertionError as e:
            raise AssertionError("workload %r qb=%d kb=%d: %s" % (wl, qb, kb, e))


@pytest.mark.parametrize("rows", list(range(1, 26)) + [56, 96])
def test_hilbert_order_any_grid_matches_oracle(rows):
    for cols in list(range(1, 26)) + [56, 96]:
        wl = dict(grid=[rows, cols], order="hilbert", pattern=dict(kind="band", left=1, right=1))
        p = _plan(wl, 16, 16)
        assert np.array_equal(p.order().astype(np.int64), oracle.hilbert_grid(rows, cols)), \
            (rows, cols)


def test_hilbert_needs_2d_grid():
    for grid in ([64], [4, 4, 4]):
        wl = dict(grid=grid, order="hilbert", pattern=dict(kind="band", left=5, right=5),
                  D=64, dtype="bf16")
        with pytest.raises(na.NaError) as ei:
            na.Plan(wl, host_only=True)
        assert ei.value.status == na.NA_ERR_UNSUPPORTED


@pytest.mark.parametrize("field,value", [
    ("ndim", 0), ("ndim", 4), ("grid", [0, 4, 1]), ("order", 7), ("dtype", 9), ("head_dim", 0),
    ("window", [0, 3, 1]), ("stride", [3, 0, 1]), ("dilation", [1, 0, 1]), ("causal", [2, 0, 0]),
    ("boundary", [5, 0, 0]), ("window_left", [-3, -1, -1]), ("q_block", -1), ("kv_block", -5),
    ("stride", [4, 1, 1]), ("shift", [1, 0, 0]), ("shift", [-1, 0, 0]),
])
def test_invalid_descriptors(field, value):
    d = na.desc_from_workload(dict(grid=[4, 4], pattern=dict(kind="na", window=[3, 3]), D=64,
                                   dtype="bf16"))
    if isinstance(value, list):
        for i, x in enumerate(value):
            getattr(d, field)[i] = x
    else:
        setattr(d, field, value)
    with pytest.raises(na.NaError) as ei:
        na.Plan(d, host_only=True)
    assert ei.value.status == na.NA_ERR_INVALID_ARG


def test_tiled_needs_tiles():
    d = na.desc_from_workload(dict(grid=[4, 4], order="tiled", tile=[2, 2],
                                   pattern=dict(kind="na", window=[3, 3]), D=64, dtype="bf16"))
    d.tile[1] = 0
    with pytest.raises(na.NaError) as ei:
        na.Plan(d, host_only=True)
    assert ei.value.status == na.NA_ERR_INVALID_ARG


def test_causal_flag_equals_left_extent():
    base = dict(grid=[200], D=64, dtype="bf16")
    a = na.desc_from_workload(dict(base, pattern=dict(kind="band", left=19, right=0)))
    b = na.desc_from_workload(dict(base, pattern=dict(kind="na", window=[20])))
    b.causal[0] = 1
    pa, pb = na.Plan(a, host_only=True), na.Plan(b, host_only=True)
    assert np.array_equal(pa.classes(), pb.classes())
    assert pa.stats == pb.stats


def test_host_only_plan_cannot_run():
    torch = pytest.importorskip("torch")
    p = na.Plan(W.CONFIGS["na2d_bf16"], host_only=True)
    t = na.Tensor(16, 0, 0, 64)
    st = na.lib().na_forward(p._h, 1, 1, t, t, t, t, None, 0.1, 0, None, 0, None)
    assert st == na.NA_ERR_PLAN_MISMATCH
    del torch


def test_hilbert_page_workloads_reproduce_printed_sparsity():
    """At the page's block size (128 x 128) the workloads built for the Hilbert
    page's Tables 1-3 have the empty-block ratios printed there: HWA 96x96 8x8
    98.61 %, HWA 128x128 16x16 98.44 %, HSA 96x96 95.87 %."""
    printed = {"hwa96_bf16": 98.61, "hwa128_bf16": 98.44, "hsa96_bf16": 95.87}
    for name, pct in printed.items():
        st = na.Plan(W.HILBERT_PAGE[name], host_only=True, q_block=128, kv_block=128).stats
        assert round(100.0 * st["n_empty"] / (st["n_q_tiles"] * st["n_kv_tiles"]), 2) == pct, name


def test_block_causal_video_closed_form():
    """STA causal in time: the first 6-frame chunk sees 6 frames, the other
    four see 12; in space every query sees 3x5 whole 8x8 tiles (24 x 40,
    shifted inside).  Pairs per head = 3840 * (6 * 6 * 960 + 24 * 12 * 960)."""
    wl = W.GNA["sta3d_causal_t_bf16"]
    st = na.Plan(wl, host_only=True, q_block=128, kv_block=64).stats
    assert st["attended_pairs"] == 48 * 80 * (6 * 6 * 960 + 24 * 12 * 960) == 1194393600
    # tile-aligned: every visited tile pair is full (a query tile lies in one
    # 384-token tile whose key tiles are all attended or all not)
    assert st["n_partial"] == 0
    # per query tile: chunk 0 attends 1 chunk, the others 2, each of 15 spatial tiles
    # of 6 key tiles (64 keys) per 384-token tile
    assert st["n_full"] == 3 * 60 * (1 * 15 * 6) + 3 * 240 * (2 * 15 * 6)


def test_patch_order_same_neighbourhoods_denser_tiles():
    """8x8 patch order for the 64x64 13x13 neighbourhood workload: identical
    neighbourhoods (pairs), 308 instead of 442 visited tile pairs."""
    a = na.Plan(W.CONFIGS["na2d_bf16"], host_only=True, q_block=128, kv_block=64)
    b = na.Plan(W.GNA["na2d_tiled_bf16"], host_only=True, q_block=128, kv_block=64)
    assert a.stats["attended_pairs"] == b.stats["attended_pairs"] == 692224
    assert a.stats["n_partial"] + a.stats["n_full"] == 442
    assert b.stats["n_partial"] + b.stats["n_full"] == 308


def test_speedup_bounds():
    # perfectly block-sparse: the tile bound equals the flop bound, 115200 / 40320
    sb = na.Plan(W.CONFIGS["sta3d_bf16"], host_only=True, q_block=128).speedup_bounds()
    assert sb["flop"] == pytest.approx(115200 / 40320) and sb["tile"] == pytest.approx(300 / 105)
    assert sb["useful_fraction"] == 1.0
    # row-major neighbourhood attention: flop bound 4096^2 / 692224, tile bound
    # 32 * 64 / 442; useful fraction 692224 / (442 * 128 * 64)
    sb = na.Plan(W.CONFIGS["na2d_bf16"], host_only=True, q_block=128).speedup_bounds()
    assert sb["flop"] == pytest.approx(4096 ** 2 / 692224)
    assert sb["tile"] == pytest.approx(2048 / 442)
    assert sb["useful_fraction"] == pytest.approx(692224 / (442 * 128 * 64))
    # ragged tiles count at their true size: a dense 100-token window
    sb = na.Plan(dict(grid=[100], pattern=dict(kind="band", left=100, right=100), D=64,
                      dtype="bf16"), host_only=True, q_block=128).speedup_bounds()
    assert sb == {"flop": 1.0, "tile": 1.0, "useful_fraction": 1.0}


def test_speedup_bounds_match_class_matrix():
    # the C call against the same bounds counted here from the class matrix
    rng = np.random.default_rng(5)
    for _ in range(40):
        n = int(rng.integers(1, 700))
        wl = dict(grid=[n], pattern=dict(kind="band", left=int(rng.integers(0, 90)),
                                         right=int(rng.integers(0, 90))), D=64, dtype="bf16")
        qb = int(rng.choice([64, 128, 256]))
        p = na.Plan(wl, host_only=True, q_block=qb)
        st, cls = p.stats, p.classes()
        qs = np.minimum(st["q_block"], n - np.arange(st["n_q_tiles"]) * st["q_block"])
        ks = np.minimum(st["kv_block"], n - np.arange(st["n_kv_tiles"]) * st["kv_block"])
        inside = int(np.sum(qs[:, None] * ks[None, :] * (cls != 0)))
        visited = int(np.count_nonzero(cls))
        got = p.speedup_bounds()
        assert got["flop"] == pytest.approx(n * n / st["attended_pairs"])
        assert got["tile"] == pytest.approx(cls.size / visited)
        assert got["useful_fraction"] == pytest.approx(st["attended_pairs"] / inside)


def test_pi_partner_tile_maps():
    """pi-Attention's partner (pi-Attention, Eqs. 8-9) in the tile map: union
    and fixed fusion put the partners into the map, the separate variant keeps
    the window's map and counts the partners as attended pairs."""
    rng = np.random.default_rng(77)
    for it in range(120):
        mode = ["union", "fixed_fusion", "separate"][it % 3]
        skip = int(rng.integers(1, 80))
        both = int(rng.integers(0, 2))
        if rng.random() < 0.3:
            side = int(rng.integers(2, 12))
            wl = dict(grid=[side, int(rng.integers(2, 12))], order="hilbert")
        else:
            wl = dict(grid=[int(rng.integers(1, 300))])
        base = rng.choice(["band", "na", "blocked"])
        if base == "band":
            pat = dict(kind="band", left=int(rng.integers(0, 20)), right=int(rng.integers(0, 5)))
        elif base == "na":
            pat = dict(kind="na", window=[int(rng.integers(1, 30))])
        else:
            pat = dict(kind="blocked", window=[int(rng.integers(1, 30))])
        pat.update(skip=skip, skip_both=both, skip_mode=mode, skip_prior=0.3)
        wl["pattern"] = pat
        n = oracle.num_tokens(wl)
        qb = int(rng.choice([16, 32, 64, 128]))
        kb = int(rng.choice([16, 32, 64]))
        try:
            _compare(wl, qb, kb)
        except AssertionError as e:
            raise AssertionError("workload %r qb=%d kb=%d: %s" % (wl, qb, kb, e))


@pytest.mark.parametrize("pattern,status", [
    (dict(kind="na", window=[3, 3], skip=4), "unsupported"),          # two pattern dimensions
    (dict(kind="na", window=[3, 3], skip=-1), "invalid"),
    (dict(kind="na", window=[3, 3], skip=4, skip_both=2), "invalid"),
])
def test_pi_partner_invalid_2d(pattern, status):
    d = na.desc_from_workload(dict(grid=[6, 6], pattern=pattern, D=64, dtype="bf16"))
    with pytest.raises(na.NaError) as ei:
        na.Plan(d, host_only=True)
    want = na.NA_ERR_UNSUPPORTED if status == "unsupported" else na.NA_ERR_INVALID_ARG
    assert ei.value.status == want


@pytest.mark.parametrize("prior", [0.0, 1.0, -0.5, float("nan")])
def test_pi_fixed_fusion_needs_prior_in_open_interval(prior):
    d = na.desc_from_workload(dict(grid=[64], D=64, dtype="bf16",
                                   pattern=dict(kind="band", left=4, right=0, skip=16,
                                                skip_mode="fixed_fusion", skip_prior=prior)))
    with pytest.raises(na.NaError) as ei:
        na.Plan(d, host_only=True)
    assert ei.value.status == na.NA_ERR_INVALID_ARG


@pytest.mark.parametrize("name", [n for n in list(W.HILBERT_PAGE) + list(W.GNA) + list(W.PI_ATTENTION)
                                  if n != "sta3d_causal_t_bf16"])
def test_named_workload_tile_maps(name):
    """Every named workload's tile map (classes, pair counts, order) equals the
    oracle's at the library's default tiles and at 64-query tiles."""
    wl = W.ALL[name]
    p = na.Plan(wl, host_only=True)
    _compare(wl, p.stats["q_block"], p.stats["kv_block"])
    _compare(wl, 64, 64)

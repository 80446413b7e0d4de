"""Seeded random sweep of the HIP kernels against the fp64 oracle.

Each case draws a grid of one to three dimensions (sizes unrelated to any
tile, down to a single token), a pattern (neighbourhood attention with
strides, stride phases, dilation and causal dimensions; slide attention;
blocked and shifted windows; 1-D bands; sliding tiles; Hilbert orders with a
1-D pattern on the curve; on 1-D and Hilbert patterns, pi-Attention's partner
in its union, fixed-fusion and separate-softmax forms), an order (row-major,
tiled with random tiles, Hilbert), a dtype and head_dim the kernels support
and one of the query tiles available for it. Every output element and every
lse is compared with the oracle at the parity tolerances (bf16: max-abs 2e-2,
relative L2 5e-3, lse 1e-3, with 2^-8 of the reference added elementwise for
the separate softmax, whose output is not bounded by max |v|; fp32: 1e-5).
Every third bf16 case whose query tile the gradients support also compares dq,
dk and dv (relative L2 1e-2, max-abs 2e-2 of the largest reference magnitude).
"""
import os

import numpy as np
import pytest

import oracle
from dimensional_sparse_local_amd import workloads as W

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

N_CASES = 160
TOL = {"fp32": dict(abs=1e-5, rel=None, lse=1e-5), "bf16": dict(abs=2e-2, rel=5e-3, lse=1e-3)}
Q_BLOCKS = {("bf16", 64): [64, 128, 192, 256], ("bf16", 128): [128, 192, 256, 384],
            ("fp32", 32): [0], ("fp32", 64): [0]}


def _na():
    from dimensional_sparse_local_amd import na

    if not os.path.exists(na._LIB_PATH):
        raise RuntimeError("libna.so missing: the HIP path must be built")
    return na


def _case(i):
    """Workload and query tile of case i (deterministic)."""
    rng = np.random.default_rng(7000 + i)
    dtype = "bf16" if rng.random() < 0.8 else "fp32"
    D = int(rng.choice([64, 128] if dtype == "bf16" else [32, 64]))
    q_block = int(rng.choice(Q_BLOCKS[(dtype, D)]))
    kind = str(rng.choice(["na", "sa", "blocked", "band", "sta", "hilbert"]))
    order, tile = "row_major", None
    if kind == "band":
        grid = [int(rng.integers(1, 1500))]
        pat = dict(kind="band", left=int(rng.integers(0, 300)), right=int(rng.integers(0, 300)))
    elif kind == "hilbert":
        grid = [int(rng.integers(1, 48)), int(rng.integers(1, 48))]
        order = "hilbert"
        sub = str(rng.choice(["band", "blocked", "na"]))
        if sub == "band":
            pat = dict(kind="band", left=int(rng.integers(0, 200)), right=int(rng.integers(0, 200)))
        elif sub == "blocked":
            w = int(rng.integers(1, 130))
            pat = dict(kind="blocked", window=[w], shift=[int(rng.integers(0, w))])
        else:
            pat = dict(kind="na", window=[int(rng.integers(1, 160))])
    elif kind == "sta":
        ndim = int(rng.integers(1, 4))
        tile = [int(rng.integers(1, 9)) for _ in range(ndim)]
        grid = [t * int(rng.integers(1, 5)) for t in tile]
        pat = dict(kind="sta", tile=tile, window_tiles=[int(rng.integers(1, 4)) for _ in range(ndim)])
        order = "tiled" if rng.random() < 0.7 else "row_major"
        if order == "row_major":
            tile = None
    else:
        ndim = int(rng.integers(1, 4))
        hi = {1: 900, 2: 40, 3: 14}[ndim]
        grid = [int(rng.integers(1, hi)) for _ in range(ndim)]
        window = [int(rng.integers(1, min(g + 3, 24))) for g in grid]
        pat = dict(kind=kind, window=window)
        if kind in ("na", "sa"):
            pat["stride"] = [int(rng.integers(1, min(3, w) + 1)) for w in window]
            pat["shift"] = [int(rng.integers(0, s)) for s in pat["stride"]]
            pat["dilation"] = [int(rng.integers(1, 3)) for _ in grid]
            pat["causal"] = [int(rng.random() < 0.3) for _ in grid]
        else:
            pat["shift"] = [int(rng.integers(0, w)) for w in window]
        if rng.random() < 0.3:
            order = "tiled"
            tile = [int(rng.integers(1, 5)) for _ in grid]
    if (len(grid) == 1 or order == "hilbert") and kind != "sta" and rng.random() < 0.4:
        # pi-Attention's partner on the 1-D pattern axis, in one of its three forms
        pat["skip"] = int(rng.integers(1, 300))
        pat["skip_both"] = int(rng.random() < 0.3)
        mode = str(rng.choice(["union", "fixed_fusion", "separate"]))
        if mode == "fixed_fusion" and (dtype != "bf16" or q_block in (192, 384)):
            mode = "union"   # the logit bias exists in the 32-query-per-wave bf16 kernels
        pat["skip_mode"] = mode
        if mode == "fixed_fusion":
            pat["skip_prior"] = float(rng.uniform(0.05, 0.95))
    wl = dict(name="random_%d" % i, B=int(rng.integers(1, 3)), H=int(rng.integers(1, 4)), D=D,
              dtype=dtype, grid=grid, order=order, pattern=pat, seed=9000 + i)
    if tile is not None:
        wl["tile"] = tile
    return wl, q_block


@pytest.mark.parametrize("i", range(N_CASES))
def test_random_case(i):
    na = _na()
    wl, q_block = _case(i)
    print("case %d: %s q_block=%d" % (i, {k: wl[k] for k in ("B", "H", "D", "dtype", "grid", "order",
                                                             "pattern")}, q_block), flush=True)
    plan = na.Plan(wl, q_block=q_block)
    q, k, v = W.make_qkv(wl, device="cuda")
    scale = W.default_scale(wl)
    # every other case asks for the split tail (a no-op where the launch has
    # no split mode); these small grids split every query tile
    out, lse = plan.forward(q, k, v, scale=scale, split_tail=i % 2 == 1)
    torch.cuda.synchronize()
    ref, ref_lse = oracle.attention(wl, q.cpu(), k.cpu(), v.cpu(), scale)
    t = TOL[wl["dtype"]]
    o = out.float().cpu().numpy().astype(np.float64)
    l = lse.cpu().numpy().astype(np.float64)
    assert np.all(np.isfinite(o))
    bound = t["abs"]
    if wl["pattern"].get("skip") and wl["pattern"]["skip_mode"] == "separate" and wl["dtype"] == "bf16":
        # the window branch's average plus a whole partner row: not bounded by
        # max |v|, each part rounded to bf16 once (2^-9 relative)
        bound = t["abs"] + 2.0 ** -8 * np.abs(ref)
    excess = float(np.max(np.abs(o - ref) - bound))
    assert excess <= 0, "error above bound by %.3e" % excess
    if t["rel"] is not None and np.linalg.norm(ref) > 0:
        rel = float(np.linalg.norm(o - ref) / np.linalg.norm(ref))
        assert rel <= t["rel"], "rel-L2 %.3e" % rel
    finite = np.isfinite(ref_lse)
    assert np.array_equal(np.isfinite(l), finite)
    if finite.any():
        assert float(np.max(np.abs(l[finite] - ref_lse[finite]))) <= t["lse"]
    if wl["dtype"] == "bf16" and plan.stats["q_block"] in (128, 256) and i % 3 == 0:
        g = W.make_dout(wl, device="cuda")
        grads = plan.backward(q, k, v, out, lse, g, scale=scale)
        torch.cuda.synchronize()
        refs = oracle.attention_backward(wl, q.cpu(), k.cpu(), v.cpu(), g.cpu(), scale)
        for name, got, want in zip(("dq", "dk", "dv"), grads, refs):
            a = got.float().cpu().numpy().astype(np.float64)
            nw = np.linalg.norm(want)
            if nw == 0:
                assert np.all(a == 0), name
                continue
            rel = float(np.linalg.norm(a - want) / nw)
            mx = float(np.max(np.abs(a - want)) / np.max(np.abs(want)))
            print("  %s rel-L2 %.2e max %.2e" % (name, rel, mx), flush=True)
            assert rel <= 1e-2 and mx <= 2e-2, name


def test_cases_are_valid_plans():
    """Every drawn workload is accepted by the planner (host-only plan): the
    sweep exercises kernels, not descriptor validation."""
    na = _na()
    for i in range(N_CASES):
        wl, q_block = _case(i)
        na.Plan(wl, q_block=q_block, host_only=True)

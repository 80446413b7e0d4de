"""GPU parity of the gradients: na_backward (through the C ABI) against the
fp64 oracle's gradients on the same bf16 bits of q, k, v and dout.

Tolerance (bf16): relative L2 error <= 1e-2 and max-abs error <= 2e-2 times
the largest reference magnitude, for each of dq, dk, dv.  Sources of error,
all from the bf16 arithmetic of the kernel: P and dS are rounded to bf16
(relative 2^-9 each) before their MFMA products; delta_i = dout_i . out_i is
taken from the bf16-rounded forward output (relative 2^-9 on out); S, dP and
the accumulations are fp32.  A rounding error of relative 2^-9 per term
leaves a relative L2 error of the sums of about 2^-9 ~ 2e-3; the bounds leave
a factor of five for the cancellation in dP - delta.
"""
import numpy as np
import pytest

import oracle
from dimensional_sparse_local_amd import workloads as W

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

REL_L2 = 1e-2
MAX_REL = 2e-2


def _na():
    from dimensional_sparse_local_amd import na

    return na


def _grad_case(wl, q_block=0, seed=None):
    na = _na()
    print("case %s grid=%s B=%d H=%d D=%d q_block=%d" % (wl["name"], wl["grid"], wl["B"], wl["H"],
                                                        wl["D"], q_block), flush=True)
    plan = na.Plan(wl, q_block=q_block)
    q, k, v = W.make_qkv(wl, device="cuda", seed=seed)
    g = W.make_dout(wl, device="cuda", seed=seed)
    scale = W.default_scale(wl)
    out, lse = plan.forward(q, k, v, scale=scale)
    dq, dk, dv = plan.backward(q, k, v, out, lse, g, scale=scale)
    torch.cuda.synchronize()
    ref = oracle.attention_backward(wl, q.cpu(), k.cpu(), v.cpu(), g.cpu(), scale)
    errs = {}
    for name, got, want in zip(("dq", "dk", "dv"), (dq, dk, dv), ref):
        a = got.float().cpu().numpy().astype(np.float64)
        assert np.all(np.isfinite(a)), "%s: %s not finite" % (wl["name"], name)
        top = np.max(np.abs(want))
        rel = np.linalg.norm(a - want) / max(np.linalg.norm(want), 1e-30)
        mx = np.max(np.abs(a - want)) / max(top, 1e-30)
        errs[name] = (rel, mx)
    print("  errors (rel-L2, max-abs / max|ref|): %s" % {k: ("%.2e" % r, "%.2e" % m)
                                                         for k, (r, m) in errs.items()}, flush=True)
    for name, (rel, mx) in errs.items():
        assert rel <= REL_L2 and mx <= MAX_REL, "%s %s: rel-L2 %.3e, max %.3e" % (wl["name"], name,
                                                                                 rel, mx)


SMALL = [
    W.scaled(W.CONFIGS["na2d_bf16"], name="na2d_small", B=1, H=2, grid=[24, 20],
             pattern=dict(kind="na", window=[7, 5])),
    W.scaled(W.CONFIGS["sta3d_bf16"], name="sta3d_small", H=2, grid=[12, 16, 24],
             pattern=dict(kind="sta", tile=[6, 8, 8], window_tiles=[1, 1, 3])),
    W.scaled(W.CONFIGS["sta3d_bf16"], name="sta3d_small_d64", H=1, D=64, grid=[6, 16, 40],
             pattern=dict(kind="sta", tile=[6, 8, 8], window_tiles=[1, 1, 3])),
    W.scaled(W.CONFIGS["hilbert_band_bf16"], name="hilbert_small", B=2, H=2, grid=[32, 32],
             pattern=dict(kind="band", left=37, right=37)),
    W.scaled(W.CONFIGS["causal1d_bf16"], name="causal_small", H=2, grid=[1000],
             pattern=dict(kind="band", left=99, right=0)),
    W.scaled(W.CONFIGS["causal1d_bf16"], name="causal_small_d64", H=2, D=64, grid=[333],
             pattern=dict(kind="band", left=70, right=0)),
    W.scaled(W.CONFIGS["na2d_bf16"], name="sa3d_ragged", B=1, H=1, grid=[5, 7, 9],
             pattern=dict(kind="sa", window=[3, 5, 3])),
    W.scaled(W.CONFIGS["na2d_bf16"], name="gna_stride_dil", B=1, H=2, grid=[19, 23],
             pattern=dict(kind="na", window=[7, 5], stride=[3, 2], dilation=[2, 1])),
    W.scaled(W.CONFIGS["na2d_bf16"], name="blocked_tiled", B=1, H=1, grid=[16, 16],
             order="tiled", tile=[4, 8], pattern=dict(kind="blocked", window=[4, 8])),
    W.scaled(W.CONFIGS["causal1d_bf16"], name="band_d128_ragged", H=2, grid=[3000],
             pattern=dict(kind="band", left=600, right=0)),
    W.scaled(W.CONFIGS["na2d_bf16"], name="na2d_d128_ragged", B=1, H=2, D=128, grid=[40, 50],
             pattern=dict(kind="na", window=[9, 11])),
]


@pytest.mark.parametrize("q_block", [128, 256])
@pytest.mark.parametrize("wl", SMALL, ids=[w["name"] for w in SMALL])
def test_backward_small(wl, q_block):
    _grad_case(wl, q_block=q_block)


def test_backward_empty_rows_and_unattended_keys():
    """Queries whose window excludes themselves (the first has none) and keys
    no query attends (the last): zero gradients there, parity elsewhere."""
    na = _na()
    wl = W.scaled(W.CONFIGS["causal1d_bf16"], name="strict_past", H=1, grid=[300],
                  pattern=dict(kind="band", left=10, right=0))
    d = na.desc_from_workload(wl)
    d.window[0] = 10
    d.window_left[0] = 10          # keys [x - 10, x - 1]
    plan = na.Plan(d)
    q, k, v = W.make_qkv(wl, device="cuda")
    g = W.make_dout(wl, device="cuda")
    out, lse = plan.forward(q, k, v, scale=0.1)
    dq, dk, dv = plan.backward(q, k, v, out, lse, g, scale=0.1)
    torch.cuda.synchronize()
    assert torch.all(dq[:, :, 0] == 0)
    assert torch.all(dk[:, :, -1] == 0) and torch.all(dv[:, :, -1] == 0)
    ref_wl = W.scaled(wl, pattern=dict(kind="band", left=10, right=-1))
    ref = oracle.attention_backward(ref_wl, q.cpu(), k.cpu(), v.cpu(), g.cpu(), 0.1)
    for got, want in zip((dq, dk, dv), ref):
        a = got.float().cpu().numpy()
        assert np.linalg.norm(a - want) / np.linalg.norm(want) <= REL_L2


def test_backward_full_size_na2d():
    _grad_case(W.CONFIGS["na2d_bf16"])


def test_backward_hilbert_full_grid():
    _grad_case(W.scaled(W.CONFIGS["hilbert_band_bf16"], name="hilbert_full_grid", B=1, H=2))


def _sample_rows(wl, n_random, seed=0):
    grid = wl["grid"]
    corners = set()
    for c in np.ndindex(*([2] * len(grid))):
        corners.add(int(np.ravel_multi_index([(g - 1) * b for g, b in zip(grid, c)], grid)))
    rng = np.random.default_rng(seed)
    rnd = rng.choice(W.num_tokens(wl), size=n_random, replace=False)
    return np.array(sorted(corners | set(int(x) for x in rnd)), dtype=np.int64)


def _compare(label, got, want):
    got = got.float().cpu().numpy().astype(np.float64)
    assert np.all(np.isfinite(got)), label
    rel = np.linalg.norm(got - want) / max(np.linalg.norm(want), 1e-30)
    mx = np.max(np.abs(got - want)) / max(np.max(np.abs(want)), 1e-30)
    print("  %s: rel-L2 %.2e max %.2e" % (label, rel, mx), flush=True)
    assert rel <= REL_L2 and mx <= MAX_REL, "%s: rel-L2 %.3e, max %.3e" % (label, rel, mx)


def _full_size_grads(name):
    na = _na()
    wl = W.CONFIGS[name]
    print("case %s (full size)" % name, flush=True)
    plan = na.Plan(wl)
    q, k, v = W.make_qkv(wl, device="cuda")
    g = W.make_dout(wl, device="cuda")
    scale = W.default_scale(wl)
    out, lse = plan.forward(q, k, v, scale=scale)
    dq, dk, dv = plan.backward(q, k, v, out, lse, g, scale=scale)
    torch.cuda.synchronize()
    return wl, scale, (q, k, v, g), (dq, dk, dv)


def _head(x, h):
    return x[:, h:h + 1].contiguous().cpu()


def test_backward_full_size_causal():
    """The 1-D causal window at full size (32768 tokens, 4096 keys), launched
    as the benchmark launches its backward pass: dq, dk and dv of the last
    head compared element by element, every row, and dq of the first head on
    sampled rows."""
    wl, scale, (q, k, v, g), (dq, dk, dv) = _full_size_grads("causal1d_bf16")
    N, h = W.num_tokens(wl), int(wl["H"]) - 1
    args = [_head(x, h) for x in (q, k, v, g)]
    all_rows = np.arange(N, dtype=np.int64)
    ref_dq = oracle.attention_backward_dq(wl, *args, scale, all_rows)
    _compare("dq head %d" % h, dq[:, h:h + 1], ref_dq)
    ref_dk, ref_dv = oracle.attention_backward_kv(wl, *args, scale, all_rows)
    _compare("dk head %d" % h, dk[:, h:h + 1], ref_dk)
    _compare("dv head %d" % h, dv[:, h:h + 1], ref_dv)
    rows = _sample_rows(wl, 64, seed=wl["seed"])
    ref0 = oracle.attention_backward_dq(wl, *[_head(x, 0) for x in (q, k, v, g)], scale, rows)
    _compare("dq head 0 rows", dq[:, 0:1][:, :, rows], ref0)


def test_backward_full_size_sta3d():
    """The 3-D sliding-tile map at full size (30x48x80, 3x5x7 tiles of
    6x8x8), launched as the benchmark launches its backward pass.  dq: sampled
    rows (grid corners and random rows) of the first and last heads.  dk and
    dv: element by element on 16 random key rows from each of the two corner
    tiles of the grid, for one head.  The oracle's cost for a key is every
    query that attends it, each with its whole row: a corner tile is attended
    by 24 query tiles (2x3x4), an interior one by 105.  Over all keys, the
    identities sum_j dk_j = 0 (adding one vector to every key leaves the
    attention unchanged) and sum_j dv_j = sum_i dout_i (the rows of P sum to
    one)."""
    wl, scale, (q, k, v, g), (dq, dk, dv) = _full_size_grads("sta3d_bf16")
    N, H = W.num_tokens(wl), int(wl["H"])
    for h in (0, H - 1):
        rows = _sample_rows(wl, 24, seed=wl["seed"] + h)
        ref = oracle.attention_backward_dq(wl, *[_head(x, h) for x in (q, k, v, g)], scale, rows)
        _compare("dq head %d rows" % h, dq[:, h:h + 1][:, :, rows], ref)
    # the sequence order runs tile by tile (384 tokens per 6x8x8 tile)
    order = oracle.order(wl)
    tile = 6 * 8 * 8
    rng = np.random.default_rng(wl["seed"] + 7)
    keys = np.concatenate([order[t0 + rng.choice(tile, 16, replace=False)]
                           for t0 in (0, N - tile)]).astype(np.int64)
    h = H // 2
    ref_dk, ref_dv = oracle.attention_backward_kv(wl, *[_head(x, h) for x in (q, k, v, g)], scale,
                                                  keys)
    _compare("dk head %d key rows" % h, dk[:, h:h + 1][:, :, keys], ref_dk)
    _compare("dv head %d key rows" % h, dv[:, h:h + 1][:, :, keys], ref_dv)
    sdv = dv.double().sum(dim=2)
    sg = g.double().sum(dim=2)
    e_dv = (torch.linalg.norm(sdv - sg) / torch.linalg.norm(sg)).item()
    sdk = dk.double().sum(dim=2)
    scale_dk = (dk.double().pow(2).sum(dim=2).sqrt()).norm().item()
    e_dk = torch.linalg.norm(sdk).item() / scale_dk
    print("  sum dv vs sum dout: %.2e   |sum dk| / sqrt(sum |dk|^2): %.2e" % (e_dv, e_dk), flush=True)
    assert e_dv <= 1e-3
    assert e_dk <= 2e-2


@pytest.mark.parametrize("name", ["hwa96_bf16", "hswa96_bf16", "hna56_bf16", "hsa96_bf16"])
def test_backward_hilbert_page(name):
    """Gradients on the Hilbert page's shapes (generalised curve), two batches."""
    _grad_case(W.scaled(W.HILBERT_PAGE[name], B=2))


GNA = [
    W.scaled(W.CONFIGS["na2d_bf16"], name="na3d_causal_t", B=1, H=2, grid=[8, 12, 10],
             pattern=dict(kind="na", window=[3, 5, 5], causal=[1, 0, 0])),
    W.scaled(W.GNA["sta3d_causal_t_bf16"], name="block_causal_small", H=2, grid=[18, 16, 24],
             pattern=dict(kind="na", window=[12, 16, 24], stride=[6, 8, 8], causal=[1, 0, 0])),
    W.scaled(W.CONFIGS["na2d_bf16"], name="stride_shift_2d", B=1, H=2, grid=[20, 30],
             pattern=dict(kind="na", window=[7, 9], stride=[3, 3], shift=[1, 2])),
    W.GNA["na2d_tiled_bf16"],
]


@pytest.mark.parametrize("q_block", [128, 256])
@pytest.mark.parametrize("wl", GNA, ids=[w["name"] for w in GNA])
def test_backward_gna(wl, q_block):
    _grad_case(wl, q_block=q_block)


def test_backward_unsupported_query_tiles():
    """Gradient kernels exist for 128- and 256-query tiles: plans built with 64
    (head_dim 64) or 384 (head_dim 128) query tiles refuse na_backward."""
    na = _na()
    for D, qb in ((64, 64), (128, 384)):
        wl = W.scaled(W.CONFIGS["causal1d_bf16"], name="qb%d" % qb, H=1, D=D, grid=[500],
                      pattern=dict(kind="band", left=40, right=0))
        plan = na.Plan(wl, q_block=qb)
        q, k, v = W.make_qkv(wl, device="cuda")
        out, lse = plan.forward(q, k, v, scale=0.1)
        with pytest.raises(na.NaError) as ei:
            plan.backward(q, k, v, out, lse, out, scale=0.1)
        assert ei.value.status == na.NA_ERR_UNSUPPORTED
    torch.cuda.synchronize()

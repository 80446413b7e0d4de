"""GPU parity of pi-Attention's forms ("pi-Attention: Online Efficient Sparse
Transformers for Long-Context Modeling", Sections 3.4-3.5) against the fp64
oracle on the same bits: the union working set with one softmax (Eq. 11),
fixed fusion's log-prior logits (Eqs. 16-17) and the separate softmax of
Eq. 15, causal and bidirectional, on 1-D sequences and on the Hilbert curve.
Tolerances as for every other pattern (fp32 1e-5; bf16 max-abs 2e-2, relative
L2 5e-3, lse 1e-3), since the partner only adds keys (and, for fixed fusion,
one fp32 addition to their logits).  The separate variant's output is the
window's weighted average plus a whole partner value row, so it is no longer
bounded by max |v|; where the partner branch runs as its own kernel (fp32,
and bf16 at q_block 192) the window part is rounded to bf16 and the sum
rounded again, each at most 2^-9 relative (the other bf16 kernels add the
branch before their one rounding).  Its bound is therefore elementwise:
|error| <= 2e-2 + 2^-8 |reference| (bf16), with the same relative L2 bound.
"""
import os

import numpy as np
import pytest

import oracle
from dimensional_sparse_local_amd import workloads as W

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

TOL = {"fp32": dict(abs=1e-5, rel=None, lse=1e-5), "bf16": dict(abs=2e-2, rel=5e-3, lse=1e-3)}


def _na():
    from dimensional_sparse_local_amd import na

    if not os.path.exists(na._LIB_PATH):
        raise RuntimeError("libna.so missing: the HIP path must be built")
    return na


def _check_out(wl, o, ref_out):
    t = TOL[wl["dtype"]]
    bound = t["abs"]
    if wl["pattern"].get("skip_mode") == "separate" and wl["dtype"] == "bf16":
        bound = t["abs"] + 2.0 ** -8 * np.abs(ref_out)
    excess = np.abs(o - ref_out) - bound
    assert np.all(excess <= 0), "%s: error above bound by %.3e" % (wl["name"], excess.max())


def _run(wl, q_block=0, permute_passes=False, rows=None):
    na = _na()
    print("case %s grid=%s B=%d H=%d D=%d q_block=%d pattern=%s" % (
        wl["name"], wl["grid"], wl["B"], wl["H"], wl["D"], q_block, wl["pattern"]), flush=True)
    plan = na.Plan(wl, q_block=q_block)
    q, k, v = W.make_qkv(wl, device="cuda")
    scale = W.default_scale(wl)
    out, lse = plan.forward(q, k, v, scale=scale, permute_passes=permute_passes)
    torch.cuda.synchronize()
    ref_out, ref_lse = oracle.attention(wl, q.cpu(), k.cpu(), v.cpu(), scale, rows=rows)
    t = TOL[wl["dtype"]]
    o = out.float().cpu().numpy().astype(np.float64)
    l = lse.cpu().numpy().astype(np.float64)
    if rows is not None:
        o, l = o[:, :, rows], l[:, :, rows]
    _check_out(wl, o, ref_out)
    if t["rel"] is not None:
        rel = np.linalg.norm(o - ref_out) / np.linalg.norm(ref_out)
        assert rel <= t["rel"], "%s: rel-L2 %.3e" % (wl["name"], rel)
    fin = np.isfinite(ref_lse)
    assert np.array_equal(np.isfinite(l), fin)
    assert np.max(np.abs(l[fin] - ref_lse[fin])) <= t["lse"]


def _pi(name, N=1000, left=4, right=0, skip=16, both=0, mode="union", prior=0.5, D=64,
        dtype="bf16", H=2, B=1, hilbert=None):
    pat = dict(kind="band", left=left, right=right, skip=skip, skip_both=both, skip_mode=mode,
               skip_prior=prior)
    grid, order = ([hilbert, hilbert], "hilbert") if hilbert else ([N], "row_major")
    return dict(name=name, B=B, H=H, D=D, dtype=dtype, grid=grid, order=order, pattern=pat,
                seed=40)


CASES = [
    _pi("union_causal"),
    _pi("union_both", left=8, right=8, skip=40, both=1),
    _pi("union_far", N=777, left=30, right=0, skip=300, D=128),
    _pi("fusion_causal", mode="fixed_fusion", prior=0.3),
    _pi("fusion_both", left=8, right=8, skip=40, both=1, mode="fixed_fusion", prior=0.8, D=128),
    _pi("fusion_near", N=500, left=20, right=0, skip=7, mode="fixed_fusion", prior=0.2),
    _pi("fusion_half", mode="fixed_fusion", prior=0.5),
    _pi("separate_causal", mode="separate"),
    _pi("separate_both", left=8, right=8, skip=40, both=1, mode="separate", D=128),
    _pi("separate_fp32", mode="separate", dtype="fp32", D=32, N=300),
    _pi("separate_fp32_d64", mode="separate", dtype="fp32", D=64, N=300, both=1, skip=50),
    _pi("union_fp32", dtype="fp32", D=32, N=300, skip=30, both=1),
    _pi("hilbert_fusion", left=10, right=10, skip=100, both=1, mode="fixed_fusion", prior=0.3,
        hilbert=32),
    _pi("hilbert_separate", left=10, right=10, skip=100, both=1, mode="separate", hilbert=32),
]


@pytest.mark.parametrize("wl", CASES, ids=[w["name"] for w in CASES])
def test_pi_forms(wl):
    _run(wl)


@pytest.mark.parametrize("q_block", [64, 256])
@pytest.mark.parametrize("name", ["union_both", "fusion_causal", "separate_causal"])
def test_pi_query_blocks(name, q_block):
    wl = next(w for w in CASES if w["name"] == name)
    if q_block == 64 and wl["D"] != 64:
        pytest.skip("64-query tiles exist at head_dim 64")
    _run(wl, q_block=q_block)


@pytest.mark.parametrize("name", ["hilbert_fusion", "hilbert_separate"])
def test_pi_permute_passes(name):
    _run(next(w for w in CASES if w["name"] == name), permute_passes=True)


@pytest.mark.parametrize("name", list(W.PI_ATTENTION))
def test_pi_full_size(name):
    """The page's defaults (k = 4, pi = 16) at 4 x 16 heads x 8192 tokens: every
    element of the first batch, launched as the benchmark launches it."""
    wl = W.PI_ATTENTION[name]
    na = _na()
    print("case %s full size" % name, flush=True)
    plan = na.Plan(wl)
    q, k, v = W.make_qkv(wl, device="cuda")
    scale = W.default_scale(wl)
    out, lse = plan.forward(q, k, v, scale=scale)
    torch.cuda.synchronize()
    one = W.scaled(wl, B=1)
    ref_out, ref_lse = oracle.attention(one, q[:1].cpu(), k[:1].cpu(), v[:1].cpu(), scale)
    o = out[:1].float().cpu().numpy().astype(np.float64)
    _check_out(wl, o, ref_out)
    assert np.linalg.norm(o - ref_out) / np.linalg.norm(ref_out) <= 5e-3
    assert np.max(np.abs(lse[:1].cpu().numpy() - ref_lse)) <= 1e-3


GRAD_CASES = [
    (_pi("g_union", N=600, left=6, right=0, skip=50), 0),
    (_pi("g_union_both", N=600, left=6, right=6, skip=90, both=1, D=128), 0),
    (_pi("g_fusion", N=600, left=6, right=0, skip=50, mode="fixed_fusion", prior=0.3), 0),
    (_pi("g_fusion_both", N=700, left=8, right=8, skip=40, both=1, mode="fixed_fusion", prior=0.8,
         D=128), 256),
    (_pi("g_fusion_near", N=500, left=20, right=0, skip=7, mode="fixed_fusion", prior=0.2), 256),
    (_pi("g_fusion_hilbert", left=10, right=10, skip=100, both=1, mode="fixed_fusion", prior=0.3,
         hilbert=32), 128),
    (_pi("g_separate", N=600, left=6, right=0, skip=50, mode="separate"), 0),
    (_pi("g_separate_both", N=700, left=8, right=8, skip=40, both=1, mode="separate", D=128), 256),
    (_pi("g_separate_near", N=500, left=20, right=0, skip=7, both=1, mode="separate"), 128),
    (_pi("g_separate_hilbert", left=10, right=10, skip=100, both=1, mode="separate", hilbert=32),
     128),
]


@pytest.mark.parametrize("wl,q_block", GRAD_CASES, ids=[w["name"] for w, _ in GRAD_CASES])
def test_pi_gradients(wl, q_block):
    """The union form is an ordinary neighbourhood; fixed fusion's log-priors are
    constants added to the recomputed logits (same kernels, a partner bit plane);
    the separate variant adds the partner branch's gradients to the window
    branch's, whose row sums use the window output alone."""
    na = _na()
    print("case %s q_block=%d" % (wl["name"], q_block), flush=True)
    plan = na.Plan(wl, q_block=q_block)
    q, k, v = W.make_qkv(wl, device="cuda")
    g = W.make_dout(wl, device="cuda")
    scale = W.default_scale(wl)
    out, lse = plan.forward(q, k, v, scale=scale)
    dq, dk, dv = plan.backward(q, k, v, out, lse, g, scale=scale)
    torch.cuda.synchronize()
    ref = oracle.attention_backward(wl, q.cpu(), k.cpu(), v.cpu(), g.cpu(), scale)
    for name, got, want in zip(("dq", "dk", "dv"), (dq, dk, dv), ref):
        a = got.float().cpu().numpy().astype(np.float64)
        rel = np.linalg.norm(a - want) / np.linalg.norm(want)
        mx = np.max(np.abs(a - want)) / np.max(np.abs(want))
        assert rel <= 1e-2 and mx <= 2e-2, "%s %s rel-L2 %.3e max %.3e" % (wl["name"], name, rel, mx)


@pytest.mark.parametrize("q_block,D", [(192, 64), (384, 128)])
def test_pi_fixed_fusion_unsupported_tiles(q_block, D):
    """The logit-bias forward exists for 64 (head_dim 64), 128 and 256 query tiles."""
    na = _na()
    wl = _pi("fusion_qb%d" % q_block, N=500, mode="fixed_fusion", prior=0.3, D=D)
    plan = na.Plan(wl, q_block=q_block)
    q, k, v = W.make_qkv(wl, device="cuda")
    with pytest.raises(na.NaError) as ei:
        plan.forward(q, k, v, scale=0.125)
    assert ei.value.status == na.NA_ERR_UNSUPPORTED

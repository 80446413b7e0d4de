"""GPU parity for tensors of more than 2^31 elements, where the byte offset of
a (batch, head) slice passes 4 GiB: the forward pass at the 3-D sliding-tile
shape with 8 batches (as the benchmark launches it, 384-query tiles), its
gradients, the Hilbert band gather at head_dim 64 and the fp32 kernel.

Each case checks sampled query rows of the first, a middle and the last
slice against the fp64 oracle (tolerances as in the other parity tests) and
compares the last slice bit for bit with a run of the same plan on that slice
alone: every workgroup's arithmetic is independent of where its slice sits,
so any addressing error shows as a difference.
"""
import os

import numpy as np
import pytest

import oracle
from dimensional_sparse_local_amd import workloads as W

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

TOL = {"fp32": dict(abs=1e-5, lse=1e-5), "bf16": dict(abs=2e-2, lse=1e-3)}
REL_L2 = 1e-2
MAX_REL = 2e-2


def _na():
    from dimensional_sparse_local_amd import na

    if not os.path.exists(na._LIB_PATH):
        raise RuntimeError("libna.so missing: the HIP path must be built")
    return na


def _rows(wl, n_random, seed):
    rng = np.random.default_rng(seed)
    n = W.num_tokens(wl)
    rnd = rng.choice(n, size=min(n_random, n), replace=False)
    return np.array(sorted({0, n - 1} | set(int(x) for x in rnd)), dtype=np.int64)


def _slices(wl):
    B, H = int(wl["B"]), int(wl["H"])
    return [(0, 0), (B // 2, H // 2), (B - 1, H - 1)]


def _free():
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


LARGE_FWD = [
    # 8 x 24 x 115,200 x 128 = 2.83e9 elements per tensor
    (W.scaled(W.CONFIGS["sta3d_bf16"], name="sta3d_b8", B=8), 384),
    # 4 x 528 x 16,384 x 64 = 2.21e9 elements, Hilbert gather fused in the kernel
    (W.scaled(W.CONFIGS["hilbert_band_bf16"], name="hilbert_band_h528", H=528), 0),
    # 1024 x 1025 x 64 x 32 = 2.15e9 fp32 elements
    (W.scaled(W.CONFIGS["na2d_fp32"], name="na2d_fp32_many", B=1024, H=1025), 0),
]


@pytest.mark.parametrize("wl,q_block", LARGE_FWD, ids=[w["name"] for w, _ in LARGE_FWD])
def test_forward_beyond_2e31_elements(wl, q_block):
    na = _na()
    n_el = int(wl["B"]) * int(wl["H"]) * W.num_tokens(wl) * int(wl["D"])
    assert n_el > 2 ** 31
    print("case %s B=%d H=%d elements/tensor=%d q_block=%d" % (wl["name"], wl["B"], wl["H"], n_el,
                                                                q_block), flush=True)
    plan = na.Plan(wl, q_block=q_block)
    q, k, v = W.make_qkv(wl, device="cuda")
    scale = W.default_scale(wl)
    out, lse = plan.forward(q, k, v, scale=scale)
    torch.cuda.synchronize()
    t = TOL[wl["dtype"]]
    one = W.scaled(wl, B=1, H=1)
    rows = _rows(wl, 16, seed=int(wl["seed"]))
    for b, h in _slices(wl):
        qs, ks, vs = (x[b:b + 1, h:h + 1].contiguous() for x in (q, k, v))
        ref, ref_lse = oracle.attention(one, qs.cpu(), ks.cpu(), vs.cpu(), scale, rows=rows)
        o = out[b, h, rows].float().cpu().numpy()
        l = lse[b, h, rows].cpu().numpy()
        err = float(np.max(np.abs(o - ref[0, 0])))
        lerr = float(np.max(np.abs(l - ref_lse[0, 0])))
        print("  slice (%d, %d): max-abs %.3e lse %.3e" % (b, h, err, lerr), flush=True)
        assert err <= t["abs"] and lerr <= t["lse"], (b, h)
    b, h = _slices(wl)[-1]
    qs, ks, vs = (x[b:b + 1, h:h + 1].contiguous() for x in (q, k, v))
    o1, l1 = plan.forward(qs, ks, vs, scale=scale)
    torch.cuda.synchronize()
    assert torch.equal(o1[0, 0], out[b, h]) and torch.equal(l1[0, 0], lse[b, h])
    del q, k, v, out, lse, qs, ks, vs, o1, l1
    _free()


def test_backward_beyond_2e31_elements():
    """Gradients at the 3-D sliding-tile shape with 8 batches (2.83e9 elements
    per tensor): dq rows of three slices against the oracle; dq, dk and dv of
    the last slice bit for bit against that slice run alone."""
    na = _na()
    wl = W.scaled(W.CONFIGS["sta3d_bf16"], name="sta3d_b8", B=8)
    print("case sta3d_b8 backward", flush=True)
    plan = na.Plan(wl)
    q, k, v = W.make_qkv(wl, device="cuda")
    g = W.make_dout(wl, device="cuda")
    scale = W.default_scale(wl)
    out, lse = plan.forward(q, k, v, scale=scale)
    dq, dk, dv = plan.backward(q, k, v, out, lse, g, scale=scale)
    torch.cuda.synchronize()
    one = W.scaled(wl, B=1, H=1)
    rows = _rows(wl, 12, seed=int(wl["seed"]))
    for b, h in _slices(wl):
        qs, ks, vs, gs = (x[b:b + 1, h:h + 1].contiguous().cpu() for x in (q, k, v, g))
        ref = oracle.attention_backward_dq(one, qs, ks, vs, gs, scale, rows)[0, 0]
        got = dq[b, h, rows].float().cpu().numpy()
        rel = np.linalg.norm(got - ref) / np.linalg.norm(ref)
        mx = np.max(np.abs(got - ref)) / np.max(np.abs(ref))
        print("  slice (%d, %d): dq rows rel-L2 %.2e max %.2e" % (b, h, rel, mx), flush=True)
        assert rel <= REL_L2 and mx <= MAX_REL, (b, h)
    b, h = _slices(wl)[-1]
    qs, ks, vs, gs = (x[b:b + 1, h:h + 1].contiguous() for x in (q, k, v, g))
    o1, l1 = plan.forward(qs, ks, vs, scale=scale)
    g1 = plan.backward(qs, ks, vs, o1, l1, gs, scale=scale)
    torch.cuda.synchronize()
    for name, one_slice, big in zip(("dq", "dk", "dv"), g1, (dq, dk, dv)):
        assert torch.equal(one_slice[0, 0], big[b, h]), name
    del q, k, v, g, out, lse, dq, dk, dv, qs, ks, vs, gs, o1, l1, g1
    _free()


def test_slice_at_the_2e31_element_limit():
    """Rows spread so that one (batch, head) slice spans exactly the largest
    accepted extent ((N - 1) * stride_n + D <= 2^31 - 1 elements, byte offsets
    up to 4 GiB) run and match the oracle; one stride step more is rejected
    on the host with NA_ERR_UNSUPPORTED before anything is launched."""
    na = _na()
    wl = W.scaled(W.CONFIGS["na2d_bf16"], name="slice_limit", B=1, H=1, grid=[8, 8],
                  pattern=dict(kind="na", window=[3, 3]))
    N, D = W.num_tokens(wl), int(wl["D"])
    fits = ((2 ** 31 - 1 - D) // (N - 1)) // 8 * 8   # a multiple of 16 bytes
    over = fits + 8
    assert (N - 1) * fits + D <= 2 ** 31 - 1 < (N - 1) * over + D
    plan = na.Plan(wl)
    q0, k0, v0 = W.make_qkv(wl, device="cuda")
    scale = W.default_scale(wl)

    def spread(x, s):
        base = torch.zeros((N - 1) * s + D, dtype=x.dtype, device="cuda")
        y = base.as_strided((1, 1, N, D), (N * s, N * s, s, 1))
        y.copy_(x)
        return y

    print("case slice_limit stride_n=%d (extent %d elements)" % (fits, (N - 1) * fits + D), flush=True)
    q, k, v, out = (spread(x, fits) for x in (q0, k0, v0, torch.zeros_like(q0)))
    _, lse = plan.forward(q, k, v, out=out, scale=scale)
    torch.cuda.synchronize()
    ref, ref_lse = oracle.attention(wl, q0.cpu(), k0.cpu(), v0.cpu(), scale)
    err = float(np.max(np.abs(out.float().cpu().numpy() - ref)))
    lerr = float(np.max(np.abs(lse.cpu().numpy() - ref_lse)))
    print("  max-abs %.3e lse %.3e" % (err, lerr), flush=True)
    assert err <= TOL["bf16"]["abs"] and lerr <= TOL["bf16"]["lse"]
    del q, k, v, out
    _free()
    q = spread(q0, over)
    with pytest.raises(na.NaError) as ei:
        plan.forward(q, k0, v0, scale=scale)
    assert ei.value.status == na.NA_ERR_UNSUPPORTED
    del q
    _free()

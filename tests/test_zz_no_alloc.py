"""na_backward_noalloc (the backward pass with the library's fixed per-GPU
scratch, for callers that cannot allocate) against na_backward with a
caller-supplied workspace: the same kernels on the same delta rows, so the
gradients must be bit-identical.  Three calls in a row on one GPU, each
smaller than the one before it and each with different contents left in the
scratch by the previous call; then a size past the scratch is refused before
any device work."""
import pytest

from dimensional_sparse_local_amd import workloads as W

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


def _na():
    from dimensional_sparse_local_amd import na

    return na


CALLS = [
    W.scaled(W.CONFIGS["causal1d_bf16"], name="noalloc_band_d128", B=2, H=4, grid=[5000],
             pattern=dict(kind="band", left=600, right=0)),
    W.scaled(W.CONFIGS["na2d_bf16"], name="noalloc_na2d_d64", B=1, H=2, grid=[30, 41],
             pattern=dict(kind="na", window=[7, 9])),
    W.scaled(W.CONFIGS["causal1d_bf16"], name="noalloc_pi_separate", B=1, H=2, D=64,
             grid=[700], pattern=dict(kind="band", left=50, right=0, skip=97,
                                      skip_mode="separate")),
]


def test_noalloc_matches_workspace_backward():
    na = _na()
    sizes = [w["B"] * w["H"] * W.num_tokens(w) for w in CALLS]
    assert sizes == sorted(sizes, reverse=True)
    for wl in CALLS:
        print("case %s B=%d H=%d N=%d D=%d" % (wl["name"], wl["B"], wl["H"], W.num_tokens(wl),
                                              wl["D"]), flush=True)
        plan = na.Plan(wl)
        q, k, v = W.make_qkv(wl, device="cuda")
        g = W.make_dout(wl, device="cuda")
        scale = W.default_scale(wl)
        out, lse = plan.forward(q, k, v, scale=scale)
        ref = plan.backward(q, k, v, out, lse, g, scale=scale)
        got = tuple(torch.full_like(x, float("nan")) for x in (q, k, v))
        plan.backward_noalloc(q, k, v, out, lse, g, got, scale=scale)
        torch.cuda.synchronize()
        for name, a, b in zip(("dq", "dk", "dv"), got, ref):
            assert torch.equal(a, b), "%s %s differs from na_backward" % (wl["name"], name)


def test_noalloc_refuses_beyond_scratch():
    na = _na()
    limit_rows = na.NA_BACKWARD_NOALLOC_MAX_BYTES // 4
    wl = W.scaled(W.CONFIGS["causal1d_bf16"], name="noalloc_too_big", B=2, H=3, D=64,
                  grid=[limit_rows // 6 + 1], pattern=dict(kind="band", left=3, right=0))
    plan = na.Plan(wl)
    x = torch.zeros((2, 3, plan.n_tokens, 64), dtype=torch.bfloat16, device="cuda")
    lse = torch.zeros((2, 3, plan.n_tokens), dtype=torch.float32, device="cuda")
    with pytest.raises(na.NaError) as ei:
        plan.backward_noalloc(x, x, x, x, lse, x, (x, x, x), scale=0.1)
    assert ei.value.status == na.NA_ERR_INVALID_ARG
    assert "scratch" in str(ei.value)
    torch.cuda.synchronize()

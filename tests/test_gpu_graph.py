"""The hot path under HIP graph capture: a forward with the split tail (the
attention kernel and its merge kernel, workspace supplied by the caller) and
the allocation-free backward (na_backward_noalloc, delta rows in the
library's fixed per-GPU scratch) captured into one torch.cuda.CUDAGraph and
replayed several times, with eager work and synchronisations between the
replays; every replay must reproduce the eager results bit for bit (the
kernels are deterministic).  Nothing in the captured calls allocates or
clears memory."""
import pytest

from dimensional_sparse_local_amd import workloads as W

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


def _na():
    from dimensional_sparse_local_amd import na

    return na


@pytest.mark.parametrize("D", [64, 128])
def test_forward_and_noalloc_backward_replay(D):
    na = _na()
    wl = W.scaled(W.CONFIGS["causal1d_bf16"], name="graph_band_d%d" % D, B=2, H=3, D=D,
                  grid=[1500], pattern=dict(kind="band", left=300, right=0))
    plan = na.Plan(wl, q_block=256)
    assert plan.stats["resident_workgroups"] > 0
    q, k, v = W.make_qkv(wl, device="cuda")
    g = W.make_dout(wl, device="cuda")
    scale = W.default_scale(wl)
    B, H, N = wl["B"], wl["H"], plan.n_tokens
    ws = torch.empty(int(na.lib().na_forward_workspace_bytes(plan._h, B, H, na.NA_FWD_SPLIT_TAIL)),
                     dtype=torch.uint8, device="cuda")
    assert ws.numel() > 0
    out = torch.empty_like(q)
    lse = torch.empty((B, H, N), dtype=torch.float32, device="cuda")
    grads = tuple(torch.empty_like(x) for x in (q, k, v))

    # eager results (the split forward and the workspace backward)
    ref_out, ref_lse = plan.forward(q, k, v, scale=scale, split_tail=True, workspace=ws)
    ref_grads = plan.backward(q, k, v, ref_out, ref_lse, g, scale=scale)
    torch.cuda.synchronize()

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):   # warm-up on the capture stream's kind
        plan.forward(q, k, v, out=out, lse=lse, scale=scale, split_tail=True, workspace=ws)
        plan.backward_noalloc(q, k, v, out, lse, g, grads, scale=scale)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()

    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        plan.forward(q, k, v, out=out, lse=lse, scale=scale, split_tail=True, workspace=ws)
        plan.backward_noalloc(q, k, v, out, lse, g, grads, scale=scale)
    torch.cuda.synchronize()

    for rep in range(3):
        # eager work between the replays: clobber every output and the workspace
        out.fill_(float("nan"))
        lse.fill_(float("nan"))
        ws.fill_(0xFF)
        for x in grads:
            x.fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, ref_out), "replay %d: out" % rep
        assert torch.equal(lse, ref_lse), "replay %d: lse" % rep
        for name, a, b in zip(("dq", "dk", "dv"), grads, ref_grads):
            assert torch.equal(a, b), "replay %d: %s" % (rep, name)

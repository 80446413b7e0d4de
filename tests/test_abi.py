"""The C-ABI library loads and exports every function include/na.h declares,
and the host-side status / error surface works without a GPU."""
import ctypes
import os
import re

import pytest

from dimensional_sparse_local_amd import na
from dimensional_sparse_local_amd import workloads as W

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
pytestmark = pytest.mark.skipif(not os.path.exists(na._LIB_PATH), reason="libna.so not built")


def declared_functions():
    text = open(os.path.join(ROOT, "include", "na.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(na_[a-z_]+)\s*\(", text)))


def test_every_declared_symbol_is_exported():
    names = declared_functions()
    assert len(names) >= 11
    lib = ctypes.CDLL(na._LIB_PATH)
    missing = [n for n in names if not hasattr(lib, n)]
    assert not missing, missing


def test_status_strings_and_version():
    lib = na.lib()
    assert lib.na_abi_version() == na.ABI_VERSION == 7
    for s in range(6):
        assert lib.na_status_string(s)
    assert lib.na_status_string(99) == b"unknown status"


def test_null_arguments():
    lib = na.lib()
    assert lib.na_plan_create(None, 0, None) == na.NA_ERR_INVALID_ARG
    h = ctypes.c_void_p()
    assert lib.na_plan_create(None, 0, ctypes.byref(h)) == na.NA_ERR_INVALID_ARG
    assert b"NULL" in lib.na_last_error()
    assert lib.na_plan_destroy(None) == na.NA_OK
    assert lib.na_plan_get_stats(None, None) == na.NA_ERR_INVALID_ARG
    assert lib.na_forward(None, 1, 1, None, None, None, None, None, 1.0, 0, None, 0, None) \
        == na.NA_ERR_INVALID_ARG
    assert lib.na_permute(None, 1, 1, None, None, 0, None) == na.NA_ERR_INVALID_ARG
    assert lib.na_forward_workspace_bytes(None, 1, 1, 0) == 0
    assert lib.na_backward(None, 1, 1, None, None, None, None, None, None, None, None, None, 1.0,
                           None, 0, None) == na.NA_ERR_INVALID_ARG
    assert lib.na_backward_workspace_bytes(None, 1, 1) == 0
    assert lib.na_plan_get_bounds(None, None) == na.NA_ERR_INVALID_ARG


def test_unknown_flags():
    lib = na.lib()
    d = na.desc_from_workload(dict(grid=[8], pattern=dict(kind="band", left=1, right=1), D=64))
    h = ctypes.c_void_p()
    assert lib.na_plan_create(ctypes.byref(d), 0x10, ctypes.byref(h)) == na.NA_ERR_INVALID_ARG


def test_small_output_buffers():
    p = na.Plan(dict(grid=[300], pattern=dict(kind="band", left=3, right=3), D=64), host_only=True)
    buf = (ctypes.c_uint8 * 1)()
    assert na.lib().na_plan_get_classes(p._h, buf, 1) == na.NA_ERR_INVALID_ARG
    ob = (ctypes.c_int32 * 2)()
    assert na.lib().na_plan_get_order(p._h, ob, 2) == na.NA_ERR_INVALID_ARG


def test_workspace_size():
    p = na.Plan(dict(grid=[32, 32], order="hilbert", pattern=dict(kind="band", left=3, right=3),
                     D=64), host_only=True)
    assert na.lib().na_forward_workspace_bytes(p._h, 2, 3, 0) == 0
    ws = na.lib().na_forward_workspace_bytes(p._h, 2, 3, na.NA_FWD_PERMUTE_PASSES)
    assert ws >= 4 * 2 * 3 * 1024 * 64 * 2 + 2 * 3 * 1024 * 4


# ---------------------------------------------------------------------------
# The binding checks every tensor's (B, H) before any device call: the C ABI
# sees pointers and strides only, so a tensor with fewer batches or heads than
# q would be written past its end.  These run on the CPU (host-only plan, CPU
# tensors): the shape check comes first and raises ValueError.
# ---------------------------------------------------------------------------

def _bh_case():
    torch = pytest.importorskip("torch")
    wl = dict(grid=[64], pattern=dict(kind="band", left=2, right=2), D=64, dtype="bf16")
    plan = na.Plan(wl, host_only=True)
    mk = lambda B, H: torch.zeros((B, H, 64, 64), dtype=torch.bfloat16)
    return torch, plan, mk


def test_forward_rejects_out_with_fewer_heads():
    torch, plan, mk = _bh_case()
    q = mk(2, 3)
    with pytest.raises(ValueError, match="out"):
        plan.forward(q, mk(2, 3), mk(2, 3), out=mk(2, 2))
    with pytest.raises(ValueError, match="out"):
        plan.forward(q, mk(2, 3), mk(2, 3), out=mk(1, 3))


def test_forward_rejects_k_v_mismatch():
    torch, plan, mk = _bh_case()
    with pytest.raises(ValueError, match="k"):
        plan.forward(mk(2, 3), mk(2, 1), mk(2, 3))
    with pytest.raises(ValueError, match="v"):
        plan.forward(mk(2, 3), mk(2, 3), mk(1, 3))


@pytest.mark.parametrize("which", [0, 1, 2])
def test_backward_rejects_small_grads(which):
    torch, plan, mk = _bh_case()
    x = mk(2, 3)
    lse = torch.zeros((2, 3, 64), dtype=torch.float32)
    grads = [mk(2, 3), mk(2, 3), mk(2, 3)]
    grads[which] = mk(2, 1)
    with pytest.raises(ValueError, match=("dq", "dk", "dv")[which]):
        plan.backward(x, x, x, x, lse, x, grads=tuple(grads))


def test_backward_rejects_dout_mismatch():
    torch, plan, mk = _bh_case()
    x = mk(2, 3)
    lse = torch.zeros((2, 3, 64), dtype=torch.float32)
    with pytest.raises(ValueError, match="dout"):
        plan.backward(x, x, x, x, lse, mk(2, 2))


def test_permute_rejects_small_out():
    torch, plan, mk = _bh_case()
    with pytest.raises(ValueError, match="out"):
        plan.permute(mk(2, 3), out=mk(2, 2))


def test_backward_noalloc_refuses_before_device_work():
    """The scratch limit and the plan checks of na_backward_noalloc come
    before any HIP call, so a host-only plan shows them without a GPU."""
    L = na.lib()
    assert L.na_backward_noalloc(None, 1, 1, *([None] * 9), 0.1, None) == na.NA_ERR_INVALID_ARG
    limit_rows = na.NA_BACKWARD_NOALLOC_MAX_BYTES // 4
    big = na.Plan(W.scaled(W.CONFIGS["causal1d_bf16"], B=2, H=3, D=64,
                           grid=[limit_rows // 6 + 1], pattern=dict(kind="band", left=3, right=0)),
                  host_only=True)
    st = L.na_backward_noalloc(big._h, 2, 3, *([None] * 9), 0.1, None)
    assert st == na.NA_ERR_INVALID_ARG
    assert b"scratch" in L.na_last_error()
    st = L.na_backward_noalloc(big._h, 1, 3, *([None] * 9), 0.1, None)   # fits: 3 * N rows
    assert st == na.NA_ERR_PLAN_MISMATCH
    assert L.na_backward_noalloc(big._h, 0, 3, *([None] * 9), 0.1, None) == na.NA_ERR_INVALID_ARG


def test_split_tail_flag_on_host_only_plan():
    """A host-only plan has no device to size a round of workgroups for: the
    split tail needs no workspace there, and unknown forward flags are
    refused."""
    L = na.lib()
    plan = na.Plan(W.scaled(W.CONFIGS["causal1d_bf16"], H=2, grid=[3000],
                            pattern=dict(kind="band", left=600, right=0)),
                   host_only=True, q_block=384)
    assert int(L.na_forward_workspace_bytes(plan._h, 1, 2, na.NA_FWD_SPLIT_TAIL)) == 0
    st = L.na_forward(plan._h, 1, 2, None, None, None, None, None, 0.1, 4, None, 0, None)
    assert st in (na.NA_ERR_INVALID_ARG, na.NA_ERR_PLAN_MISMATCH)


def test_na_log_prints_plan_statistics():
    """NA_LOG=1 makes plan creation print one line of tile-map statistics to
    stderr; without it the library prints nothing."""
    import subprocess
    import sys

    code = ("import sys; sys.path.insert(0, %r)\n"
            "from dimensional_sparse_local_amd import na, workloads as W\n"
            "na.Plan(W.CONFIGS['na2d_fp32'], host_only=True)\n") % ROOT
    env = dict(os.environ)
    env.pop("NA_LOG", None)
    quiet = subprocess.run([sys.executable, "-c", code], env=env, capture_output=True, text=True)
    assert quiet.returncode == 0, quiet.stderr
    assert "na: plan" not in quiet.stderr
    env["NA_LOG"] = "1"
    loud = subprocess.run([sys.executable, "-c", code], env=env, capture_output=True, text=True)
    assert loud.returncode == 0, loud.stderr
    lines = [l for l in loud.stderr.splitlines() if l.startswith("na: plan")]
    assert len(lines) == 1
    assert "N=64 " in lines[0] and "pairs_per_head=576 " in lines[0] and "host-only" in lines[0]


def test_tile_order_of_causal_and_other_maps():
    """A one-dimensional map whose walks grow along the sequence (a causal
    window) dispatches its query tiles longest first; a two-sided band and a
    2-D neighbourhood keep ascending order (the plan line of NA_LOG=1)."""
    import subprocess
    import sys

    code = ("import sys; sys.path.insert(0, %r)\n"
            "from dimensional_sparse_local_amd import na, workloads as W\n"
            "c = W.CONFIGS['causal1d_bf16']\n"
            "na.Plan(W.scaled(c, H=2, grid=[3000], pattern=dict(kind='band', left=600, right=0)), host_only=True)\n"
            "na.Plan(W.scaled(c, H=2, grid=[3000], pattern=dict(kind='band', left=600, right=600)), host_only=True)\n"
            "na.Plan(W.CONFIGS['na2d_fp32'], host_only=True)\n") % ROOT
    env = dict(os.environ, NA_LOG="1")
    run = subprocess.run([sys.executable, "-c", code], env=env, capture_output=True, text=True)
    assert run.returncode == 0, run.stderr
    lines = [l for l in run.stderr.splitlines() if l.startswith("na: plan")]
    assert len(lines) == 3
    assert "tile_order=descending " in lines[0]
    assert "tile_order=ascending " in lines[1]
    assert "tile_order=ascending " in lines[2]

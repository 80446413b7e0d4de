"""The C-ABI library loads and exports every function include/na.h declares,
and the host-side status / error surface works without a GPU."""
import ctypes
import os
import re

import pytest

from dimensional_sparse_local_amd import na

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
    assert lib.na_abi_version() == na.ABI_VERSION == 3
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

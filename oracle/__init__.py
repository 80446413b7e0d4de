"""Plain fp64 CPU oracle for N-dimensional local attention — TEST INFRASTRUCTURE.

Only the tests, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  The product path (the GPU library and
its Python binding) never does, and shares no code with it.

The arithmetic lives in ``oracle.c`` (plain C, fp64, OpenMP over query rows);
this module only builds it with gcc, loads it with ctypes and translates a
workload description (plain data, see ``dimensional_sparse_local_amd.workloads``)
into the oracle's own rule descriptors:

* ``na``      -> sliding window shifted inside at the borders (neighbourhood
                 attention; "Generalized Neighborhood Attention", abstract),
* ``sa``      -> sliding window cut at the borders (slide attention),
* ``band``    -> 1-D window [x-left, x+right] cut at the ends ("pi-Attention",
                 Eq. 5; causal when right = 0),
* ``blocked`` -> non-overlapping windows (window attention),
* ``sta``     -> sliding tile attention ("ENA: Efficient N-dimensional
                 Attention", tiles share one window that moves tile by tile).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

ORC_WINDOW, ORC_BLOCKED, ORC_STA = 0, 1, 2
ORDERS = {"row_major": 0, "tiled": 1, "hilbert": 2}


class _Rule(ctypes.Structure):
    _fields_ = [
        ("kind", ctypes.c_int32),
        ("clamp", ctypes.c_int32),
        ("w", ctypes.c_int64),
        ("left", ctypes.c_int64),
        ("stride", ctypes.c_int64),
        ("dil", ctypes.c_int64),
        ("tile", ctypes.c_int64),
        ("wt", ctypes.c_int64),
        ("shift", ctypes.c_int64),
        ("causal", ctypes.c_int64),
    ]


class _Spec(ctypes.Structure):
    _fields_ = [
        ("ndim", ctypes.c_int32),
        ("grid", ctypes.c_int64 * 3),
        ("order", ctypes.c_int32),
        ("tile", ctypes.c_int64 * 3),
        ("rule", _Rule * 3),
        ("skip", ctypes.c_int64),
        ("skip_both", ctypes.c_int32),
        ("skip_mode", ctypes.c_int32),
        ("skip_prior", ctypes.c_double),
    ]


SKIP_MODES = {"union": 0, "fixed_fusion": 1, "separate": 2}


def build(force: bool = False) -> str:
    """Compile oracle.c into liboracle.so with gcc (fp64, OpenMP)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(
            ["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared", _SRC, "-o", tmp, "-lm"]
        )
        os.replace(tmp, _LIB)
    return _LIB


def build_sanitized(path: str) -> str:
    """Compile oracle.c with AddressSanitizer and UndefinedBehaviorSanitizer
    into `path` (for the CPU sanitizer run of the pins; load it with the
    sanitizer runtime preloaded)."""
    tmp = path + ".tmp%d" % os.getpid()
    subprocess.check_call(
        ["gcc", "-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
         "-fno-sanitize-recover=undefined", "-std=c11", "-fopenmp", "-fPIC", "-shared", _SRC,
         "-o", tmp, "-lm"]
    )
    os.replace(tmp, path)
    return path


_lib = None


def lib():
    global _lib
    if _lib is None:
        build()
        L = ctypes.CDLL(_LIB)
        P = ctypes.POINTER
        L.orc_num_tokens.argtypes = [P(_Spec)]
        L.orc_num_tokens.restype = ctypes.c_int64
        L.orc_order.argtypes = [P(_Spec), ctypes.c_void_p]
        L.orc_hilbert.argtypes = [ctypes.c_int64, ctypes.c_void_p]
        L.orc_hilbert_grid.argtypes = [ctypes.c_int64, ctypes.c_int64, ctypes.c_void_p]
        L.orc_rule_set.argtypes = [P(_Rule), ctypes.c_int64, ctypes.c_int64, ctypes.c_void_p]
        L.orc_rule_set.restype = ctypes.c_int64
        L.orc_neighbors.argtypes = [P(_Spec), ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64,
                                    ctypes.c_void_p]
        L.orc_neighbors.restype = ctypes.c_int64
        L.orc_attended_pairs.argtypes = [P(_Spec)]
        L.orc_attended_pairs.restype = ctypes.c_int64
        L.orc_attention.argtypes = [P(_Spec), ctypes.c_int64, ctypes.c_int64, ctypes.c_int64,
                                    ctypes.c_int32, ctypes.c_void_p, ctypes.c_void_p,
                                    ctypes.c_void_p, ctypes.c_double, ctypes.c_void_p,
                                    ctypes.c_int64, ctypes.c_void_p, ctypes.c_void_p,
                                    ctypes.c_int32]
        L.orc_attention_backward.argtypes = [P(_Spec), ctypes.c_int64, ctypes.c_int64,
                                             ctypes.c_int64, ctypes.c_int32, ctypes.c_void_p,
                                             ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                             ctypes.c_double, ctypes.c_void_p, ctypes.c_void_p,
                                             ctypes.c_void_p, ctypes.c_int32]
        L.orc_attention_backward_dq_rows.argtypes = [P(_Spec), ctypes.c_int64, ctypes.c_int64,
                                                     ctypes.c_int64, ctypes.c_int32,
                                                     ctypes.c_void_p, ctypes.c_void_p,
                                                     ctypes.c_void_p, ctypes.c_void_p,
                                                     ctypes.c_double, ctypes.c_void_p,
                                                     ctypes.c_int64, ctypes.c_void_p,
                                                     ctypes.c_int32]
        L.orc_attention_backward_kv_rows.argtypes = [P(_Spec), ctypes.c_int64, ctypes.c_int64,
                                                     ctypes.c_int64, ctypes.c_int32,
                                                     ctypes.c_void_p, ctypes.c_void_p,
                                                     ctypes.c_void_p, ctypes.c_void_p,
                                                     ctypes.c_double, ctypes.c_void_p,
                                                     ctypes.c_int64, ctypes.c_void_p,
                                                     ctypes.c_void_p, ctypes.c_int32]
        L.orc_tile_classes.argtypes = [P(_Spec), ctypes.c_int64, ctypes.c_int64, ctypes.c_void_p,
                                       P(ctypes.c_int64), ctypes.c_int32]
        L.orc_max_threads.restype = ctypes.c_int32
        _lib = L
    return _lib


def max_threads() -> int:
    return int(lib().orc_max_threads())


# --------------------------------------------------------------------------
# Workload description -> oracle descriptor
# --------------------------------------------------------------------------

def _rule_for(pattern: dict, d: int) -> _Rule:
    kind = pattern["kind"]
    r = _Rule()
    r.stride, r.dil, r.tile, r.wt = 1, 1, 1, 1
    if kind in ("na", "sa"):
        w = int(pattern["window"][d])
        r.kind, r.w, r.left = ORC_WINDOW, w, w // 2
        r.clamp = 1 if kind == "na" else 0
        r.stride = int(pattern.get("stride", [1, 1, 1])[d])
        r.dil = int(pattern.get("dilation", [1, 1, 1])[d])
        r.shift = int(pattern.get("shift", [0, 0, 0])[d])
        if int(pattern.get("causal", [0, 0, 0])[d]):
            # causal dimension: the w positions ending at the query, cut at the start
            r.left, r.clamp, r.causal = w - 1, 0, 1
    elif kind == "band":
        left, right = int(pattern["left"]), int(pattern["right"])
        r.kind, r.clamp, r.w, r.left = ORC_WINDOW, 0, left + right + 1, left
    elif kind == "blocked":
        r.kind, r.w = ORC_BLOCKED, int(pattern["window"][d])
        r.shift = int(pattern.get("shift", [0, 0, 0])[d])
    elif kind == "sta":
        r.kind = ORC_STA
        r.tile = int(pattern["tile"][d])
        r.wt = int(pattern["window_tiles"][d])
    else:
        raise ValueError("unknown pattern kind %r" % kind)
    return r


def spec(workload: dict) -> _Spec:
    """Oracle descriptor for a workload description (plain dict)."""
    s = _Spec()
    grid = [int(g) for g in workload["grid"]]
    s.ndim = len(grid)
    for d in range(3):
        s.grid[d] = grid[d] if d < len(grid) else 1
    order = workload.get("order", "row_major")
    s.order = ORDERS[order]
    tile = workload.get("tile") or [1] * len(grid)
    for d in range(3):
        s.tile[d] = int(tile[d]) if d < len(tile) else 1
    pat = workload["pattern"]
    if order == "hilbert":
        s.rule[0] = _rule_for(pat, 0)
    else:
        for d in range(len(grid)):
            s.rule[d] = _rule_for(pat, d)
    # pi-Attention's online partner (1-D patterns only)
    s.skip = int(pat.get("skip", 0))
    if s.skip and order != "hilbert" and len(grid) != 1:
        raise ValueError("the skip partner needs a 1-D pattern (1-D grid or Hilbert order)")
    s.skip_both = int(pat.get("skip_both", 0))
    s.skip_mode = SKIP_MODES[pat.get("skip_mode", "union")]
    s.skip_prior = float(pat.get("skip_prior", 0.5))
    return s


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


def num_tokens(workload: dict) -> int:
    s = spec(workload)
    return int(lib().orc_num_tokens(ctypes.byref(s)))


def order(workload: dict) -> np.ndarray:
    """perm[p] = row-major token at sequence position p."""
    s = spec(workload)
    n = num_tokens(workload)
    perm = np.empty(n, dtype=np.int64)
    if lib().orc_order(ctypes.byref(s), _ptr(perm)) != 0:
        raise ValueError("order not defined for this grid")
    return perm


def hilbert(n: int) -> np.ndarray:
    perm = np.empty(n * n, dtype=np.int64)
    if lib().orc_hilbert(n, _ptr(perm)) != 0:
        raise ValueError("Hilbert order needs a power-of-two side")
    return perm


def hilbert_grid(rows: int, cols: int) -> np.ndarray:
    """Generalised Hilbert curve over a rows x cols grid (perm[p] = row * cols + col)."""
    perm = np.empty(rows * cols, dtype=np.int64)
    if lib().orc_hilbert_grid(rows, cols, _ptr(perm)) != 0:
        raise ValueError("grid must be at least 1 x 1")
    return perm


def rule_set(pattern: dict, d: int, length: int, x: int) -> np.ndarray:
    r = _rule_for(pattern, d)
    out = np.empty(max(length, 1), dtype=np.int64)
    n = lib().orc_rule_set(ctypes.byref(r), length, x, _ptr(out))
    return out[:n].copy()


def neighbors(workload: dict, token: int) -> np.ndarray:
    s = spec(workload)
    n = num_tokens(workload)
    perm = order(workload)
    pos = np.empty(n, dtype=np.int64)
    pos[perm] = np.arange(n, dtype=np.int64)
    out = np.empty(n, dtype=np.int64)
    c = lib().orc_neighbors(ctypes.byref(s), _ptr(perm), _ptr(pos), int(token), _ptr(out))
    return out[:c].copy()


def attended_pairs(workload: dict) -> int:
    s = spec(workload)
    return int(lib().orc_attended_pairs(ctypes.byref(s)))


def _raw(x) -> tuple[np.ndarray, int]:
    """(contiguous raw array, dtype code) for a numpy array or CPU torch tensor.
    Code 0: bf16 bit patterns (uint16); 1: float32; 2: float64."""
    if hasattr(x, "detach"):  # a torch tensor
        import torch

        x = x.detach().cpu().contiguous()
        if x.dtype == torch.bfloat16:
            return np.ascontiguousarray(x.view(torch.int16).numpy().view(np.uint16)), 0
        if x.dtype == torch.float64:
            return np.ascontiguousarray(x.numpy()), 2
        return np.ascontiguousarray(x.float().numpy()), 1
    x = np.asarray(x)
    if x.dtype == np.uint16:
        return np.ascontiguousarray(x), 0
    if x.dtype == np.float64:
        return np.ascontiguousarray(x), 2
    return np.ascontiguousarray(x, dtype=np.float32), 1


def attention(workload: dict, q, k, v, scale: float, rows=None, threads: int = 0):
    """fp64 softmax attention over N(i) for the given row-major query tokens.

    q, k, v: [B, H, N, D] (bf16 torch tensors, uint16 bf16 bit arrays, or
    float32).  Returns (out [B, H, R, D] fp64, lse [B, H, R] fp64) where R is
    len(rows) (all N tokens when rows is None)."""
    s = spec(workload)
    qa, dt = _raw(q)
    ka, dk = _raw(k)
    va, dv = _raw(v)
    assert dt == dk == dv, "q, k, v must share a dtype"
    B, H, N, D = qa.shape
    assert N == num_tokens(workload)
    if rows is None:
        rows_a = None
        R = N
    else:
        rows_a = np.ascontiguousarray(np.asarray(rows, dtype=np.int64))
        R = rows_a.shape[0]
    out = np.empty((B, H, R, D), dtype=np.float64)
    lse = np.empty((B, H, R), dtype=np.float64)
    rc = lib().orc_attention(ctypes.byref(s), B, H, D, dt, _ptr(qa), _ptr(ka), _ptr(va),
                             float(scale), _ptr(rows_a) if rows_a is not None else None, R,
                             _ptr(out), _ptr(lse), int(threads))
    if rc != 0:
        raise ValueError("oracle attention failed (%d)" % rc)
    return out, lse


def attention_backward(workload: dict, q, k, v, dout, scale: float, threads: int = 0):
    """fp64 gradients (dq, dk, dv), each [B, H, N, D], of sum(out * dout) where
    out = attention(workload, q, k, v, scale) over all rows.  Inputs as for
    attention(); dout of the same dtype."""
    s = spec(workload)
    qa, dt = _raw(q)
    ka, dk_ = _raw(k)
    va, dv_ = _raw(v)
    ga, dg = _raw(dout)
    assert dt == dk_ == dv_ == dg, "q, k, v, dout must share a dtype"
    B, H, N, D = qa.shape
    assert N == num_tokens(workload)
    dq = np.empty((B, H, N, D), dtype=np.float64)
    dk = np.empty_like(dq)
    dv = np.empty_like(dq)
    rc = lib().orc_attention_backward(ctypes.byref(s), B, H, D, dt, _ptr(qa), _ptr(ka), _ptr(va),
                                      _ptr(ga), float(scale), _ptr(dq), _ptr(dk), _ptr(dv),
                                      int(threads))
    if rc != 0:
        raise ValueError("oracle backward failed (%d)" % rc)
    return dq, dk, dv


def attention_backward_dq(workload: dict, q, k, v, dout, scale: float, rows, threads: int = 0):
    """fp64 dq [B, H, len(rows), D] of the same gradients for the listed
    row-major query tokens only."""
    s = spec(workload)
    qa, dt = _raw(q)
    ka, dk_ = _raw(k)
    va, dv_ = _raw(v)
    ga, dg = _raw(dout)
    assert dt == dk_ == dv_ == dg, "q, k, v, dout must share a dtype"
    B, H, N, D = qa.shape
    rows_a = np.ascontiguousarray(np.asarray(rows, dtype=np.int64))
    dq = np.empty((B, H, rows_a.shape[0], D), dtype=np.float64)
    rc = lib().orc_attention_backward_dq_rows(ctypes.byref(s), B, H, D, dt, _ptr(qa), _ptr(ka),
                                              _ptr(va), _ptr(ga), float(scale), _ptr(rows_a),
                                              rows_a.shape[0], _ptr(dq), int(threads))
    if rc != 0:
        raise ValueError("oracle backward rows failed (%d)" % rc)
    return dq


def attention_backward_kv(workload: dict, q, k, v, dout, scale: float, keys, threads: int = 0):
    """fp64 (dk, dv), each [B, H, len(keys), D], of the same gradients for the
    listed row-major key tokens only (distinct).  Every query whose
    neighbourhood holds a listed key runs its full row gradient; cheap when
    the listed keys share few queries (keys of one tile)."""
    s = spec(workload)
    qa, dt = _raw(q)
    ka, dk_ = _raw(k)
    va, dv_ = _raw(v)
    ga, dg = _raw(dout)
    assert dt == dk_ == dv_ == dg, "q, k, v, dout must share a dtype"
    B, H, N, D = qa.shape
    keys_a = np.ascontiguousarray(np.asarray(keys, dtype=np.int64))
    dk = np.empty((B, H, keys_a.shape[0], D), dtype=np.float64)
    dv = np.empty_like(dk)
    rc = lib().orc_attention_backward_kv_rows(ctypes.byref(s), B, H, D, dt, _ptr(qa), _ptr(ka),
                                              _ptr(va), _ptr(ga), float(scale), _ptr(keys_a),
                                              keys_a.shape[0], _ptr(dk), _ptr(dv), int(threads))
    if rc != 0:
        raise ValueError("oracle backward key rows failed (%d)" % rc)
    return dk, dv


def tile_classes(workload: dict, q_block: int, kv_block: int, threads: int = 0):
    """(classes uint8 [n_q_tiles, n_kv_tiles], attended pairs) over the
    sequence order: 0 empty, 1 partial, 2 full."""
    s = spec(workload)
    n = num_tokens(workload)
    nqt = -(-n // q_block)
    nkt = -(-n // kv_block)
    cls = np.empty((nqt, nkt), dtype=np.uint8)
    pairs = ctypes.c_int64(0)
    rc = lib().orc_tile_classes(ctypes.byref(s), q_block, kv_block, _ptr(cls),
                                ctypes.byref(pairs), int(threads))
    if rc != 0:
        raise ValueError("oracle tile classes failed (%d)" % rc)
    return cls, int(pairs.value)

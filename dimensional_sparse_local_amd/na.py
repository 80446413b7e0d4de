"""Thin ctypes binding of libna.so (include/na.h).

Argument marshalling only: every step of the attention runs inside the
library.  PyTorch supplies device memory and the current HIP stream.  If the
library has not been built, every call fails loudly: there is no fallback.
"""
from __future__ import annotations

import ctypes
import math
import os

import numpy as np

_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libna.so")

NA_OK, NA_ERR_INVALID_ARG, NA_ERR_UNSUPPORTED, NA_ERR_OUT_OF_MEMORY, NA_ERR_DEVICE, \
    NA_ERR_PLAN_MISMATCH = range(6)
NA_ORDER_ROW_MAJOR, NA_ORDER_TILED, NA_ORDER_HILBERT = 0, 1, 2
NA_BOUND_CLAMP, NA_BOUND_TRUNCATE = 0, 1
NA_BF16, NA_F32 = 0, 1
NA_PLAN_HOST_ONLY = 1
NA_FWD_PERMUTE_PASSES = 1
NA_FWD_SPLIT_TAIL = 2
NA_BACKWARD_NOALLOC_MAX_BYTES = 16 << 20

ORDERS = {"row_major": NA_ORDER_ROW_MAJOR, "tiled": NA_ORDER_TILED, "hilbert": NA_ORDER_HILBERT}
NA_SKIP_UNION, NA_SKIP_FIXED_FUSION, NA_SKIP_SEPARATE = 0, 1, 2
SKIP_MODES = {"union": NA_SKIP_UNION, "fixed_fusion": NA_SKIP_FIXED_FUSION,
              "separate": NA_SKIP_SEPARATE}
DTYPES = {"bf16": NA_BF16, "fp32": NA_F32}

I3 = ctypes.c_int32 * 3


class Desc(ctypes.Structure):
    _fields_ = [
        ("ndim", ctypes.c_int32), ("grid", I3), ("order", ctypes.c_int32), ("tile", I3),
        ("window", I3), ("window_left", I3), ("stride", I3), ("dilation", I3), ("causal", I3),
        ("boundary", I3), ("q_block", ctypes.c_int32), ("kv_block", ctypes.c_int32),
        ("head_dim", ctypes.c_int32), ("dtype", ctypes.c_int32), ("shift", I3),
        ("skip", ctypes.c_int32), ("skip_both", ctypes.c_int32), ("skip_mode", ctypes.c_int32),
        ("skip_prior", ctypes.c_float),
    ]


class Stats(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int64) for n in (
        "n_tokens", "q_block", "kv_block", "n_q_tiles", "n_kv_tiles", "n_empty", "n_partial",
        "n_full", "attended_pairs", "resident_workgroups")]


class Bounds(ctypes.Structure):
    _fields_ = [("flop", ctypes.c_double), ("tile", ctypes.c_double),
                ("useful_fraction", ctypes.c_double)]


class Tensor(ctypes.Structure):
    _fields_ = [("ptr", ctypes.c_void_p), ("stride_b", ctypes.c_int64),
                ("stride_h", ctypes.c_int64), ("stride_n", ctypes.c_int64)]


class NaError(RuntimeError):
    def __init__(self, status: int, detail: str):
        super().__init__("%s: %s" % (_STATUS.get(status, "status %d" % status), detail))
        self.status = status


_STATUS = {NA_ERR_INVALID_ARG: "invalid argument", NA_ERR_UNSUPPORTED: "unsupported",
           NA_ERR_OUT_OF_MEMORY: "out of memory", NA_ERR_DEVICE: "device error",
           NA_ERR_PLAN_MISMATCH: "plan mismatch"}

_lib = None
ABI_VERSION = 7  # NA_ABI_VERSION of include/na.h that Desc mirrors


def lib():
    """The loaded library; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            raise RuntimeError("libna.so is not built (run: python -m "
                               "dimensional_sparse_local_amd.build); no fallback exists")
        L = ctypes.CDLL(_LIB_PATH)
        P, vp, i64, u32 = ctypes.POINTER, ctypes.c_void_p, ctypes.c_int64, ctypes.c_uint32
        L.na_plan_create.argtypes = [P(Desc), u32, P(vp)]
        L.na_plan_destroy.argtypes = [vp]
        L.na_plan_get_stats.argtypes = [vp, P(Stats)]
        L.na_plan_get_bounds.argtypes = [vp, P(Bounds)]
        L.na_plan_get_classes.argtypes = [vp, vp, ctypes.c_size_t]
        L.na_plan_get_order.argtypes = [vp, vp, ctypes.c_size_t]
        L.na_forward_workspace_bytes.argtypes = [vp, i64, i64, u32]
        L.na_forward_workspace_bytes.restype = ctypes.c_size_t
        L.na_forward.argtypes = [vp, i64, i64, P(Tensor), P(Tensor), P(Tensor), P(Tensor), vp,
                                 ctypes.c_float, u32, vp, ctypes.c_size_t, vp]
        L.na_permute.argtypes = [vp, i64, i64, P(Tensor), P(Tensor), ctypes.c_int32, vp]
        L.na_backward_workspace_bytes.argtypes = [vp, i64, i64]
        L.na_backward_workspace_bytes.restype = ctypes.c_size_t
        L.na_backward.argtypes = [vp, i64, i64, P(Tensor), P(Tensor), P(Tensor), P(Tensor),
                                  P(Tensor), vp, P(Tensor), P(Tensor), P(Tensor), ctypes.c_float,
                                  vp, ctypes.c_size_t, vp]
        L.na_backward_noalloc.argtypes = [vp, i64, i64, P(Tensor), P(Tensor), P(Tensor),
                                          P(Tensor), P(Tensor), vp, P(Tensor), P(Tensor),
                                          P(Tensor), ctypes.c_float, vp]
        L.na_status_string.argtypes = [ctypes.c_int]
        L.na_status_string.restype = ctypes.c_char_p
        L.na_last_error.restype = ctypes.c_char_p
        L.na_abi_version.restype = ctypes.c_int32
        for f in ("na_plan_create", "na_plan_destroy", "na_plan_get_stats", "na_plan_get_bounds",
                  "na_plan_get_classes",
                  "na_plan_get_order", "na_forward", "na_permute", "na_backward",
                  "na_backward_noalloc"):
            getattr(L, f).restype = ctypes.c_int
        if L.na_abi_version() != ABI_VERSION:
            raise RuntimeError("libna.so has ABI version %d, this binding expects %d (rebuild)"
                               % (L.na_abi_version(), ABI_VERSION))
        _lib = L
    return _lib


def _same_bh(B: int, H: int, **tensors):
    """Raise ValueError unless every given tensor (None skipped) is 4-D with
    leading dimensions (B, H)."""
    for name, x in tensors.items():
        if x is None:
            continue
        if x.dim() != 4 or (int(x.shape[0]), int(x.shape[1])) != (B, H):
            raise ValueError("%s has shape %s; it must be [B, H, N, D] with B=%d, H=%d"
                             % (name, tuple(x.shape), B, H))


def _check(status: int):
    if status != NA_OK:
        raise NaError(status, lib().na_last_error().decode())


# ---------------------------------------------------------------------------
# Workload description -> plan descriptor
# ---------------------------------------------------------------------------

def desc_from_workload(w: dict, q_block: int = 0, kv_block: int = 0) -> Desc:
    d = Desc()
    grid = [int(g) for g in w["grid"]]
    d.ndim = len(grid)
    for i in range(3):
        d.grid[i] = grid[i] if i < len(grid) else 1
        d.window[i] = d.stride[i] = d.dilation[i] = 1
        d.window_left[i] = -1
    order = w.get("order", "row_major")
    d.order = ORDERS[order]
    if order == "tiled":
        for i, t in enumerate(w["tile"]):
            d.tile[i] = int(t)
    pat = w["pattern"]
    kind = pat["kind"]
    pdims = 1 if order == "hilbert" else len(grid)
    for i in range(pdims):
        if kind in ("na", "sa"):
            d.window[i] = int(pat["window"][i])
            d.stride[i] = int(pat.get("stride", [1, 1, 1])[i])
            d.shift[i] = int(pat.get("shift", [0, 0, 0])[i])
            d.dilation[i] = int(pat.get("dilation", [1, 1, 1])[i])
            d.causal[i] = int(pat.get("causal", [0, 0, 0])[i])
            d.boundary[i] = NA_BOUND_CLAMP if kind == "na" else NA_BOUND_TRUNCATE
        elif kind == "band":
            left, right = int(pat["left"]), int(pat["right"])
            d.window[i] = left + right + 1
            d.window_left[i] = left
            d.boundary[i] = NA_BOUND_TRUNCATE
        elif kind == "blocked":
            # non-overlapping windows: a window of w whose stride is w, cut at the end;
            # shifted windows move the group boundaries back by `shift`
            d.window[i] = d.stride[i] = int(pat["window"][i])
            d.shift[i] = int(pat.get("shift", [0, 0, 0])[i])
            d.boundary[i] = NA_BOUND_TRUNCATE
        elif kind == "sta":
            # sliding tile attention: window of (tiles * tile) positions moving one
            # whole tile at a time, shifted inside the grid
            t, wt = int(pat["tile"][i]), int(pat["window_tiles"][i])
            if grid[i] % t:
                raise ValueError("sliding tile attention needs whole tiles (grid %% tile == 0)")
            d.window[i] = wt * t
            d.stride[i] = t
            # the group leader sits t//2 into its tile; start wt//2 tiles earlier
            d.window_left[i] = t * (wt // 2) + t // 2
            d.boundary[i] = NA_BOUND_CLAMP
        else:
            raise ValueError("unknown pattern kind %r" % kind)
    # pi-Attention's online partner (1-D patterns)
    d.skip = int(pat.get("skip", 0))
    d.skip_both = int(pat.get("skip_both", 0))
    d.skip_mode = SKIP_MODES[pat.get("skip_mode", "union")]
    d.skip_prior = float(pat.get("skip_prior", 0.5))
    d.q_block, d.kv_block = int(q_block), int(kv_block)
    d.head_dim = int(w["D"])
    d.dtype = DTYPES[w.get("dtype", "bf16")]
    return d


def forward_launch(w: dict) -> tuple[dict, int, bool]:
    """(kernel-side workload, query tile, split tail) for the forward pass
    alone, the fastest measured launch of each shape:

    * bf16, head_dim 128, no fixed-fusion bias: the 16x16x32 MFMA kernel with
      48 queries per wave, at 384-query tiles (8 waves: each staged K/V tile
      serves 1.5x the queries of a 256-query tile) unless the tile map's
      useful fraction there is more than 2 points below that at 192-query
      tiles (4 waves, two workgroups per CU), as on the 1-D causal window
      (0.915 against 0.955: 1.86 ms at 192 against 1.93 at 384, one box);
      with the split tail, so that a last round of workgroups that would
      leave most compute units idle is spread over all of them;
    * bf16, head_dim 64, 2-D neighbourhood or slide window in row-major order:
      8x8 patch order inside the kernel (q, k, v, out stay row-major) makes the
      visited tile pairs denser, and 64-query tiles give the short walks more
      workgroups;
    * otherwise the library defaults (the workload as given, query tile 0,
      no split: on the short, latency-bound walks of the head_dim-64
      workloads the merge kernel's launch costs more than a split tail saves,
      e.g. 47 -> 56 us on the 96x96 shifted Hilbert windows).

    The gradient kernels take 128- or 256-query tiles: a plan made for the
    backward pass keeps the defaults."""
    pat = w["pattern"]
    bias = pat.get("skip", 0) > 0 and pat.get("skip_mode", "union") == "fixed_fusion"
    if w.get("dtype", "bf16") == "bf16" and int(w["D"]) == 128 and not bias:
        u384 = Plan(w, host_only=True, q_block=384).speedup_bounds()["useful_fraction"]
        u192 = Plan(w, host_only=True, q_block=192).speedup_bounds()["useful_fraction"]
        return w, (384 if u384 >= u192 - 0.02 else 192), True
    if (w.get("dtype", "bf16") == "bf16" and int(w["D"]) == 64
            and w.get("order", "row_major") == "row_major" and len(w["grid"]) == 2
            and pat["kind"] in ("na", "sa")):
        return dict(w, order="tiled", tile=[8, 8]), 64, False
    return w, 0, False


class Plan:
    """A tile map built once per shape (na_plan_create) and run many times."""

    def __init__(self, workload_or_desc, host_only: bool = False, q_block: int = 0,
                 kv_block: int = 0):
        if isinstance(workload_or_desc, Desc):
            desc = workload_or_desc
        else:
            desc = desc_from_workload(workload_or_desc, q_block, kv_block)
        self.desc = desc
        self._h = ctypes.c_void_p()
        _check(lib().na_plan_create(ctypes.byref(desc), NA_PLAN_HOST_ONLY if host_only else 0,
                                    ctypes.byref(self._h)))
        st = Stats()
        _check(lib().na_plan_get_stats(self._h, ctypes.byref(st)))
        self.stats = {n: int(getattr(st, n)) for n, _ in Stats._fields_}
        self.dtype = "fp32" if desc.dtype == NA_F32 else "bf16"
        self.head_dim = int(desc.head_dim)

    def close(self):
        if getattr(self, "_h", None) and self._h.value:
            lib().na_plan_destroy(self._h)
            self._h = ctypes.c_void_p()

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    @property
    def n_tokens(self) -> int:
        return self.stats["n_tokens"]

    def classes(self) -> np.ndarray:
        nq, nk = self.stats["n_q_tiles"], self.stats["n_kv_tiles"]
        out = np.empty((nq, nk), dtype=np.uint8)
        _check(lib().na_plan_get_classes(self._h, out.ctypes.data_as(ctypes.c_void_p), out.size))
        return out

    def order(self) -> np.ndarray:
        out = np.empty(self.n_tokens, dtype=np.int32)
        _check(lib().na_plan_get_order(self._h, out.ctypes.data_as(ctypes.c_void_p), out.size))
        return out

    def effective_flops(self, B: int, H: int) -> int:
        """Unmasked QK^T + PV flops: 4 * D * attended pairs * B * H."""
        return 4 * self.head_dim * self.stats["attended_pairs"] * B * H

    def speedup_bounds(self) -> dict:
        """Upper bounds on the speedup of this pattern over dense attention of
        the same length and tile sizes, from the tile map alone (the kind of
        bound the "Generalized Neighborhood Attention" page's simulator gives,
        abstract: realistic rather than flop-count bounds):

        * ``flop``: N^2 / attended pairs, what counting flops promises;
        * ``tile``: dense tile pairs / non-empty tile pairs, what a kernel that
          skips empty tiles and pays full price for every other tile can reach;
        * ``useful_fraction``: attended pairs / pairs inside non-empty tiles
          (1.0 when every visited tile is full: a perfectly block-sparse map).
        """
        b = Bounds()
        _check(lib().na_plan_get_bounds(self._h, ctypes.byref(b)))
        return {"flop": b.flop, "tile": b.tile, "useful_fraction": b.useful_fraction}

    # -- device calls --------------------------------------------------------

    def _tensor(self, x, name):
        import torch

        want = torch.float32 if self.dtype == "fp32" else torch.bfloat16
        if x.dtype != want or x.dim() != 4 or not x.is_cuda:
            raise ValueError("%s must be a [B, H, N, D] %s device tensor" % (name, want))
        if x.shape[2] != self.n_tokens or x.shape[3] != self.head_dim or x.stride(3) != 1:
            raise ValueError("%s has shape %s / strides %s; the plan wants N=%d, D=%d with D "
                             "contiguous" % (name, tuple(x.shape), x.stride(), self.n_tokens,
                                             self.head_dim))
        return Tensor(x.data_ptr(), x.stride(0), x.stride(1), x.stride(2))

    def forward(self, q, k, v, out=None, lse=True, scale=None, permute_passes=False,
                split_tail=False, workspace=None, stream=None):
        """(out, lse) for [B, H, N, D] tensors in row-major token order.
        split_tail: NA_FWD_SPLIT_TAIL (the last round's query tiles split over
        the idle compute units; 48-query-per-wave kernels only)."""
        import torch

        B, H = int(q.shape[0]), int(q.shape[1])
        # every tensor the kernels write or read must cover (B, H): the C ABI
        # takes pointers and strides only, so a smaller one would be overrun
        _same_bh(B, H, k=k, v=v, out=out)
        if out is None:
            out = torch.empty_like(q, memory_format=torch.contiguous_format)
        if lse is True:
            lse = torch.empty((B, H, self.n_tokens), dtype=torch.float32, device=q.device)
        elif lse is False:
            lse = None
        if lse is not None and (lse.dtype != torch.float32 or not lse.is_contiguous()
                                or tuple(lse.shape) != (B, H, self.n_tokens)):
            raise ValueError("lse must be a contiguous float32 [B, H, N] tensor")
        if scale is None:
            scale = 1.0 / math.sqrt(self.head_dim)
        flags = ((NA_FWD_PERMUTE_PASSES if permute_passes else 0)
                 | (NA_FWD_SPLIT_TAIL if split_tail else 0))
        ws_bytes = int(lib().na_forward_workspace_bytes(self._h, B, H, flags))
        if ws_bytes and workspace is None:
            workspace = torch.empty(ws_bytes, dtype=torch.uint8, device=q.device)
        if ws_bytes:   # the library checks the size the caller actually supplied
            ws_bytes = workspace.numel() * workspace.element_size()
        if stream is None:
            stream = torch.cuda.current_stream(q.device).cuda_stream
        ts = [self._tensor(x, n) for x, n in ((q, "q"), (k, "k"), (v, "v"), (out, "out"))]
        _check(lib().na_forward(self._h, B, H, ctypes.byref(ts[0]), ctypes.byref(ts[1]),
                                ctypes.byref(ts[2]), ctypes.byref(ts[3]),
                                ctypes.c_void_p(lse.data_ptr() if lse is not None else None),
                                float(scale), flags,
                                ctypes.c_void_p(workspace.data_ptr() if ws_bytes else None),
                                ws_bytes, ctypes.c_void_p(stream)))
        return out, lse

    def backward(self, q, k, v, out, lse, dout, scale=None, grads=None, workspace=None,
                 stream=None):
        """(dq, dk, dv): gradients of sum(out * dout) for the forward's out and
        lse over the same q, k, v and scale.  grads: optional preallocated
        (dq, dk, dv)."""
        import torch

        B, H = int(q.shape[0]), int(q.shape[1])
        _same_bh(B, H, k=k, v=v, out=out, dout=dout)
        if grads is not None:
            if len(grads) != 3:
                raise ValueError("grads must be (dq, dk, dv)")
            _same_bh(B, H, dq=grads[0], dk=grads[1], dv=grads[2])
        if (lse.dtype != torch.float32 or not lse.is_contiguous()
                or tuple(lse.shape) != (B, H, self.n_tokens)):
            raise ValueError("lse must be a contiguous float32 [B, H, N] tensor")
        if scale is None:
            scale = 1.0 / math.sqrt(self.head_dim)
        if grads is None:
            grads = tuple(torch.empty_like(x, memory_format=torch.contiguous_format)
                          for x in (q, k, v))
        dq, dk, dv = grads
        ws_bytes = int(lib().na_backward_workspace_bytes(self._h, B, H))
        if workspace is None:
            workspace = torch.empty(ws_bytes, dtype=torch.uint8, device=q.device)
        ws_bytes = workspace.numel() * workspace.element_size()
        if stream is None:
            stream = torch.cuda.current_stream(q.device).cuda_stream
        ts = [self._tensor(x, n) for x, n in ((q, "q"), (k, "k"), (v, "v"), (out, "out"),
                                              (dout, "dout"), (dq, "dq"), (dk, "dk"), (dv, "dv"))]
        _check(lib().na_backward(self._h, B, H, *[ctypes.byref(t) for t in ts[:5]],
                                 ctypes.c_void_p(lse.data_ptr()),
                                 *[ctypes.byref(t) for t in ts[5:]], float(scale),
                                 ctypes.c_void_p(workspace.data_ptr()), ws_bytes,
                                 ctypes.c_void_p(stream)))
        return dq, dk, dv

    def backward_noalloc(self, q, k, v, out, lse, dout, grads, scale=None, stream=None):
        """na_backward_noalloc: the gradients into the caller's (dq, dk, dv)
        with the library's fixed per-GPU scratch (B * H * N <= 4,194,304);
        nothing is allocated.  Calls that overlap on one GPU race."""
        import torch

        B, H = int(q.shape[0]), int(q.shape[1])
        _same_bh(B, H, k=k, v=v, out=out, dout=dout)
        if len(grads) != 3:
            raise ValueError("grads must be (dq, dk, dv)")
        _same_bh(B, H, dq=grads[0], dk=grads[1], dv=grads[2])
        if (lse.dtype != torch.float32 or not lse.is_contiguous()
                or tuple(lse.shape) != (B, H, self.n_tokens)):
            raise ValueError("lse must be a contiguous float32 [B, H, N] tensor")
        if scale is None:
            scale = 1.0 / math.sqrt(self.head_dim)
        dq, dk, dv = grads
        if stream is None:
            stream = torch.cuda.current_stream(q.device).cuda_stream
        ts = [self._tensor(x, n) for x, n in ((q, "q"), (k, "k"), (v, "v"), (out, "out"),
                                              (dout, "dout"), (dq, "dq"), (dk, "dk"), (dv, "dv"))]
        _check(lib().na_backward_noalloc(self._h, B, H, *[ctypes.byref(t) for t in ts[:5]],
                                         ctypes.c_void_p(lse.data_ptr()),
                                         *[ctypes.byref(t) for t in ts[5:]], float(scale),
                                         ctypes.c_void_p(stream)))
        return dq, dk, dv

    def permute(self, x, inverse=False, out=None, stream=None):
        """Rows gathered into the plan's order (or scattered back with inverse)."""
        import torch

        _same_bh(int(x.shape[0]), int(x.shape[1]), out=out)
        if out is None:
            out = torch.empty_like(x, memory_format=torch.contiguous_format)
        if stream is None:
            stream = torch.cuda.current_stream(x.device).cuda_stream
        a, b = self._tensor(x, "in"), self._tensor(out, "out")
        _check(lib().na_permute(self._h, int(x.shape[0]), int(x.shape[1]), ctypes.byref(a),
                                ctypes.byref(b), 1 if inverse else 0, ctypes.c_void_p(stream)))
        return out

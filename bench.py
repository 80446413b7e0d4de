"""Benchmark: one step = one forward of the N-D local-attention hot path over one
batch of synthetic input, by default the 3-D sliding-tile workload (batch 1,
24 heads, head_dim 128, 30x48x80 tokens, 6x8x8 tiles, 3x5x7-tile window).

Prints ONE JSON line: effective TFLOP/s (only unmasked QK^T + PV flops,
4 * D * attended pairs * B * H per step), the roofline of the attention kernel
(MFMA bound against the MI355X dense peak of the dtype, or HBM bound against
8 TB/s when moving every tensor once takes longer than the flops at peak),
and the fp64 CPU oracle timed on a bounded sample of the same workload as a
reported baseline.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "effective TFLOP/s (unmasked FLOPs) + % bf16 MFMA peak, 3D sliding-tile attn"
PEAK_TFLOPS = {"bf16": 2516.6, "fp32": 157.3}  # MI355X dense MFMA (published)
PEAK_HBM_GBS = 8000.0                           # MI355X HBM3E (published)
ELEM_BYTES = {"bf16": 2, "fp32": 4}
PROFILE_PMC = os.path.join(ROOT, "profiles", "attn_fwd_sta3d_pmc.md")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def read_traffic(kernel_sig: str, workload: str, q_block: int):
    """HBM bytes per launch from the committed rocprofv3 PMC summary, if it
    was taken on the current kernel source, this workload and query tile (null
    otherwise)."""
    try:
        with open(PROFILE_PMC) as f:
            for line in f:
                if line.startswith("traffic_json:"):
                    d = json.loads(line.split(":", 1)[1])
                    if (d.get("kernel_sig") == kernel_sig and d.get("workload") == workload
                            and d.get("q_block", 256) == q_block):
                        return d.get("bytes_per_launch")
    except OSError:
        pass
    return None


def kernel_signature() -> str:
    import hashlib

    h = hashlib.sha256()
    for name in ("attn_fwd.hip", "attn_common.h"):
        with open(os.path.join(ROOT, "dimensional_sparse_local_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def cpu_baseline(wl, q, k, v, scale, target_s: float):
    """The oracle as it stands, on all host cores, over a bounded sample of
    query rows of one (batch, head) of the same workload."""
    import numpy as np

    import oracle

    q1, k1, v1 = (x[:1, :1].cpu().contiguous() for x in (q, k, v))
    n = q1.shape[2]
    rng = np.random.default_rng(0)
    order = rng.permutation(n)
    threads = oracle.max_threads()

    def run(count):
        rows = np.sort(order[:count]).astype(np.int64)
        t0 = time.perf_counter()
        oracle.attention(wl, q1, k1, v1, scale, rows=rows)
        dt = time.perf_counter() - t0
        if len(rows) == n:
            pairs = oracle.attended_pairs(wl)   # every row: the exact count
        else:
            # rows differ in their key counts (borders, causal starts): estimate
            # from a uniform subset of the sample, not from its first rows
            sub = rng.choice(rows, size=min(len(rows), 256), replace=False)
            pairs = sum(len(oracle.neighbors(wl, int(r))) for r in sub) * len(rows) / len(sub)
        return dt, pairs, len(rows)

    dt, _, c = run(min(n, 4 * threads))
    per_row = dt / c
    count = int(min(n, max(c, target_s / max(per_row, 1e-9))))
    dt, pairs, c = run(count)
    flops = 4.0 * int(wl["D"]) * pairs
    model = "unknown CPU"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
            "sample": "%d query rows of batch 0, head 0 (%.3g effective flops) in %.1f s, fp64, "
                      "OpenMP, %d threads on %s" % (c, flops, dt, threads, model)}


def main():
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default=None, help="workload name (default: the headline)")
    ap.add_argument("--q-block", type=int, default=0,
                    help="query tile; 0 = the forward pass takes 384 at head_dim 128 when every "
                         "visited tile pair is full at 384 (sliding-tile maps: each staged K/V "
                         "tile then serves 1.5x the queries), else the library default")
    ap.add_argument("--permute-passes", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--pass", dest="which", choices=("forward", "backward"), default="forward",
                    help="time the forward (default) or the backward pass (dq, dk, dv from the "
                         "forward's out and lse; effective flops 10 * D per attended pair: the "
                         "recomputed score and the dP, dV, dK, dQ products)")
    ap.add_argument("--vs-dense", action="store_true",
                    help="also time dense attention of the same shape on the same kernel (window "
                         "= whole grid) and report the measured speedup beside the tile map's "
                         "speedup bounds")
    ap.add_argument("--copy-probe", action="store_true",
                    help="run only the row-permute kernel over 268,435,456 bytes (read once, "
                         "written once): the known-size copy that calibrates HBM counters")
    args = ap.parse_args()

    if args.gpus != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path. The "
              "(batch, head) slices are independent, so N GPUs would each run this kernel on "
              "1/N of them with no communication. Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import torch

    from dimensional_sparse_local_amd import na
    from dimensional_sparse_local_amd import workloads as W

    if args.copy_probe:
        wl = dict(name="copy_probe", B=1, H=4, D=128, dtype="bf16", grid=[512, 512],
                  order="hilbert", pattern=dict(kind="band", left=1, right=1), seed=0)
        plan = na.Plan(wl)
        x = W.make_qkv(wl, device="cuda:0")[0]
        y = torch.empty_like(x)
        for _ in range(3):
            plan.permute(x, out=y)
        torch.cuda.synchronize()
        print(json.dumps({"copy_probe_bytes_read": x.numel() * 2,
                          "copy_probe_bytes_written": y.numel() * 2, "launches": 3}))
        return

    name = args.workload or W.HEADLINE
    wl = W.ALL[name]
    B, H, D = int(wl["B"]), int(wl["H"]), int(wl["D"])
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    q_block = args.q_block
    internal = None
    if q_block == 0 and args.which == "forward" and D == 128 and wl["dtype"] == "bf16":
        if na.Plan(wl, host_only=True, q_block=384).stats["n_partial"] == 0:
            q_block = 384
    if (q_block == 0 and args.which == "forward" and D == 64 and wl["dtype"] == "bf16"
            and wl["order"] == "row_major" and len(wl["grid"]) == 2
            and wl["pattern"]["kind"] in ("na", "sa")):
        # the token order inside the kernel is free (q, k, v, out stay row-major):
        # 8x8 patches make the visited tile pairs denser, 64-query tiles give
        # the short walks more workgroups
        internal = dict(order="tiled", tile=[8, 8])
        q_block = 64
    plan = na.Plan(W.scaled(wl, **internal) if internal else wl, q_block=q_block)
    flops = plan.effective_flops(B, H)
    q, k, v = W.make_qkv(wl, device=dev)
    scale = W.default_scale(wl)
    out = torch.empty_like(q)
    lse = torch.empty((B, H, plan.n_tokens), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream(dev)
    log("bench: %s plan %s" % (name, plan.stats))

    def step():
        plan.forward(q, k, v, out=out, lse=lse, scale=scale, permute_passes=args.permute_passes)

    if args.which == "backward":
        if args.permute_passes:
            raise SystemExit("--permute-passes applies to the forward pass only")
        dout = W.make_dout(wl, device=dev)
        step()
        grads = tuple(torch.empty_like(x) for x in (q, k, v))
        ws = torch.empty(int(na.lib().na_backward_workspace_bytes(plan._h, B, H)),
                         dtype=torch.uint8, device=dev)
        flops = flops * 10 // 4

        def step():
            plan.backward(q, k, v, out, lse, dout, scale=scale, grads=grads, workspace=ws)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    log("bench: warmup done")
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record(stream)
    for _ in range(args.steps):
        step()
    end.record(stream)
    torch.cuda.synchronize()
    ms = start.elapsed_time(end) / args.steps
    log("bench: %.3f ms/step" % ms)
    tflops = flops / (ms * 1e-3) / 1e12
    peak = PEAK_TFLOPS[wl["dtype"]]
    # Algorithmic HBM bytes per step: every tensor read or written once
    # (forward: q, k, v in, out and fp32 lse out; backward: q, k, v, out, dout
    # and lse in, dq, dk, dv out).
    n_rows = B * H * plan.n_tokens
    row_tensors = 4 if args.which == "forward" else 8
    alg_bytes = n_rows * (row_tensors * D * ELEM_BYTES[wl["dtype"]] + 4)
    hbm_bound = alg_bytes / (PEAK_HBM_GBS * 1e9) > flops / (peak * 1e12)
    gbs = alg_bytes / (ms * 1e-3) / 1e9

    sparsity = None
    if args.vs_dense:
        if args.which != "forward" or args.permute_passes:
            raise SystemExit("--vs-dense times the plain forward pass only")
        n_tok = plan.n_tokens
        if wl["order"] == "hilbert":
            dense_pat = dict(kind="band", left=n_tok, right=n_tok)
        else:
            dense_pat = dict(kind="na", window=list(wl["grid"]))
        dense = na.Plan(W.scaled(wl, pattern=dense_pat), q_block=q_block)
        dense_out = torch.empty_like(q)
        dense_lse = torch.empty_like(lse)

        def dense_step():
            dense.forward(q, k, v, out=dense_out, lse=dense_lse, scale=scale)

        dense_steps = max(2, args.steps // 4)
        for _ in range(2):
            dense_step()
        torch.cuda.synchronize()
        start.record(stream)
        for _ in range(dense_steps):
            dense_step()
        end.record(stream)
        torch.cuda.synchronize()
        dense_ms = start.elapsed_time(end) / dense_steps
        log("bench: dense %.3f ms/step" % dense_ms)
        sparsity = {"dense_ms_per_step": round(dense_ms, 4),
                    "dense_tflops": round(dense.effective_flops(B, H) / (dense_ms * 1e-3) / 1e12, 3),
                    "speedup_vs_dense": round(dense_ms / ms, 4),
                    "bounds": {k: round(x, 4) for k, x in plan.speedup_bounds().items()}}

    cpu = None
    if not args.no_cpu_baseline and args.which == "forward":
        log("bench: timing the CPU oracle (~%.0f s)" % args.cpu_seconds)
        cpu = cpu_baseline(wl, q, k, v, scale, args.cpu_seconds)

    sig = kernel_signature()
    if name == W.HEADLINE and args.which == "forward":
        metric = METRIC
    else:
        metric = "effective TFLOP/s (unmasked FLOPs), %s%s" % (
            wl.get("note", name), ", backward pass" if args.which == "backward" else "")
    traffic = read_traffic(sig, name, plan.stats["q_block"]) if args.which == "forward" else None
    if hbm_bound:
        roof = {"bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": round(gbs / PEAK_HBM_GBS, 4)}
    else:
        roof = {"bound": "mfma", "achieved": round(tflops, 3), "peak": peak, "unit": "TFLOP/s",
                "frac": round(tflops / peak, 4)}
    roof.update({"traffic": traffic, "algorithmic_bytes": alg_bytes, "kernel_sig": sig})
    line = {
        "metric": metric,
        "value": round(tflops, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": wl["dtype"],
        "data": "synthetic",
        "config": {"workload": name, "batch": B, "heads": H, "head_dim": D, "grid": wl["grid"],
                   "order": wl["order"], "pattern": wl["pattern"],
                   "q_block": plan.stats["q_block"], "kv_block": plan.stats["kv_block"],
                   "attended_pairs_per_head": plan.stats["attended_pairs"],
                   "effective_flops_per_step": flops,
                   "pct_of_peak": round(100.0 * tflops / peak, 2),
                   "permute_passes": bool(args.permute_passes), "pass": args.which,
                   "internal_order": internal or {"order": wl["order"]}},
        "roofline": roof,
        "cpu_baseline": cpu,
    }
    if sparsity is not None:
        line["sparsity"] = sparsity
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()

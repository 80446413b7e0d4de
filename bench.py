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


def read_traffic(kernel_sig: str, workload: str, q_block: int, split_tail: bool, passes: bool):
    """HBM bytes per launch of the attention kernel from the committed
    rocprofv3 PMC summary, if it was taken on the current kernel source, this
    workload, query tile and launch flags (null otherwise)."""
    try:
        with open(PROFILE_PMC) as f:
            for line in f:
                if line.startswith("traffic_json:"):
                    d = json.loads(line.split(":", 1)[1])
                    if (d.get("kernel_sig") == kernel_sig and d.get("workload") == workload
                            and d.get("q_block", 256) == q_block
                            and bool(d.get("split_tail", False)) == split_tail
                            and bool(d.get("permute_passes", False)) == passes):
                        return d.get("bytes_per_launch")
    except OSError:
        pass
    return None


def _stats(xs):
    ys = sorted(xs)
    n = len(ys)
    med = ys[n // 2] if n % 2 else 0.5 * (ys[n // 2 - 1] + ys[n // 2])
    return {"median": round(med, 4), "min": round(ys[0], 4), "max": round(ys[-1], 4),
            "mean": round(sum(ys) / n, 4)}


def kernel_signature() -> str:
    """sha256[:16] of the source of the 48-query-per-wave forward kernel and
    its combine kernel (the part of attn_fwd.hip from the 16x16x32 helpers to
    the fp32 kernel), attn_common.h and the planner (plan.cpp: the walk order
    of each tile row and the dispatch order of the tiles): the code the
    committed traffic counters were taken on."""
    import hashlib

    csrc = os.path.join(ROOT, "dimensional_sparse_local_amd", "csrc")
    with open(os.path.join(csrc, "attn_fwd.hip"), "rb") as f:
        text = f.read()
    start = text.index(b"__device__ __forceinline__ float quad_max(float x) {")
    end = text.index(b"// fp32: one wave, 32 queries", start)
    h = hashlib.sha256()
    h.update(text[start:end])
    for name in ("attn_common.h", "plan.cpp"):
        with open(os.path.join(csrc, name), "rb") as f:
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
    ap.add_argument("--warmup", type=int, default=None,
                    help="untimed warm-up steps (default: as many as fill 1 s, at least 5: the "
                         "clock ramps up over the first tens of milliseconds of load, which "
                         "a sub-millisecond step would otherwise time)")
    ap.add_argument("--workload", default=None, help="workload name (default: the headline)")
    ap.add_argument("--q-block", type=int, default=0,
                    help="query tile; 0 = the forward pass takes the launch of "
                         "na.forward_launch (384 with the split tail at head_dim 128 in bf16; 8x8 "
                         "patch order and 64 at head_dim 64 for 2-D windows in row-major order), "
                         "the backward pass the library default")
    ap.add_argument("--permute-passes", action="store_true")
    ap.add_argument("--graph", action="store_true",
                    help="capture one step into a HIP graph and time its replays (no host "
                         "launch between steps; measured slower than direct launches for these "
                         "one- or two-kernel steps, e.g. 38.3 against 32.6 us on the 64x64 "
                         "neighbourhood: the direct launches are not host-bound)")
    ap.add_argument("--no-split-tail", action="store_true",
                    help="run the forward without NA_FWD_SPLIT_TAIL even where its launch "
                         "takes it")
    ap.add_argument("--rounds", type=int, default=0,
                    help="also time the Hilbert page's protocol after the timed steps: this many "
                         "rounds of 100 iterations, each after 25 untimed ones (a quarter of "
                         "the round), reported as the median, min and max of the rounds' mean "
                         "step times under \"rounds_ms\" (10 on the page; 0 = off)")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--pass", dest="which", choices=("forward", "backward", "permute"),
                    default="forward",
                    help="time the forward (default), the backward pass (dq, dk, dv from the "
                         "forward's out and lse; effective flops 10 * D per attended pair: the "
                         "recomputed score and the dP, dV, dK, dQ products), or the row gather "
                         "along the plan's order alone (q into sequence order; GB/s of rows read "
                         "and written against 8 TB/s)")
    ap.add_argument("--vs-dense", action="store_true",
                    help="also time dense attention of the same shape on the same kernel (window "
                         "= whole grid) and report the measured speedup beside the tile map's "
                         "speedup bounds")
    ap.add_argument("--plan-times", action="store_true",
                    help="only time host plan creation (tile map, CSR, masks; no device upload) "
                         "for the five named workloads in their forward launch: median of 3, one "
                         "JSON line each (runs without a GPU)")
    ap.add_argument("--copy-probe", action="store_true",
                    help="run only the row-permute kernel over 268,435,456 bytes (read once, "
                         "written once): the known-size copy that calibrates HBM counters")
    args = ap.parse_args()

    if args.gpus != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path. The "
              "(batch, head) slices are independent, so N GPUs would each run this kernel on "
              "1/N of them with no communication. Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    if args.plan_times:
        from dimensional_sparse_local_amd import na
        from dimensional_sparse_local_amd import workloads as W

        for name in ("na2d_fp32", "na2d_bf16", "sta3d_bf16", "hilbert_band_bf16",
                     "causal1d_bf16"):
            wl, q_block, _ = na.forward_launch(W.CONFIGS[name])
            ts = []
            for _ in range(3):
                t0 = time.perf_counter()
                plan = na.Plan(wl, host_only=True, q_block=q_block)
                ts.append(time.perf_counter() - t0)
            st = plan.stats
            print(json.dumps({"workload": name, "plan_ms": round(sorted(ts)[1] * 1e3, 2),
                              "q_block": st["q_block"], "n_q_tiles": st["n_q_tiles"],
                              "n_kv_tiles": st["n_kv_tiles"],
                              "non_empty": st["n_partial"] + st["n_full"]}), flush=True)
        return

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
    kernel_wl, q_block, split = wl, args.q_block, False
    if q_block == 0 and args.which == "forward":
        kernel_wl, q_block, split = na.forward_launch(wl)
    split = split and not args.no_split_tail
    internal = kernel_wl is not wl
    plan = na.Plan(kernel_wl, q_block=q_block)
    flops = plan.effective_flops(B, H)
    q, k, v = W.make_qkv(wl, device=dev)
    scale = W.default_scale(wl)
    out = torch.empty_like(q)
    lse = torch.empty((B, H, plan.n_tokens), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream(dev)
    # the forward's workspace (permute passes, split tail), allocated once
    flags = ((na.NA_FWD_PERMUTE_PASSES if args.permute_passes else 0)
             | (na.NA_FWD_SPLIT_TAIL if split else 0))
    ws_bytes = int(na.lib().na_forward_workspace_bytes(plan._h, B, H, flags))
    fwd_ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev) if ws_bytes else None
    log("bench: %s plan %s split_tail=%s workspace=%d" % (name, plan.stats, split, ws_bytes))

    def step():
        plan.forward(q, k, v, out=out, lse=lse, scale=scale, permute_passes=args.permute_passes,
                     split_tail=split, workspace=fwd_ws)

    if args.which == "permute":
        if wl["order"] == "row_major" or internal:
            raise SystemExit("--pass permute needs a workload with a tiled or Hilbert order")
        gathered = torch.empty_like(q)
        flops = 0

        def step():
            plan.permute(q, out=gathered)

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

    if args.warmup is None:
        args.warmup = 0
        t_warm = time.perf_counter()
        while args.warmup < 5 or time.perf_counter() - t_warm < 1.0:
            step()
            args.warmup += 1
            if args.warmup % 8 == 0:
                torch.cuda.synchronize()
    else:
        for _ in range(args.warmup):
            step()
    torch.cuda.synchronize()
    if args.graph:
        # one step captured into a HIP graph and replayed: no host launch
        # cost between steps (the launches of a step are the same kernels)
        side = torch.cuda.Stream()
        side.wait_stream(stream)
        with torch.cuda.stream(side):
            step()
        stream.wait_stream(side)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            step()
        torch.cuda.synchronize()
        step = graph.replay
        for _ in range(args.warmup):
            step()
        torch.cuda.synchronize()
    log("bench: warmup done")
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    # one HIP event after each step, on the stream the kernels run on: the
    # per-step times (each step is one launch of the hot path)
    marks = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    torch.cuda.synchronize()
    start.record(stream)
    for i in range(args.steps):
        step()
        marks[i].record(stream)
    end.record(stream)
    torch.cuda.synchronize()
    ms = start.elapsed_time(end) / args.steps
    per_step = [start.elapsed_time(marks[0])] + [marks[i - 1].elapsed_time(marks[i])
                                                  for i in range(1, args.steps)]
    step_stats = _stats(per_step)
    log("bench: %.3f ms/step (median %.3f, min %.3f, max %.3f)"
        % (ms, step_stats["median"], step_stats["min"], step_stats["max"]))
    rounds_stats = None
    if args.rounds > 0:
        # "Hilbert-Guided Sparse Local Attention", Methodology in Plain English:
        # the median over repeated rounds of 100 iterations, a quarter of each
        # round run first as warm-up
        round_ms = []
        for _ in range(args.rounds):
            for _ in range(25):
                step()
            r0 = torch.cuda.Event(enable_timing=True)
            r1 = torch.cuda.Event(enable_timing=True)
            r0.record(stream)
            for _ in range(100):
                step()
            r1.record(stream)
            torch.cuda.synchronize()
            round_ms.append(r0.elapsed_time(r1) / 100)
        rounds_stats = dict(_stats(round_ms), rounds=args.rounds, iterations=100, warmup=25)
        log("bench: rounds of 100: median %.4f ms (min %.4f, max %.4f)"
            % (rounds_stats["median"], rounds_stats["min"], rounds_stats["max"]))
    tflops = flops / (ms * 1e-3) / 1e12
    peak = PEAK_TFLOPS[wl["dtype"]]
    # Algorithmic HBM bytes per step: every tensor read or written once
    # (forward: q, k, v in, out and fp32 lse out; backward: q, k, v, out, dout
    # and lse in, dq, dk, dv out).
    # Permute: each row read once and written once.
    n_rows = B * H * plan.n_tokens
    if args.which == "permute":
        alg_bytes = n_rows * 2 * D * ELEM_BYTES[wl["dtype"]]
    else:
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
    value, unit = round(tflops, 3), "TFLOP/s"
    if name == W.HEADLINE and args.which == "forward":
        metric = METRIC
    elif args.which == "permute":
        metric = "row gather along the plan's order (GB/s read + written), %s" % wl.get("note", name)
        value, unit = round(gbs, 1), "GB/s"
    else:
        metric = "effective TFLOP/s (unmasked FLOPs), %s%s" % (
            wl.get("note", name), ", backward pass" if args.which == "backward" else "")
    traffic = (read_traffic(sig, name, plan.stats["q_block"], split, bool(args.permute_passes))
               if args.which == "forward" else None)
    if hbm_bound:
        roof = {"bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": round(gbs / PEAK_HBM_GBS, 4)}
    else:
        roof = {"bound": "mfma", "achieved": round(tflops, 3), "peak": peak, "unit": "TFLOP/s",
                "frac": round(tflops / peak, 4)}
    roof.update({"traffic": traffic, "algorithmic_bytes": alg_bytes, "kernel_sig": sig,
                 "traffic_source": ("rocprofv3 FETCH_SIZE + WRITE_SIZE on this kernel source, "
                                    "committed in profiles/attn_fwd_sta3d_pmc.md"
                                    if traffic is not None else None)})
    line = {
        "metric": metric,
        "value": value,
        "unit": unit,
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "step_ms": step_stats,
        **({"rounds_ms": rounds_stats} if rounds_stats else {}),
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
                   "permute_passes": bool(args.permute_passes), "split_tail": split,
                   "graph": bool(args.graph),
                   "pass": args.which,
                   "internal_order": ({k: kernel_wl[k] for k in ("order", "tile")} if internal
                                      else {"order": wl["order"]})},
        "roofline": roof,
        "cpu_baseline": cpu,
    }
    if sparsity is not None:
        line["sparsity"] = sparsity
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()

#!/usr/bin/env python3
"""Benchmark of the sparse COO layer's hot path on one MI355X.

Workload: one 10000 x 10000 layer at 95 % unstructured sparsity (nnz =
5,000,000 uniform random positions), fp32 values, int32 indices, trained with
the batch sweep B in {1, 2, 4, 8, 16, 32, 64}.  One *step* is one training
iteration at every batch size of the sweep, each iteration being forward
Y = X W^T, MSE gradient, backward (dX and dW on the support) and an SGD update
(lr 0.01) of the values, issued as one snack_train_step_mse call per
iteration; after every 10th iteration the layer drops the 30 %
smallest-|w| entries and regrows as many at random empty positions (SET-style,
nnz fixed).  Inputs are synthetic (seeded N(0,1) activations and targets) and
resident in device memory before the timed region starts.

Printed: one JSON line.  `value` is the achieved algorithmic bandwidth over
the timed region -- the bytes the method must move for forward + backward
(28 nnz + 4 B (3K + 2M)), the MSE gradient (12 B M) and SGD (12 nnz), per
iteration, divided by the wall time of the whole timed region, which also
contains the drop/regrow calls (they add time but no credited bytes).  That
region runs without instrumentation; the same number of steps then runs a
second time with HIP events around every kernel class, which gives
`per_batch` (forward+backward microseconds per iteration: fwd, dX, dW and
their activation transposes) and `roofline` (the dominant kernel against the
8 TB/s HBM peak).  `cold` times forward + backward once per repetition right
after a 512 MiB write that evicts the Infinity Cache and the L2s (the triple
then streams from HBM; the warm figures above run with it cache-resident).
`cpu_baseline` is the fp64 oracle timed on one host core on a bounded sample.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "SpMM fwd+bwd µs/iter + achieved GB/s, 10000² at 95% sparse, batch 1–64"
HBM_PEAK_GBPS = 8000.0


def fwd_bwd_bytes(nnz, M, K, B):
    return 28 * nnz + 4 * B * (3 * K + 2 * M)


def kernel_bytes(kind, nnz, M, K, B):
    # per launch, algorithmic: what the kernel's part of the method must move
    if kind == "spmm_forward":
        # the triple (12 B / entry), X once, Y once
        return 12 * nnz + 4 * B * (K + M)
    if kind == "spmm_dx":
        # column pass of the fused backward + SGD: index + value read per entry; written per entry, the
        # value after its SGD step, and at the 64-column tile also dW in column order (the canonical dW is
        # permuted from it there; narrower tiles recompute it over the row view); dY, X once; dX once
        per_entry = 12 + (4 if B > 32 else 0)
        return per_entry * nnz + 4 * B * (M + 2 * K)
    raise KeyError(kind)


TRAFFIC_FILES = {"spmm_dx (B=64)": os.path.join(ROOT, "profiles", "spmm_dx_b64_traffic.md")}
KERNEL_SOURCE = os.path.join(ROOT, "coo_spmm_amd", "csrc", "spmm.hip")


def measured_traffic(kernel_label):
    """HBM bytes per launch from the committed counter summary of this kernel, or None when there is
    none or when the kernel source changed since the counters were taken."""
    import hashlib
    path = TRAFFIC_FILES.get(kernel_label)
    if not path or not os.path.exists(path):
        return None
    fields = {}
    for line in open(path):
        if ":" in line and not line.startswith(("#", "|", " ")):
            k, v = line.split(":", 1)
            fields[k.strip()] = v.strip()
    if "traffic_bytes_per_launch" not in fields or "source_sha256" not in fields:
        return None
    if hashlib.sha256(open(KERNEL_SOURCE, "rb").read()).hexdigest() != fields["source_sha256"]:
        return None
    return int(fields["traffic_bytes_per_launch"])


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=30)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--batches", default="1,2,4,8,16,32,64")
    ap.add_argument("--prune-every", type=int, default=10)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-profile", action="store_true", help="time without per-kernel HIP events")
    ap.add_argument("--cold-reps", type=int, default=3,
                    help="cold forward + backward timings per batch size, each after a 512 MiB write that "
                         "evicts the Infinity Cache and the L2s (0: skip)")
    ap.add_argument("--copy-probe-mb", type=int, default=0,
                    help="before timing, run one plain device copy of this many MiB (a reference dispatch of known "
                         "size for hardware byte counters)")
    ap.add_argument("--layers", choices=("gpt2",), default=None,
                    help="instead of the default workload: time forward, backward and the one-call training step "
                         "of the GPT-2-small MLP layer shapes (768 -> 3072 and 3072 -> 768 at 90 and 99 %% "
                         "sparsity) at 64, 256 and 1024 tokens; prints one JSON line of per-layer timings")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)
    if args.layers == "gpt2":
        return layer_shapes(args)

    import numpy as np
    import torch

    import coo_spmm_amd as L
    from snack_inputs import normal, random_layer, weight_std

    torch.cuda.set_device(0)
    if args.copy_probe_mb > 0:
        n = args.copy_probe_mb * (1 << 20) // 4
        src = torch.ones(n, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    M = K = 10000
    sparsity = 95
    nnz = M * K * (100 - sparsity) // 100
    batches = [int(b) for b in args.batches.split(",")]
    n_drop = nnz * 3 // 10
    lr = 0.01

    rows, cols, vals = random_layer(M, K, nnz, "c4/s95", weight_std(K, sparsity))
    layer = L.SnackLayer(M, K, torch.from_numpy(rows).cuda(), torch.from_numpy(cols).cuda(),
                         torch.from_numpy(vals).cuda(), seed=2024)
    layer.reserve(max(batches))
    bufs = {}
    for B in batches:
        X = torch.from_numpy(normal((B, K), f"c4/X/{B}")).cuda()
        T = torch.from_numpy(normal((B, M), f"c4/T/{B}")).cuda()
        bufs[B] = dict(X=X, T=T, Y=torch.empty(B, M, device="cuda"), dY=torch.empty(B, M, device="cuda"),
                       dX=torch.empty(B, K, device="cuda"), dW=torch.empty(nnz, device="cuda"))
    stream = torch.cuda.current_stream()

    it_counter = [0]

    def iteration(B):
        b = bufs[B]
        # forward, MSE gradient, backward (dX, dW) and the SGD step in one call (the same
        # results, bit for bit, as snack_forward + snack_mse_grad + snack_backward_sgd)
        L.snack_train_step_mse(layer.h, b["X"], b["T"], b["Y"], b["dY"], b["dX"], b["dW"], 2.0 / (B * M), lr,
                               stream)
        it_counter[0] += 1
        if args.prune_every > 0 and it_counter[0] % args.prune_every == 0:
            L.snack_profile_set_tag(-1)
            L.snack_prune_regrow(layer.h, n_drop, stream)

    def step():
        for B in batches:
            L.snack_profile_set_tag(B)
            iteration(B)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    cls = L.profile_class_ids()

    # timed pass 1: the value -- no instrumentation inside the timed region
    L.snack_profile_enable(False)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    wall = t1 - t0

    # timed pass 2: the same steps again with HIP events around every kernel class
    # (per-batch breakdown and the roofline kernel); events cost host time, so this
    # pass is slower and is not used for the value
    wall_prof = None
    if not args.no_profile:
        L.snack_profile_reset()
        L.snack_profile_enable(True)
        torch.cuda.synchronize()
        t2 = time.perf_counter()
        for _ in range(args.steps):
            step()
        torch.cuda.synchronize()
        wall_prof = time.perf_counter() - t2
        L.snack_profile_enable(False)

    # cold: forward + backward alone, each right after a 512 MiB write (more than the 256 MB Infinity
    # Cache plus the L2s), so the triple and the index come from HBM; timed with events on the launch stream
    cold = None
    if args.cold_reps > 0:
        flush = torch.empty((512 << 20) // 4, dtype=torch.float32, device="cuda")
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        cold = {"reps": args.cold_reps, "flush_mib": 512, "per_batch": {}}
        for B in batches:
            b = bufs[B]
            ts = []
            for rep in range(args.cold_reps):
                flush.fill_(float(rep + 1))
                e0.record(stream)
                L.snack_forward(layer.h, b["X"], b["Y"], stream)
                L.snack_backward(layer.h, b["X"], b["dY"], b["dX"], b["dW"], stream)
                e1.record(stream)
                e1.synchronize()
                ts.append(e0.elapsed_time(e1) * 1e3)
            us = sorted(ts)[len(ts) // 2]
            cold["per_batch"][str(B)] = {"fwd_bwd_us": round(us, 2),
                                         "fwd_bwd_GBps": round(fwd_bwd_bytes(nnz, M, K, B) / (us * 1e-6) / 1e9, 1)}
        del flush

    iters_per_b = args.steps
    credited = sum((fwd_bwd_bytes(nnz, M, K, B) + 12 * B * M + 12 * nnz) * iters_per_b for B in batches)
    value_gbps = credited / wall / 1e9

    per_batch = {}
    dominant = None
    for B in batches:
        d = {}
        tot_us = 0.0
        for name in ("spmm_forward", "spmm_dx", "sddmm_dw", "transpose", "vals_t_refresh", "sgd", "elementwise"):
            n, ms = L.snack_profile_read_tag(cls[name], B)
            d[name + "_us"] = round(ms * 1e3 / max(iters_per_b, 1), 3)
            if name in ("spmm_forward", "spmm_dx", "sddmm_dw", "transpose", "vals_t_refresh"):
                tot_us += ms * 1e3 / max(iters_per_b, 1)
            if name in ("spmm_forward", "spmm_dx") and n > 0:
                if dominant is None or ms > dominant[3]:
                    dominant = (name, B, n, ms)
        d["fwd_bwd_us"] = round(tot_us, 3)
        if tot_us > 0:
            gbps = fwd_bwd_bytes(nnz, M, K, B) / (tot_us * 1e-6) / 1e9
            d["fwd_bwd_GBps"] = round(gbps, 1)
            d["fwd_bwd_frac_of_hbm"] = round(gbps / HBM_PEAK_GBPS, 4)
        per_batch[str(B)] = d
    n_pr, ms_pr = L.snack_profile_read_tag(cls["prune_regrow"], -1)

    roofline = None
    if dominant is not None:
        name, B, n, ms = dominant
        per_launch = kernel_bytes(name, nnz, M, K, B)
        achieved = per_launch * n / (ms * 1e-3) / 1e9
        roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                    "frac": round(achieved / HBM_PEAK_GBPS, 4), "traffic": measured_traffic(f"{name} (B={B})"),
                    "kernel": f"{name} (B={B})", "avg_launch_us": round(ms * 1e3 / n, 3),
                    "bytes_per_launch": per_launch}

    out = {
        "metric": METRIC,
        "value": round(value_gbps, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(wall * 1e3 / args.steps, 4),
        "ms_per_step_instrumented": round(wall_prof * 1e3 / args.steps, 4) if wall_prof else None,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": ("10000x10000 COO layer, 95% sparse (nnz 5,000,000), batch sweep "
                                f"{'/'.join(map(str, batches))}; fwd + MSE grad + bwd(dX, dW) + SGD per batch; "
                                f"drop/regrow 30% every {args.prune_every} iterations"),
                   "M": M, "K": K, "nnz": nnz, "batches": batches, "n_drop": n_drop, "lr": lr,
                   "parallelism": "single GPU"},
        "per_batch": per_batch,
        "prune_regrow_us_per_call": round(ms_pr * 1e3 / n_pr, 1) if n_pr else None,
        "prune_regrow_calls": n_pr,
        "roofline": roofline,
        "cold": cold,
    }

    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(layer, M, K, nnz, batches, lr)

    layer.close()
    print(json.dumps(out), flush=True)


def layer_shapes(args):
    """Per-layer timings of the GPT-2-small MLP shapes (not the default workload):
    synthetic N(0,1) activations and targets, uniform random supports; each
    call timed with events over `--steps` repetitions after `--warmup`."""
    import torch
    import coo_spmm_amd as L
    from snack_inputs import normal, random_layer

    torch.cuda.set_device(0)
    res = {}
    for (M, K) in ((3072, 768), (768, 3072)):
        for sp in (90, 99):
            nnz = M * K * (100 - sp) // 100
            r, c, v = random_layer(M, K, nnz, f"gpt2/{M}x{K}/{sp}")
            layer = L.SnackLayer(M, K, torch.from_numpy(r).cuda(), torch.from_numpy(c).cuda(),
                                 torch.from_numpy(v).cuda())
            try:
                layer.reserve(1024)
                for B in (64, 256, 1024):
                    X = torch.from_numpy(normal((B, K), f"gpt2/X/{K}/{B}")).cuda()
                    T = torch.from_numpy(normal((B, M), f"gpt2/T/{M}/{B}")).cuda()
                    Y = torch.empty(B, M, device="cuda"); dY = torch.empty(B, M, device="cuda")
                    dX = torch.empty(B, K, device="cuda"); dW = torch.empty(nnz, device="cuda")
                    calls = {
                        "fwd": lambda: L.snack_forward(layer.h, X, Y),
                        "bwd": lambda: L.snack_backward(layer.h, X, dY, dX, dW),
                        "train_step": lambda: L.snack_train_step_mse(layer.h, X, T, Y, dY, dX, dW,
                                                                     2.0 / (B * M), 0.0),
                    }
                    d = {}
                    for name, f in calls.items():
                        for _ in range(args.warmup):
                            f()
                        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                        torch.cuda.synchronize()
                        e0.record()
                        for _ in range(args.steps):
                            f()
                        e1.record()
                        e1.synchronize()
                        d[name + "_us"] = round(e0.elapsed_time(e1) * 1e3 / args.steps, 2)
                    d["fwd_TFLOPs"] = round(2.0 * B * nnz / (d["fwd_us"] * 1e-6) / 1e12, 2)
                    d["bwd_TFLOPs"] = round(4.0 * B * nnz / (d["bwd_us"] * 1e-6) / 1e12, 2)
                    res[f"{M}x{K}/s{sp}/B{B}"] = d
            finally:
                layer.close()
    print(json.dumps({"layers": "gpt2-small MLP shapes", "data": "synthetic", "dtype": "f32",
                      "steps": args.steps, "warmup": args.warmup, "timings": res}))


def cpu_baseline(layer, M, K, nnz, batches, lr, min_seconds=10.0, max_steps=20):
    """The fp64 oracle as it stands, one host core, on a bounded sample of the
    workload: whole sweep steps (forward, MSE gradient, dX, dW and SGD for every
    batch size, no drop/regrow) repeated until about ten seconds have passed."""
    import numpy as np

    import oracle
    from snack_inputs import normal

    r, c, v = (t.cpu().numpy() for t in layer.export())
    inputs = [(B, normal((B, K), f"c4/X/{B}"), normal((B, M), f"c4/T/{B}")) for B in batches]
    credited = 0
    steps = 0
    t0 = time.perf_counter()
    while True:
        for B, X, T in inputs:
            Y, _ = oracle.forward(M, K, r, c, v, X)
            dY = oracle.mse_grad(Y.astype(np.float32), T).astype(np.float32)
            oracle.backward_dx(M, K, r, c, v, dY)
            dW, _ = oracle.backward_dw(M, K, r, c, X, dY)
            v = oracle.sgd(v, dW.astype(np.float32), lr).astype(np.float32)
            credited += fwd_bwd_bytes(nnz, M, K, B) + 12 * B * M + 12 * nnz
        steps += 1
        dt = time.perf_counter() - t0
        if dt >= min_seconds or steps >= max_steps:
            break
    try:
        cores = len(os.sched_getaffinity(0))
    except Exception:
        cores = os.cpu_count()
    return {"value": round(credited / dt / 1e9, 4), "unit": "GB/s", "cores": 1, "kind": "oracle",
            "sample": "%d sweep step(s) (fwd, MSE grad, dX, dW, SGD for B = %s) without drop/regrow; "
                      "single-threaded fp64 C oracle; %.1f s; host has %s usable cores"
                      % (steps, "/".join(map(str, batches)), dt, cores),
            "seconds": round(dt, 2)}


if __name__ == "__main__":
    main()

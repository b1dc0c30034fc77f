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
the per-kernel-class breakdown in `per_batch` and `roofline` (the dominant
kernel against its binding floor: the 8 TB/s HBM peak or the 78.6 TFLOP/s
non-packed fp32 FMA rate).  `per_batch[B].fwd_bwd_us` is one whole training
iteration at that batch size (forward, MSE gradient, dX, dW, SGD), timed back
to back with one pair of events around all of them, credited with the
forward + backward bytes only.  `cold` times forward + backward once per repetition right
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
# fp32 FMA issue rate without packed-fp32 instructions (which this build keeps
# off): 256 CUs x 4 SIMDs x 16 lanes x 2 flops x 2.4 GHz
VALU_PEAK_TFLOPS = 78.6


def fwd_bwd_bytes(nnz, M, K, B):
    return 28 * nnz + 4 * B * (3 * K + 2 * M)


def fwd_bwd_flops(nnz, B):
    # forward, dX and dW: one multiply-add per stored entry and batch column each
    return 6 * B * nnz


def kernel_flops(kind, nnz, B):
    if kind == "spmm_forward":
        return 2 * B * nnz
    if kind == "spmm_dx":
        # the column pass computes dX and, fused into it, dW (in column order at the 64-column tile;
        # narrower tiles recompute the canonical dW in their row pass instead)
        return (4 if B > 32 else 2) * B * nnz
    raise KeyError(kind)


def roofline_entry(bytes_, flops, seconds):
    """Both floors of one timed piece of work: achieved HBM-side bandwidth against
    8 TB/s and achieved fp32 rate against the non-packed VALU rate, and which of
    the two floors (time at peak) is the higher, i.e. binds."""
    gbps = bytes_ / seconds / 1e9
    tflops = flops / seconds / 1e12
    t_hbm = bytes_ / (HBM_PEAK_GBPS * 1e9)
    t_alu = flops / (VALU_PEAK_TFLOPS * 1e12)
    return {"GBps": round(gbps, 1), "frac_hbm": round(gbps / HBM_PEAK_GBPS, 4),
            "TFLOPs": round(tflops, 2), "frac_valu": round(tflops / VALU_PEAK_TFLOPS, 4),
            "binding": "alu" if t_alu > t_hbm else "hbm",
            "floor_us": round(max(t_hbm, t_alu) * 1e6, 2)}


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
    ap.add_argument("--no-configs", action="store_true",
                    help="skip the legs of the other workloads (500x500 layer, 5000x5000 sparsity sweep against a "
                         "masked-dense matmul, 10000x10000 SGD at batch 4, GPT-2-small MLP stack)")
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

    # whole iterations: each batch size's training steps timed back to back between one pair of events
    # on the launch stream (no per-kernel events, no drop/regrow): the per-batch time of record
    whole = {}
    L.snack_profile_enable(False)
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    for B in batches:
        b = bufs[B]
        torch.cuda.synchronize()
        ev0.record(stream)
        for _ in range(args.steps):
            L.snack_train_step_mse(layer.h, b["X"], b["T"], b["Y"], b["dY"], b["dX"], b["dW"], 2.0 / (B * M), lr,
                                   stream)
        ev1.record(stream)
        ev1.synchronize()
        whole[B] = ev0.elapsed_time(ev1) * 1e3 / args.steps

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
        # the kernel classes' event sum (each class bracketed by its own events) and the whole
        # iteration (forward, MSE gradient, backward, SGD) timed back to back: the latter is the
        # figure of record; it also holds the MSE gradient and the SGD step
        d["kernel_event_sum_us"] = round(tot_us, 3)
        tot_us = whole[B]
        d["fwd_bwd_us"] = round(tot_us, 3)
        if tot_us > 0:
            r = roofline_entry(fwd_bwd_bytes(nnz, M, K, B), fwd_bwd_flops(nnz, B), tot_us * 1e-6)
            d["fwd_bwd_GBps"] = r["GBps"]
            d["fwd_bwd_frac_of_hbm"] = r["frac_hbm"]
            d["fwd_bwd_TFLOPs"] = r["TFLOPs"]
            d["fwd_bwd_frac_of_valu"] = r["frac_valu"]
            d["binding_floor"] = r["binding"]
            d["floor_us"] = r["floor_us"]
            d["frac_of_binding_floor"] = round(r["floor_us"] / tot_us, 4)
        per_batch[str(B)] = d
    n_pr, ms_pr = L.snack_profile_read_tag(cls["prune_regrow"], -1)

    roofline = None
    if dominant is not None:
        name, B, n, ms = dominant
        per_launch = kernel_bytes(name, nnz, M, K, B)
        flops = kernel_flops(name, nnz, B)
        r = roofline_entry(per_launch, flops, ms * 1e-3 / n)
        if r["binding"] == "hbm":
            main = {"bound": "hbm", "achieved": r["GBps"], "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                    "frac": r["frac_hbm"]}
        else:
            main = {"bound": "alu", "achieved": r["TFLOPs"], "peak": VALU_PEAK_TFLOPS, "unit": "TFLOP/s",
                    "frac": r["frac_valu"]}
        roofline = dict(main, traffic=measured_traffic(f"{name} (B={B})"), kernel=f"{name} (B={B})",
                        avg_launch_us=round(ms * 1e3 / n, 3), bytes_per_launch=per_launch, flops_per_launch=flops,
                        hbm={"achieved": r["GBps"], "peak": HBM_PEAK_GBPS, "unit": "GB/s", "frac": r["frac_hbm"]},
                        alu={"achieved": r["TFLOPs"], "peak": VALU_PEAK_TFLOPS, "unit": "TFLOP/s",
                             "frac": r["frac_valu"]})

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
    del bufs
    if not args.no_configs:
        out["configs"] = config_legs()
    print(json.dumps(out), flush=True)


def _event_us(f, reps, warmup=10):
    """Mean microseconds per call of f over reps calls, timed with events on the
    current stream (where the library launches when given no stream)."""
    import torch
    for _ in range(warmup):
        f()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(reps):
        f()
    e1.record()
    e1.synchronize()
    return e0.elapsed_time(e1) * 1e3 / reps


def config_legs():
    """The other workloads of the measurement plan, each timed on its own (synthetic inputs of the
    workloads' shapes; supports uniform random without replacement, values N(0, 1/sqrt(fan-in)))."""
    import torch
    import coo_spmm_amd as L
    from snack_inputs import normal, random_layer, weight_std

    def make(M, K, sp, key, seed=1, max_batch=None):
        nnz = M * K * (100 - sp) // 100
        r, c, v = random_layer(M, K, nnz, key, weight_std(K, sp) if (M, K) != (500, 500) else 0.2)
        return L.SnackLayer(M, K, torch.from_numpy(r).cuda(), torch.from_numpy(c).cuda(),
                            torch.from_numpy(v).cuda(), seed=seed, max_batch=max_batch)

    res = {}
    print("[bench] 500x500 layer, 95 %, batch 1", file=sys.stderr, flush=True)
    lay = make(500, 500, 95, "c1/layer")
    X = torch.from_numpy(normal((1, 500), "c1/X")).cuda()
    dY = torch.from_numpy(normal((1, 500), "c1/dY")).cuda()
    Y = torch.empty(1, 500, device="cuda"); dX = torch.empty(1, 500, device="cuda")
    dW = torch.empty(lay.nnz, device="cuda")
    fw = _event_us(lambda: L.snack_forward(lay.h, X, Y), 1000)
    bw = _event_us(lambda: L.snack_backward(lay.h, X, dY, dX, dW), 1000)
    fb = _event_us(lambda: (L.snack_forward(lay.h, X, Y), L.snack_backward(lay.h, X, dY, dX, dW)), 1000)
    res["c1_500x500_s95_b1"] = {"reps": 1000, "fwd_us": round(fw, 2), "bwd_us": round(bw, 2),
                                "fwd_bwd_us": round(fb, 2), "nnz": lay.nnz,
                                "note": "launch-bound (0.36 MB of compulsory bytes)"}
    lay.close()

    print("[bench] 5000x5000 sparsity sweep against a masked-dense matmul", file=sys.stderr, flush=True)
    sweep = {}
    for sp in (50, 70, 90, 95, 99):
        lay = make(5000, 5000, sp, f"c2/layer/s{sp}")
        r, c, v = lay.export()
        Wd = torch.zeros(5000, 5000, device="cuda")
        Wd[r.long(), c.long()] = v          # W materialised with zeros: the Dense+Mask comparator
        for B in (1, 2):
            X = torch.from_numpy(normal((B, 5000), f"c2/X/{B}")).cuda()
            Y = torch.empty(B, 5000, device="cuda")
            Yd = torch.empty(B, 5000, device="cuda")
            fw = _event_us(lambda: L.snack_forward(lay.h, X, Y), 1000)
            dn = _event_us(lambda: torch.matmul(X, Wd.t(), out=Yd), 1000)
            sweep[f"s{sp}/b{B}"] = {"nnz": lay.nnz, "fwd_us": round(fw, 2), "masked_dense_fwd_us": round(dn, 2),
                                    "speedup_vs_masked_dense": round(dn / fw, 2),
                                    "fwd_GBps": round((12 * lay.nnz + 4 * B * 10000) / (fw * 1e-6) / 1e9, 1)}
        del Wd
        lay.close()
    res["c2_5000x5000_fwd_sweep"] = dict(sweep, reps=1000, comparator="torch.matmul with W materialised (zeros off "
                                                                       "the support), 100 MB fp32")

    print("[bench] 10000x10000 at batch 4, 100 SGD iterations", file=sys.stderr, flush=True)
    c3 = {}
    B = 4
    for sp in (90, 95, 99):
        torch.cuda.synchronize()
        torch.cuda.reset_peak_memory_stats()
        base_alloc = torch.cuda.memory_allocated()
        lay = make(10000, 10000, sp, f"c3/layer/s{sp}")
        Xs = [torch.from_numpy(normal((B, 10000), f"c3/X/s{sp}/{i}")).cuda() for i in range(10)]
        Ts = [torch.from_numpy(normal((B, 10000), f"c3/T/s{sp}/{i}")).cuda() for i in range(10)]
        Y = torch.empty(B, 10000, device="cuda"); dY = torch.empty(B, 10000, device="cuda")
        dX = torch.empty(B, 10000, device="cuda"); dW = torch.empty(lay.nnz, device="cuda")

        def run(n):
            for i in range(n):
                L.snack_train_step_mse(lay.h, Xs[i % 10], Ts[i % 10], Y, dY, dX, dW, 2.0 / (B * 10000), 0.01)

        run(10)
        reps = sorted(_event_us(lambda: run(100), 1, warmup=0) / 100 for _ in range(5))
        torch.cuda.synchronize()
        torch_peak = torch.cuda.max_memory_allocated() - base_alloc
        c3[f"s{sp}"] = {"nnz": lay.nnz, "us_per_iter_median_of_5": round(reps[2], 2),
                        "us_per_iter_min": round(reps[0], 2),
                        "peak_device_MB": round((lay.device_bytes() + torch_peak) / 1e6, 1),
                        "layer_device_MB": round(lay.device_bytes() / 1e6, 1),
                        "fwd_bwd_sgd_GBps": round((28 * lay.nnz + 4 * B * 50000 + 12 * lay.nnz)
                                                  / (reps[2] * 1e-6) / 1e9, 1)}
        del Xs, Ts
        lay.close()
    res["c3_10000x10000_b4_sgd"] = dict(c3, iterations=100, warmup=10, lr=0.01,
                                        step="snack_train_step_mse (forward, MSE gradient, dX, dW, SGD)",
                                        peak_memory="layer device bytes + torch peak for the caller's tensors")

    print("[bench] inference at batch 1: 5000x5000 layers, bf16 values, a chained stack", file=sys.stderr, flush=True)
    inf = {}
    for sp in (90, 95, 99):
        lay = make(5000, 5000, sp, f"c2/layer/s{sp}")
        X = torch.from_numpy(normal((1, 5000), "n3/X")).cuda()
        Y = torch.empty(1, 5000, device="cuda")
        fw = _event_us(lambda: L.snack_forward_infer(lay.h, X, Y), 2000)
        fb = _event_us(lambda: L.snack_forward_infer(lay.h, X, Y, bf16_values=True), 2000)
        inf[f"s{sp}"] = {"nnz": lay.nnz, "fp32_values_us": round(fw, 2), "bf16_values_us": round(fb, 2),
                         "bytes_per_entry": {"fp32": 6, "bf16": 4},
                         "bf16_GBps_of_12B_triple": round(12 * lay.nnz / (fb * 1e-6) / 1e9, 1)}
        lay.close()
    layers = [make(5000, 5000, 95, f"n3/chain/{i}") for i in range(4)]
    acts = [L.ACT_GELU, L.ACT_GELU, L.ACT_GELU, L.ACT_NONE]
    X = torch.from_numpy(normal((1, 5000), "n3/chain/X")).cuda()
    Ys = [torch.empty(1, 5000, device="cuda") for _ in layers]
    eager = _event_us(lambda: L.snack_forward_chain([l.h for l in layers], acts, X, Ys, bf16_values=True), 500)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        L.snack_forward_chain([l.h for l in layers], acts, X, Ys, bf16_values=True)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        L.snack_forward_chain([l.h for l in layers], acts, X, Ys, bf16_values=True)
    replay = _event_us(graph.replay, 500)
    del graph
    for l in layers:
        l.close()
    inf["chain_4x5000x5000_s95_gelu"] = {"eager_us": round(eager, 2), "graph_replay_us": round(replay, 2),
                                         "values": "bf16"}
    res["n3_inference_b1"] = dict(inf, reps=2000, note="snack_forward_infer: 16-bit column indices, fp32 or bf16 "
                                                       "values, GELU fused into the stores")

    print("[bench] gradient-driven drop/regrow at 10000x10000, 95 %", file=sys.stderr, flush=True)
    lay = make(10000, 10000, 95, "c4/s95", seed=2024)
    grad = {}
    for B in (4, 64):
        X = torch.from_numpy(normal((B, 10000), f"rigl/X/{B}")).cuda()
        dY = torch.from_numpy(normal((B, 10000), f"rigl/dY/{B}")).cuda()
        n = lay.nnz * 3 // 10
        us = _event_us(lambda: L.snack_prune_regrow_grad(lay.h, n, X, dY), 5, warmup=1)
        # five sweeps over the 10^8 cells, each one fused multiply-add per cell and batch row
        flops = 5 * 2.0 * B * 10000 * 10000
        grad[f"b{B}"] = {"us_per_call": round(us, 1), "score_TFLOPs": round(flops / (us * 1e-6) / 1e12, 2),
                         "frac_valu": round(flops / (us * 1e-6) / 1e12 / VALU_PEAK_TFLOPS, 4)}
    lay.close()
    res["n2_gradient_regrow_10000x10000_s95"] = dict(grad, n_drop="30 % of 5,000,000",
                                                     step="drop the smallest |w|, regrow at the empty cells of "
                                                          "largest |dY^T X| for a batch of B rows")

    print("[bench] row-local drop/regrow at 10000x10000, 95 %", file=sys.stderr, flush=True)
    lay = make(10000, 10000, 95, "c4/s95", seed=2024)
    rows_leg = {"random_us_per_call": round(_event_us(lambda: L.snack_prune_regrow_rows(
        lay.h, 3, 10, L.REGROW_RANDOM), 10, warmup=1), 1)}
    for B in (4, 64):
        X = torch.from_numpy(normal((B, 10000), f"rigl/X/{B}")).cuda()
        dY = torch.from_numpy(normal((B, 10000), f"rigl/dY/{B}")).cuda()
        rows_leg[f"gradient_b{B}_us_per_call"] = round(_event_us(lambda: L.snack_prune_regrow_rows(
            lay.h, 3, 10, L.REGROW_GRADIENT, X, dY), 5, warmup=1), 1)
    lay.close()
    res["n4_row_local_regrow_10000x10000_s95"] = dict(
        rows_leg, drop="floor(3 n_i / 10) of every row i", step="each row drops its smallest |w| and regrows as "
                                                                "many cells inside itself (random, or largest "
                                                                "|dY^T X| for a batch of B rows)")

    print("[bench] GPT-2-small MLP stack, 1024 tokens", file=sys.stderr, flush=True)
    c5 = {}
    tokens = 1024
    for sp in (90, 99):
        layers = []
        for b in range(12):
            for (M, K, name) in ((3072, 768, "fc"), (768, 3072, "proj")):
                layers.append(make(M, K, sp, f"c5/s{sp}/{b}/{name}", seed=500 + len(layers), max_batch=tokens))
        Xs = [torch.from_numpy(normal((tokens, 768), f"c5/s{sp}/X/{i}")).cuda() for i in range(4)]
        Ts = [torch.from_numpy(normal((tokens, 768), f"c5/s{sp}/T/{i}")).cuda() for i in range(4)]
        acts = [None] + [torch.empty(tokens, l.M, device="cuda") for l in layers]   # input of layer i+1
        pre = [torch.empty(tokens, 3072, device="cuda") for _ in range(12)]      # c_fc outputs
        grads = [torch.empty(tokens, l.K, device="cuda") for l in layers]        # dX of layer i
        dWs = [torch.empty(l.nnz, device="cuda") for l in layers]
        dYl = torch.empty(tokens, 768, device="cuda")
        gpre = torch.empty(tokens, 3072, device="cuda")

        def step(i):
            X, T = Xs[i % 4], Ts[i % 4]
            h = X
            for j, l in enumerate(layers[:-1]):
                if j % 2 == 0:
                    L.snack_forward(l.h, h, pre[j // 2])
                    L.snack_gelu_fwd(pre[j // 2], acts[j + 1])
                else:
                    L.snack_forward(l.h, h, acts[j + 1])
                h = acts[j + 1]
            last = layers[-1]
            # the last layer: forward, MSE gradient, backward and SGD in one call
            L.snack_train_step_mse(last.h, h, T, acts[-1], dYl, grads[-1], dWs[-1], 2.0 / (tokens * 768), 0.01)
            g = grads[-1]
            for j in range(len(layers) - 2, -1, -1):
                l = layers[j]
                x_in = X if j == 0 else acts[j]
                if j % 2 == 0:
                    L.snack_gelu_bwd(pre[j // 2], g, gpre)
                    L.snack_backward_sgd(l.h, x_in, gpre, None if j == 0 else grads[j], dWs[j], 0.01)
                else:
                    L.snack_backward_sgd(l.h, x_in, g, grads[j], dWs[j], 0.01)
                g = grads[j]

        steps = 20
        for i in range(3):
            step(i)
        us = _event_us(lambda: [step(i) for i in range(steps)], 1, warmup=0) / steps

        def prune_all():
            for l in layers:
                L.snack_prune_regrow(l.h, l.nnz * 3 // 10)
        pr = _event_us(prune_all, 1, warmup=0)
        nnz_all = sum(l.nnz for l in layers)
        c5[f"s{sp}"] = {"us_per_step": round(us, 1), "steps": steps,
                        "drop_regrow_all_24_layers_us": round(pr, 1),
                        "us_per_step_with_drop_regrow_every_50": round(us + pr / 50, 1),
                        "TFLOPs": round(6.0 * tokens * nnz_all / (us * 1e-6) / 1e12, 2),
                        "nnz_per_layer": [layers[0].nnz, layers[1].nnz]}
        for l in layers:
            l.close()
        del Xs, Ts, acts, pre, grads, dWs
    res["c5_gpt2_small_mlp_stack_1024_tokens"] = dict(
        c5, step="forward through 24 sparse layers with GELU after each c_fc, MSE gradient, backward with SGD "
                 "through all 24 (the first layer without dX)")
    return res


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


class OracleParts:
    """Work split of the oracle's calls over host threads with every output
    element summed in the same order as one call: the forward by ranges of
    output rows (contiguous runs of the row-sorted triple), dX by ranges of
    input columns (each thread gets the entries of its columns, in their
    order), dW and SGD by ranges of slots.  The oracle's C routines release
    the interpreter lock, so the threads run in parallel."""

    def __init__(self, M, K, r, c, nthreads):
        import numpy as np
        self.M, self.K, self.n = M, K, nthreads
        nnz = r.shape[0]
        rb = [M * t // nthreads for t in range(nthreads + 1)]
        kb = np.searchsorted(r, rb).tolist()
        self.fwd = [(rb[t], rb[t + 1], kb[t], kb[t + 1]) for t in range(nthreads)]
        cb = [K * t // nthreads for t in range(nthreads + 1)]
        self.dx = []
        for t in range(nthreads):
            sel = np.nonzero((c >= cb[t]) & (c < cb[t + 1]))[0]
            self.dx.append((cb[t], cb[t + 1], sel, np.ascontiguousarray(r[sel]), np.ascontiguousarray(c[sel])))
        self.slots = [(nnz * t // nthreads, nnz * (t + 1) // nthreads) for t in range(nthreads)]

    def forward(self, pool, r, c, v, X):
        import numpy as np
        import oracle
        Y = np.empty((X.shape[0], self.M), np.float64)

        def one(p):
            r0, r1, k0, k1 = p
            Yt, _ = oracle.forward(self.M, self.K, r[k0:k1], c[k0:k1], v[k0:k1], X)
            Y[:, r0:r1] = Yt[:, r0:r1]
        list(pool.map(one, self.fwd))
        return Y

    def backward_dx(self, pool, r, c, v, dY):
        import numpy as np
        import oracle
        dX = np.empty((dY.shape[0], self.K), np.float64)

        def one(p):
            c0, c1, sel, rs, cs = p
            d, _ = oracle.backward_dx(self.M, self.K, rs, cs, v[sel], dY)
            dX[:, c0:c1] = d[:, c0:c1]
        list(pool.map(one, self.dx))
        return dX

    def backward_dw(self, pool, r, c, X, dY):
        import numpy as np
        import oracle
        dW = np.empty(r.shape[0], np.float64)

        def one(p):
            k0, k1 = p
            dW[k0:k1], _ = oracle.backward_dw(self.M, self.K, r[k0:k1], c[k0:k1], X, dY)
        list(pool.map(one, self.slots))
        return dW

    def sgd(self, pool, v, g, lr):
        import numpy as np
        import oracle
        out = np.empty(v.shape[0], np.float64)

        def one(p):
            k0, k1 = p
            out[k0:k1] = oracle.sgd(v[k0:k1], g[k0:k1], lr)
        list(pool.map(one, self.slots))
        return out


def cpu_baseline(layer, M, K, nnz, batches, lr, min_seconds=10.0, max_steps=20):
    """The fp64 oracle as it stands, one host core, on a bounded sample of the
    workload: whole sweep steps (forward, MSE gradient, dX, dW and SGD for every
    batch size, no drop/regrow) repeated until about ten seconds have passed.
    `all_cores`: the same sample with the oracle's calls split over every usable
    host core (OracleParts; the results are the one-core results bit for bit)."""
    import numpy as np
    from concurrent.futures import ThreadPoolExecutor

    import oracle
    from snack_inputs import normal

    r, c, v = (t.cpu().numpy() for t in layer.export())
    v_start = v.copy()
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
    one_core = {"value": round(credited / dt / 1e9, 4), "unit": "GB/s", "cores": 1, "kind": "oracle",
                "sample": "%d sweep step(s) (fwd, MSE grad, dX, dW, SGD for B = %s) without drop/regrow; "
                          "single-threaded fp64 C oracle; %.1f s; host has %s usable cores"
                          % (steps, "/".join(map(str, batches)), dt, cores),
                "seconds": round(dt, 2)}

    # the same steps with the calls split over every usable core (at most 16, the machine's CPU share)
    nt = max(1, min(16, cores or 1))
    parts = OracleParts(M, K, r, c, nt)
    v = v_start.copy()
    credited_p, steps_p = 0, 0
    with ThreadPoolExecutor(nt) as pool:
        t0 = time.perf_counter()
        while steps_p < steps:
            for B, X, T in inputs:
                Y = parts.forward(pool, r, c, v, X)
                dY = oracle.mse_grad(Y.astype(np.float32), T).astype(np.float32)
                parts.backward_dx(pool, r, c, v, dY)
                dW = parts.backward_dw(pool, r, c, X, dY)
                v = parts.sgd(pool, v, dW.astype(np.float32), lr).astype(np.float32)
                credited_p += fwd_bwd_bytes(nnz, M, K, B) + 12 * B * M + 12 * nnz
            steps_p += 1
        dt_p = time.perf_counter() - t0
    one_core["all_cores"] = {"value": round(credited_p / dt_p / 1e9, 4), "unit": "GB/s", "cores": nt,
                             "kind": "oracle", "seconds": round(dt_p, 2),
                             "sample": "the same %d sweep step(s), the oracle's calls split over %d threads by output "
                                       "rows (forward), input columns (dX) and slots (dW, SGD); bit-identical to the "
                                       "one-core run" % (steps_p, nt)}
    return one_core


if __name__ == "__main__":
    main()

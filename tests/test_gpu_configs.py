"""The five workloads at their full sizes, HIP path against the oracle.

c1  500x500 at 95 %, batch 1: forward, dX and dW, every element; the index
    structures bit-exact.
c2  5000x5000 at 50/70/90/95/99 %, batches 1 and 2: forward, every element
    (at 50 % the rows hold ~2500 entries, the densest layer of the suite).
c3  10000x10000 at 90/95/99 %, batch 4: 100 SGD iterations (lr 0.01, MSE
    against fresh N(0,1) targets), teacher-forced checks at iterations 0, 1,
    50 and 99: the GPU's values and that iteration's inputs go to the oracle,
    which recomputes Y, dY, dX, dW and the SGD update.
c4  10000x10000 at 95 %, the batch sweep 1..64 one batch size per iteration,
    drop/regrow of 30 % after every 10th iteration: teacher-forced checks of
    iterations 1, 10, 11, 20 and bit-exact drop/regrow against the oracle.
c5  GPT-2-small MLP stack (12 x [768->3072, GELU, 3072->768]) at 90 and 99 %,
    1024 tokens: every layer checked in step 1 (forward, GELU, backward,
    SGD), 50 steps, drop/regrow of every layer, every layer checked again in
    the step after it.

Tolerance: |gpu - oracle| <= 1e-5 * sum|terms| + 1e-6 per element; integer
results bit-exact.  Inputs come from the seeded generators of the workloads.
"""
import numpy as np
import pytest

import oracle
from snack_inputs import normal, random_layer, weight_std, nnz_for
from tests.gpu_util import say, lib, dev, host, assert_close

pytestmark = pytest.mark.gpu


def _sgd_close(got, v, g, lr, ulps=2):
    ref = oracle.sgd(v, g, lr)
    got = np.asarray(got, np.float32).astype(np.float64)
    big = np.maximum(np.abs(v.astype(np.float64)), np.abs(lr * g.astype(np.float64)))
    spacing = np.spacing(big.astype(np.float32)).astype(np.float64)
    return np.abs(got - ref) <= ulps * spacing + 1e-30


def _layer(M, K, sp, key, seed=1, max_batch=None):
    L = lib()
    rows, cols, vals = random_layer(M, K, nnz_for(M, K, sp), key, weight_std(K, sp))
    return (L.SnackLayer(M, K, dev(rows), dev(cols), dev(vals), seed=seed, max_batch=max_batch),
            (rows, cols, vals))


def _export(layer):
    return tuple(host(t) for t in layer.export())


def test_c1_500_square_95_batch1():
    M = K = 500
    layer, (rows, cols, vals) = _layer(M, K, 95, "c1/layer")
    try:
        ref = oracle.canonicalize(M, K, rows, cols, vals)
        r, c, v = _export(layer)
        assert np.array_equal(r, ref["rows"]) and np.array_equal(c, ref["cols"])
        assert np.array_equal(v.view(np.uint32), ref["vals"].view(np.uint32))
        rp, pm, rt, cp = (host(t) for t in layer.export_index())
        assert np.array_equal(rp, ref["row_ptr"]) and np.array_equal(cp, ref["col_ptr"])
        assert np.array_equal(pm, ref["perm"]) and np.array_equal(rt, ref["rows_t"])
        X = normal((1, K), "c1/X"); dY = normal((1, M), "c1/dY")
        say("c1 forward/backward")
        Y = layer.forward(dev(X)); dX, dW = layer.backward(dev(X), dev(dY))
        Yr, Ya = oracle.forward(M, K, r, c, v, X)
        assert_close("c1 Y", host(Y), Yr, Ya)
        dXr, dXa = oracle.backward_dx(M, K, r, c, v, dY)
        assert_close("c1 dX", host(dX), dXr, dXa)
        dWr, dWa = oracle.backward_dw(M, K, r, c, X, dY)
        assert_close("c1 dW", host(dW), dWr, dWa)
    finally:
        layer.close()


@pytest.mark.parametrize("sp", [50, 70, 90, 95, 99])
def test_c2_5000_square_sparsity_sweep_forward(sp):
    M = K = 5000
    layer, _ = _layer(M, K, sp, f"c2/layer/s{sp}")
    try:
        r, c, v = _export(layer)
        assert r.shape[0] == nnz_for(M, K, sp)
        for B in (1, 2):
            X = normal((B, K), f"c2/X/s{sp}/b{B}")
            say("c2 forward sparsity", sp, "B", B)
            Y = layer.forward(dev(X))
            Yr, Ya = oracle.forward(M, K, r, c, v, X)
            assert_close(f"c2 s={sp} B={B} Y", host(Y), Yr, Ya)
    finally:
        layer.close()


def _check_iteration(tag, layer, M, K, r, c, v, X, T, Y, dY, dX, dW, lr):
    """Teacher-forced check of one training iteration that has just run on the GPU."""
    Yg, dYg, dXg, dWg = host(Y), host(dY), host(dX), host(dW)
    Yr, Ya = oracle.forward(M, K, r, c, v, X)
    assert_close(f"{tag} Y", Yg, Yr, Ya)
    dYr = oracle.mse_grad(Yg, T)
    assert_close(f"{tag} dY", dYg, dYr, np.abs(dYr), rel=2e-7, atol=1e-12)
    dXr, dXa = oracle.backward_dx(M, K, r, c, v, dYg)
    assert_close(f"{tag} dX", dXg, dXr, dXa)
    dWr, dWa = oracle.backward_dw(M, K, r, c, X, dYg)
    assert_close(f"{tag} dW", dWg, dWr, dWa)
    v_new = host(layer.export()[2])
    assert _sgd_close(v_new, v, dWg, lr).all(), f"{tag} SGD update"
    return v_new


@pytest.mark.parametrize("sp", [90, 95, 99])
def test_c3_10000_square_batch4_100_sgd_iterations(sp):
    import torch
    L = lib()
    M = K = 10000
    B, lr, iters = 4, 0.01, 100
    checks = {0, 1, 50, iters - 1}
    layer, _ = _layer(M, K, sp, f"c3/layer/s{sp}")
    Y = torch.empty(B, M, device="cuda"); dY = torch.empty(B, M, device="cuda")
    dX = torch.empty(B, K, device="cuda"); dW = torch.empty(layer.nnz, device="cuda")
    try:
        for it in range(iters):
            X = normal((B, K), f"c3/X/s{sp}/{it}"); T = normal((B, M), f"c3/T/s{sp}/{it}")
            if it in checks:
                r, c, v = _export(layer)
                say("c3 sparsity", sp, "checked iteration", it)
            Xd, Td = dev(X), dev(T)
            L.snack_forward(layer.h, Xd, Y)
            L.snack_mse_grad(Y, Td, dY, 2.0 / (B * M))
            L.snack_backward(layer.h, Xd, dY, dX, dW)
            L.snack_sgd_step(layer.h, dW, lr)
            if it in checks:
                _check_iteration(f"c3 s={sp} it={it}", layer, M, K, r, c, v, X, T, Y, dY, dX, dW, lr)
    finally:
        layer.close()


def test_c4_10000_square_batch_sweep_with_drop_regrow():
    import torch
    L = lib()
    M = K = 10000
    batches = (1, 2, 4, 8, 16, 32, 64)
    lr, period, iters, seed = 0.01, 10, 20, 4242
    # every iteration of the first sweep (t = 1..7: batches 1, 2, 4, 8, 16, 32, 64), the last
    # before the first drop/regrow (t = 10, batch 4), the first after it (t = 11, batch 8),
    # batch 64 after it (t = 14) and the last before the second (t = 20, batch 32)
    checks = {1, 2, 3, 4, 5, 6, 7, 10, 11, 14, 20}
    layer, _ = _layer(M, K, 95, "c4/layer", seed=seed)
    nnz = layer.nnz
    n_drop = nnz * 3 // 10
    dW = torch.empty(nnz, device="cuda")
    try:
        for t in range(1, iters + 1):
            B = batches[(t - 1) % len(batches)]
            X = normal((B, K), f"c4/X/{t}"); T = normal((B, M), f"c4/T/{t}")
            Y = torch.empty(B, M, device="cuda"); dY = torch.empty(B, M, device="cuda")
            dX = torch.empty(B, K, device="cuda")
            if t in checks:
                r, c, v = _export(layer)
                say("c4 checked iteration", t, "B", B)
            Xd, Td = dev(X), dev(T)
            L.snack_forward(layer.h, Xd, Y)
            L.snack_mse_grad(Y, Td, dY, 2.0 / (B * M))
            L.snack_backward(layer.h, Xd, dY, dX, dW)
            L.snack_sgd_step(layer.h, dW, lr)
            if t in checks:
                _check_iteration(f"c4 t={t} B={B}", layer, M, K, r, c, v, X, T, Y, dY, dX, dW, lr)
            if t % period == 0:
                r0, c0, v0 = _export(layer)
                epoch = layer.epoch
                say("c4 drop/regrow after iteration", t, "epoch", epoch)
                layer.prune_regrow(n_drop)
                o = oracle.prune_regrow(M, K, r0, c0, v0, n_drop, seed, epoch)
                r1, c1, v1 = _export(layer)
                assert r1.shape[0] == nnz
                assert np.array_equal(r1, o[0]) and np.array_equal(c1, o[1])
                assert np.array_equal(v1.view(np.uint32), o[2].view(np.uint32))
                ref = oracle.canonicalize(M, K, r1, c1, v1)
                rp, pm, rt, cp = (host(x) for x in layer.export_index())
                assert np.array_equal(rp, ref["row_ptr"]) and np.array_equal(cp, ref["col_ptr"])
                assert np.array_equal(pm, ref["perm"]) and np.array_equal(rt, ref["rows_t"])
    finally:
        layer.close()


class _Stack:
    """The GPT-2-small MLP stack: 12 blocks of sparse c_fc (768 -> 3072), GELU,
    sparse c_proj (3072 -> 768), chained with no residual or normalisation."""

    def __init__(self, sp, blocks=12, seed0=500):
        self.layers = []
        for b in range(blocks):
            for (M, K, name) in ((3072, 768, "fc"), (768, 3072, "proj")):
                layer, _ = _layer(M, K, sp, f"c5/s{sp}/{b}/{name}", seed=seed0 + len(self.layers),
                                  max_batch=1024)
                self.layers.append(layer)

    def close(self):
        for layer in self.layers:
            layer.close()


def _c5_step(stack, L, X, T, lr, record):
    """One forward + backward + SGD step through the stack; returns the recorded
    per-layer tensors (inputs, outputs, gradients) when record is set."""
    import torch
    acts = [X]        # input of layer i
    pre = []          # c_fc outputs (GELU inputs)
    rec = []
    h = X
    for i, layer in enumerate(stack.layers):
        y = torch.empty(h.shape[0], layer.M, device="cuda")
        L.snack_forward(layer.h, h, y)
        if i % 2 == 0:
            pre.append(y)
            g = torch.empty_like(y)
            L.snack_gelu_fwd(y, g)
            h = g
        else:
            h = y
        acts.append(h)
    out = h
    dY = torch.empty_like(out)
    L.snack_mse_grad(out, T, dY, 2.0 / out.numel())
    g = dY
    grads = [None] * len(stack.layers)
    for i in range(len(stack.layers) - 1, -1, -1):
        layer = stack.layers[i]
        if i % 2 == 0:
            dpre = torch.empty_like(pre[i // 2])
            L.snack_gelu_bwd(pre[i // 2], g, dpre)
            g_in = dpre
        else:
            g_in = g
        dX = torch.empty(acts[i].shape[0], layer.K, device="cuda")
        dW = torch.empty(layer.nnz, device="cuda")
        vals_before = host(layer.export()[2]) if record else None
        L.snack_backward(layer.h, acts[i], g_in, dX, dW)
        L.snack_sgd_step(layer.h, dW, lr)
        if record:
            grads[i] = dict(x=host(acts[i]), y=host(pre[i // 2]) if i % 2 == 0 else host(acts[i + 1]),
                            dy=host(g_in), dx=host(dX), dw=host(dW), v=vals_before)
            if i % 2 == 0:
                grads[i]["gelu_out"] = host(acts[i + 1])
                grads[i]["gelu_dout"] = host(g)
        g = dX
    return grads if record else None


def _check_c5_step(stack, grads, lr, tag):
    # supports and updated values come off the GPU first; the oracle then runs on
    # host threads (its C routines release the interpreter lock)
    from concurrent.futures import ThreadPoolExecutor
    import os
    meta = []
    for i, layer in enumerate(stack.layers):
        r, c, v_after = _export(layer)
        meta.append((layer.M, layer.K, r, c, v_after))

    def ref(i):
        M, K, r, c, _ = meta[i]
        d = grads[i]
        out = dict(Y=oracle.forward(M, K, r, c, d["v"], d["x"]),
                   dX=oracle.backward_dx(M, K, r, c, d["v"], d["dy"]),
                   dW=oracle.backward_dw(M, K, r, c, d["x"], d["dy"]))
        if i % 2 == 0:
            out["gelu"] = oracle.gelu_fwd(d["y"])
            out["gelu_b"] = oracle.gelu_bwd(d["y"], d["gelu_dout"])
        return out

    say(tag, "oracle on", len(meta), "layers")
    with ThreadPoolExecutor(max_workers=min(16, os.cpu_count() or 1)) as ex:
        refs = list(ex.map(ref, range(len(meta))))
    for i, o in enumerate(refs):
        d = grads[i]
        assert_close(f"{tag} layer {i} Y", d["y"], *o["Y"])
        if i % 2 == 0:
            assert_close(f"{tag} layer {i} GELU", d["gelu_out"], o["gelu"], np.abs(o["gelu"]), rel=1e-6, atol=1e-7)
            assert_close(f"{tag} layer {i} GELU'", d["dy"], o["gelu_b"], np.abs(o["gelu_b"]), rel=1e-6, atol=1e-12)
        assert_close(f"{tag} layer {i} dX", d["dx"], *o["dX"])
        assert_close(f"{tag} layer {i} dW", d["dw"], *o["dW"])
        assert _sgd_close(meta[i][4], d["v"], d["dw"], lr).all(), f"{tag} layer {i} SGD"


@pytest.mark.parametrize("sp", [90, 99])
def test_c5_gpt2_mlp_stack(sp):
    L = lib()
    tokens, lr, period = 1024, 0.01, 50
    stack = _Stack(sp)
    try:
        X = dev(normal((tokens, 768), f"c5/s{sp}/X/0")); T = dev(normal((tokens, 768), f"c5/s{sp}/T/0"))
        say("c5 sparsity", sp, "step 1")
        grads = _c5_step(stack, L, X, T, lr, record=True)
        _check_c5_step(stack, grads, lr, f"c5 s={sp} step 1")
        for step in range(2, period + 1):
            X = dev(normal((tokens, 768), f"c5/s{sp}/X/{step}")); T = dev(normal((tokens, 768), f"c5/s{sp}/T/{step}"))
            _c5_step(stack, L, X, T, lr, record=False)
        for i, layer in enumerate(stack.layers):
            r0, c0, v0 = _export(layer)
            epoch = layer.epoch
            say("c5 sparsity", sp, "drop/regrow layer", i)
            layer.prune_regrow(layer.nnz * 3 // 10)
            o = oracle.prune_regrow(layer.M, layer.K, r0, c0, v0, layer.nnz * 3 // 10, 500 + i, epoch)
            r1, c1, v1 = _export(layer)
            assert np.array_equal(r1, o[0]) and np.array_equal(c1, o[1])
            assert np.array_equal(v1.view(np.uint32), o[2].view(np.uint32))
        X = dev(normal((tokens, 768), f"c5/s{sp}/X/{period + 1}"))
        T = dev(normal((tokens, 768), f"c5/s{sp}/T/{period + 1}"))
        say("c5 sparsity", sp, "step after drop/regrow")
        grads = _c5_step(stack, L, X, T, lr, record=True)
        _check_c5_step(stack, grads, lr, f"c5 s={sp} step {period + 1}")
    finally:
        stack.close()

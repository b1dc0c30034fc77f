"""Training loop on the GPU (forward, MSE gradient, backward, SGD, drop/regrow),
checked step by step against the oracle with teacher forcing: every check feeds
the oracle the GPU's own values and inputs of that iteration, so fp32 and fp64
trajectories are never compared after they drift apart.

Also checks the layer's two value copies stay bit-identical (vals_t ==
vals[perm]) after SGD updates both of them from dW produced in each order."""
import numpy as np
import pytest

import oracle
from snack_inputs import normal, random_layer, weight_std
from tests.gpu_util import say, lib, dev, host, assert_close

pytestmark = pytest.mark.gpu


def _sgd_close(got, v, g, lr, ulps=2):
    """fp32 evaluation of v - lr*g (with lr rounded to fp32) is within a couple
    of ulps of the larger operand of the exact fp64 update."""
    ref = oracle.sgd(v, g, lr)
    got = np.asarray(got, np.float32).astype(np.float64)
    big = np.maximum(np.abs(v.astype(np.float64)), np.abs(lr * g.astype(np.float64)))
    spacing = np.spacing(big.astype(np.float32)).astype(np.float64)
    return np.abs(got - ref) <= ulps * spacing + 1e-30


@pytest.mark.parametrize("B", [1, 3, 8, 16, 40, 64, 100])
def test_training_steps_teacher_forced(B):
    import torch
    L = lib()
    M, K, sp = 700, 900, 90
    nnz = M * K * (100 - sp) // 100
    rows, cols, vals = random_layer(M, K, nnz, f"train/{B}", weight_std(K, sp))
    say("training create B", B)
    layer = L.SnackLayer(M, K, dev(rows), dev(cols), dev(vals), seed=77, max_batch=B)
    lr = 0.01
    Y = torch.empty(B, M, device="cuda"); dY = torch.empty(B, M, device="cuda")
    dX = torch.empty(B, K, device="cuda"); dW = torch.empty(nnz, device="cuda")
    try:
        for it in range(6):
            X = normal((B, K), f"train/{B}/X/{it}"); T = normal((B, M), f"train/{B}/T/{it}")
            r, c, v = (host(t) for t in layer.export())
            Xd, Td = dev(X), dev(T)
            say("training iteration", it, "B", B)
            L.snack_forward(layer.h, Xd, Y)
            L.snack_mse_grad(Y, Td, dY, 2.0 / (B * M))
            L.snack_backward(layer.h, Xd, dY, dX, dW)
            L.snack_sgd_step(layer.h, dW, lr)
            Yg, dYg, dXg, dWg = host(Y), host(dY), host(dX), host(dW)
            Yr, Ya = oracle.forward(M, K, r, c, v, X)
            assert_close(f"Y it={it}", Yg, Yr, Ya)
            dYr = oracle.mse_grad(Yg, T)
            assert_close(f"dY it={it}", dYg, dYr, np.abs(dYr), rel=2e-7, atol=1e-12)
            dXr, dXa = oracle.backward_dx(M, K, r, c, v, dYg)
            assert_close(f"dX it={it}", dXg, dXr, dXa)
            dWr, dWa = oracle.backward_dw(M, K, r, c, X, dYg)
            assert_close(f"dW it={it}", dWg, dWr, dWa)
            v_new = host(layer.export()[2])
            assert _sgd_close(v_new, v, dWg, lr).all()
            rp, pm, rt, cp, vt = (host(t) for t in layer.export_index(with_values=True))
            assert np.array_equal(vt.view(np.uint32), v_new[pm].view(np.uint32)), "value copies diverged"
            if it == 2:
                say("training prune B", B)
                layer.prune_regrow(nnz * 3 // 10)
                o = oracle.prune_regrow(M, K, r, c, v_new, nnz * 3 // 10, 77, 0)
                r2, c2, v2 = (host(t) for t in layer.export())
                assert np.array_equal(r2, o[0]) and np.array_equal(c2, o[1])
                assert np.array_equal(v2.view(np.uint32), o[2].view(np.uint32))
    finally:
        layer.close()


@pytest.mark.parametrize("M,K,nnz", [(1500, 1100, 80000), (1000, 800, 200000), (12000, 300, 1800000)])
def test_dw_row_and_column_orders_bit_identical(M, K, nnz):
    """dW from the backward (canonical order) equals the transposed-order copy
    the layer keeps, bit for bit, for every batch plan -- on short keys (the
    segmented kernels), on long keys (the key-major kernels), and where one
    view's gathered operand fits in LDS and the other's does not."""
    import torch
    L = lib()
    rows, cols, vals = random_layer(M, K, nnz, f"dwt/{M}x{K}")
    layer = L.SnackLayer(M, K, dev(rows), dev(cols), dev(vals))
    try:
        for B in (1, 2, 4, 8, 16, 32, 64):
            X = dev(normal((B, K), f"dwt/{M}x{K}/X/{B}")); dY = dev(normal((B, M), f"dwt/{M}x{K}/dY/{B}"))
            say("dwt orders B", B)
            v0 = host(layer.export()[2])
            dX, dW = layer.backward(X, dY)
            layer.sgd_step(dW, 1.0)         # updates both copies from dW and its transposed twin
            v1 = host(layer.export()[2])
            rp, pm, rt, cp, vt = (host(t) for t in layer.export_index(with_values=True))
            assert np.array_equal(vt.view(np.uint32), v1[pm].view(np.uint32))
            # and the canonical update is exactly v - dW in fp32
            assert np.array_equal(v1, (v0 - host(dW)).astype(np.float32))
    finally:
        layer.close()


@pytest.mark.parametrize("M,K,nnz", [(2000, 1500, 300000), (768, 3072, 23593), (10000, 10000, 5_000_000)])
def test_backward_sgd_matches_backward_then_sgd(M, K, nnz):
    """The fused backward + SGD step equals snack_backward followed by
    snack_sgd_step bit for bit (dX, dW and both value copies), for every batch
    plan; twice per plan, so the second call starts from stepped values.  The
    768 x 3072 layer's short keys take the fallback (no in-place step)."""
    L = lib()
    rows, cols, vals = random_layer(M, K, nnz, f"fused/{M}x{K}")
    a = L.SnackLayer(M, K, dev(rows), dev(cols), dev(vals), max_batch=100)
    b = L.SnackLayer(M, K, dev(rows), dev(cols), dev(vals), max_batch=100)
    lr = 0.01
    try:
        for B in (1, 2, 3, 4, 8, 16, 32, 64, 100):
            X = dev(normal((B, K), f"fused/{M}x{K}/X/{B}"))
            dY = dev(normal((B, M), f"fused/{M}x{K}/dY/{B}"))
            for it in range(2):
                say("fused backward+sgd", M, K, "B", B, "it", it)
                dXa, dWa = a.backward(X, dY)
                a.sgd_step(dWa, lr)
                dXb, dWb = b.backward_sgd(X, dY, lr)
                assert np.array_equal(host(dXa).view(np.uint32), host(dXb).view(np.uint32)), f"dX B={B}"
                assert np.array_equal(host(dWa).view(np.uint32), host(dWb).view(np.uint32)), f"dW B={B}"
                va, vb = host(a.export()[2]), host(b.export()[2])
                assert np.array_equal(va.view(np.uint32), vb.view(np.uint32)), f"values B={B}"
                _, pm, _, _, vta = (host(t) for t in a.export_index(with_values=True))
                _, _, _, _, vtb = (host(t) for t in b.export_index(with_values=True))
                assert np.array_equal(vta.view(np.uint32), vtb.view(np.uint32)), f"column-order values B={B}"
                assert np.array_equal(vtb.view(np.uint32), vb[pm].view(np.uint32)), f"copies diverged B={B}"
        # without dX the column pass does not run: the step falls back to the separate update
        X = dev(normal((8, K), f"fused/{M}x{K}/X/nodx")); dY = dev(normal((8, M), f"fused/{M}x{K}/dY/nodx"))
        _, dWa = a.backward(X, dY, want_dx=False)
        a.sgd_step(dWa, lr)
        _, dWb = b.backward_sgd(X, dY, lr, want_dx=False)
        assert np.array_equal(host(dWa).view(np.uint32), host(dWb).view(np.uint32))
        assert np.array_equal(host(a.export()[2]).view(np.uint32), host(b.export()[2]).view(np.uint32))
    finally:
        a.close()
        b.close()


@pytest.mark.parametrize("M,K,nnz", [(10000, 10000, 5_000_000), (2000, 1500, 300000), (768, 3072, 23593)])
def test_train_step_matches_separate_calls(M, K, nnz):
    """The one-call training step (forward, MSE gradient, backward, SGD) equals
    snack_forward + snack_mse_grad + snack_backward_sgd bit for bit (Y, dY, dX,
    dW and both value copies) for every batch plan, twice per plan.  The layers
    reach the forward that writes dY beside Y (slice reduction or key stores)
    and the paths where the gradient is a separate pass."""
    import torch
    L = lib()
    rows, cols, vals = random_layer(M, K, nnz, f"tstep/{M}x{K}")
    a = L.SnackLayer(M, K, dev(rows), dev(cols), dev(vals), max_batch=449)
    b = L.SnackLayer(M, K, dev(rows), dev(cols), dev(vals), max_batch=449)
    lr = 0.01
    u32 = lambda t: host(t).view(np.uint32)
    try:
        for B in (1, 2, 3, 4, 8, 16, 32, 64, 100, 449):
            X = dev(normal((B, K), f"tstep/{M}x{K}/X/{B}"))
            T = dev(normal((B, M), f"tstep/{M}x{K}/T/{B}"))
            scale = 2.0 / (B * M)
            for it in range(2):
                say("train step", M, K, "B", B, "it", it)
                Ya = torch.empty(B, M, device="cuda"); dYa = torch.empty(B, M, device="cuda")
                L.snack_forward(a.h, X, Ya)
                L.snack_mse_grad(Ya, T, dYa, scale)
                dXa, dWa = a.backward_sgd(X, dYa, lr)
                Yb, dYb, dXb, dWb = b.train_step_mse(X, T, lr, scale=scale)
                for name, x, y in (("Y", Ya, Yb), ("dY", dYa, dYb), ("dX", dXa, dXb), ("dW", dWa, dWb)):
                    assert np.array_equal(u32(x), u32(y)), f"{name} B={B} it={it}"
                assert np.array_equal(u32(a.export()[2]), u32(b.export()[2])), f"values B={B}"
                _, pm, _, _, vtb = (host(t) for t in b.export_index(with_values=True))
                assert np.array_equal(vtb.view(np.uint32), host(b.export()[2])[pm].view(np.uint32)), f"copies B={B}"
        # without dX
        X = dev(normal((8, K), f"tstep/{M}x{K}/X/nodx")); T = dev(normal((8, M), f"tstep/{M}x{K}/T/nodx"))
        Ya = torch.empty(8, M, device="cuda"); dYa = torch.empty(8, M, device="cuda")
        L.snack_forward(a.h, X, Ya)
        L.snack_mse_grad(Ya, T, dYa, 2.0 / (8 * M))
        _, dWa = a.backward_sgd(X, dYa, lr, want_dx=False)
        _, _, _, dWb = b.train_step_mse(X, T, lr, want_dx=False)
        assert np.array_equal(u32(dWa), u32(dWb))
        assert np.array_equal(u32(a.export()[2]), u32(b.export()[2]))
    finally:
        a.close()
        b.close()


@pytest.mark.parametrize("M,K,nnz", [(1, 1, 1), (1, 300, 17), (300, 1, 29), (7, 9, 0), (64, 4096, 20000)])
def test_train_step_small_and_degenerate_shapes(M, K, nnz):
    """The one-call training step on one-row, one-column, empty and short-key
    layers over ragged batch plans: bit for bit the separate calls."""
    import torch
    L = lib()
    rows, cols, vals = random_layer(M, K, nnz, f"tstep-small/{M}x{K}")
    a = L.SnackLayer(M, K, dev(rows), dev(cols), dev(vals), max_batch=65)
    b = L.SnackLayer(M, K, dev(rows), dev(cols), dev(vals), max_batch=65)
    u32 = lambda t: host(t).view(np.uint32)
    try:
        for B in (1, 2, 3, 5, 8, 13, 33, 64, 65):
            X = dev(normal((B, K), f"tstep-small/{M}x{K}/X/{B}"))
            T = dev(normal((B, M), f"tstep-small/{M}x{K}/T/{B}"))
            say("train step small", M, K, nnz, "B", B)
            Ya = torch.empty(B, M, device="cuda"); dYa = torch.empty(B, M, device="cuda")
            L.snack_forward(a.h, X, Ya)
            L.snack_mse_grad(Ya, T, dYa, 2.0 / (B * M))
            dXa, dWa = a.backward_sgd(X, dYa, 0.01)
            Yb, dYb, dXb, dWb = b.train_step_mse(X, T, 0.01)
            for name, x, y in (("Y", Ya, Yb), ("dY", dYa, dYb), ("dX", dXa, dXb)):
                assert np.array_equal(u32(x), u32(y)), f"{name} B={B}"
            if nnz:
                assert np.array_equal(u32(dWa), u32(dWb)), f"dW B={B}"
                assert np.array_equal(u32(a.export()[2]), u32(b.export()[2])), f"values B={B}"
    finally:
        a.close()
        b.close()


@pytest.mark.parametrize("B", [1, 16, 64])
def test_sgd_step_with_gradient_changed_in_place(B):
    """A caller may change dW between snack_backward and snack_sgd_step
    (clipping, scaling): the step uses the dW it is given, and the layer's
    column-ordered value copy follows the canonical values exactly, so the next
    backward's dX is the oracle's for the stepped values."""
    import torch
    L = lib()
    M, K, nnz = 900, 700, 63000
    rows, cols, vals = random_layer(M, K, nnz, f"inplace/{B}")
    layer = L.SnackLayer(M, K, dev(rows), dev(cols), dev(vals))
    lr = 0.01
    try:
        X = normal((B, K), f"inplace/X/{B}")
        dY = normal((B, M), f"inplace/dY/{B}")
        say("in-place dW B", B)
        v0 = host(layer.export()[2])
        dX, dW = layer.backward(dev(X), dev(dY))
        dW.mul_(-3.0)   # the caller rescales the gradient in place
        g = host(dW)
        layer.sgd_step(dW, lr)
        r, c, v1 = (host(t) for t in layer.export())
        want = (v0.astype(np.float64) - np.float64(np.float32(lr)) * g.astype(np.float64))
        assert _sgd_close(v1, v0, g, lr).all()
        assert np.abs(v1 - want).max() <= 1e-6 * (1 + np.abs(want).max())
        _, pm, _, _, vt = (host(t) for t in layer.export_index(with_values=True))
        assert np.array_equal(vt.view(np.uint32), v1[pm].view(np.uint32))
        # the next backward reads the column-ordered copy
        dY2 = normal((B, M), f"inplace/dY2/{B}")
        dX2, _ = layer.backward(dev(X), dev(dY2), want_dw=False)
        assert_close(f"dX after in-place step B={B}", host(dX2), *oracle.backward_dx(M, K, r, c, v1, dY2))
    finally:
        layer.close()

"""HIP path vs the fp64 oracle, element by element, through the C ABI.

Floating outputs: |gpu - oracle| <= 1e-5 * sum|terms| + 1e-6 per element.
Integer work (canonical order, row pointer, transposed index): bit-exact.
"""
import numpy as np
import pytest

import oracle
from snack_inputs import random_layer, normal, weight_std
from tests.gpu_util import say, lib, dev, host, assert_close

pytestmark = pytest.mark.gpu


def _make(M, K, nnz, key, std=None):
    rows, cols, vals = random_layer(M, K, nnz, key, std)
    return rows, cols, vals


def _check_layer_vs_oracle(M, K, nnz, batches, key, std=None, check_index=True, triple=None):
    import torch
    L = lib()
    rows, cols, vals = triple if triple is not None else _make(M, K, nnz, key, std)
    ref = oracle.canonicalize(M, K, rows, cols, vals)
    say("create", key, M, K, nnz)
    layer = L.SnackLayer(M, K, dev(rows), dev(cols), dev(vals), seed=1, max_batch=max(batches))
    try:
        if check_index:
            r, c, v = layer.export()
            assert np.array_equal(host(r), ref["rows"])
            assert np.array_equal(host(c), ref["cols"])
            assert np.array_equal(host(v).view(np.uint32), ref["vals"].view(np.uint32))
            rp, pm, rt, cp = layer.export_index()
            assert np.array_equal(host(rp), ref["row_ptr"])
            assert np.array_equal(host(cp), ref["col_ptr"])
            if nnz:
                assert np.array_equal(host(pm), ref["perm"])
                assert np.array_equal(host(rt), ref["rows_t"])
        for B in batches:
            X = normal((B, K), f"{key}/X/{B}")
            dY = normal((B, M), f"{key}/dY/{B}")
            say("forward/backward", key, "B", B)
            Xd, dYd = dev(X), dev(dY)
            Y = layer.forward(Xd)
            dX, dW = layer.backward(Xd, dYd)
            Yr, Ya = oracle.forward(M, K, ref["rows"], ref["cols"], ref["vals"], X)
            assert_close(f"Y B={B}", host(Y), Yr, Ya)
            dXr, dXa = oracle.backward_dx(M, K, ref["rows"], ref["cols"], ref["vals"], dY)
            assert_close(f"dX B={B}", host(dX), dXr, dXa)
            dWr, dWa = oracle.backward_dw(M, K, ref["rows"], ref["cols"], X, dY)
            assert_close(f"dW B={B}", host(dW), dWr, dWa)
    finally:
        layer.close()


@pytest.mark.parametrize("M,K,nnz", [(1, 1, 1), (1, 300, 17), (300, 1, 29), (7, 9, 0), (37, 53, 400),
                                     (130, 70, 2000), (64, 4096, 20000)])
def test_small_shapes_all_batch_plans(M, K, nnz):
    _check_layer_vs_oracle(M, K, nnz, (1, 2, 3, 4, 5, 8, 13, 16, 17, 32, 33, 64, 65, 130), f"gpu/small/{M}x{K}")


@pytest.mark.parametrize("M,K,nnz", [(4096, 64, 20000), (1000, 800, 200000)])
def test_long_keys_wide_batches(M, K, nnz):
    # hundreds of entries per row and per column: the key-major kernels and the
    # column-order dW permuted into canonical order
    _check_layer_vs_oracle(M, K, nnz, (1, 2, 3, 4, 5, 8, 9, 16, 24, 32, 40, 64, 65), f"gpu/longkeys/{M}x{K}")


def test_wide_batches_over_skewed_short_keys():
    # more than one 64-column batch tile over views whose keys average few entries (the wide-batch
    # short-key passes), with a skewed degree: three rows and three columns far longer than the rest,
    # most rows and columns empty, and batches that end inside a 64-column block
    from snack_inputs import rng_for
    M, K = 700, 500
    g = rng_for("gpu/wide/skew")
    pos = set()
    for r in (3, 350, 699):                      # long rows
        pos.update(r * K + int(c) for c in g.choice(K, 300, replace=False))
    for c in (0, 250, 499):                      # long columns
        pos.update(int(r) * K + c for r in g.choice(M, 400, replace=False))
    for p in g.choice(M * K, 1500, replace=False):   # a sprinkle elsewhere
        pos.add(int(p))
    pos = np.array(sorted(pos), np.int64)
    rows, cols = (pos // K).astype(np.int32), (pos % K).astype(np.int32)
    vals = normal((pos.shape[0],), "gpu/wide/skew/v")
    _check_layer_vs_oracle(M, K, pos.shape[0], (65, 100, 128, 191, 257), "gpu/wide/skew",
                           triple=(rows, cols, vals))


def test_slice_tiled_several_batch_tiles():
    # long keys with operands of three and four slices per view; at 449 and 500
    # columns (eight 64-column tiles, the first with a last tile of one column)
    # the slice-tiled forward and column passes run one grid row per tile (the
    # column pass writing one dW slab per tile, added up and permuted into
    # canonical order afterwards); at 65 columns the workgroups would have too
    # few entries and the key-major kernels and a separate dW pass run instead
    _check_layer_vs_oracle(2000, 1500, 300000, (65, 449, 500), "gpu/multitile/2000x1500", check_index=False)


@pytest.mark.parametrize("transpose", [False, True])
def test_keyed_keys_longer_than_chunks(transpose):
    # keys of ~1400 entries (several chunks each, so chunks that start inside a
    # key hold no key of their own) and one empty key, on the key-major path;
    # transposed, the same structure reaches the column view
    n, L_ = 8, 3000
    rng = np.random.default_rng(11)
    r, c = [], []
    for key in range(n):
        if key == 3:
            continue
        idx = np.sort(rng.choice(L_, 1400, replace=False))
        r.append(np.full(idx.shape[0], key)); c.append(idx)
    r = np.concatenate(r).astype(np.int32); c = np.concatenate(c).astype(np.int32)
    perm = rng.permutation(r.shape[0])
    r, c = r[perm], c[perm]
    v = rng.standard_normal(r.shape[0]).astype(np.float32)
    M, K = (n, L_) if not transpose else (L_, n)
    if transpose:
        r, c = c, r
    _check_layer_vs_oracle(M, K, r.shape[0], (1, 2, 3, 4, 5, 8, 16, 64), f"gpu/keyedlong/{int(transpose)}",
                           triple=(r, c, v))


def test_non_finite_activations_outside_the_support():
    # +inf in a feature no entry reads (feature 0, the first staged row of the
    # first slice) and in an output gradient no entry reads: entries the
    # kernels neutralise must add exactly zero, so every output stays finite
    # and matches the oracle
    import torch
    L = lib()
    M, K, nnz = 1000, 800, 200000
    rows, cols, vals = _make(M, K, nnz, "gpu/nonfinite")
    keep = (cols != 0) & (rows != 0)
    rows, cols, vals = rows[keep], cols[keep], vals[keep]
    ref = oracle.canonicalize(M, K, rows, cols, vals)
    layer = L.SnackLayer(M, K, dev(rows), dev(cols), dev(vals), seed=1)
    try:
        for B in (1, 2, 4, 8, 16, 32, 64):
            X = normal((B, K), f"gpu/nonfinite/X/{B}")
            dY = normal((B, M), f"gpu/nonfinite/dY/{B}")
            X[:, 0] = np.inf
            dY[:, 0] = np.inf
            say("non-finite outside the support B", B)
            Y = host(layer.forward(dev(X)))
            dX, dW = (host(t) for t in layer.backward(dev(X), dev(dY)))
            assert np.isfinite(Y).all() and np.isfinite(dX[:, 1:]).all() and np.isfinite(dW).all()
            Yr, Ya = oracle.forward(M, K, ref["rows"], ref["cols"], ref["vals"], X)
            assert_close(f"Y B={B}", Y, Yr, Ya)
            dXr, dXa = oracle.backward_dx(M, K, ref["rows"], ref["cols"], ref["vals"], dY)
            assert_close(f"dX B={B}", dX, dXr, dXa)
            dWr, dWa = oracle.backward_dw(M, K, ref["rows"], ref["cols"], X, dY)
            assert_close(f"dW B={B}", dW, dWr, dWa)
    finally:
        layer.close()


@pytest.mark.parametrize("M,K,nnz", [(130, 70, 2000), (1000, 800, 200000)])
def test_backward_dx_only_and_dw_only(M, K, nnz):
    # a first layer needs no dX; a frozen layer needs no dW: both paths alone
    L = lib()
    key = f"gpu/partial/{M}x{K}"
    rows, cols, vals = _make(M, K, nnz, key)
    ref = oracle.canonicalize(M, K, rows, cols, vals)
    layer = L.SnackLayer(M, K, dev(rows), dev(cols), dev(vals), seed=1, max_batch=65)
    try:
        for B in (1, 4, 16, 64, 65):
            X = normal((B, K), f"{key}/X/{B}")
            dY = normal((B, M), f"{key}/dY/{B}")
            say("partial backward", key, "B", B)
            dX, _ = layer.backward(dev(X), dev(dY), want_dw=False)
            dXr, dXa = oracle.backward_dx(M, K, ref["rows"], ref["cols"], ref["vals"], dY)
            assert_close(f"dX-only B={B}", host(dX), dXr, dXa)
            _, dW = layer.backward(dev(X), dev(dY), want_dx=False)
            dWr, dWa = oracle.backward_dw(M, K, ref["rows"], ref["cols"], X, dY)
            assert_close(f"dW-only B={B}", host(dW), dWr, dWa)
    finally:
        layer.close()


def test_long_rows_and_columns_span_many_chunks():
    # a row longer than a chunk, a dense column, and many empty rows/columns
    M, K = 50, 6000
    rng = np.random.default_rng(5)
    rows = np.concatenate([np.full(5000, 3), np.arange(50), rng.integers(10, 20, 300)])
    cols = np.concatenate([np.arange(5000), np.full(50, 5500), rng.integers(5001, 5499, 300)])
    pos = np.unique(rows.astype(np.int64) * K + cols)
    rng.shuffle(pos)
    r, c = (pos // K).astype(np.int32), (pos % K).astype(np.int32)
    v = rng.standard_normal(pos.shape[0]).astype(np.float32)
    import torch
    L = lib()
    ref = oracle.canonicalize(M, K, r, c, v)
    say("create long rows", M, K, pos.shape[0])
    layer = L.SnackLayer(M, K, dev(r), dev(c), dev(v))
    try:
        for B in (1, 4, 33):
            X = normal((B, K), f"long/X/{B}"); dY = normal((B, M), f"long/dY/{B}")
            say("long rows B", B)
            Y = layer.forward(dev(X)); dX, dW = layer.backward(dev(X), dev(dY))
            Yr, Ya = oracle.forward(M, K, ref["rows"], ref["cols"], ref["vals"], X)
            assert_close("Y", host(Y), Yr, Ya)
            dXr, dXa = oracle.backward_dx(M, K, ref["rows"], ref["cols"], ref["vals"], dY)
            assert_close("dX", host(dX), dXr, dXa)
            dWr, dWa = oracle.backward_dw(M, K, ref["rows"], ref["cols"], X, dY)
            assert_close("dW", host(dW), dWr, dWa)
    finally:
        layer.close()


def test_worked_example_exact():
    # "Padded-CSR" section 6.1, nn.Linear layout: Y^T = [[23, 5, 23], [28, 10, 28]]
    import torch
    L = lib()
    rows = np.array([2, 0, 1, 2, 0], np.int32); cols = np.array([2, 1, 0, 1, 3], np.int32)
    vals = np.array([4, 3, 5, 1, 2], np.float32)
    say("worked example")
    layer = L.SnackLayer(3, 4, dev(rows), dev(cols), dev(vals))
    X = dev(np.array([[1, 3, 5, 7], [2, 4, 6, 8]], np.float32))
    Y = host(layer.forward(X))
    assert Y.tolist() == [[23, 5, 23], [28, 10, 28]]
    layer.close()


def test_integer_data_bit_exact():
    import torch
    L = lib()
    M, K, nnz = 200, 300, 6000
    rows, cols, _ = random_layer(M, K, nnz, "gpu/int")
    rng = np.random.default_rng(11)
    vals = rng.integers(-8, 9, nnz).astype(np.float32)
    layer = L.SnackLayer(M, K, dev(rows), dev(cols), dev(vals))
    ref = oracle.canonicalize(M, K, rows, cols, vals)
    for B in (1, 3, 64):
        X = rng.integers(-8, 9, (B, K)).astype(np.float32)
        dY = rng.integers(-8, 9, (B, M)).astype(np.float32)
        say("integer exact B", B)
        Y = layer.forward(dev(X)); dX, dW = layer.backward(dev(X), dev(dY))
        Yr, _ = oracle.forward(M, K, ref["rows"], ref["cols"], ref["vals"], X)
        dXr, _ = oracle.backward_dx(M, K, ref["rows"], ref["cols"], ref["vals"], dY)
        dWr, _ = oracle.backward_dw(M, K, ref["rows"], ref["cols"], X, dY)
        assert np.array_equal(host(Y).astype(np.float64), Yr)
        assert np.array_equal(host(dX).astype(np.float64), dXr)
        assert np.array_equal(host(dW).astype(np.float64), dWr)
    layer.close()


def test_repeat_runs_bit_identical():
    import torch
    L = lib()
    M, K, nnz = 3000, 2000, 300000
    rows, cols, vals = random_layer(M, K, nnz, "gpu/det")
    layer = L.SnackLayer(M, K, dev(rows), dev(cols), dev(vals))
    for B in (1, 16, 64):
        X = dev(normal((B, K), "det/X")); dY = dev(normal((B, M), "det/dY"))
        say("determinism B", B)
        a = [host(t) for t in (layer.forward(X),) + layer.backward(X, dY)]
        for _ in range(3):
            b = [host(t) for t in (layer.forward(X),) + layer.backward(X, dY)]
            for x, y in zip(a, b):
                assert np.array_equal(x.view(np.uint32), y.view(np.uint32))
    layer.close()


def test_create_errors_leave_no_layer():
    L = lib()
    say("create errors")
    with pytest.raises(L.SnackError) as e:
        L.SnackLayer(4, 4, dev(np.array([0, 4], np.int32)), dev(np.array([0, 0], np.int32)))
    assert e.value.code == L.ERR_INDEX_RANGE
    with pytest.raises(L.SnackError) as e:
        L.SnackLayer(4, 4, dev(np.array([1, 2, 1], np.int32)), dev(np.array([3, 3, 3], np.int32)))
    assert e.value.code == L.ERR_DUPLICATE
    with pytest.raises(L.SnackError) as e:
        L.SnackLayer(4, 4, dev(np.array([1, -1], np.int32)), dev(np.array([3, 3], np.int32)))
    assert e.value.code == L.ERR_INDEX_RANGE


def test_reserve_covers_every_batch_up_to_it():
    """After snack_layer_reserve(max_batch), calls at any batch up to it
    allocate nothing: the workspace is sized for the largest plan, which need
    not be max_batch's own (the batch-tiled buffers have size limits)."""
    L = lib()
    M, K, nnz = 2000, 1500, 300000
    rows, cols, vals = _make(M, K, nnz, "gpu/reserve", None)
    layer = L.SnackLayer(M, K, dev(rows), dev(cols), dev(vals), seed=1)
    try:
        layer.reserve(600)
        before = layer.device_bytes()
        for B in (600, 1, 8, 64, 65, 449, 500, 130):
            say("reserve", "B", B)
            X = dev(normal((B, K), f"gpu/reserve/X/{B}"))
            dY = dev(normal((B, M), f"gpu/reserve/dY/{B}"))
            layer.forward(X)
            layer.backward(X, dY)
            assert layer.device_bytes() == before, f"B={B} grew the workspace"
    finally:
        layer.close()


def test_batch_beyond_reserve_is_refused_cleanly():
    """Forward, backward and the fused training calls allocate nothing: a layer
    reserves batches up to 64 at create, a larger batch is refused with
    SNACK_ERR_WORKSPACE before anything is launched (outputs untouched, device
    bytes unchanged), batches up to the reserve run, and after
    snack_layer_reserve the larger batch runs too.  Batches above 2^20 are
    refused as unsupported."""
    import torch
    L = lib()
    M, K, nnz = 2000, 1500, 300000
    rows, cols, vals = _make(M, K, nnz, "gpu/refuse", None)
    layer = L.SnackLayer(M, K, dev(rows), dev(cols), dev(vals), seed=1)
    try:
        before = layer.device_bytes()
        B = 600   # its feature-major copies alone (9 MB) exceed what batches up to 64 need here (2.4 MB)
        X = dev(normal((B, K), "gpu/refuse/X"))
        T = dev(normal((B, M), "gpu/refuse/T"))
        dY = dev(normal((B, M), "gpu/refuse/dY"))
        Y = torch.full((B, M), 7.0, device="cuda")
        dX = torch.full((B, K), 7.0, device="cuda")
        dW = torch.full((nnz,), 7.0, device="cuda")
        v0 = host(layer.export()[2])
        say("refuse: B", B, "beyond the default reserve")
        calls = (
            lambda: L.snack_forward(layer.h, X, Y),
            lambda: L.snack_backward(layer.h, X, dY, dX, dW),
            lambda: L.snack_backward(layer.h, X, dY, dX, None),
            lambda: L.snack_backward_sgd(layer.h, X, dY, dX, dW, 0.01),
            lambda: L.snack_train_step_mse(layer.h, X, T, Y, dY.clone(), dX, dW, 2.0 / (B * M), 0.01),
        )
        for f in calls:
            with pytest.raises(L.SnackError) as e:
                f()
            assert e.value.code == L.ERR_WORKSPACE
        torch.cuda.synchronize()
        assert layer.device_bytes() == before
        assert bool((Y == 7.0).all()) and bool((dX == 7.0).all()) and bool((dW == 7.0).all())
        assert np.array_equal(host(layer.export()[2]).view(np.uint32), v0.view(np.uint32))
        for b in (1, 2, 4, 8, 16, 32, 64):
            say("refuse: B", b, "inside the default reserve")
            Xb = dev(normal((b, K), f"gpu/refuse/X/{b}"))
            Tb = dev(normal((b, M), f"gpu/refuse/T/{b}"))
            layer.forward(Xb)
            layer.train_step_mse(Xb, Tb, 0.0)
        torch.cuda.synchronize()
        assert layer.device_bytes() == before
        layer.reserve(B)
        assert layer.device_bytes() > before
        say("refuse: B", B, "after reserve")
        L.snack_forward(layer.h, X, Y)
        Yr, Ya = oracle.forward(M, K, *(host(t) for t in layer.export()), host(X))
        assert_close("Y after reserve", host(Y), Yr, Ya)
        with pytest.raises(L.SnackError) as e:
            layer.reserve(2 ** 20 + 1)
        assert e.value.code == L.ERR_UNSUPPORTED
    finally:
        layer.close()
    small = L.SnackLayer(3, 1, dev(np.array([0, 2], np.int32)), dev(np.array([0, 0], np.int32)),
                         dev(np.array([1.0, 2.0], np.float32)))
    try:
        Xh = torch.zeros((2 ** 20 + 1, 1), device="cuda")
        Yh = torch.zeros((2 ** 20 + 1, 3), device="cuda")
        say("refuse: B above 2^20")
        with pytest.raises(L.SnackError) as e:
            L.snack_forward(small.h, Xh, Yh)
        assert e.value.code == L.ERR_UNSUPPORTED
    finally:
        small.close()

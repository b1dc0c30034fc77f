"""Row-local drop / regrow on the GPU vs the oracle (through the C ABI): every
row drops floor(n_i * num / den) of its smallest |w| and regrows as many cells
inside itself, at random (SET) or at the largest |dY^T X| (RigL); positions,
kept values and the +0 of grown entries bit-exact, and both index views."""
import numpy as np
import pytest

import oracle
from snack_inputs import normal, random_layer, rng_for
from tests.gpu_util import say, lib, dev, host, assert_close

pytestmark = pytest.mark.gpu

SEED = 5


def _check_views(layer, M, K, cur, nnz):
    ci = oracle.canonicalize(M, K, *cur)
    rp, pm, rt, cp = (host(t) for t in layer.export_index())
    assert np.array_equal(rp, ci["row_ptr"]) and np.array_equal(cp, ci["col_ptr"])
    if nnz:
        assert np.array_equal(pm, ci["perm"]) and np.array_equal(rt, ci["rows_t"])


def _data(B, M, K, key, data):
    if data == "int":
        g = rng_for(f"{key}/int")
        return (g.integers(-2, 3, size=(B, K)).astype(np.float32), g.integers(-2, 3, size=(B, M)).astype(np.float32))
    if data == "zero":
        return normal((B, K), f"{key}/X"), np.zeros((B, M), np.float32)
    return normal((B, K), f"{key}/X"), normal((B, M), f"{key}/dY")


def _run(M, K, nnz, mode, fracs, key, B=3, data="normal", layer_in=None):
    L = lib()
    if layer_in is None:
        rows, cols, v = random_layer(M, K, nnz, key)
    else:
        rows, cols, v = layer_in
        nnz = rows.shape[0]
    ref = oracle.canonicalize(M, K, rows, cols, v)
    say("rows create", key, M, K, nnz, "mode", mode)
    layer = L.SnackLayer(M, K, dev(rows), dev(cols), dev(v), seed=SEED)
    cur = (ref["rows"], ref["cols"], ref["vals"])
    try:
        for i, (num, den) in enumerate(fracs):
            epoch = layer.epoch
            say("rows", key, "round", i, "frac", num, den)
            if mode == L.REGROW_GRADIENT:
                X, dY = _data(B, M, K, f"{key}/{i}", data)
                layer.prune_regrow_rows(num, den, mode, dev(X), dev(dY))
                o = oracle.prune_regrow_rows(M, K, *cur, num, den, 1, X=X, dY=dY)
            else:
                layer.prune_regrow_rows(num, den, mode)
                o = oracle.prune_regrow_rows(M, K, *cur, num, den, 0, seed=SEED, epoch=epoch)
            r, c, vv = (host(t) for t in layer.export())
            assert np.array_equal(r, o[0]) and np.array_equal(c, o[1]), f"{key} round {i}: positions"
            assert np.array_equal(vv.view(np.uint32), o[2].view(np.uint32)), f"{key} round {i}: values"
            assert layer.epoch == epoch + 1
            cur = o
            _check_views(layer, M, K, cur, nnz)
    finally:
        layer.close()


SHAPES = [(6, 5, 14), (40, 30, 300), (1, 300, 17), (300, 1, 29), (33, 31, 500), (64, 64, 2000), (7, 3, 21),
          (500, 500, 12500), (257, 129, 3300), (300, 700, 21000)]
FRACS = ((3, 10), (1, 2), (1, 1), (1, 7))


@pytest.mark.parametrize("M,K,nnz", SHAPES)
def test_random_row_regrow_matches_oracle(M, K, nnz):
    L = lib()
    _run(M, K, nnz, L.REGROW_RANDOM, FRACS, f"gpu/rows/set/{M}x{K}")


@pytest.mark.parametrize("M,K,nnz", SHAPES)
def test_gradient_row_regrow_matches_oracle(M, K, nnz):
    L = lib()
    _run(M, K, nnz, L.REGROW_GRADIENT, FRACS, f"gpu/rows/rigl/{M}x{K}")


@pytest.mark.parametrize("B", [1, 17, 64])
def test_gradient_row_regrow_batch_sizes(B):
    L = lib()
    _run(300, 450, 13500, L.REGROW_GRADIENT, ((3, 10),), f"gpu/rows/rigl/b{B}", B=B)


def test_gradient_row_regrow_ties_and_zero_gradient():
    L = lib()
    # small integer data: many cells of a row share the threshold score
    _run(120, 450, 13500, L.REGROW_GRADIENT, ((3, 10), (1, 2)), "gpu/rows/rigl/ties", data="int")
    # zero gradient: every empty cell ties, the smallest columns are taken
    _run(50, 300, 3000, L.REGROW_GRADIENT, ((3, 10),), "gpu/rows/rigl/zero", data="zero")


def test_empty_and_full_rows():
    # rows 0 and 5 empty, rows 2 and 7 full, the rest ragged
    L = lib()
    M, K = 9, 40
    g = rng_for("gpu/rows/edges")
    pos = []
    for i in range(M):
        if i in (0, 5):
            continue
        n = K if i in (2, 7) else int(g.integers(1, K))
        pos.extend(i * K + np.sort(g.choice(K, n, replace=False)))
    pos = np.array(pos, np.int64)
    rows, cols = (pos // K).astype(np.int32), (pos % K).astype(np.int32)
    v = normal((pos.shape[0],), "gpu/rows/edges/v")
    for mode in (L.REGROW_RANDOM, L.REGROW_GRADIENT):
        _run(M, K, 0, mode, ((3, 10), (1, 1)), f"gpu/rows/edges/{mode}", layer_in=(rows, cols, v))


def test_random_row_regrow_full_scale_exact():
    # 10000 x 10000 at 95 %: 30 % of every row, exact against the oracle
    L = lib()
    _run(10000, 10000, 5_000_000, L.REGROW_RANDOM, ((3, 10),), "gpu/rows/c4/set")


def test_gradient_row_regrow_full_scale_sampled_rows():
    # 10000 x 10000 at 95 %, batch 4: rows are independent, so sampled rows are
    # checked exactly against the oracle run on just those rows
    L = lib()
    M = K = 10000
    nnz, B = 5_000_000, 4
    rows, cols, v = random_layer(M, K, nnz, "gpu/rows/c4/rigl")
    ref = oracle.canonicalize(M, K, rows, cols, v)
    X = normal((B, K), "gpu/rows/c4/rigl/X")
    dY = normal((B, M), "gpu/rows/c4/rigl/dY")
    layer = L.SnackLayer(M, K, dev(rows), dev(cols), dev(v), seed=SEED)
    try:
        say("rows rigl full scale")
        layer.prune_regrow_rows(3, 10, L.REGROW_GRADIENT, dev(X), dev(dY))
        r, c, vv = (host(t) for t in layer.export())
        assert np.array_equal(np.bincount(r, minlength=M), np.bincount(ref["rows"], minlength=M))
        sample = np.unique(np.concatenate([[0, M - 1], rng_for("gpu/rows/c4/rigl/sample").choice(M, 60)]))
        sel = np.isin(ref["rows"], sample)
        sub = np.searchsorted(sample, ref["rows"][sel]).astype(np.int32)
        o = oracle.prune_regrow_rows(sample.shape[0], K, sub, ref["cols"][sel], ref["vals"][sel], 3, 10, 1,
                                     X=X, dY=np.ascontiguousarray(dY[:, sample]))
        got = np.isin(r, sample)
        assert np.array_equal(r[got], sample[o[0]]) and np.array_equal(c[got], o[1])
        assert np.array_equal(vv[got].view(np.uint32), o[2].view(np.uint32))
    finally:
        layer.close()


def test_training_after_row_regrow_matches_oracle():
    # forward and backward run on the rebuilt views
    L = lib()
    M, K, nnz, B = 200, 300, 6000, 8
    rows, cols, v = random_layer(M, K, nnz, "gpu/rows/train")
    layer = L.SnackLayer(M, K, dev(rows), dev(cols), dev(v), seed=SEED)
    try:
        layer.prune_regrow_rows(3, 10, L.REGROW_RANDOM)
        X = normal((B, K), "gpu/rows/train/X")
        dY = normal((B, M), "gpu/rows/train/dY")
        r, c, vv = (host(t) for t in layer.export())
        Y = layer.forward(dev(X))
        dX, dW = layer.backward(dev(X), dev(dY))
        assert_close("Y", host(Y), *oracle.forward(M, K, r, c, vv, X))
        assert_close("dX", host(dX), *oracle.backward_dx(M, K, r, c, vv, dY))
        assert_close("dW", host(dW), *oracle.backward_dw(M, K, r, c, X, dY))
    finally:
        layer.close()


def test_row_regrow_argument_errors():
    import torch
    L = lib()
    rows, cols, v = random_layer(20, 30, 100, "gpu/rows/err")
    layer = L.SnackLayer(20, 30, dev(rows), dev(cols), dev(v))
    try:
        X = torch.zeros(2, 30, device="cuda")
        dY = torch.zeros(2, 20, device="cuda")
        for num, den in ((2, 1), (-1, 3), (1, 0)):
            with pytest.raises(L.SnackError):
                layer.prune_regrow_rows(num, den, L.REGROW_RANDOM)
        with pytest.raises(L.SnackError):
            layer.prune_regrow_rows(1, 2, 7)
        with pytest.raises(L.SnackError):
            layer.prune_regrow_rows(1, 2, L.REGROW_GRADIENT)       # no batch given
        layer.prune_regrow_rows(0, 1, L.REGROW_GRADIENT, X, dY)   # nothing moves: only the epoch advances
        assert layer.epoch == 1
    finally:
        layer.close()

"""Gradient-driven drop / regrow on the GPU vs the oracle (through the C ABI):
the drop of the n smallest |w| and the regrow at the empty cells of largest
|dL/dW| for a batch, bit-exact (positions, kept values, +0 for grown ones)."""
import numpy as np
import pytest

import oracle
from snack_inputs import normal, random_layer, rng_for
from tests.gpu_util import say, lib, dev, host

pytestmark = pytest.mark.gpu


def _run(M, K, nnz, B, fracs, key, data="normal"):
    L = lib()
    rows, cols, v = random_layer(M, K, nnz, key)
    ref = oracle.canonicalize(M, K, rows, cols, v)
    say("rigl create", key, M, K, nnz, "B", B)
    layer = L.SnackLayer(M, K, dev(rows), dev(cols), dev(v), seed=5)
    cur = (ref["rows"], ref["cols"], ref["vals"])
    try:
        for i, frac in enumerate(fracs):
            if data == "int":
                g = rng_for(f"{key}/int/{i}")
                X = g.integers(-2, 3, size=(B, K)).astype(np.float32)
                dY = g.integers(-2, 3, size=(B, M)).astype(np.float32)
            elif data == "zero":
                X = normal((B, K), f"{key}/X/{i}")
                dY = np.zeros((B, M), np.float32)
            else:
                X = normal((B, K), f"{key}/X/{i}")
                dY = normal((B, M), f"{key}/dY/{i}")
            n_drop = int(nnz * frac)
            say("rigl", key, "round", i, "n_drop", n_drop)
            epoch = layer.epoch
            layer.prune_regrow_grad(n_drop, dev(X), dev(dY))
            o = oracle.prune_regrow_grad(M, K, cur[0], cur[1], cur[2], n_drop, X, dY)
            r, c, vv = (host(t) for t in layer.export())
            assert np.array_equal(r, o[0]) and np.array_equal(c, o[1]), f"{key} round {i}: positions"
            assert np.array_equal(vv.view(np.uint32), o[2].view(np.uint32)), f"{key} round {i}: values"
            assert layer.epoch == epoch + 1
            cur = o
            ci = oracle.canonicalize(M, K, *cur)
            rp, pm, rt, cp = (host(t) for t in layer.export_index())
            assert np.array_equal(rp, ci["row_ptr"]) and np.array_equal(cp, ci["col_ptr"])
            if nnz:
                assert np.array_equal(pm, ci["perm"]) and np.array_equal(rt, ci["rows_t"])
    finally:
        layer.close()


@pytest.mark.parametrize("M,K,nnz,B", [(6, 5, 14, 2), (40, 30, 300, 3), (1, 300, 17, 5), (300, 1, 29, 4),
                                       (500, 500, 12500, 4), (300, 700, 21000, 17), (257, 129, 3300, 40),
                                       (3000, 700, 105000, 64)])
def test_gradient_regrow_matches_oracle(M, K, nnz, B):
    _run(M, K, nnz, B, (0.3, 0.5, 1.0), f"gpu/rigl/{M}x{K}")


def test_gradient_regrow_ties_at_the_threshold():
    # small integer data: many cells share the threshold score across tiles, so
    # the position-order ranking of ties is exercised
    _run(600, 450, 13500, 3, (0.3, 0.1), "gpu/rigl/ties", data="int")


def test_gradient_regrow_zero_gradient_takes_first_empty_cells():
    _run(200, 300, 3000, 2, (0.3,), "gpu/rigl/zero", data="zero")


def test_gradient_regrow_full_scale_dominance():
    # 10000 x 10000 at 95 %, batch 4: drop 30 %, regrow at the largest |dY^T X|.  The
    # exact oracle would sort 96.5 M cells; here: the drop is the n smallest |w|, nnz is
    # kept, grown values are +0 on cells empty after the drop, and every grown cell's
    # |G| (dense, fp64) is at least every other empty cell's, within fp32 accumulation.
    L = lib()
    M = K = 10000
    nnz, B = 5_000_000, 4
    rows, cols, v = random_layer(M, K, nnz, "gpu/rigl/c4")
    ref = oracle.canonicalize(M, K, rows, cols, v)
    layer = L.SnackLayer(M, K, dev(rows), dev(cols), dev(v), seed=5)
    try:
        X = normal((B, K), "gpu/rigl/c4/X")
        dY = normal((B, M), "gpu/rigl/c4/dY")
        n_drop = nnz * 3 // 10
        say("rigl full scale")
        layer.prune_regrow_grad(n_drop, dev(X), dev(dY))
        r, c, vv = (host(t) for t in layer.export())
        pos = r.astype(np.int64) * K + c
        assert pos.shape[0] == nnz and np.all(np.diff(pos) > 0)
        # the kept entries: all but the n_drop smallest |v| (order key: |v| bits, then slot)
        old_pos = ref["rows"].astype(np.int64) * K + ref["cols"]
        drop_order = np.lexsort((np.arange(nnz), np.abs(ref["vals"]).view(np.uint32)))
        kept_mask = np.ones(nnz, bool)
        kept_mask[drop_order[:n_drop]] = False
        kept_pos = old_pos[kept_mask]
        assert np.all(np.isin(kept_pos, pos))
        is_kept = np.isin(pos, kept_pos)
        assert np.array_equal(vv[is_kept].view(np.uint32), ref["vals"][kept_mask].view(np.uint32))
        grown = pos[~is_kept]
        assert grown.shape[0] == n_drop and np.all(vv[~is_kept].view(np.uint32) == 0)
        G = np.abs(dY.astype(np.float64).T @ X.astype(np.float64)).reshape(-1)
        occupied = np.zeros(M * K, bool)
        occupied[kept_pos] = True
        occupied[grown] = True
        rest = G[~occupied]                                    # empty cells not grown
        err = 1e-5 * (np.abs(dY.astype(np.float64)).T @ np.abs(X.astype(np.float64))).max()
        assert G[grown].min() >= rest.max() - 2 * err
        del G, rest, occupied
        # the grown cells' own fp32 keys are those the oracle computes
        sample = grown[:: max(1, grown.shape[0] // 2000)]
        keys = np.array([oracle.grow_key(M, K, X, dY, p // K, p % K) for p in sample], np.uint32)
        assert keys.min() > 0
    finally:
        layer.close()


def test_gradient_regrow_argument_errors():
    import torch
    L = lib()
    rows, cols, v = random_layer(20, 30, 100, "gpu/rigl/err")
    layer = L.SnackLayer(20, 30, dev(rows), dev(cols), dev(v))
    try:
        X = torch.zeros(2, 30, device="cuda")
        dY = torch.zeros(2, 20, device="cuda")
        with pytest.raises(L.SnackError):
            layer.prune_regrow_grad(101, X, dY)
        with pytest.raises(L.SnackError):
            layer.prune_regrow_grad(-1, X, dY)
        layer.prune_regrow_grad(0, X, dY)              # nothing to move: only the epoch advances
        assert layer.epoch == 1
    finally:
        layer.close()

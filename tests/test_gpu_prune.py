"""Drop / regrow on the GPU vs the oracle: bit-exact triples and index."""
import numpy as np
import pytest

import oracle
from snack_inputs import normal, random_layer
from tests.gpu_util import say, lib, dev, host, assert_close

pytestmark = pytest.mark.gpu


def _run(M, K, nnz, fracs, key, seed=12345, vals=None, rounds=1):
    L = lib()
    rows, cols, v = random_layer(M, K, nnz, key)
    if vals is not None:
        v = vals
    ref = oracle.canonicalize(M, K, rows, cols, v)
    say("prune create", key, M, K, nnz)
    layer = L.SnackLayer(M, K, dev(rows), dev(cols), dev(v), seed=seed)
    cur = (ref["rows"], ref["cols"], ref["vals"])
    try:
        epoch = 0
        for _ in range(rounds):
            for frac in fracs:
                n_drop = int(nnz * frac)
                say("prune", key, "n_drop", n_drop, "epoch", epoch)
                layer.prune_regrow(n_drop)
                o = oracle.prune_regrow(M, K, cur[0], cur[1], cur[2], n_drop, seed, epoch)
                epoch += 1
                r, c, vv = (host(t) for t in layer.export())
                assert np.array_equal(r, o[0]) and np.array_equal(c, o[1])
                assert np.array_equal(vv.view(np.uint32), o[2].view(np.uint32))
                assert layer.epoch == epoch
                cur = o[:3]
                ci = oracle.canonicalize(M, K, *cur)
                rp, pm, rt, cp = (host(t) for t in layer.export_index())
                assert np.array_equal(rp, ci["row_ptr"]) and np.array_equal(cp, ci["col_ptr"])
                if nnz:
                    assert np.array_equal(pm, ci["perm"]) and np.array_equal(rt, ci["rows_t"])
    finally:
        layer.close()


@pytest.mark.parametrize("M,K,nnz", [(6, 5, 14), (40, 30, 300), (500, 500, 12500), (64, 64, 4096),
                                     (3000, 700, 105000), (600, 600, 180000)])
def test_prune_regrow_matches_oracle(M, K, nnz):
    _run(M, K, nnz, (0.3, 0.0, 0.5, 1.0), f"gpu/prune/{M}x{K}")


def test_prune_ties_signed_zero_nan():
    M, K, nnz = 30, 40, 600
    rng = np.random.default_rng(3)
    vals = rng.choice(np.array([0.0, -0.0, 0.25, -0.25, 1.0, np.nan, 2.0], np.float32), nnz)
    _run(M, K, nnz, (0.1, 0.3, 0.6), "gpu/prune/ties", vals=vals)


@pytest.mark.parametrize("M,K,nnz,cap", [(500, 500, 12500, 24), (64, 64, 4096, 16)])
def test_prune_bucket_overflow_retries(M, K, nnz, cap, monkeypatch):
    # tiny buckets overflow on most batches: each is taken again at half size
    # (and the rebuild queued behind the first batch is replaced), the result
    # being the same as with one large batch
    monkeypatch.setenv("SNACK_GROW_BUCKET_CAP", str(cap))
    _run(M, K, nnz, (0.3, 0.05), f"gpu/prune/overflow/{M}x{K}")


def test_prune_full_scale_10000_square():
    # 10000 x 10000 at 95 %: drop 30 % of 5,000,000 twice (two epochs)
    _run(10000, 10000, 5_000_000, (0.3,), "gpu/prune/c4", rounds=2)


def test_prune_regions_wider_than_one_pass():
    # 50000 x 50000 = 2.5e9 cells: the grow step's regions are wider than one
    # LDS pass, so each is claimed in several; the column view takes the sort path
    _run(50000, 50000, 200_000, (0.3, 0.7), "gpu/prune/wide")


@pytest.mark.parametrize("M,K", [(3000, 3000), (1700, 6100)])
def test_batch_tiled_passes_after_drop_regrow(M, K):
    """Drop/regrow rebuilds the slice tables the batch-tiled kernels read; the
    forward and backward that follow match the oracle for every batch tile,
    on both views (keys long enough that the tables have two or more slices)."""
    L = lib()
    nnz = M * K // 20
    rows, cols, v = random_layer(M, K, nnz, f"gpu/prune/tiles/{M}x{K}")
    layer = L.SnackLayer(M, K, dev(rows), dev(cols), dev(v), seed=31)
    try:
        say("tiles after prune", M, K)
        layer.prune_regrow(nnz * 3 // 10)
        r, c, vv = (host(t) for t in layer.export())
        for B in (8, 16, 32, 64):
            X = normal((B, K), f"gpu/prune/tiles/{M}x{K}/X/{B}")
            dY = normal((B, M), f"gpu/prune/tiles/{M}x{K}/dY/{B}")
            say("tiles after prune B", B)
            Y = host(layer.forward(dev(X)))
            dX, dW = (host(t) for t in layer.backward(dev(X), dev(dY)))
            assert_close(f"Y B={B}", Y, *oracle.forward(M, K, r, c, vv, X))
            assert_close(f"dX B={B}", dX, *oracle.backward_dx(M, K, r, c, vv, dY))
            assert_close(f"dW B={B}", dW, *oracle.backward_dw(M, K, r, c, X, dY))
    finally:
        layer.close()


@pytest.mark.parametrize("M,K,nnz", [(500, 500, 12500), (3000, 700, 105000)])
def test_resume_from_export_continues_drop_regrow(M, K, nnz):
    """Checkpoint / resume: export the triple after some drop/regrow epochs,
    create a new layer from it with the same seed, set its epoch, and the next
    drop/regrow calls give bit for bit what the uninterrupted layer gives (and
    what the oracle gives at that epoch)."""
    import torch
    L = lib()
    seed = 777
    rows, cols, v = random_layer(M, K, nnz, f"gpu/resume/{M}x{K}")
    n_drop = nnz * 3 // 10
    a = L.SnackLayer(M, K, dev(rows), dev(cols), dev(v), seed=seed)
    b = None
    try:
        for _ in range(2):
            a.prune_regrow(n_drop)
        assert a.epoch == 2
        say("resume: checkpoint at epoch", a.epoch)
        r, c, vv = a.export()
        epoch = a.epoch
        # the checkpoint crosses the host, as a saved state would
        r, c, vv = (torch.from_numpy(host(t)).cuda() for t in (r, c, vv))
        b = L.SnackLayer(M, K, r, c, vv, seed=seed)
        b.epoch = epoch
        cur = (host(r), host(c), host(vv))
        for step in range(2):
            say("resume: drop/regrow after resume", step)
            a.prune_regrow(n_drop)
            b.prune_regrow(n_drop)
            ta = [host(t) for t in a.export()]
            tb = [host(t) for t in b.export()]
            assert np.array_equal(ta[0], tb[0]) and np.array_equal(ta[1], tb[1])
            assert np.array_equal(ta[2].view(np.uint32), tb[2].view(np.uint32))
            o = oracle.prune_regrow(M, K, cur[0], cur[1], cur[2], n_drop, seed, epoch + step)
            assert np.array_equal(tb[0], o[0]) and np.array_equal(tb[1], o[1])
            assert np.array_equal(tb[2].view(np.uint32), o[2].view(np.uint32))
            assert a.epoch == b.epoch == epoch + step + 1
            cur = o[:3]
        # a fresh layer left at epoch 0 draws another stream: the epoch matters
        c0 = L.SnackLayer(M, K, dev(cur[0]), dev(cur[1]), dev(cur[2]), seed=seed)
        try:
            c0.prune_regrow(n_drop)
            o0 = oracle.prune_regrow(M, K, cur[0], cur[1], cur[2], n_drop, seed, 0)
            r0 = host(c0.export()[0])
            assert np.array_equal(r0, o0[0])
            o4 = oracle.prune_regrow(M, K, cur[0], cur[1], cur[2], n_drop, seed, 4)
            assert not (np.array_equal(o0[0], o4[0]) and np.array_equal(o0[1], o4[1]))
        finally:
            c0.close()
    finally:
        a.close()
        if b is not None:
            b.close()

"""Pins of the oracle's gradient regrow (drop the smallest |w|, grow at the empty
cells of largest |dL/dW| -- the "Padded-CSR" post, section 4.3: RigL grows at
high-gradient locations; SNACK paper, Tables 8-9).  CPU only.

The gradient of the layer's loss with respect to the dense weight is
dL/dW = dY^T X (Padded-CSR, section 7.1), so the brute force below computes it
with a plain numpy matrix product, masks the cells occupied after the drop,
and takes the n largest |G| with ties broken by the smaller linear position.
With small integer data every product and sum is exact in fp32, so the
oracle's fp32 decision must match the brute force exactly; with random data
the brute force in fp64 bounds what the fp32 decision may differ on.
"""
import numpy as np
import pytest

import oracle
from snack_inputs import normal, random_layer, rng_for


def _brute(M, K, rows, cols, vals, n_drop, X, dY):
    """Brute force: (kept positions, their values, grown positions), all from numpy."""
    nnz = rows.shape[0]
    mags = np.abs(vals.astype(np.float32)).view(np.uint32)
    order = np.lexsort((np.arange(nnz), mags))            # by (|v| bits, slot)
    dropped = np.zeros(nnz, bool)
    dropped[order[:n_drop]] = True
    pos = rows.astype(np.int64) * K + cols
    kept_pos = pos[~dropped]
    kept_val = vals[~dropped]
    G = dY.astype(np.float64).T @ X.astype(np.float64)   # [M, K]
    occupied = np.zeros(M * K, bool)
    occupied[kept_pos] = True
    cells = np.nonzero(~occupied)[0]
    score = np.abs(G.reshape(-1)[cells])
    pick = np.lexsort((cells, -score))[:n_drop]            # larger |G| first, then smaller position
    return kept_pos, kept_val, np.sort(cells[pick]), G


def _canon(M, K, seed_key, nnz):
    r, c, v = random_layer(M, K, nnz, seed_key)
    ref = oracle.canonicalize(M, K, r, c, v)
    return ref["rows"], ref["cols"], ref["vals"]


def _split(M, K, o):
    r, c, v = o
    return r.astype(np.int64) * K + c, v


@pytest.mark.parametrize("M,K,nnz,B,frac", [(7, 11, 30, 3, 0.3), (12, 5, 20, 1, 0.5), (9, 9, 81, 2, 0.3),
                                            (16, 13, 60, 4, 1.0), (5, 40, 37, 6, 0.1)])
def test_integer_data_matches_dense_brute_force_exactly(M, K, nnz, B, frac):
    rows, cols, vals = _canon(M, K, f"rigl/int/{M}x{K}", nnz)
    g = rng_for(f"rigl/int/data/{M}x{K}")
    X = g.integers(-3, 4, size=(B, K)).astype(np.float32)
    dY = g.integers(-3, 4, size=(B, M)).astype(np.float32)
    n_drop = int(nnz * frac)
    o = oracle.prune_regrow_grad(M, K, rows, cols, vals, n_drop, X, dY)
    pos, v = _split(M, K, o)
    kept_pos, kept_val, grown, _ = _brute(M, K, rows, cols, vals, n_drop, X, dY)
    assert np.array_equal(pos, np.sort(np.concatenate([kept_pos, grown])))
    is_grown = np.isin(pos, grown)
    assert np.array_equal(v[~is_grown].view(np.uint32), kept_val.view(np.uint32))
    assert np.all(v[is_grown].view(np.uint32) == 0)         # +0.0 exactly


def test_random_data_grown_scores_dominate():
    # fp32 accumulation may order near-equal scores differently from fp64, but
    # never by more than the accumulation error
    M, K, nnz, B = 40, 55, 400, 8
    rows, cols, vals = _canon(M, K, "rigl/rand", nnz)
    X = normal((B, K), "rigl/rand/X")
    dY = normal((B, M), "rigl/rand/dY")
    n_drop = 120
    o = oracle.prune_regrow_grad(M, K, rows, cols, vals, n_drop, X, dY)
    pos, v = _split(M, K, o)
    kept_pos, _, grown_bf, G = _brute(M, K, rows, cols, vals, n_drop, X, dY)
    grown = np.setdiff1d(pos, kept_pos)
    assert grown.shape[0] == n_drop
    occupied = np.zeros(M * K, bool)
    occupied[kept_pos] = True
    empty = np.nonzero(~occupied)[0]
    not_grown = np.setdiff1d(empty, grown)
    S = np.abs(G.reshape(-1))
    err = 1e-5 * (np.abs(dY.astype(np.float64)).T @ np.abs(X.astype(np.float64))).reshape(-1)
    assert S[grown].min() >= S[not_grown].max() - 2 * err.max()
    # and the sets agree away from near-ties
    assert np.setdiff1d(grown, grown_bf).shape[0] <= 2


def test_zero_gradient_grows_the_first_empty_cells():
    M, K, nnz, B = 10, 10, 30, 2
    rows, cols, vals = _canon(M, K, "rigl/zero", nnz)
    X = normal((B, K), "rigl/zero/X")
    dY = np.zeros((B, M), np.float32)
    n_drop = 9
    o = oracle.prune_regrow_grad(M, K, rows, cols, vals, n_drop, X, dY)
    pos, _ = _split(M, K, o)
    kept_pos, _, _, _ = _brute(M, K, rows, cols, vals, n_drop, X, dY)
    occupied = np.zeros(M * K, bool)
    occupied[kept_pos] = True
    first = np.nonzero(~occupied)[0][:n_drop]               # every score 0: smallest positions
    assert np.array_equal(np.setdiff1d(pos, kept_pos), first)


def test_just_dropped_cell_with_the_largest_gradient_is_regrown():
    # 3 x 3, entries at (0,0) value 0.1 and (2,2) value 5; dropping one removes (0,0);
    # the gradient is largest exactly at (0,0), so it is grown back (with value +0)
    M = K = 3
    rows = np.array([0, 2], np.int32); cols = np.array([0, 2], np.int32); vals = np.array([0.1, 5.0], np.float32)
    X = np.array([[10.0, 1.0, 1.0]], np.float32)
    dY = np.array([[10.0, 1.0, 1.0]], np.float32)            # G = dY^T X: G[0,0] = 100, others <= 10
    r, c, v = oracle.prune_regrow_grad(M, K, rows, cols, vals, 1, X, dY)
    assert r.tolist() == [0, 2] and c.tolist() == [0, 2]
    assert v[0] == 0.0 and np.signbit(v[0]) == False and v[1] == 5.0


def test_negative_gradient_counts_by_magnitude_and_orientation():
    # a non-square layer: G is [M, K] = dY^T X; the largest |G| is negative
    M, K = 2, 3
    rows = np.array([0], np.int32); cols = np.array([0], np.int32); vals = np.array([1.0], np.float32)
    X = np.array([[1.0, -7.0, 2.0]], np.float32)
    dY = np.array([[1.0, 3.0]], np.float32)                  # G[1,1] = -21, G[1,2] = 6, G[0,1] = -7
    r, c, v = oracle.prune_regrow_grad(M, K, rows, cols, vals, 1, X, dY)
    # the entry (|1|) is dropped; the best empty cell is (1, 1)
    assert r.tolist() == [1] and c.tolist() == [1] and v.tolist() == [0.0]


def test_grow_key_is_the_fp32_fma_chain_and_nan_counts_as_zero():
    M, K = 1, 2
    X = np.array([[1.0, np.nan], [2.0, 1.0]], np.float32)
    dY = np.array([[0.5], [-3.0]], np.float32)
    # cell (0, 0): 0.5 * 1 + (-3) * 2 = -5.5
    assert oracle.grow_key(M, K, X, dY, 0, 0) == int(np.array([5.5], np.float32).view(np.uint32)[0])
    assert oracle.grow_key(M, K, X, dY, 0, 1) == 0


def test_invariants_and_degenerate_counts():
    M, K, nnz, B = 20, 17, 100, 3
    rows, cols, vals = _canon(M, K, "rigl/inv", nnz)
    X = normal((B, K), "rigl/inv/X")
    dY = normal((B, M), "rigl/inv/dY")
    # n_drop = 0: unchanged
    r, c, v = oracle.prune_regrow_grad(M, K, rows, cols, vals, 0, X, dY)
    assert np.array_equal(r, rows) and np.array_equal(c, cols) and np.array_equal(v.view(np.uint32),
                                                                                  vals.view(np.uint32))
    for n_drop in (1, 30, nnz):
        r, c, v = oracle.prune_regrow_grad(M, K, rows, cols, vals, n_drop, X, dY)
        pos = r.astype(np.int64) * K + c
        assert pos.shape[0] == nnz                             # nnz preserved
        assert np.all(np.diff(pos) > 0)                        # canonical, distinct
        assert int((v == 0).sum()) >= n_drop                   # grown entries are +0
    with pytest.raises(oracle.OracleError):
        oracle.prune_regrow_grad(M, K, rows, cols, vals, nnz + 1, X, dY)

"""Pins of the oracle's row-local drop / regrow (every row keeps its number of
entries: the "Padded-CSR" post, section 8.3, says SparseLab's SET and RigL keep
per-row nnz fixed, so both the drop and the regrow happen inside each row).
CPU only.

Row i with n_i entries drops d_i = floor(n_i * num / den): its smallest |v|
(order key: IEEE bits of |v|, then slot).  It grows d_i cells of the same row
that are empty after its drop, value +0.0:
  mode 0 (random, SET): the row's candidate stream, SplitMix64 outputs
      (whose output mix is pinned to the published values in
      test_oracle_prune_pins.py) replayed here by an independent Python
      implementation of the stream's definition;
  mode 1 (gradient, RigL): the d_i empty cells of largest |dY^T X| in the row,
      ties by smaller column; with small integer data every product and sum is
      exact in fp32, so a dense numpy product decides exactly.
"""
import numpy as np
import pytest

import oracle
from snack_inputs import normal, random_layer, rng_for

GAMMA = 0x9E3779B97F4A7C15
MASK = 2**64 - 1


def _canon(M, K, key, nnz):
    r, c, v = random_layer(M, K, nnz, key)
    ref = oracle.canonicalize(M, K, r, c, v)
    return ref["rows"], ref["cols"], ref["vals"]


def _drop_by_row(M, rows, vals, num, den):
    """Brute force: per row, the slots of the d_i smallest (|v| bits, slot); returns a kept mask."""
    kept = np.ones(rows.shape[0], bool)
    mags = np.abs(vals.astype(np.float32)).view(np.uint32)
    for i in range(M):
        s = np.nonzero(rows == i)[0]
        d = s.shape[0] * num // den
        order = s[np.lexsort((s, mags[s]))]
        kept[order[:d]] = False
    return kept


def _mix(z):
    z = ((z ^ (z >> 30)) * 0xBF58476D1CE4E5B9) & MASK
    z = ((z ^ (z >> 27)) * 0x94D049BB133111EB) & MASK
    return z ^ (z >> 31)


def _row_stream(seed, epoch, row, K):
    """The random stream of one row, from its stated definition."""
    s = _mix((seed ^ _mix(((epoch << 32) + row) & MASK)) & MASK)
    t = 0
    while True:
        u = _mix((s + (t + 1) * GAMMA) & MASK)
        yield (u * K) >> 64
        t += 1


def _check_common(M, K, rows, cols, vals, num, den, out):
    r, c, v = out
    assert r.shape == rows.shape
    assert np.array_equal(np.bincount(r, minlength=M), np.bincount(rows, minlength=M))   # per-row nnz kept
    pos = r.astype(np.int64) * K + c
    assert np.all(np.diff(pos) > 0)                                                      # canonical, distinct
    kept = _drop_by_row(M, rows, vals, num, den)
    old_pos = rows.astype(np.int64) * K + cols
    kept_pos = old_pos[kept]
    assert np.all(np.isin(kept_pos, pos))
    is_kept = np.isin(pos, kept_pos)
    assert np.array_equal(v[is_kept].view(np.uint32), vals[kept].view(np.uint32))
    assert np.all(v[~is_kept].view(np.uint32) == 0)                                       # +0.0 exactly
    return pos[~is_kept], kept_pos


@pytest.mark.parametrize("M,K,nnz,num,den", [(7, 11, 30, 3, 10), (12, 40, 200, 1, 2), (9, 9, 81, 3, 10),
                                             (5, 64, 120, 1, 1), (30, 17, 100, 1, 3)])
def test_random_regrow_replays_the_row_streams(M, K, nnz, num, den):
    rows, cols, vals = _canon(M, K, f"rows/set/{M}x{K}", nnz)
    seed, epoch = 0x1234_5678_9ABC_DEF0, 3
    out = oracle.prune_regrow_rows(M, K, rows, cols, vals, num, den, 0, seed=seed, epoch=epoch)
    grown, kept_pos = _check_common(M, K, rows, cols, vals, num, den, out)
    kept_set = set(kept_pos.tolist())
    expect = []
    for i in range(M):
        d = int((rows == i).sum()) * num // den
        got = []
        for t, c in enumerate(_row_stream(seed, epoch, i, K)):
            if len(got) == d or t >= 64 * K + 4096:
                break
            p = i * K + c
            if p not in kept_set and p not in got:
                got.append(p)
        assert len(got) == d, "the stream always finds the empty cells of these rows"
        expect.extend(got)
    assert np.array_equal(np.sort(grown), np.sort(np.array(expect, np.int64)))
    assert oracle.row_candidate(seed, epoch, 2, 0, K) == next(_row_stream(seed, epoch, 2, K))


def test_random_regrow_is_uniform_over_the_rows_empty_cells():
    # one row of 64 columns with 8 entries, fully regrown over 4000 epochs: each
    # of the 64 columns should be chosen about 4000 * 8 / 64 = 500 times
    M, K = 1, 64
    rows = np.zeros(8, np.int32)
    cols = np.arange(0, 64, 8, dtype=np.int32)
    vals = np.arange(1, 9, dtype=np.float32)
    hits = np.zeros(K, np.int64)
    for e in range(4000):
        r, c, _ = oracle.prune_regrow_rows(M, K, rows, cols, vals, 1, 1, 0, seed=7, epoch=e)
        hits[c] += 1
    chi2 = float(((hits - 500.0) ** 2 / 500.0).sum())
    assert chi2 < 120.0          # 63 degrees of freedom: p < 1e-5 above this


@pytest.mark.parametrize("M,K,nnz,B,num,den", [(7, 11, 30, 3, 3, 10), (12, 5, 20, 1, 1, 2), (9, 9, 81, 2, 3, 10),
                                               (16, 13, 60, 4, 1, 1), (5, 40, 37, 6, 1, 10), (20, 30, 300, 2, 1, 3)])
def test_gradient_regrow_matches_dense_brute_force_exactly(M, K, nnz, B, num, den):
    rows, cols, vals = _canon(M, K, f"rows/rigl/{M}x{K}", nnz)
    g = rng_for(f"rows/rigl/data/{M}x{K}")
    X = g.integers(-3, 4, size=(B, K)).astype(np.float32)
    dY = g.integers(-3, 4, size=(B, M)).astype(np.float32)
    out = oracle.prune_regrow_rows(M, K, rows, cols, vals, num, den, 1, X=X, dY=dY)
    grown, kept_pos = _check_common(M, K, rows, cols, vals, num, den, out)
    G = np.abs(dY.astype(np.float64).T @ X.astype(np.float64))
    occupied = np.zeros(M * K, bool)
    occupied[kept_pos] = True
    expect = []
    for i in range(M):
        d = int((rows == i).sum()) * num // den
        cand = np.nonzero(~occupied[i * K:(i + 1) * K])[0]
        pick = cand[np.lexsort((cand, -G[i, cand]))][:d]     # larger |G| first, then smaller column
        expect.extend((i * K + pick).tolist())
    assert np.array_equal(np.sort(grown), np.sort(np.array(expect, np.int64)))


def test_gradient_regrow_random_data_dominates_within_the_row():
    M, K, nnz, B = 30, 60, 500, 8
    rows, cols, vals = _canon(M, K, "rows/rigl/rand", nnz)
    X = normal((B, K), "rows/rigl/rand/X")
    dY = normal((B, M), "rows/rigl/rand/dY")
    out = oracle.prune_regrow_rows(M, K, rows, cols, vals, 3, 10, 1, X=X, dY=dY)
    grown, kept_pos = _check_common(M, K, rows, cols, vals, 3, 10, out)
    G = np.abs(dY.astype(np.float64).T @ X.astype(np.float64))
    err = 1e-5 * (np.abs(dY.astype(np.float64)).T @ np.abs(X.astype(np.float64))).max()
    occupied = np.zeros(M * K, bool)
    occupied[kept_pos] = True
    occupied[grown] = True
    for i in range(M):
        gi = grown[grown // K == i] % K
        if gi.shape[0] == 0:
            continue
        rest = np.nonzero(~occupied[i * K:(i + 1) * K])[0]
        if rest.shape[0]:
            assert G[i, gi].min() >= G[i, rest].max() - 2 * err


def test_just_dropped_cell_is_regrown_when_its_gradient_is_largest():
    # row 0 holds (0,0)=0.1 and (0,2)=5; dropping half removes (0,0); its gradient is the row's largest
    M, K = 2, 3
    rows = np.array([0, 0, 1], np.int32); cols = np.array([0, 2, 1], np.int32)
    vals = np.array([0.1, 5.0, 2.0], np.float32)
    X = np.array([[10.0, 1.0, 1.0]], np.float32)
    dY = np.array([[10.0, 1.0]], np.float32)
    r, c, v = oracle.prune_regrow_rows(M, K, rows, cols, vals, 1, 2, 1, X=X, dY=dY)
    # row 1 (one entry) drops floor(1/2) = 0 entries
    assert r.tolist() == [0, 0, 1] and c.tolist() == [0, 2, 1]
    assert v[0] == 0.0 and not np.signbit(v[0]) and v[1] == 5.0 and v[2] == 2.0


def test_degenerate_fractions_and_rows():
    M, K, nnz = 25, 19, 160
    rows, cols, vals = _canon(M, K, "rows/degenerate", nnz)
    X = normal((3, K), "rows/degenerate/X")
    dY = normal((3, M), "rows/degenerate/dY")
    for mode in (0, 1):
        kw = dict(seed=11, epoch=4) if mode == 0 else dict(X=X, dY=dY)
        r, c, v = oracle.prune_regrow_rows(M, K, rows, cols, vals, 0, 1, mode, **kw)   # nothing moves
        assert np.array_equal(r, rows) and np.array_equal(c, cols)
        assert np.array_equal(v.view(np.uint32), vals.view(np.uint32))
        out = oracle.prune_regrow_rows(M, K, rows, cols, vals, 1, 1, mode, **kw)        # every entry moves
        _check_common(M, K, rows, cols, vals, 1, 1, out)
        assert np.all(out[2].view(np.uint32) == 0)
    # one column: every row's single cell is dropped and is the only empty cell, so it comes back as +0
    rows1 = np.array([0, 2, 3], np.int32); cols1 = np.zeros(3, np.int32); vals1 = np.array([1.0, -2.0, 3.0], np.float32)
    for mode in (0, 1):
        kw = dict(seed=1) if mode == 0 else dict(X=np.ones((1, 1), np.float32), dY=np.ones((1, 4), np.float32))
        r, c, v = oracle.prune_regrow_rows(4, 1, rows1, cols1, vals1, 1, 1, mode, **kw)
        assert r.tolist() == [0, 2, 3] and c.tolist() == [0, 0, 0] and v.tolist() == [0.0, 0.0, 0.0]
    with pytest.raises(oracle.OracleError):
        oracle.prune_regrow_rows(M, K, rows, cols, vals, 2, 1, 0)
    with pytest.raises(oracle.OracleError):
        oracle.prune_regrow_rows(M, K, rows, cols, vals, 1, 0, 0)

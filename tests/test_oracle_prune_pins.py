"""Pins of the oracle's drop/regrow (CPU only).

The drop rule (smallest |w| first, ties by canonical slot) and the grow rule
(uniform over the positions that are empty after the drop, nnz kept fixed)
follow the DST update of the "Padded-CSR" post, section 4.3, applied in place on
the triple as in the SNACK paper's Figure 1.  The pages name no random
generator: the candidate stream is SplitMix64, pinned here to its published
outputs; the rest is pinned by an independent set-based brute force on tiny
matrices, by invariants and by a chi-square uniformity test.
"""
import json
import os
import struct

import numpy as np
import pytest

import oracle
from snack_inputs import random_layer, rng_for
from tests.conftest import GOLDEN


def _canon(M, K, key, nnz, vals=None):
    rows, cols, v = random_layer(M, K, nnz, key)
    out = oracle.canonicalize(M, K, rows, cols, v if vals is None else vals)
    return out["rows"], out["cols"], out["vals"]


def test_splitmix64_published_outputs():
    g = json.load(open(os.path.join(GOLDEN, "splitmix64.json")))
    gamma = 0x9E3779B97F4A7C15
    for i, h in enumerate(g["outputs_hex"]):
        assert oracle.splitmix64_mix((gamma * (i + 1)) % 2**64) == int(h, 16)
        # candidate t of epoch 0 with seed 0 is output t; with N = 2^32 the
        # multiply-shift keeps the top 32 bits
        assert oracle.regrow_candidate(0, 0, i, 2**32) == int(h, 16) >> 32
        assert oracle.regrow_candidate(0, 0, i, 1) == 0


def test_candidate_epoch_and_seed_offsets():
    gamma = 0x9E3779B97F4A7C15
    N = 1000003
    for seed, epoch, t in ((5, 0, 0), (123456789, 3, 17), (2**63 + 11, 1, 2**20)):
        x = (seed + ((epoch << 40) + t + 1) * gamma) % 2**64
        u = oracle.splitmix64_mix(x)
        assert oracle.regrow_candidate(seed, epoch, t, N) == (u * N) >> 64


def _brute_prune_regrow(M, K, rows, cols, vals, n_drop, seed, epoch):
    """Independent set-based restatement: rank every entry by (|v| bits, slot),
    drop the first n_drop, grow from the candidate stream into a Python set."""
    def mag(v):
        return struct.unpack("<I", struct.pack("<f", abs(float(v))))[0]
    order = sorted(range(len(vals)), key=lambda k: (mag(vals[k]), k))
    drop = set(order[:n_drop])
    kept = {int(rows[k]) * K + int(cols[k]): np.float32(vals[k]) for k in range(len(vals)) if k not in drop}
    grown = {}
    t = 0
    while len(grown) < n_drop:
        p = oracle.regrow_candidate(seed, epoch, t, M * K)
        t += 1
        if p in kept or p in grown:
            continue
        grown[p] = np.float32(0.0)
    allp = dict(kept); allp.update(grown)
    keys = sorted(allp)
    return (np.array([p // K for p in keys], np.int32), np.array([p % K for p in keys], np.int32),
            np.array([allp[p] for p in keys], np.float32), t)


def test_tiny_enumeration_with_ties_and_signed_zero():
    M, K = 6, 5
    rows, cols, _ = _canon(M, K, "prune/tiny", 14)
    vals = np.array([0.5, -0.0, 0.25, 0.0, -0.25, 1.0, -0.5, 0.25, 2.0, -1.0, 0.125, np.nan, -0.125, 0.0],
                    np.float32)
    for n_drop in range(0, 15):
        for epoch in (0, 1, 7):
            got = oracle.prune_regrow(M, K, rows, cols, vals, n_drop, 99, epoch)
            ref = _brute_prune_regrow(M, K, rows, cols, vals, n_drop, 99, epoch)
            assert np.array_equal(got[0], ref[0]) and np.array_equal(got[1], ref[1])
            assert np.array_equal(got[2].view(np.uint32), ref[2].view(np.uint32))
            assert got[3] == ref[3]


def test_drop_order_examples():
    # 1 x 6 row: |v| = [0, 0, .25, .25, nan, 1]; -0 ties +0, ties go by slot, NaN is never dropped first
    rows = np.zeros(6, np.int32); cols = np.arange(6, dtype=np.int32)
    vals = np.array([-0.0, 0.0, 0.25, -0.25, np.nan, 1.0], np.float32)
    M, K = 1, 6
    # with a full row there is nowhere new to grow, so the grown set is exactly the dropped positions
    for n_drop, expect_zeroed in ((1, {0}), (2, {0, 1}), (3, {0, 1, 2}), (4, {0, 1, 2, 3}), (5, {0, 1, 2, 3, 5})):
        r, c, v, _ = oracle.prune_regrow(M, K, rows, cols, vals, n_drop, 1, 0)
        assert c.tolist() == list(range(6))
        changed = {i for i in range(6) if not (np.isnan(v[i]) and np.isnan(vals[i]))
                   and v[i].view(np.uint32) != vals[i].view(np.uint32)}
        # dropped-and-regrown positions hold +0.0; position 0 and 1 held +-0 already
        zeroed = {i for i in range(6) if v[i].view(np.uint32) == 0}
        assert expect_zeroed <= zeroed
        assert changed <= expect_zeroed


@pytest.mark.parametrize("M,K,nnz,frac", [(40, 30, 300, 0.3), (64, 64, 2048, 0.5), (17, 23, 391, 1.0),
                                          (50, 50, 1, 1.0), (10, 10, 100, 0.3)])
def test_invariants(M, K, nnz, frac):
    rows, cols, vals = _canon(M, K, f"prune/inv/{M}", nnz)
    n_drop = int(nnz * frac)
    r, c, v, used = oracle.prune_regrow(M, K, rows, cols, vals, n_drop, 7, 2)
    assert r.shape[0] == nnz                                   # nnz preserved
    p = r.astype(np.int64) * K + c
    assert np.all(np.diff(p) > 0)                              # canonical and distinct
    mags = np.abs(vals).view(np.uint32)
    order = np.lexsort((np.arange(nnz), mags))
    dropped = set((rows.astype(np.int64) * K + cols)[order[:n_drop]].tolist())
    keptpos = (rows.astype(np.int64) * K + cols)[order[n_drop:]]
    newpos = dict(zip(p.tolist(), v.view(np.uint32).tolist()))
    old = dict(zip((rows.astype(np.int64) * K + cols).tolist(), vals.view(np.uint32).tolist()))
    for q in keptpos.tolist():                                 # kept values bit-identical
        assert newpos[q] == old[q]
    grown = set(newpos) - set(keptpos.tolist())
    assert len(grown) == n_drop
    assert all(newpos[q] == 0 for q in grown)                  # regrown at +0.0
    assert used >= n_drop
    assert len(dropped) == n_drop


def test_regrow_is_uniform_chi_square():
    """Rows and columns of grown positions over many epochs are uniform."""
    M, K = 40, 50
    rows, cols, vals = _canon(M, K, "prune/chi", 200)
    n_drop = 60
    order = np.lexsort((np.arange(rows.shape[0]), np.abs(vals).view(np.uint32)))
    kept = order[n_drop:]
    keep = set((rows[kept].astype(np.int64) * K + cols[kept]).tolist())
    rh = np.zeros(M); ch = np.zeros(K)
    for e in range(150):
        r, c, v, _ = oracle.prune_regrow(M, K, rows, cols, vals, n_drop, 4242, e)
        for rr, cc in zip(r.tolist(), c.tolist()):
            if rr * K + cc not in keep:
                rh[rr] += 1; ch[cc] += 1
    assert rh.sum() == 150 * n_drop
    from scipy.stats import chisquare
    # grown positions are uniform over the cells left empty by the drop, so the
    # expected count of a row (column) is proportional to its empty cells
    occ = np.zeros((M, K), bool); occ[rows[kept], cols[kept]] = True
    er = (~occ).sum(1).astype(float); ec = (~occ).sum(0).astype(float)
    assert chisquare(rh, er / er.sum() * rh.sum()).pvalue > 1e-4
    assert chisquare(ch, ec / ec.sum() * ch.sum()).pvalue > 1e-4


def test_invalid_drop_counts():
    rows, cols, vals = _canon(5, 5, "prune/bad", 10)
    with pytest.raises(oracle.OracleError):
        oracle.prune_regrow(5, 5, rows, cols, vals, 11, 0, 0)
    with pytest.raises(oracle.OracleError):
        oracle.prune_regrow(5, 5, rows, cols, vals, -1, 0, 0)

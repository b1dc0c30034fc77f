"""Pins of the fp64 oracle to things other than itself (CPU only).

Each test states what fixes the expected value: a worked example printed on
the pages (tests/golden), a dense brute-force product, an identity of the
mathematics (adjointness, finite differences, linearity), or a special case
with a closed form.  They are chosen so that a dropped term, a wrong sign or
index, or a transposed operand in the oracle fails at least one of them.
"""
import json
import os

import numpy as np
import pytest

import oracle
from snack_inputs import random_layer, normal, rng_for
from tests.conftest import GOLDEN


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _dense(M, K, rows, cols, vals):
    W = np.zeros((M, K), np.float64)
    W[rows, cols] = vals
    return W


# --------------------------------------------------------------------------
# Worked examples printed on the pages
# --------------------------------------------------------------------------

def test_toy_4x6_sorted_coo_and_row_pointer():
    g = _golden("pcsr_toy_4x6.json")
    rows, cols, vals = map(np.array, (g["coo_rows"], g["coo_cols"], g["coo_values"]))
    shuffle = np.array([3, 0, 4, 2, 1])  # any arrival order must canonicalise the same way
    out = oracle.canonicalize(g["M"], g["K"], rows[shuffle], cols[shuffle], vals[shuffle])
    assert out["rows"].tolist() == g["coo_rows"]
    assert out["cols"].tolist() == g["csr_col_indices"]
    assert out["vals"].tolist() == g["csr_values"]
    assert out["row_ptr"].tolist() == g["row_start"] == g["csr_row_ptr"]
    assert np.array_equal(_dense(g["M"], g["K"], out["rows"], out["cols"], out["vals"]), np.array(g["dense"]))


def test_csr_insertion_example_is_a_canonical_resort():
    g = _golden("pcsr_insert.json")
    t = _golden("pcsr_toy_4x6.json")
    ins = g["insert"]
    rows = np.array(t["coo_rows"] + [ins["row"]])
    cols = np.array(t["coo_cols"] + [ins["col"]])
    vals = np.array(t["coo_values"] + [ins["value"]], np.float32)
    out = oracle.canonicalize(g["M"], g["K"], rows, cols, vals)
    assert out["vals"].tolist() == g["after_values"]
    assert out["cols"].tolist() == g["after_col_indices"]
    assert out["row_ptr"].tolist() == g["after_row_ptr"]


def test_table7_coo_csr_csc():
    g = _golden("snack_table7.json")
    out = oracle.canonicalize(g["M"], g["K"], g["coo_row"], g["coo_col"], g["coo_data"])
    assert out["vals"].tolist() == g["csr_data"]
    assert out["cols"].tolist() == g["csr_col"]
    assert out["row_ptr"].tolist() == g["csr_indptr"]
    # CSC = the canonical values gathered through perm
    assert out["vals"][out["perm"]].tolist() == g["csc_data"]
    assert out["rows_t"].tolist() == g["csc_row"]
    assert out["col_ptr"].tolist() == g["csc_indptr"]
    assert out["perm"].tolist() == [1, 2, 0]


def test_spmm_worked_example_in_linear_layout():
    g = _golden("pcsr_spmm_3x4.json")
    e = np.array(g["entries"])
    rows, cols, vals = e[:, 0].astype(np.int32), e[:, 1].astype(np.int32), e[:, 2].astype(np.float32)
    X = np.array(g["X_page"], np.float32).T.copy()     # [B=2, K=4]
    Y, A = oracle.forward(g["M"], g["K"], rows, cols, vals, X)
    assert np.array_equal(Y, np.array(g["Y_page"], np.float64).T)
    # every term is non-negative here, so the abs-sum equals the sum
    assert np.array_equal(A, Y)


# --------------------------------------------------------------------------
# Dense brute force (the Dense+Mask definition): tiny random shapes, including
# empty rows / columns, nnz = 0, and degenerate M or K of 1.
# --------------------------------------------------------------------------

SHAPES = [(1, 1, 1, 1), (1, 7, 3, 2), (7, 1, 4, 3), (6, 5, 0, 2), (9, 13, 20, 1), (16, 11, 60, 5),
          (33, 17, 100, 4), (5, 40, 190, 3)]


@pytest.mark.parametrize("M,K,nnz,B", SHAPES)
def test_forward_dx_dw_match_dense_masked_products(M, K, nnz, B):
    key = f"pin/brute/{M}x{K}x{nnz}"
    rows, cols, vals = random_layer(M, K, nnz, key)
    X = normal((B, K), key + "/X")
    dY = normal((B, M), key + "/dY")
    W = _dense(M, K, rows, cols, vals)
    Y, YA = oracle.forward(M, K, rows, cols, vals, X)
    np.testing.assert_allclose(Y, X.astype(np.float64) @ W.T, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(YA, np.abs(X.astype(np.float64)) @ np.abs(W).T, rtol=1e-12, atol=1e-12)
    dX, _ = oracle.backward_dx(M, K, rows, cols, vals, dY)
    np.testing.assert_allclose(dX, dY.astype(np.float64) @ W, rtol=1e-12, atol=1e-12)
    dW, _ = oracle.backward_dw(M, K, rows, cols, X, dY)
    full = dY.astype(np.float64).T @ X.astype(np.float64)          # [M, K] dense gradient
    np.testing.assert_allclose(dW, full[rows, cols], rtol=1e-12, atol=1e-12)
    # scattered back, the sparse gradient equals the masked dense one, exactly 0 off-support
    dWd = np.zeros((M, K))
    dWd[rows, cols] = dW
    support = _dense(M, K, rows, cols, np.ones(nnz)) != 0
    np.testing.assert_allclose(dWd, full * support, rtol=1e-12, atol=1e-12)
    assert np.all(dWd[~support] == 0)


def test_stored_zero_gets_a_gradient_and_contributes_nothing():
    rows = np.array([0, 1]); cols = np.array([1, 0]); vals = np.array([0.0, 2.0], np.float32)
    X = np.array([[3.0, 5.0]], np.float32); dY = np.array([[7.0, 11.0]], np.float32)
    Y, _ = oracle.forward(2, 2, rows, cols, vals, X)
    assert Y.tolist() == [[0.0, 6.0]]
    dW, _ = oracle.backward_dw(2, 2, rows, cols, X, dY)
    assert dW.tolist() == [7.0 * 5.0, 11.0 * 3.0]


# --------------------------------------------------------------------------
# Identities
# --------------------------------------------------------------------------

def test_adjoint_identity():
    M, K, B = 37, 29, 6
    rows, cols, vals = random_layer(M, K, 200, "pin/adjoint")
    X = normal((B, K), "pin/adjoint/X"); dY = normal((B, M), "pin/adjoint/dY")
    Y, _ = oracle.forward(M, K, rows, cols, vals, X)
    dX, _ = oracle.backward_dx(M, K, rows, cols, vals, dY)
    dW, _ = oracle.backward_dw(M, K, rows, cols, X, dY)
    a = np.sum(Y * dY.astype(np.float64))
    b = np.sum(dX * X.astype(np.float64))
    c = np.sum(dW * vals.astype(np.float64))
    assert abs(a - b) <= 1e-10 * (abs(a) + 1) and abs(a - c) <= 1e-10 * (abs(a) + 1)


def test_finite_differences_of_mse_loss():
    M, K, B = 12, 9, 3
    rows, cols, vals = random_layer(M, K, 40, "pin/fd")
    X = normal((B, K), "pin/fd/X"); T = normal((B, M), "pin/fd/T")

    def loss(v, x):
        Y, _ = oracle.forward(M, K, rows, cols, v, x)
        return np.mean((Y - T.astype(np.float64)) ** 2)

    Y, _ = oracle.forward(M, K, rows, cols, vals, X)
    dY = oracle.mse_grad(Y.astype(np.float32), T)
    np.testing.assert_allclose(dY, 2 * (Y.astype(np.float32).astype(np.float64) - T) / (B * M), rtol=1e-12)
    dY32 = dY.astype(np.float32)
    dW, _ = oracle.backward_dw(M, K, rows, cols, X, dY32)
    dX, _ = oracle.backward_dx(M, K, rows, cols, vals, dY32)
    h = 2.0 ** -10
    for k in (0, 7, 21, 39):
        vp, vm = vals.copy(), vals.copy()
        vp[k] += np.float32(h); vm[k] -= np.float32(h)
        fd = (loss(vp, X) - loss(vm, X)) / (float(vp[k]) - float(vm[k]))
        assert abs(fd - dW[k]) <= 2e-6 * (abs(fd) + 1e-3)
    for (b, c) in ((0, 0), (1, 4), (2, 8)):
        xp, xm = X.copy(), X.copy()
        xp[b, c] += np.float32(h); xm[b, c] -= np.float32(h)
        fd = (loss(vals, xp) - loss(vals, xm)) / (float(xp[b, c]) - float(xm[b, c]))
        assert abs(fd - dX[b, c]) <= 2e-6 * (abs(fd) + 1e-3)


# --------------------------------------------------------------------------
# Special cases with closed forms
# --------------------------------------------------------------------------

def test_identity_and_permutation_weights_copy_exactly():
    n, B = 50, 4
    X = normal((B, n), "pin/ident/X")
    eye = np.arange(n)
    Y, _ = oracle.forward(n, n, eye, eye, np.ones(n, np.float32), X)
    assert np.array_equal(Y, X.astype(np.float64))
    p = rng_for("pin/perm").permutation(n)
    Y, _ = oracle.forward(n, n, eye, p, np.ones(n, np.float32), X)
    assert np.array_equal(Y, X[:, p].astype(np.float64))
    dX, _ = oracle.backward_dx(n, n, eye, p, np.ones(n, np.float32), X)  # W^T is the inverse permutation
    inv = np.empty(n, int); inv[p] = eye
    assert np.array_equal(dX, X[:, inv].astype(np.float64))


def test_full_density_is_dense_gemm():
    M, K, B = 8, 6, 3
    pos = np.arange(M * K)
    rows, cols = pos // K, pos % K
    vals = normal(M * K, "pin/full/v")
    X = normal((B, K), "pin/full/X")
    Y, _ = oracle.forward(M, K, rows, cols, vals, X)
    np.testing.assert_allclose(Y, X.astype(np.float64) @ vals.astype(np.float64).reshape(M, K).T, rtol=1e-12)


def test_integer_data_exact():
    M, K, B = 30, 40, 5
    rng = rng_for("pin/int")
    rows, cols, _ = random_layer(M, K, 300, "pin/int")
    vals = rng.integers(-8, 9, 300).astype(np.float32)
    X = rng.integers(-8, 9, (B, K)).astype(np.float32)
    Y, _ = oracle.forward(M, K, rows, cols, vals, X)
    W = np.zeros((M, K), np.int64); W[rows, cols] = vals.astype(np.int64)
    assert np.array_equal(Y, (X.astype(np.int64) @ W.T).astype(np.float64))


def test_canonicalize_matches_lexsort_and_transposed_view():
    M, K = 23, 19
    rows, cols, vals = random_layer(M, K, 150, "pin/canon")
    out = oracle.canonicalize(M, K, rows, cols, vals)
    order = np.lexsort((cols, rows))
    assert np.array_equal(out["rows"], rows[order]) and np.array_equal(out["cols"], cols[order])
    assert np.array_equal(out["vals"], vals[order])
    torder = np.lexsort((out["rows"], out["cols"]))
    assert np.array_equal(out["perm"], torder)
    assert np.array_equal(out["rows_t"], out["rows"][torder])
    assert np.array_equal(out["row_ptr"], np.concatenate([[0], np.cumsum(np.bincount(rows, minlength=M))]))
    assert np.array_equal(out["col_ptr"], np.concatenate([[0], np.cumsum(np.bincount(cols, minlength=K))]))


def test_canonicalize_rejects_bad_input():
    with pytest.raises(oracle.OracleError) as e:
        oracle.canonicalize(3, 3, [0, 3], [0, 0], [1, 1])
    assert e.value.code == oracle.RANGE
    with pytest.raises(oracle.OracleError) as e:
        oracle.canonicalize(3, 3, [0, 1, 0], [2, 2, 2], [1, 1, 1])
    assert e.value.code == oracle.DUPLICATE
    with pytest.raises(oracle.OracleError) as e:
        oracle.canonicalize(3, 3, [0, -1], [0, 0], [1, 1])
    assert e.value.code == oracle.RANGE


# --------------------------------------------------------------------------
# Training-loop glue
# --------------------------------------------------------------------------

def test_gelu_closed_forms_and_derivative():
    x = np.linspace(-6, 6, 97).astype(np.float32)
    g = oracle.gelu_fwd(x)
    assert g[48] == 0.0                                   # gelu(0) = 0
    np.testing.assert_allclose(g - oracle.gelu_fwd(-x), x, rtol=0, atol=1e-15)  # gelu(x) - gelu(-x) = x
    assert abs(g[-1] - 6.0) < 1e-7 and abs(g[0]) < 1e-7
    # derivative by central differences of the forward
    h = 2.0 ** -12
    xs = np.array([-2.5, -0.75, 0.0, 0.3, 1.9], np.float32)
    d = oracle.gelu_bwd(xs, np.ones_like(xs))
    fd = (oracle.gelu_fwd(xs + np.float32(h)) - oracle.gelu_fwd(xs - np.float32(h))) / (2 * h)
    np.testing.assert_allclose(d, fd, rtol=1e-6, atol=1e-7)
    assert abs(d[2] - 0.5) < 1e-15                          # gelu'(0) = 1/2


def test_gelu_pinned_to_normal_table_values():
    # GELU(x) = x * Phi(x) with Phi the standard normal CDF, so its values at +-1
    # and its slope at 1 are fixed by the normal table: Phi(1) = 0.8413447460685429,
    # phi(1) = exp(-1/2) / sqrt(2 pi) = 0.24197072451914337.  A missing 1/sqrt(2)
    # inside erf (x * (1 + erf(x)) / 2 gives 0.9213503964748575 at 1) or the tanh
    # approximation (0.8411919906082768 at 1) fails these by far more than the
    # tolerance.
    phi1_cdf = 0.8413447460685429
    phi1_pdf = 0.24197072451914337
    x = np.array([1.0, -1.0, 2.0], np.float32)
    g = oracle.gelu_fwd(x)
    assert abs(g[0] - phi1_cdf) < 1e-15
    assert abs(g[1] - (-(1.0 - phi1_cdf))) < 1e-15              # Phi(-1) = 1 - Phi(1)
    assert abs(g[2] - 2.0 * 0.9772498680518208) < 1e-15         # Phi(2) from the table
    d = oracle.gelu_bwd(x, np.ones_like(x))
    assert abs(d[0] - (phi1_cdf + phi1_pdf)) < 1e-15            # Phi(1) + 1 * phi(1)
    assert abs(d[1] - ((1.0 - phi1_cdf) - phi1_pdf)) < 1e-15    # Phi(-1) + (-1) * phi(-1)
    # the chain rule: the incoming gradient scales the derivative
    d2 = oracle.gelu_bwd(x[:1], np.array([-3.0], np.float32))
    assert abs(d2[0] + 3.0 * (phi1_cdf + phi1_pdf)) < 1e-14


def test_sgd_closed_form():
    v = np.array([1.0, -2.0, 0.5], np.float32); g = np.array([10.0, 0.0, -4.0], np.float32)
    assert oracle.sgd(v, g, 0.25).tolist() == [1.0 - 2.5, -2.0, 0.5 + 1.0]

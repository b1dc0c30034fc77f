"""fp64 CPU oracle for the truly sparse COO layer -- TEST INFRASTRUCTURE ONLY.

Only the test-suite, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  The product library (``coo_spmm_amd``)
never imports, links or calls it, and the two share no code: the oracle is the
plain C file ``snack_oracle.c`` (loops in double) plus this ctypes wrapper.

What each function computes, and the passage it follows, is documented in
``snack_oracle.c``.  In short (W is [M, K], X is [B, K], dY is [B, M]):

* ``canonicalize``  -- sort by (row, col), row pointer, transposed index
  ("Padded-CSR" post, sections 3.2 and 7.2; SNACK paper, Table 7).
* ``forward``       -- Y = X W^T  (SNACK paper, Figure 1; Padded-CSR 6.1).
* ``backward_dx``   -- dX = dY W  (Padded-CSR 7.1).
* ``backward_dw``   -- dW on the support (Padded-CSR 7.1; SNACK Figure 1).
* ``prune_regrow``  -- SET-style drop of the smallest |w|, uniform regrow
  (Padded-CSR 4.3; SNACK Figure 1).  The candidate stream is SplitMix64:
  parity of the stream itself is pinned only to SplitMix64's published output
  and a uniformity test, since the pages name no generator.
* ``prune_regrow_rows`` -- row-local variants: every row keeps its nnz, drops
  its smallest |w| and regrows inside itself, at random or by gradient
  (Padded-CSR 8.3: SparseLab's SET and RigL keep per-row nnz fixed).
* ``round_bf16``    -- values rounded to bf16 for the inference forward with a
  narrower value stream (Padded-CSR 9.3).
* ``prune_regrow_grad`` -- the same drop, regrow at the empty cells of largest
  |dL/dW| for a batch (Padded-CSR 4.3: RigL grows "at high-gradient
  locations"; SNACK Tables 8-9).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "snack_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

OK, INVALID, RANGE, DUPLICATE, NOMEM = 0, 1, 2, 3, 4


def build(force: bool = False) -> str:
    """Compile the oracle with gcc (plain -O2, no fast-math)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


_lib = None


def _load():
    global _lib
    if _lib is None:
        build()
        lib = ctypes.CDLL(_LIB)
        P = ctypes.c_void_p
        i32, i64, u64, f64 = ctypes.c_int32, ctypes.c_int64, ctypes.c_uint64, ctypes.c_double
        lib.oracle_canonicalize.argtypes = [i32, i32, i64, P, P, P, P, P, P, P, P, P, P]
        lib.oracle_canonicalize.restype = ctypes.c_int
        lib.oracle_forward.argtypes = [i32, i32, i64, P, P, P, i32, P, P, P]
        lib.oracle_forward.restype = None
        lib.oracle_backward_dx.argtypes = [i32, i32, i64, P, P, P, i32, P, P, P]
        lib.oracle_backward_dx.restype = None
        lib.oracle_backward_dw.argtypes = [i32, i32, i64, P, P, i32, P, P, P, P]
        lib.oracle_backward_dw.restype = None
        lib.oracle_mse_grad.argtypes = [i64, P, P, P]
        lib.oracle_gelu_fwd.argtypes = [i64, P, P]
        lib.oracle_gelu_bwd.argtypes = [i64, P, P, P]
        lib.oracle_sgd.argtypes = [i64, P, P, f64, P]
        lib.oracle_splitmix64_mix.argtypes = [u64]
        lib.oracle_splitmix64_mix.restype = u64
        lib.oracle_regrow_candidate.argtypes = [u64, u64, u64, u64]
        lib.oracle_regrow_candidate.restype = u64
        lib.oracle_prune_regrow.argtypes = [i32, i32, i64, P, P, P, i64, u64, u64, P, P, P, P]
        lib.oracle_prune_regrow.restype = ctypes.c_int
        lib.oracle_row_candidate.argtypes = [u64, u64, i32, u64, i32]
        lib.oracle_row_candidate.restype = i32
        lib.oracle_prune_regrow_rows.argtypes = [i32, i32, i64, P, P, P, i64, i64, ctypes.c_int, u64, u64, i32, P, P,
                                                 P, P, P]
        lib.oracle_prune_regrow_rows.restype = ctypes.c_int
        lib.oracle_round_bf16.argtypes = [ctypes.c_float]
        lib.oracle_round_bf16.restype = ctypes.c_float
        lib.oracle_grow_key.argtypes = [i32, i32, i32, P, P, i32, i32]
        lib.oracle_grow_key.restype = ctypes.c_uint32
        lib.oracle_prune_regrow_grad.argtypes = [i32, i32, i64, P, P, P, i64, i32, P, P, P, P, P]
        lib.oracle_prune_regrow_grad.restype = ctypes.c_int
        _lib = lib
    return _lib


def _p(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _i32(a):
    return np.ascontiguousarray(a, dtype=np.int32)


def _f32(a):
    return np.ascontiguousarray(a, dtype=np.float32)


class OracleError(RuntimeError):
    def __init__(self, code):
        super().__init__({1: "invalid argument", 2: "index out of range", 3: "duplicate position",
                          4: "out of memory"}.get(code, str(code)))
        self.code = code


def canonicalize(M, K, rows, cols, vals):
    """Returns dict(rows, cols, vals, row_ptr, perm, rows_t, col_ptr); raises OracleError."""
    rows, cols, vals = _i32(rows), _i32(cols), _f32(vals)
    nnz = rows.shape[0]
    out = dict(rows=np.empty(nnz, np.int32), cols=np.empty(nnz, np.int32), vals=np.empty(nnz, np.float32),
               row_ptr=np.empty(M + 1, np.int32), perm=np.empty(nnz, np.int32),
               rows_t=np.empty(nnz, np.int32), col_ptr=np.empty(K + 1, np.int32))
    rc = _load().oracle_canonicalize(M, K, nnz, _p(rows), _p(cols), _p(vals), _p(out["rows"]), _p(out["cols"]),
                                     _p(out["vals"]), _p(out["row_ptr"]), _p(out["perm"]), _p(out["rows_t"]),
                                     _p(out["col_ptr"]))
    if rc != OK:
        raise OracleError(rc)
    return out


def forward(M, K, rows, cols, vals, X):
    """Y[b, i] = sum_k v_k X[b, c_k] over r_k = i, in fp64; returns (Y, abs_sum)."""
    rows, cols, vals, X = _i32(rows), _i32(cols), _f32(vals), _f32(X)
    B = X.shape[0]
    assert X.shape == (B, K)
    Y = np.empty((B, M), np.float64)
    A = np.empty((B, M), np.float64)
    _load().oracle_forward(M, K, rows.shape[0], _p(rows), _p(cols), _p(vals), B, _p(X), _p(Y), _p(A))
    return Y, A


def backward_dx(M, K, rows, cols, vals, dY):
    rows, cols, vals, dY = _i32(rows), _i32(cols), _f32(vals), _f32(dY)
    B = dY.shape[0]
    assert dY.shape == (B, M)
    dX = np.empty((B, K), np.float64)
    A = np.empty((B, K), np.float64)
    _load().oracle_backward_dx(M, K, rows.shape[0], _p(rows), _p(cols), _p(vals), B, _p(dY), _p(dX), _p(A))
    return dX, A


def backward_dw(M, K, rows, cols, X, dY):
    rows, cols, X, dY = _i32(rows), _i32(cols), _f32(X), _f32(dY)
    B = X.shape[0]
    assert X.shape == (B, K) and dY.shape == (B, M)
    nnz = rows.shape[0]
    dW = np.empty(nnz, np.float64)
    A = np.empty(nnz, np.float64)
    _load().oracle_backward_dw(M, K, nnz, _p(rows), _p(cols), B, _p(X), _p(dY), _p(dW), _p(A))
    return dW, A


def mse_grad(Y, T):
    Y, T = _f32(Y), _f32(T)
    out = np.empty(Y.shape, np.float64)
    _load().oracle_mse_grad(Y.size, _p(Y), _p(T), _p(out))
    return out


def gelu_fwd(X):
    X = _f32(X)
    out = np.empty(X.shape, np.float64)
    _load().oracle_gelu_fwd(X.size, _p(X), _p(out))
    return out


def gelu_bwd(X, dY):
    X, dY = _f32(X), _f32(dY)
    out = np.empty(X.shape, np.float64)
    _load().oracle_gelu_bwd(X.size, _p(X), _p(dY), _p(out))
    return out


def sgd(v, g, lr):
    v, g = _f32(v), _f32(g)
    out = np.empty(v.shape, np.float64)
    _load().oracle_sgd(v.size, _p(v), _p(g), float(lr), _p(out))
    return out


def splitmix64_mix(z):
    return int(_load().oracle_splitmix64_mix(ctypes.c_uint64(z & (2**64 - 1))))


def regrow_candidate(seed, epoch, t, N):
    return int(_load().oracle_regrow_candidate(seed & (2**64 - 1), epoch, t, N))


def prune_regrow(M, K, rows, cols, vals, n_drop, seed, epoch):
    """Canonical triple in, canonical triple out (nnz unchanged).  Returns (rows, cols, vals, candidates_used)."""
    rows, cols, vals = _i32(rows), _i32(cols), _f32(vals)
    nnz = rows.shape[0]
    o_r, o_c, o_v = np.empty(nnz, np.int32), np.empty(nnz, np.int32), np.empty(nnz, np.float32)
    used = ctypes.c_uint64(0)
    rc = _load().oracle_prune_regrow(M, K, nnz, _p(rows), _p(cols), _p(vals), int(n_drop), seed & (2**64 - 1),
                                     int(epoch), _p(o_r), _p(o_c), _p(o_v), ctypes.byref(used))
    if rc != OK:
        raise OracleError(rc)
    return o_r, o_c, o_v, int(used.value)


def grow_key(M, K, X, dY, r, c):
    """The regrow score key of cell (r, c): IEEE bits of |sum_b dY[b, r] X[b, c]| accumulated in fp32 with
    one fused multiply-add per batch row, in batch order (a NaN counts as 0)."""
    X, dY = _f32(X), _f32(dY)
    B = X.shape[0]
    assert X.shape == (B, K) and dY.shape == (B, M)
    return int(_load().oracle_grow_key(M, K, B, _p(X), _p(dY), int(r), int(c)))


def prune_regrow_grad(M, K, rows, cols, vals, n_drop, X, dY):
    """Drop the n_drop smallest |v| (as prune_regrow), grow n_drop empty cells with the largest gradient
    score for the batch (X [B, K], dY [B, M]); canonical triple in and out."""
    rows, cols, vals, X, dY = _i32(rows), _i32(cols), _f32(vals), _f32(X), _f32(dY)
    nnz = rows.shape[0]
    B = X.shape[0]
    assert X.shape == (B, K) and dY.shape == (B, M)
    o_r, o_c, o_v = np.empty(nnz, np.int32), np.empty(nnz, np.int32), np.empty(nnz, np.float32)
    rc = _load().oracle_prune_regrow_grad(M, K, nnz, _p(rows), _p(cols), _p(vals), int(n_drop), B, _p(X), _p(dY),
                                          _p(o_r), _p(o_c), _p(o_v))
    if rc != OK:
        raise OracleError(rc)
    return o_r, o_c, o_v


def row_candidate(seed, epoch, row, t, K):
    return int(_load().oracle_row_candidate(seed & (2**64 - 1), int(epoch), int(row), int(t), int(K)))


def prune_regrow_rows(M, K, rows, cols, vals, num, den, mode, seed=0, epoch=0, X=None, dY=None):
    """Row-local drop / regrow (each row keeps its nnz): canonical triple in and out.  mode 0: random regrow
    inside the row; mode 1: regrow at the row's empty cells of largest |dY^T X| for the batch (X, dY)."""
    rows, cols, vals = _i32(rows), _i32(cols), _f32(vals)
    nnz = rows.shape[0]
    B = 0
    if mode == 1:
        X, dY = _f32(X), _f32(dY)
        B = X.shape[0]
        assert X.shape == (B, K) and dY.shape == (B, M)
    o_r, o_c, o_v = np.empty(nnz, np.int32), np.empty(nnz, np.int32), np.empty(nnz, np.float32)
    rc = _load().oracle_prune_regrow_rows(M, K, nnz, _p(rows), _p(cols), _p(vals), int(num), int(den), int(mode),
                                          seed & (2**64 - 1), int(epoch), B, _p(X), _p(dY), _p(o_r), _p(o_c),
                                          _p(o_v))
    if rc != OK:
        raise OracleError(rc)
    return o_r, o_c, o_v


def round_bf16(v):
    """Each value rounded to bf16 (nearest, ties to even), returned as float32."""
    v = _f32(v)
    f = _load().oracle_round_bf16
    return np.array([f(float(x)) for x in v.reshape(-1)], np.float32).reshape(v.shape)


def tolerance_ok(got, ref, abs_sum, rel=1e-5, atol=1e-6):
    """Per-element acceptance |got - ref| <= rel * sum|terms| + atol."""
    got = np.asarray(got, np.float64)
    return np.abs(got - ref) <= rel * abs_sum + atol

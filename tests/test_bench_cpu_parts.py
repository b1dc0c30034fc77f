"""The all-cores CPU baseline splits the oracle's calls over threads; every
output must equal the one-call oracle bit for bit (CPU)."""
import numpy as np

import oracle
from bench import OracleParts
from snack_inputs import normal, random_layer


def test_oracle_parts_bit_identical_to_one_call():
    from concurrent.futures import ThreadPoolExecutor
    M, K, nnz = 97, 83, 2100
    rows, cols, vals = random_layer(M, K, nnz, "bench/parts")
    ref = oracle.canonicalize(M, K, rows, cols, vals)
    r, c, v = ref["rows"], ref["cols"], ref["vals"]
    for nt in (1, 3, 7):
        parts = OracleParts(M, K, r, c, nt)
        with ThreadPoolExecutor(nt) as pool:
            for B in (1, 5):
                X = normal((B, K), f"bench/parts/X/{B}")
                dY = normal((B, M), f"bench/parts/dY/{B}")
                assert np.array_equal(parts.forward(pool, r, c, v, X), oracle.forward(M, K, r, c, v, X)[0])
                assert np.array_equal(parts.backward_dx(pool, r, c, v, dY), oracle.backward_dx(M, K, r, c, v, dY)[0])
                dW = parts.backward_dw(pool, r, c, X, dY)
                assert np.array_equal(dW, oracle.backward_dw(M, K, r, c, X, dY)[0])
                g = dW.astype(np.float32)
                assert np.array_equal(parts.sgd(pool, v, g, 0.01), oracle.sgd(v, g, 0.01))

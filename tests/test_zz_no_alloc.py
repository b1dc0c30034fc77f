"""snack_forward_noalloc (the forward whose scratch is a static device array)
against snack_forward, through the C ABI: bit for bit on two calls in a row,
the second with a smaller batch, and no device memory allocated by the layer
for it.  Runs alone in a fresh process as well as after the other tests."""
import numpy as np
import pytest

from snack_inputs import normal, random_layer
from tests.gpu_util import say, lib, dev, host

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("M,K,nnz,batches", [
    (10000, 10000, 5_000_000, (64, 8, 1)),     # slice-tiled pass with partial sums, then a narrow plan
    (2000, 1500, 300_000, (130, 33, 2)),       # several 64-column tiles, then smaller plans
    (37, 53, 400, (17, 3)),                    # short keys: no partial sums
])
def test_forward_noalloc_matches_forward(M, K, nnz, batches):
    import torch
    L = lib()
    key = f"noalloc/{M}x{K}"
    rows, cols, vals = random_layer(M, K, nnz, key)
    layer = L.SnackLayer(M, K, dev(rows), dev(cols), dev(vals), max_batch=max(batches))
    try:
        before = layer.device_bytes()
        for B in batches:
            X = dev(normal((B, K), f"{key}/X/{B}"))
            Y0 = torch.full((B, M), 3.0, device="cuda")
            Y1 = torch.full((B, M), -3.0, device="cuda")
            say("noalloc forward", M, K, "B", B)
            L.snack_forward(layer.h, X, Y0)
            L.snack_forward_noalloc(layer.h, X, Y1)
            assert np.array_equal(host(Y0).view(np.uint32), host(Y1).view(np.uint32)), f"B={B}"
        assert layer.device_bytes() == before
    finally:
        layer.close()


def test_forward_noalloc_refuses_plans_beyond_its_scratch():
    import torch
    L = lib()
    M = K = 10000
    rows, cols, vals = random_layer(M, K, 5_000_000, "noalloc/limit")
    layer = L.SnackLayer(M, K, dev(rows), dev(cols), dev(vals), max_batch=65)
    try:
        B = 65   # two 64-column tiles: about 87 MB of partial sums and transposed input
        X = dev(normal((B, K), "noalloc/limit/X"))
        Y = torch.full((B, M), 5.0, device="cuda")
        say("noalloc limit B", B)
        with pytest.raises(L.SnackError) as e:
            L.snack_forward_noalloc(layer.h, X, Y)
        assert e.value.code == L.ERR_WORKSPACE
        assert bool((Y == 5.0).all())
        L.snack_forward(layer.h, X, Y)   # the layer's own workspace covers it
        Y1 = torch.empty(64, M, device="cuda")
        Y0 = torch.empty(64, M, device="cuda")
        L.snack_forward_noalloc(layer.h, X[:64].contiguous(), Y1)
        L.snack_forward(layer.h, X[:64].contiguous(), Y0)
        assert np.array_equal(host(Y0).view(np.uint32), host(Y1).view(np.uint32))
    finally:
        layer.close()

"""The inference forward (16-bit indices, fp32 or bf16 values, fused GELU) and
the chained forward through the C ABI: bit-identity with the training path's
calls where the arithmetic is the same, the oracle (with bf16-rounded values)
where it is not, and replay of a captured HIP graph."""
import numpy as np
import pytest

import oracle
from snack_inputs import normal, random_layer, weight_std
from tests.gpu_util import say, lib, dev, host, assert_close

pytestmark = pytest.mark.gpu


def _layer(M, K, sp, key):
    L = lib()
    nnz = M * K * (100 - sp) // 100
    r, c, v = random_layer(M, K, nnz, key, weight_std(K, sp))
    return L.SnackLayer(M, K, dev(r), dev(c), dev(v), seed=3)


def _u32(t):
    return host(t).view(np.uint32)


@pytest.mark.parametrize("M,K,sp", [(10000, 10000, 95), (5000, 5000, 99), (3000, 4000, 90), (97, 300, 80)])
def test_infer_fp32_equals_forward_and_gelu(M, K, sp):
    import torch
    L = lib()
    layer = _layer(M, K, sp, f"infer/{M}x{K}/{sp}")
    try:
        for B in (1, 2, 3, 4):
            X = dev(normal((B, K), f"infer/{M}x{K}/X/{B}"))
            say("infer fp32", M, K, sp, "B", B)
            Y0 = torch.empty(B, M, device="cuda"); Y1 = torch.empty(B, M, device="cuda")
            G0 = torch.empty(B, M, device="cuda"); G1 = torch.empty(B, M, device="cuda")
            L.snack_forward(layer.h, X, Y0)
            L.snack_forward_infer(layer.h, X, Y1)
            assert np.array_equal(_u32(Y0), _u32(Y1)), f"B={B}"
            L.snack_gelu_fwd(Y0, G0)
            L.snack_forward_infer(layer.h, X, G1, act=L.ACT_GELU)
            assert np.array_equal(_u32(G0), _u32(G1)), f"GELU B={B}"
    finally:
        layer.close()


@pytest.mark.parametrize("M,K,sp", [(10000, 10000, 95), (5000, 5000, 90), (97, 300, 80)])
def test_infer_bf16_values_against_oracle(M, K, sp):
    import torch
    L = lib()
    layer = _layer(M, K, sp, f"infer16/{M}x{K}/{sp}")
    try:
        r, c, v = (host(t) for t in layer.export())
        vb = oracle.round_bf16(v)
        for B in (1, 4):
            X = normal((B, K), f"infer16/{M}x{K}/X/{B}")
            say("infer bf16", M, K, sp, "B", B)
            Y = torch.empty(B, M, device="cuda")
            L.snack_forward_infer(layer.h, dev(X), Y, bf16_values=True)
            assert_close(f"bf16 Y B={B}", host(Y), *oracle.forward(M, K, r, c, vb, X))
        # a value change (an SGD step) remakes the bf16 copy before the next call
        dW = torch.from_numpy(normal((layer.nnz,), f"infer16/{M}x{K}/dW")).cuda()
        layer.sgd_step(dW, 0.5)
        v2 = host(layer.export()[2])
        X = normal((2, K), f"infer16/{M}x{K}/X2")
        Y = torch.empty(2, M, device="cuda")
        L.snack_forward_infer(layer.h, dev(X), Y, bf16_values=True)
        assert_close("bf16 Y after a step", host(Y), *oracle.forward(M, K, r, c, oracle.round_bf16(v2), X))
    finally:
        layer.close()


def test_infer_refuses_what_it_does_not_cover():
    import torch
    L = lib()
    layer = _layer(300, 400, 90, "infer/refuse")
    try:
        X = torch.zeros(5, 400, device="cuda"); Y = torch.full((5, 300), 7.0, device="cuda")
        with pytest.raises(L.SnackError) as e:
            L.snack_forward_infer(layer.h, X, Y)          # batch 5: not a 1-4 column tile
        assert e.value.code == L.ERR_UNSUPPORTED
        with pytest.raises(L.SnackError):
            L.snack_forward_infer(layer.h, X[:1].contiguous(), Y[:1].contiguous(), act=7)
        assert bool((Y == 7.0).all())
    finally:
        layer.close()


def test_chain_equals_calls_and_replays_in_a_graph():
    # a GAMLP-like stack at batch 1: four 5000 x 5000 layers at 95 %, GELU between
    import torch
    L = lib()
    layers = [_layer(5000, 5000, 95, f"chain/{i}") for i in range(4)]
    acts = [L.ACT_GELU, L.ACT_GELU, L.ACT_GELU, L.ACT_NONE]
    try:
        for bf16 in (False, True):
            X = dev(normal((1, 5000), "chain/X"))
            Ys = [torch.empty(1, 5000, device="cuda") for _ in layers]
            say("chain eager bf16", bf16)
            L.snack_forward_chain([l.h for l in layers], acts, X, Ys, bf16_values=bf16)
            ref = [torch.empty(1, 5000, device="cuda") for _ in layers]
            h = X
            for l, a, y in zip(layers, acts, ref):
                L.snack_forward_infer(l.h, h, y, act=a, bf16_values=bf16)
                h = y
            for a, b in zip(Ys, ref):
                assert np.array_equal(_u32(a), _u32(b))
            # captured once, replayed three times with eager work in between
            Xs = X.clone()
            Gs = [torch.empty(1, 5000, device="cuda") for _ in layers]
            s = torch.cuda.Stream()
            s.wait_stream(torch.cuda.current_stream())
            with torch.cuda.stream(s):
                L.snack_forward_chain([l.h for l in layers], acts, Xs, Gs, bf16_values=bf16)   # warm
            torch.cuda.current_stream().wait_stream(s)
            torch.cuda.synchronize()
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                L.snack_forward_chain([l.h for l in layers], acts, Xs, Gs, bf16_values=bf16)
            for rep in range(3):
                say("chain replay", rep, "bf16", bf16)
                Xn = normal((1, 5000), f"chain/X/{rep}")
                Xs.copy_(torch.from_numpy(Xn))
                g.replay()
                torch.cuda.synchronize()
                Ye = [torch.empty(1, 5000, device="cuda") for _ in layers]
                L.snack_forward_chain([l.h for l in layers], acts, dev(Xn), Ye, bf16_values=bf16)
                for a, b in zip(Gs, Ye):
                    assert np.array_equal(_u32(a), _u32(b)), f"replay {rep}"
            del g
    finally:
        for l in layers:
            l.close()

"""Pins of the oracle's bf16 rounding (values of the inference forward with a
narrower value stream, "Padded-CSR" post, section 9.3): against torch's own
float32 -> bfloat16 conversion (round to nearest even) and hand-checked
special cases.  CPU only."""
import numpy as np
import torch

import oracle
from snack_inputs import normal


def _torch_bf16(v):
    return torch.from_numpy(np.ascontiguousarray(v, np.float32)).to(torch.bfloat16).to(torch.float32).numpy()


def test_round_bf16_matches_torch_on_random_and_wide_ranges():
    v = np.concatenate([normal((4000,), "bf16/pin/a"),
                        normal((1000,), "bf16/pin/b") * np.float32(1e-38),   # subnormals of fp32 and bf16
                        normal((1000,), "bf16/pin/c") * np.float32(3e37)])
    got = oracle.round_bf16(v)
    assert np.array_equal(got.view(np.uint32), _torch_bf16(v).view(np.uint32))


def test_round_bf16_special_cases():
    one = np.float32(1.0)
    cases = {
        1.0: 1.0,
        1.0 + 2.0 ** -8: 1.0,                      # halfway, the even neighbour is 1
        1.0 + 3 * 2.0 ** -8: 1.0 + 2.0 ** -6,      # halfway, the even neighbour is 1 + 2^-6
        1.0 + 2.0 ** -8 + 2.0 ** -20: 1.0 + 2.0 ** -7,   # just past halfway
        -2.5: -2.5,
        2.0 ** -149: 0.0,                          # below half the smallest bf16 subnormal
        2.0 ** -133: 2.0 ** -133,                  # the smallest bf16 subnormal
    }
    for x, want in cases.items():
        assert oracle.round_bf16(np.array([x], np.float32))[0] == np.float32(want), x
    big = oracle.round_bf16(np.array([np.finfo(np.float32).max], np.float32))[0]
    assert np.isinf(big) and big > 0
    z = oracle.round_bf16(np.array([-0.0], np.float32))[0]
    assert z == 0.0 and np.signbit(z)
    assert np.isnan(oracle.round_bf16(np.array([np.nan], np.float32))[0])
    del one

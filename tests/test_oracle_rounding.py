"""Pins of the oracle's storage rounding: bf16 round-to-nearest-even against torch's own
float32 -> bfloat16 conversion (a library routine), plus hand-checked special values."""
import numpy as np
import pytest
import torch

from oracle import csa


def test_bf16_matches_torch_on_float32_values():
    rng = np.random.default_rng(7)
    x = np.concatenate([
        rng.standard_normal(200_000).astype(np.float32),
        (rng.standard_normal(20_000) * 1e-38).astype(np.float32),   # subnormal range
        (rng.standard_normal(20_000) * 1e30).astype(np.float32),
        np.array([3.3895314e38, -3.3895314e38, 1.0, -0.0, 0.0], np.float32),
    ])
    ref = torch.from_numpy(x).to(torch.bfloat16).to(torch.float64).numpy()
    got = csa.round_bf16(x.astype(np.float64))
    np.testing.assert_array_equal(got, ref)


@pytest.mark.parametrize("x,expected", [
    (1.0 + 2.0 ** -8, 1.0),                      # exact midpoint -> even (1.0)
    (1.0 + 3 * 2.0 ** -8, 1.0 + 2.0 ** -6),      # midpoint between odd and even -> even
    (1.0 + 2.0 ** -8 + 2.0 ** -30, 1.0 + 2.0 ** -7),  # just above the midpoint
    (-(1.0 + 2.0 ** -8), -1.0),
    (2.0 ** -133, 2.0 ** -133),                  # smallest bf16 subnormal
    (2.0 ** -134, 0.0),                          # half of it: tie -> even (0)
    (3.0 * 2.0 ** -134, 2.0 ** -132),            # 1.5 quanta -> 2 quanta (even)
    (2.0 ** 128, np.inf),
    ((2.0 - 2.0 ** -8) * 2.0 ** 127, np.inf),    # midpoint above the largest finite -> inf
    ((2.0 - 2.0 ** -7) * 2.0 ** 127, (2.0 - 2.0 ** -7) * 2.0 ** 127),
])
def test_bf16_special_values(x, expected):
    assert csa.round_bf16(np.array([x]))[0] == expected


def test_round_f32_is_ieee():
    x = np.array([1.0 + 2.0 ** -24, 1.0 + 3 * 2.0 ** -24, 0.1])
    assert csa.round_f32(x)[0] == 1.0
    assert csa.round_f32(x)[1] == 1.0 + 2.0 ** -22
    assert csa.round_f32(x)[2] == float(np.float32(0.1))

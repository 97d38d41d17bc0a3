"""Pins of the fusion oracle (oracle/fusion.py) against facts it does not
compute itself: bfloat16 rounding against torch's conversion and hand-made
ties, hand-computed RMSNorm rows, closed forms and invariants of RMSNorm,
PyTorch's float64 silu, and hand values of silu."""

import math

import numpy as np
import pytest
import torch

from oracle import fusion as F


def test_round_bf16_matches_torch_and_ties():
    rng = np.random.default_rng(0)
    x = rng.standard_normal(100000).astype(np.float32).astype(np.float64) * 10.0 ** rng.integers(-5, 5, 100000)
    want = torch.from_numpy(x.astype(np.float32)).to(torch.bfloat16).double().numpy()
    assert np.array_equal(F.round_bf16(x.astype(np.float32).astype(np.float64)), want)
    # exact ties: 1 + 2^-8 lies halfway between 1 and 1 + 2^-7 -> even (1);
    # 1 + 3 * 2^-8 -> 1 + 2^-6 (even); negative mirrors; exact values stay
    assert F.round_bf16(1 + 2 ** -8) == 1.0
    assert F.round_bf16(1 + 3 * 2 ** -8) == 1 + 2 ** -6
    assert F.round_bf16(-(1 + 2 ** -8)) == -1.0
    assert F.round_bf16(1 + 2 ** -8 + 2 ** -30) == 1 + 2 ** -7
    assert F.round_bf16(0.0) == 0.0 and F.round_bf16(3.0) == 3.0


def test_rmsnorm_hand_row():
    # h = [3, 4] (from x = [1, 4], r = [2, 0]): mean square 12.5
    h, y = F.add_rmsnorm([[1.0, 4.0]], [[2.0, 0.0]], [1.0, 2.0], 0.0)
    assert np.array_equal(h, [[3.0, 4.0]])
    rms = math.sqrt(12.5)
    assert np.allclose(y, [[3.0 / rms, 8.0 / rms]], rtol=0, atol=1e-15)


@pytest.mark.parametrize("seed", [1, 2])
def test_rmsnorm_invariants(seed):
    rng = np.random.default_rng(seed)
    T, D = 7, 64
    x = F.round_bf16(rng.standard_normal((T, D)))
    r = F.round_bf16(rng.standard_normal((T, D)))
    # unit weight, eps 0: every output row has mean square 1
    h, y = F.add_rmsnorm(x, r, np.ones(D), 0.0)
    assert np.allclose(np.mean(y * y, axis=1), 1.0, atol=1e-14)
    # scale invariance (power-of-two scale keeps the bf16 rounding exact)
    _, y2 = F.add_rmsnorm(4 * x, 4 * r, np.ones(D), 0.0)
    assert np.allclose(y2, y, atol=1e-14)
    # weight multiplies per column; eps shrinks every row's output
    w = rng.standard_normal(D)
    _, yw = F.add_rmsnorm(x, r, w, 0.0)
    assert np.allclose(yw, y * w, atol=1e-14)
    _, ye = F.add_rmsnorm(x, r, np.ones(D), 0.5)
    assert np.all(np.abs(ye) <= np.abs(y) + 1e-15)
    # h is the bf16 rounding of the exact sum
    assert np.array_equal(h, F.round_bf16(x + r))


def test_rmsnorm_constant_row():
    # a constant row c with eps: y = c / sqrt(c^2 + eps) (eps as a float32)
    eps = 1e-6
    _, y = F.add_rmsnorm(np.full((1, 8), 0.5), np.full((1, 8), 0.25), np.ones(8), eps)
    e = float(np.float32(eps))
    assert np.allclose(y, 0.75 / math.sqrt(0.5625 + e), rtol=0, atol=1e-15)


def test_swiglu_values():
    assert F.swiglu(0.0, 5.0) == 0.0
    assert abs(F.swiglu(1.0, 1.0) - 1.0 / (1.0 + math.exp(-1.0))) < 1e-16
    assert abs(F.swiglu(1.0, 1.0) - 0.7310585786300049) < 1e-15
    assert abs(F.swiglu(-1.0, 2.0) - (-2.0 * 0.2689414213699951)) < 1e-15
    assert abs(F.swiglu(30.0, 2.0) - 60.0) < 1e-10          # silu(g) -> g for large g
    assert abs(F.swiglu(-30.0, 2.0)) < 1e-11                 # -> 0 for very negative g
    rng = np.random.default_rng(3)
    g, u = rng.standard_normal((5, 40)) * 3, rng.standard_normal((5, 40))
    ref = (torch.nn.functional.silu(torch.from_numpy(g)) * torch.from_numpy(u)).numpy()
    assert np.allclose(F.swiglu(g, u), ref, atol=1e-15, rtol=0)

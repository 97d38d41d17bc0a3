"""Pins of the backward oracle (oracle/backward.py) against facts it does not
compute itself: the derivative of the pages' worked example worked out by
hand, central finite differences of the (separately pinned) forward oracle,
PyTorch autograd through scaled_dot_product_attention on float64 CPU
tensors, closed forms at scale 0, and two sums the softmax fixes.
test_bwd_mutants_are_caught plants plausible mistakes and shows each one
fails some pin."""

import math

import numpy as np
import pytest
import torch

from oracle import backward as OB
from oracle import exact as OA


def _rand(shape, seed, amp=1.0):
    return amp * np.random.default_rng(seed).standard_normal(shape)


def pin_worked_example_derivative():
    """Scores [0, 0, ln 3, ln 3] (q = e0, k_j = s_j e0, scale 1), values
    [0, 0, 1, 1]: o = 0.75 and weights [1, 1, 3, 3] / 8.  With do = 1:
    dv_j = p_j, ds_j = p_j (v_j - o), dq = sum_j ds_j k_j, dk_j = ds_j q."""
    d = 8
    s = np.array([0.0, 0.0, math.log(3.0), math.log(3.0)])
    vals = np.array([0.0, 0.0, 1.0, 1.0])
    q = np.zeros((1, 1, 4, d)); q[..., 0] = 1.0
    k = np.zeros((1, 1, 4, d)); k[0, 0, :, 0] = s
    v = np.zeros((1, 1, 4, d)); v[0, 0, :, 0] = vals
    do = np.zeros((1, 1, 4, d)); do[0, 0, 0, 0] = 1.0        # only row 0's output dim 0
    dq, dk, dv = OB.attention_bwd(q, k, v, do, 1.0, causal=False, workers=1)
    p = np.array([1, 1, 3, 3]) / 8.0
    ds = p * (vals - 0.75)                                   # [-3/32, -3/32, 3/32, 3/32]
    assert np.allclose(dv[0, 0, :, 0], p, atol=1e-15) and np.all(dv[0, 0, :, 1:] == 0)
    assert abs(dq[0, 0, 0, 0] - (ds * s).sum()) < 1e-15      # 3/16 * ln 3
    assert abs(dq[0, 0, 0, 0] - 3.0 / 16.0 * math.log(3.0)) < 1e-15
    assert np.all(dq[0, 0, 1:] == 0)
    assert np.allclose(dk[0, 0, :, 0], ds, atol=1e-15)


def _loss(q, k, v, do, scale, causal):
    o, _ = OA.attention(q, k, v, scale, causal, workers=1)
    return float((o * do).sum())


def pin_finite_differences(causal):
    """Central differences of the forward oracle at sampled entries."""
    B, Hq, Hkv, N, d = 1, 4, 2, 9, 6
    q, k, v = _rand((B, Hq, N, d), 1), _rand((B, Hkv, N, d), 2), _rand((B, Hkv, N, d), 3)
    do = _rand((B, Hq, N, d), 4)
    sc = 0.37
    dq, dk, dv = OB.attention_bwd(q, k, v, do, sc, causal, workers=1)
    rng = np.random.default_rng(5)
    h = 1e-6
    for name, x, g in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
        for _ in range(6):
            idx = tuple(int(rng.integers(0, n)) for n in x.shape)
            xp, xm = x.copy(), x.copy()
            xp[idx] += h
            xm[idx] -= h
            args = {"q": q, "k": k, "v": v}
            fp = _loss(*(xp if n == name else args[n] for n in "qkv"), do, sc, causal)
            fm = _loss(*(xm if n == name else args[n] for n in "qkv"), do, sc, causal)
            num = (fp - fm) / (2 * h)
            assert abs(num - g[idx]) < 1e-7, (name, idx, num, g[idx])


def pin_torch_autograd():
    """PyTorch autograd through SDPA on float64 CPU tensors (GQA, causal)."""
    B, Hq, Hkv, N, d = 2, 6, 2, 37, 16
    q, k, v = _rand((B, Hq, N, d), 10), _rand((B, Hkv, N, d), 11), _rand((B, Hkv, N, d), 12)
    do = _rand((B, Hq, N, d), 13)
    for causal in (False, True):
        sc = 1.0 / math.sqrt(d)
        tq, tk, tv = (torch.tensor(x, requires_grad=True) for x in (q, k, v))
        o = torch.nn.functional.scaled_dot_product_attention(
            tq, tk, tv, is_causal=causal, scale=float(np.float32(sc)), enable_gqa=True)
        o.backward(torch.tensor(do))
        dq, dk, dv = OB.attention_bwd(q, k, v, do, sc, causal, workers=2)
        assert np.allclose(dq, tq.grad.numpy(), atol=1e-12, rtol=0)
        assert np.allclose(dk, tk.grad.numpy(), atol=1e-12, rtol=0)
        assert np.allclose(dv, tv.grad.numpy(), atol=1e-12, rtol=0)


def pin_scale_zero(causal):
    """Uniform weights: dq = dk = 0, and dv_j = sum over rows i that see j of
    do_i / #keys(i)."""
    B, Hq, Hkv, N, d = 1, 2, 1, 11, 5
    q, k, v = _rand((B, Hq, N, d), 20), _rand((B, Hkv, N, d), 21), _rand((B, Hkv, N, d), 22)
    do = _rand((B, Hq, N, d), 23)
    dq, dk, dv = OB.attention_bwd(q, k, v, do, 0.0, causal, workers=1)
    assert np.all(dq == 0) and np.all(dk == 0)
    want = np.zeros((N, d))
    for h in range(Hq):
        for i in range(N):
            keys = range(i + 1) if causal else range(N)
            for j in keys:
                want[j] += do[0, h, i] / len(keys)
    assert np.allclose(dv[0, 0], want, atol=1e-14)


def pin_softmax_sums(causal):
    """Each weight row sums to 1 and each ds row to 0, so per kv head the dv
    rows sum to the sum of do over its query heads and the dk rows to 0."""
    B, Hq, Hkv, N, d = 2, 6, 3, 23, 8
    q, k, v = _rand((B, Hq, N, d), 30), _rand((B, Hkv, N, d), 31), _rand((B, Hkv, N, d), 32)
    do = _rand((B, Hq, N, d), 33)
    _, dk, dv = OB.attention_bwd(q, k, v, do, 0.6, causal, workers=2)
    G = Hq // Hkv
    for b in range(B):
        for g in range(Hkv):
            assert np.allclose(dk[b, g].sum(axis=0), 0.0, atol=1e-12)
            assert np.allclose(dv[b, g].sum(axis=0), do[b, g * G:(g + 1) * G].sum(axis=(0, 1)), atol=1e-12)


def pin_chunking_is_not_a_parameter():
    """Row chunks of any size give the same gradients."""
    B, Hq, Hkv, N, d = 1, 2, 1, 50, 4
    q, k, v = _rand((B, Hq, N, d), 40), _rand((B, Hkv, N, d), 41), _rand((B, Hkv, N, d), 42)
    do = _rand((B, Hq, N, d), 43)
    ref = OB.attention_bwd(q, k, v, do, 0.5, True, workers=1, chunk=N)
    for ch in (1, 7, 16):
        got = OB.attention_bwd(q, k, v, do, 0.5, True, workers=1, chunk=ch)
        for a, b in zip(got, ref):
            assert np.allclose(a, b, atol=1e-13)


ALL_PINS = [
    pin_worked_example_derivative, lambda: pin_finite_differences(False),
    lambda: pin_finite_differences(True), pin_torch_autograd,
    lambda: pin_scale_zero(False), lambda: pin_scale_zero(True),
    lambda: pin_softmax_sums(False), lambda: pin_softmax_sums(True),
    pin_chunking_is_not_a_parameter,
]


def test_worked_example_derivative():
    pin_worked_example_derivative()


@pytest.mark.parametrize("causal", [False, True])
def test_finite_differences(causal):
    pin_finite_differences(causal)


def test_torch_autograd():
    pin_torch_autograd()


@pytest.mark.parametrize("causal", [False, True])
def test_scale_zero(causal):
    pin_scale_zero(causal)


@pytest.mark.parametrize("causal", [False, True])
def test_softmax_sums(causal):
    pin_softmax_sums(causal)


def test_chunking_is_not_a_parameter():
    pin_chunking_is_not_a_parameter()


# ------------------------------------------------------ planted mistakes ----

def _mutant(no_D=False, dk_from_k=False, no_sigma_dq=False, dv_from_v=False, causal_strict=False):
    def head_bwd(q, k, v, do, sigma, causal, chunk):
        N = q.shape[0]
        dq, dk, dv = np.zeros_like(q), np.zeros_like(k), np.zeros_like(v)
        s = sigma * (q @ k.T)
        if causal:
            j, i = np.arange(N), np.arange(N)
            allowed = (j[None, :] < i[:, None]) if causal_strict else (j[None, :] <= i[:, None])
            allowed[:, 0] = True
            s = np.where(allowed, s, -np.inf)
        p = np.exp(s - s.max(axis=1, keepdims=True))
        p /= p.sum(axis=1, keepdims=True)
        dv += p.T @ (v if dv_from_v else do)
        dp = do @ v.T
        D = 0.0 if no_D else (p * dp).sum(axis=1, keepdims=True)
        ds = p * (dp - D)
        dq[:] = (1.0 if no_sigma_dq else sigma) * (ds @ k)
        dk += sigma * (ds.T @ (k if dk_from_k else q))
        return dq, dk, dv
    return head_bwd


@pytest.mark.parametrize("name,mutant", [
    ("D term dropped", _mutant(no_D=True)),
    ("dk from keys instead of queries", _mutant(dk_from_k=True)),
    ("scale missing from dq", _mutant(no_sigma_dq=True)),
    ("dv from values instead of do", _mutant(dv_from_v=True)),
    ("causal diagonal dropped", _mutant(causal_strict=True)),
])
def test_bwd_mutants_are_caught(monkeypatch, name, mutant):
    monkeypatch.setattr(OB, "_head_bwd", mutant)
    failed = 0
    for pin in ALL_PINS:
        try:
            pin()
        except (AssertionError, ValueError):
            failed += 1
    assert failed, f"no pin catches: {name}"


def test_unmutated_backward_passes_every_pin():
    for pin in ALL_PINS:
        pin()

"""GPU parity of attn_bwd against the float64 backward oracle: every element
of dq, dk and dv on ragged shapes (one row, tile edges, several tiles and a
ragged tail), causal and not, grouped and ungrouped heads, d = 64 and 128,
scales 0, negative and default, and the full causal GQA 8192-token workload;
plus determinism, the scale-0 closed form on the GPU, the fused key-side
pass against the two-pass one, and the autograd wrapper that joins
attn_fwd and attn_bwd.

Tolerance (derived in the design notes): every gradient element within
2e-2 * max(1, max |reference| of that tensor) - the bf16 output rounding is
2^-9 of the value, the bf16 weights and ds in the matrix products add a few
units of 2^-9 of the partial sums."""

import math

import numpy as np
import pytest
import torch

from exact_tiled_self_amd import attn_bwd, attn_fwd
from exact_tiled_self_amd.inputs import DENSE_CONFIGS, dense_inputs
from oracle import backward as OB
from tests.gpu_util import DEV, announce, f64

pytestmark = pytest.mark.gpu

REL = 2e-2


@pytest.fixture(autouse=True)
def _name_case(request):
    announce(request.node.nodeid)
    yield


def _dout(shape, seed):
    return torch.from_numpy(np.random.default_rng(seed).standard_normal(shape, dtype=np.float32)).to(
        torch.bfloat16)


def run(q, k, v, do, scale, causal):
    qd, kd, vd, dod = (t.to(DEV) for t in (q, k, v, do))
    o, lse = attn_fwd(qd, kd, vd, scale=scale, causal=causal)
    dq, dk, dv = attn_bwd(qd, kd, vd, o, lse, dod, scale=scale, causal=causal)
    torch.cuda.synchronize()
    return dq.cpu(), dk.cpu(), dv.cpu()


def check(q, k, v, do, scale, causal, name):
    announce(f"bwd {name} q={tuple(q.shape)} kv={tuple(k.shape)} causal={causal} scale={scale}")
    got = run(q, k, v, do, scale, causal)
    ref = OB.attention_bwd(f64(q), f64(k), f64(v), f64(do), scale, causal)
    errs = []
    for nm, g, r in zip(("dq", "dk", "dv"), got, ref):
        g = f64(g)
        assert np.isfinite(g).all(), f"{name}: {nm} not finite"
        e = float(np.abs(g - r).max())
        bound = REL * max(1.0, float(np.abs(r).max()))
        errs.append((nm, e, bound))
        assert e <= bound, f"{name}: {nm} max-abs {e} > {bound}"
    return errs


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("B,Hq,Hkv,N", [(1, 1, 1, 1), (1, 2, 2, 31), (1, 4, 2, 130), (2, 3, 3, 257),
                                        (1, 12, 2, 300), (1, 6, 1, 129)])
def test_shapes(d, causal, B, Hq, Hkv, N):
    q, k, v = dense_inputs(B=B, Hq=Hq, Hkv=Hkv, N=N, d=d, dtype="bf16", seed=N + d)
    do = _dout((B, Hq, N, d), N + d + 1)
    check(q, k, v, do, 1.0 / math.sqrt(d), causal, f"shape d{d}")


@pytest.mark.parametrize("scale", [0.0, -0.2, 0.9])
def test_scales(scale):
    q, k, v = dense_inputs(B=1, Hq=4, Hkv=2, N=200, d=128, dtype="bf16", seed=7)
    do = _dout((1, 4, 200, 128), 8)
    check(q, k, v, do, scale, True, f"scale {scale}")


def test_scale_zero_closed_form():
    """scale 0: dq = dk = 0 exactly; dv_j = sum over rows i >= j of do_i / (i + 1)."""
    q, k, v = dense_inputs(B=1, Hq=2, Hkv=1, N=70, d=64, dtype="bf16", seed=9)
    do = _dout((1, 2, 70, 64), 10)
    dq, dk, dv = run(q, k, v, do, 0.0, True)
    assert torch.all(dq == 0) and torch.all(dk == 0)
    w = 1.0 / np.arange(1, 71)
    want = np.zeros((70, 64))
    g = f64(do)[0]
    for h in range(2):
        for i in range(70):
            want[:i + 1] += g[h, i] * w[i]
    assert np.abs(f64(dv)[0, 0] - want).max() <= REL * max(1.0, np.abs(want).max())


def test_full_gqa_causal_t8192():
    cfg = DENSE_CONFIGS["gqa_causal_t8192"]
    q, k, v = dense_inputs(cfg)
    do = _dout((cfg.B, cfg.Hq, cfg.N, cfg.d), 100)
    check(q, k, v, do, cfg.scale, True, "gqa_causal_t8192")


def test_deterministic():
    q, k, v = dense_inputs(B=1, Hq=6, Hkv=2, N=777, d=128, dtype="bf16", seed=11)
    do = _dout((1, 6, 777, 128), 12)
    a = run(q, k, v, do, 0.0884, True)
    b = run(q, k, v, do, 0.0884, True)
    for x, y in zip(a, b):
        assert torch.equal(x.view(torch.int16), y.view(torch.int16))


@pytest.mark.parametrize("causal", [False, True])
def test_autograd_attention(causal):
    """attention() under torch autograd: its output is attn_fwd's and the
    gradients of a loss are attn_bwd's for that loss's upstream gradient, bit
    for bit, and the oracle's within the tolerance.  The loss reads o
    transposed, so the upstream gradient arrives as a non-contiguous view."""
    from exact_tiled_self_amd import attention
    B, Hq, Hkv, N, d = 1, 4, 2, 150, 64
    q, k, v = dense_inputs(B=B, Hq=Hq, Hkv=Hkv, N=N, d=d, dtype="bf16", seed=13)
    w = _dout((B, Hq, d, N), 14)          # weights of the loss on o^T
    qd, kd, vd = (t.to(DEV).requires_grad_() for t in (q, k, v))
    o = attention(qd, kd, vd, causal=causal)
    loss = (o.transpose(2, 3).float() * w.to(DEV).float()).sum()
    loss.backward()
    torch.cuda.synchronize()
    o_ref, lse = attn_fwd(qd.detach(), kd.detach(), vd.detach(), causal=causal)
    assert torch.equal(o.detach(), o_ref)
    do = w.transpose(2, 3).contiguous()   # d loss / d o, already bf16 values
    dq, dk, dv = attn_bwd(qd.detach(), kd.detach(), vd.detach(), o_ref, lse, do.to(DEV), causal=causal)
    torch.cuda.synchronize()
    for g, r in ((qd.grad, dq), (kd.grad, dk), (vd.grad, dv)):
        assert g.dtype == torch.bfloat16 and torch.equal(g.view(torch.int16), r.view(torch.int16))
    ref = OB.attention_bwd(f64(q), f64(k), f64(v), f64(do), 1.0 / math.sqrt(d), causal)
    for g, r in zip((qd.grad, kd.grad, vd.grad), ref):
        assert np.abs(f64(g.cpu()) - r).max() <= REL * max(1.0, float(np.abs(r).max()))


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("Hq,Hkv", [(4, 4), (6, 2)])
def test_fused_key_side_matches_two_passes(monkeypatch, d, causal, Hq, Hkv):
    """The key-side gradients in one pass (the default) and in two passes
    (dV, then dK; ATTN_BWD_TWO_PASS=1) take the same steps in the same
    order: dq, dk and dv agree bit for bit."""
    q, k, v = dense_inputs(B=1, Hq=Hq, Hkv=Hkv, N=333, d=d, dtype="bf16", seed=15 + d)
    do = _dout((1, Hq, 333, d), 16 + d)
    a = run(q, k, v, do, 1.0 / math.sqrt(d), causal)
    monkeypatch.setenv("ATTN_BWD_TWO_PASS", "1")
    b = run(q, k, v, do, 1.0 / math.sqrt(d), causal)
    for x, y in zip(a, b):
        assert torch.equal(x.view(torch.int16), y.view(torch.int16))

"""GPU parity of the fused residual-add + RMSNorm and SwiGLU activation
against the float64 oracle: the new residual bit for bit against the
oracle's bf16 rounding of the exact sum, the normalised output and the
activation within one bf16 unit in the last place of the reference
(|err| <= 2^-7 |ref| + 1e-6: the result is rounded once from fp32, and an
fp32 value within 2^-24 of a rounding midpoint may round either way), every supported row-width class (one to sixteen 16-byte chunks per
lane, ragged widths), in-place residual update, merged and separate gate/up
layouts with ragged widths, tiny and very large gate values, and the
decoder-layer shapes the bench times."""

import numpy as np
import pytest
import torch

from exact_tiled_self_amd import attn_add_rmsnorm, attn_swiglu
from oracle import fusion as F
from tests.gpu_util import DEV, announce, f64

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _name_case(request):
    announce(request.node.nodeid)
    yield


def bf(x):
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16)


def close(got, ref, name):
    g = f64(got)
    assert np.isfinite(g).all(), name
    err = np.abs(g - ref)
    bound = 2.0 ** -7 * np.abs(ref) + 1e-6
    worst = float((err / bound).max())
    assert worst <= 1.0, f"{name}: error {worst:.3f} x the bound (max abs {err.max():.3g})"


@pytest.mark.parametrize("T,D", [(1, 8), (5, 512), (7, 520), (33, 1536), (3, 4096), (2, 8192), (64, 2048)])
def test_add_rmsnorm(T, D):
    rng = np.random.default_rng(T * D)
    x, r = bf(rng.standard_normal((T, D))), bf(rng.standard_normal((T, D)) * 2)
    w = bf(1 + 0.1 * rng.standard_normal(D))
    out, rout = attn_add_rmsnorm(x.to(DEV), r.to(DEV), w.to(DEV), 1e-6)
    torch.cuda.synchronize()
    h, y = F.add_rmsnorm(f64(x), f64(r), f64(w), 1e-6)
    assert np.array_equal(f64(rout.cpu()), h)
    close(out.cpu(), y, f"rms {T}x{D}")


def test_add_rmsnorm_in_place_and_eps():
    rng = np.random.default_rng(5)
    x, r = bf(rng.standard_normal((40, 1536))), bf(rng.standard_normal((40, 1536)))
    w = bf(rng.standard_normal(1536))
    rd = r.to(DEV)
    out, rout = attn_add_rmsnorm(x.to(DEV), rd, w.to(DEV), 0.25, residual_out=rd)
    torch.cuda.synchronize()
    assert rout.data_ptr() == rd.data_ptr()
    h, y = F.add_rmsnorm(f64(x), f64(r), f64(w), 0.25)
    assert np.array_equal(f64(rd.cpu()), h)
    close(out.cpu(), y, "in place")


def test_add_rmsnorm_decoder_shape():
    """T = 8192 tokens of a 1536-wide residual stream."""
    rng = np.random.default_rng(6)
    x, r = bf(rng.standard_normal((8192, 1536))), bf(rng.standard_normal((8192, 1536)))
    w = bf(1 + 0.1 * rng.standard_normal(1536))
    out, rout = attn_add_rmsnorm(x.to(DEV), r.to(DEV), w.to(DEV), 1e-6)
    torch.cuda.synchronize()
    h, y = F.add_rmsnorm(f64(x), f64(r), f64(w), 1e-6)
    assert np.array_equal(f64(rout.cpu()), h)
    close(out.cpu(), y, "decoder shape")


@pytest.mark.parametrize("T,Fw", [(1, 8), (3, 24), (17, 1000), (64, 8960)])
@pytest.mark.parametrize("merged", [False, True])
def test_swiglu(T, Fw, merged):
    rng = np.random.default_rng(T + Fw)
    g = rng.standard_normal((T, Fw)) * 3
    g[0, 0], g[-1, -1] = 60.0, -60.0              # silu saturates both ways
    u = rng.standard_normal((T, Fw))
    gb, ub = bf(g), bf(u)
    if merged:
        gu = torch.cat([gb, ub], dim=1).contiguous().to(DEV)
        out = attn_swiglu(gu)
    else:
        out = attn_swiglu(gb.to(DEV), ub.to(DEV))
    torch.cuda.synchronize()
    close(out.cpu(), F.swiglu(f64(gb), f64(ub)), f"swiglu {T}x{Fw} merged={merged}")


def test_swiglu_decoder_shape():
    """T = 8192 tokens, intermediate width 8960, merged gate/up projection."""
    rng = np.random.default_rng(7)
    gu = bf(rng.standard_normal((8192, 2 * 8960)) * 2)
    out = attn_swiglu(gu.to(DEV))
    torch.cuda.synchronize()
    ref = F.swiglu(f64(gu[:, :8960]), f64(gu[:, 8960:]))
    close(out.cpu(), ref, "decoder shape")

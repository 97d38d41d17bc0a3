"""GPU parity of attn_fwd against the float64 oracle (element by element at
small sizes, sampled rows at the full workload sizes), plus the probes whose
answer is fixed in closed form, exact selection of masked / grouped
positions, guard regions, determinism and host-forced error paths."""

import math
import os

import numpy as np
import pytest
import torch

from exact_tiled_self_amd import AttnError, attn_fwd
from exact_tiled_self_amd.inputs import DENSE_CONFIGS, dense_inputs
from oracle import exact as OA
from tests.gpu_util import (DEV, LSE_TOL, O_TOL, announce, check_config_full, check_dense_full,
                            f64, max_abs, run_fwd)

pytestmark = pytest.mark.gpu

DT = {"bf16": torch.bfloat16, "f32": torch.float32}


@pytest.fixture(autouse=True)
def _name_case(request):
    announce(request.node.nodeid)
    yield


# ------------------------------------------------------------ sweeps ----

SWEEP_N = [1, 2, 15, 16, 17, 63, 64, 65, 127, 128, 129, 196, 577]


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("N", SWEEP_N)
def test_sweep_sizes(dtype, d, causal, N):
    q, k, v = dense_inputs(B=1, Hq=2, Hkv=1, N=N, d=d, dtype=dtype, seed=1000 + N)
    check_dense_full(q, k, v, 1.0 / math.sqrt(d), causal, f"N={N}")


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("B,Hq,Hkv,N", [(32, 8, 8, 1), (32, 8, 2, 15), (16, 16, 16, 16), (32, 8, 1, 17),
                                        (64, 4, 4, 31), (32, 8, 4, 33), (32, 8, 8, 100), (64, 12, 12, 196),
                                        (32, 8, 2, 207), (16, 16, 4, 208)])
def test_short_sequences_whole_head_kernel(B, Hq, Hkv, N, causal):
    """d = 64, N <= 208 over at least 256 heads: one workgroup per head with
    the head's whole K and V staged in LDS (the batched ViT shape).  Every
    element against the oracle, ragged N around the 16- and 32-key edges,
    grouped and shared kv heads."""
    q, k, v = dense_inputs(B=B, Hq=Hq, Hkv=Hkv, N=N, d=64, dtype="bf16", seed=600 + N + Hq)
    check_dense_full(q, k, v, 0.125, causal, f"short B{B}H{Hq}/{Hkv}N{N}")


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("B,Hq,Hkv,N,d,causal", [
    (2, 6, 2, 300, 128, True), (2, 6, 3, 260, 64, False), (3, 4, 4, 129, 64, True),
    (1, 8, 1, 520, 128, False), (1, 12, 2, 700, 128, True),
])
def test_gqa_batches(dtype, B, Hq, Hkv, N, d, causal):
    q, k, v = dense_inputs(B=B, Hq=Hq, Hkv=Hkv, N=N, d=d, dtype=dtype, seed=7 * N + Hq)
    check_dense_full(q, k, v, 1.0 / math.sqrt(d), causal, f"B{B}H{Hq}/{Hkv}N{N}")


def fp32_o_tol(scale: float, d: int) -> float:
    """The fp32 bound on o at any scale.  The stated 1e-5 is for the
    workloads' scale 1/sqrt(d).  The kernel's fp32 dot product carries a
    rounding error that the softmax sees multiplied by the scale, so at fixed
    inputs the error of o grows in proportion to |scale|; the bound follows
    it beyond 1/sqrt(d).  Measured on N(0,1) inputs (N = 150, both masks):
    max error / (1e-5 |scale| sqrt(d)) stays between 0.05 and 0.1 for scales
    -0.3 .. 2.5 and d = 64, 128, and is 0.03-0.05 of the bound at 1/sqrt(d)."""
    return O_TOL[torch.float32] * max(1.0, abs(scale) * math.sqrt(d))


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("scale", [-0.3, 0.0, 1.0, 2.5])
def test_unusual_scales(dtype, d, scale):
    """Scales far from 1/sqrt(d).  bf16: the fixed 2e-2; fp32: the bound of
    fp32_o_tol; lse: the fixed 1e-4 for both dtypes (measured <= 2.1e-5 up to
    scale 2.5)."""
    q, k, v = dense_inputs(B=1, Hq=2, Hkv=2, N=150, d=d, dtype=dtype, seed=31)
    tol = O_TOL[DT[dtype]] if dtype == "bf16" else fp32_o_tol(scale, d)
    for causal in (False, True):
        o, lse = run_fwd(q, k, v, scale, causal)
        ro, rl = OA.attention(f64(q), f64(k), f64(v), scale, causal)
        assert max_abs(f64(o), ro) <= tol
        assert max_abs(lse.double().numpy(), rl) <= LSE_TOL


# ------------------------------------------------- the pages' example ----

@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("d", [64, 128])
def test_worked_example(dtype, d):
    """Scores 0, 0, ln3, ln3 with values 0, 0, 1, 1 give 0.75 (not the 0.5 of
    averaging two blocks).  In bf16 every input is exact: k in {0, 1} and the
    scale is float32(ln 3)."""
    dt = DT[dtype]
    q = torch.zeros(1, 1, 4, d); q[..., 0] = 1.0
    k = torch.zeros(1, 1, 4, d); k[0, 0, :, 0] = torch.tensor([0.0, 0.0, 1.0, 1.0])
    v = torch.zeros(1, 1, 4, d); v[0, 0, :, 0] = torch.tensor([0.0, 0.0, 1.0, 1.0])
    o, lse = run_fwd(q.to(dt), k.to(dt), v.to(dt), math.log(3.0), False)
    o = o.double()
    if dt == torch.bfloat16:
        assert torch.all(o[0, 0, :, 0] == 0.75)
    else:
        assert torch.all((o[0, 0, :, 0] - 0.75).abs() <= 1e-7)
    assert torch.all(o[0, 0, :, 1:] == 0.0)
    assert torch.all((lse[0, 0].double() - math.log(2 + 2 * math.exp(float(np.float32(math.log(3.0)))))).abs() < 1e-6)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("reverse", [False, True])
def test_worked_example_across_tiles(dtype, reverse):
    """The same two pairs of keys placed in different key tiles (positions 0,1
    and 64,65), every other key with score about -30000 (weight exactly 0):
    the rescale between tiles must still give 0.75."""
    dt = DT[dtype]
    N, d = 256, 128
    gen = torch.Generator().manual_seed(5)
    q = torch.zeros(1, 1, N, d); q[..., 0] = 1.0
    k = torch.zeros(1, 1, N, d); k[0, 0, :, 0] = -27307.0
    v = torch.randn(1, 1, N, d, generator=gen)
    lo, hi = ((64, 65), (0, 1)) if reverse else ((0, 1), (64, 65))
    for j in lo:
        k[0, 0, j, 0] = 0.0; v[0, 0, j, 0] = 0.0
    for j in hi:
        k[0, 0, j, 0] = 1.0; v[0, 0, j, 0] = 1.0
    o, _ = run_fwd(q.to(dt), k.to(dt), v.to(dt), math.log(3.0), False)
    col = o[0, 0, :, 0].double()
    assert torch.all((col - 0.75).abs() <= (0.0 if dt == torch.bfloat16 else 1e-7))


# ------------------------------------------------------ closed forms ----

@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_uniform_scores(dtype, d, causal):
    """scale 0: o_i is the mean of the allowed values (a prefix mean when
    causal) and lse_i = ln(#allowed)."""
    N = 200
    q, k, v = dense_inputs(B=1, Hq=2, Hkv=1, N=N, d=d, dtype=dtype, seed=3)
    o, lse = run_fwd(q, k, v, 0.0, causal)
    vv = f64(v)[0, 0]
    if causal:
        expect = np.cumsum(vv, axis=0) / np.arange(1, N + 1)[:, None]
        el = np.log(np.arange(1, N + 1))
    else:
        expect = np.broadcast_to(vv.mean(axis=0), (N, d))
        el = np.full(N, math.log(N))
    for h in range(2):
        assert max_abs(f64(o)[0, h], expect) <= O_TOL[DT[dtype]]
        assert max_abs(lse[0, h].double().numpy(), el) <= LSE_TOL


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_constant_values(dtype):
    """Constant V gives that constant, whatever the scores: to one bf16 ulp
    for bf16 (the weights enter the PV product rounded to bf16 while l sums
    them in fp32, a relative difference of at most 2^-9 before the output's
    own rounding) and to 1e-6 for fp32."""
    N, d = 333, 128
    q, k, _ = dense_inputs(B=1, Hq=2, Hkv=1, N=N, d=d, dtype=dtype, seed=4, amp=3.0)
    c = torch.linspace(-2.0, 2.0, d).to(DT[dtype])
    v = c.expand(1, 1, N, d).contiguous()
    cd = c.double()
    ulp = torch.where(cd == 0, torch.zeros_like(cd), torch.exp2(torch.floor(torch.log2(cd.abs())) - 7))
    for causal in (False, True):
        o, _ = run_fwd(q, k, v, 0.3, causal)
        err = (o.double() - cd).abs()
        if dtype == "bf16":
            assert torch.all(err <= ulp), err.max().item()
        else:
            assert err.max().item() <= 1e-6


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_identity_values(dtype, d, causal):
    """V = I (N = d) turns o into the probability matrix: rows sum to 1, it
    matches the oracle, and the causal upper triangle is exactly zero."""
    N = d
    q, k, _ = dense_inputs(B=1, Hq=1, Hkv=1, N=N, d=d, dtype=dtype, seed=8)
    v = torch.eye(N).reshape(1, 1, N, N).to(DT[dtype])
    o, _ = run_fwd(q, k, v, 1.0 / math.sqrt(d), causal)
    P = f64(o)[0, 0]
    ro, _ = OA.attention(f64(q), f64(k), f64(v), 1.0 / math.sqrt(d), causal)
    assert max_abs(P, ro[0, 0]) <= O_TOL[DT[dtype]]
    assert np.allclose(P.sum(axis=1), 1.0, atol=O_TOL[DT[dtype]] * 4)
    if causal:
        assert np.all(P[np.triu_indices(N, 1)] == 0.0)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_future_spike_is_masked(dtype):
    """Causal: each row's largest score sits at the masked key j = i + 1; a
    leak through the mask would move o by O(1)."""
    N, d = 256, 64
    c = 4.0
    q = torch.zeros(1, 1, N, d)
    k = torch.zeros(1, 1, N, d)
    for i in range(N):
        q[0, 0, i, (i + 1) % d] = c
        k[0, 0, i, i % d] = c
    v = torch.randn(1, 1, N, d, generator=torch.Generator().manual_seed(11))
    dt = DT[dtype]
    check_dense_full(q.to(dt), k.to(dt), v.to(dt), 1.0, True, "future-spike")


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_gqa_head_mapping(dtype):
    """V of kv head g is the constant g + 1: query head h must give exactly
    h // (Hq / Hkv) + 1.  Also GQA equals MHA with repeated K/V, bit for bit."""
    B, Hq, Hkv, N, d = 2, 12, 3, 150, 128
    q, k, _ = dense_inputs(B=B, Hq=Hq, Hkv=Hkv, N=N, d=d, dtype=dtype, seed=21)
    v = torch.empty(B, Hkv, N, d)
    for g in range(Hkv):
        v[:, g] = g + 1.0
    v = v.to(DT[dtype])
    for causal in (False, True):
        o, _ = run_fwd(q, k, v, 0.088, causal)
        for h in range(Hq):
            want = float(h // (Hq // Hkv) + 1)
            # bf16 output rounds to the constant exactly; fp32 keeps the
            # rounding of u / l (both sums in fp32, different association)
            tol = 0.0 if dtype == "bf16" else 2e-6 * want
            assert (o[:, h].double() - want).abs().max().item() <= tol
    q, k, v = dense_inputs(B=B, Hq=Hq, Hkv=Hkv, N=N, d=d, dtype=dtype, seed=22)
    G = Hq // Hkv
    o1, l1 = run_fwd(q, k, v, 0.088, True)
    o2, l2 = run_fwd(q, k.repeat_interleave(G, 1), v.repeat_interleave(G, 1), 0.088, True)
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


# ----------------------------------------------- guards & determinism ----

@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("causal", [False, True])
def test_guard_regions(dtype, causal):
    """Inputs sit inside NaN-filled buffers and outputs inside canary-filled
    buffers: no read may leave the inputs, no write may leave the outputs."""
    B, Hq, Hkv, N, d = 1, 4, 2, 197, 128
    dt = DT[dtype]
    q, k, v = dense_inputs(B=B, Hq=Hq, Hkv=Hkv, N=N, d=d, dtype=dtype, seed=41)
    pad = 4096

    def guarded(t, fill):
        buf = torch.full((t.numel() + 2 * pad,), fill, dtype=t.dtype, device=DEV)
        view = buf[pad:pad + t.numel()].view(t.shape)
        view.copy_(t.to(DEV))
        return buf, view

    _, qd = guarded(q, float("nan"))
    _, kd = guarded(k, float("nan"))
    _, vd = guarded(v, float("nan"))
    obuf, od = guarded(torch.zeros_like(q), 1234.0)
    lbuf = torch.full((B * Hq * N + 2 * pad,), -77.0, dtype=torch.float32, device=DEV)
    ld = lbuf[pad:pad + B * Hq * N].view(B, Hq, N)
    attn_fwd(qd, kd, vd, scale=1.0 / math.sqrt(d), causal=causal, o=od, lse=ld)
    torch.cuda.synchronize()
    ro, rl = OA.attention(f64(q), f64(k), f64(v), 1.0 / math.sqrt(d), causal)
    assert max_abs(f64(od), ro) <= O_TOL[dt]
    assert max_abs(ld.cpu().double().numpy(), rl) <= LSE_TOL
    ob = obuf.cpu()
    assert torch.all(ob[:pad] == 1234.0) and torch.all(ob[-pad:] == 1234.0)
    lb = lbuf.cpu()
    assert torch.all(lb[:pad] == -77.0) and torch.all(lb[-pad:] == -77.0)


@pytest.mark.parametrize("B,Hq,Hkv,N", [(1, 12, 2, 1000), (2, 4, 4, 333), (1, 2, 1, 64)])
def test_pipelined_matches_plain(monkeypatch, B, Hq, Hkv, N):
    """Causal d = 128 runs a software-pipelined kernel; it must give exactly
    the plain kernel's o and lse (same products in the same order, only
    scheduled differently)."""
    q, k, v = dense_inputs(B=B, Hq=Hq, Hkv=Hkv, N=N, d=128, dtype="bf16", seed=40 + N)
    o1, l1 = run_fwd(q, k, v, 1.0 / math.sqrt(128), True)
    monkeypatch.setenv("ATTN_PREFILL_PLAIN", "1")
    o2, l2 = run_fwd(q, k, v, 1.0 / math.sqrt(128), True)
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))
    assert torch.equal(l1.view(torch.int32), l2.view(torch.int32))
    ro, rl = OA.attention(f64(q), f64(k), f64(v), 1.0 / math.sqrt(128), True)
    assert max_abs(f64(o1), ro) <= O_TOL[torch.bfloat16]


# (B, Hq, Hkv, N) by placement: kv heads a multiple of 8 (each XCD its own kv
# heads), 8 a multiple of the kv heads (each kv head on 8 / n_kv XCDs; with
# and without padding workgroups), and neither (plain heaviest-first order).
XCD_CASES = [(8, 2, 1, 300), (1, 16, 16, 200), (2, 8, 8, 129), (1, 12, 2, 1000), (1, 6, 1, 300),
             (1, 12, 4, 333), (1, 6, 3, 200), (3, 2, 1, 400)]


@pytest.mark.parametrize("B,Hq,Hkv,N", XCD_CASES)
def test_causal_xcd_placement(monkeypatch, B, Hq, Hkv, N):
    """The causal d = 128 units are placed on the XCDs by kv head; every
    (head, q tile) must still be computed exactly once, against its own kv
    head: the result must equal, bit for bit, the launch in plain
    heaviest-first order (ATTN_PREFILL_XCD=0), and match the oracle."""
    q, k, v = dense_inputs(B=B, Hq=Hq, Hkv=Hkv, N=N, d=128, dtype="bf16", seed=300 + N + Hq)
    scale = 1.0 / math.sqrt(128)
    o1, l1 = run_fwd(q, k, v, scale, True)
    monkeypatch.setenv("ATTN_PREFILL_XCD", "0")
    o2, l2 = run_fwd(q, k, v, scale, True)
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))
    assert torch.equal(l1.view(torch.int32), l2.view(torch.int32))
    ro, rl = OA.attention(f64(q), f64(k), f64(v), scale, True)
    assert max_abs(f64(o1), ro) <= O_TOL[torch.bfloat16]
    assert max_abs(l1.double().numpy(), rl) <= LSE_TOL


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("B,Hq,Hkv,N", [(1, 12, 2, 1000), (2, 4, 4, 333), (1, 2, 1, 31), (8, 2, 1, 300)])
def test_second_tile_config(monkeypatch, d, causal, B, Hq, Hkv, N):
    """Block-size invariance on the GPU: the key tiles may have any size
    ("FlashAttention" notes: changing the block size changes no result).
    The default launch (64-key tiles at d = 128, 32-key tiles at d = 64) and
    the plain kernel forced to the other tile size (ATTN_PREFILL_BN)
    partition the keys differently, so the running maximum is raised at
    different points; both must match the oracle and each other within the
    tolerance, and each must be deterministic."""
    q, k, v = dense_inputs(B=B, Hq=Hq, Hkv=Hkv, N=N, d=d, dtype="bf16", seed=500 + N + d)
    scale = 1.0 / math.sqrt(d)
    o1, l1 = run_fwd(q, k, v, scale, causal)
    monkeypatch.setenv("ATTN_PREFILL_BN", "32" if d == 128 else "64")
    o2, l2 = run_fwd(q, k, v, scale, causal)
    o3, l3 = run_fwd(q, k, v, scale, causal)
    assert torch.equal(o2.view(torch.int16), o3.view(torch.int16)) and torch.equal(l2, l3)
    ro, rl = OA.attention(f64(q), f64(k), f64(v), scale, causal)
    for o, lse in ((o1, l1), (o2, l2)):
        assert max_abs(f64(o), ro) <= O_TOL[torch.bfloat16]
        assert max_abs(lse.double().numpy(), rl) <= LSE_TOL
    assert max_abs(f64(o1), f64(o2)) <= O_TOL[torch.bfloat16]
    assert max_abs(l1.double().numpy(), l2.double().numpy()) <= LSE_TOL


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("B,Hq,Hkv,N", [(1, 12, 12, 196), (2, 4, 2, 333), (1, 2, 1, 17), (3, 2, 2, 100)])
def test_fp32_row_partitions(monkeypatch, causal, B, Hq, Hkv, N):
    """The fp32 d = 64 path on 16-row query blocks (default) and on 32-row
    blocks (ATTN_F32_ROWS=32): another partition of the rows and of the
    merged key blocks; both against the oracle at the fp32 bound, each
    deterministic."""
    q, k, v = dense_inputs(B=B, Hq=Hq, Hkv=Hkv, N=N, d=64, dtype="f32", seed=700 + N)
    scale = 0.125
    o1, l1 = run_fwd(q, k, v, scale, causal)
    o1b, l1b = run_fwd(q, k, v, scale, causal)
    monkeypatch.setenv("ATTN_F32_ROWS", "32")
    o2, l2 = run_fwd(q, k, v, scale, causal)
    assert torch.equal(o1, o1b) and torch.equal(l1, l1b)
    ro, rl = OA.attention(f64(q), f64(k), f64(v), scale, causal)
    for o, lse in ((o1, l1), (o2, l2)):
        assert max_abs(f64(o), ro) <= O_TOL[torch.float32]
        assert max_abs(lse.double().numpy(), rl) <= LSE_TOL


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("B,Hq,Hkv,N", [(8, 2, 1, 300), (4, 6, 2, 129), (2, 8, 8, 64), (1, 16, 8, 200)])
def test_xcd_runs_cover_every_tile(d, B, Hq, Hkv, N):
    """Non-causal launches with a multiple of 8 kv heads (over the batch) map
    the q tiles that share a kv head to one XCD in a run; every (head, q tile)
    must still be computed once, against its own kv head."""
    q, k, v = dense_inputs(B=B, Hq=Hq, Hkv=Hkv, N=N, d=d, dtype="bf16", seed=90 + N + Hq)
    o, lse = run_fwd(q, k, v, 1.0 / math.sqrt(d), False)
    ro, rl = OA.attention(f64(q), f64(k), f64(v), 1.0 / math.sqrt(d), False)
    assert max_abs(f64(o), ro) <= O_TOL[torch.bfloat16]
    assert max_abs(lse.double().numpy(), rl) <= LSE_TOL


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("spike", [4, 84])
def test_row_max_spans_both_lane_halves(d, causal, spike):
    """The row maximum must cover all keys of a tile.  In the transposed score
    layout the keys at positions 4..7 (mod 8) of each block sit in the upper
    32 lanes; put the only large score there, far enough above the rest that a
    maximum taken over the lower lanes alone would overflow 2^(c (s - m))
    (here c s ~ 277), and the output must still be that key's value row."""
    N = 200
    g = torch.Generator().manual_seed(spike + d)
    q = torch.zeros(1, 1, N, d)
    k = torch.zeros(1, 1, N, d)
    q[..., 0] = 8.0
    k[0, 0, spike, 0] = 16.0
    v = torch.randn(1, 1, N, d, generator=g)
    q, k, v = (t.to(torch.bfloat16) for t in (q, k, v))
    o, lse = run_fwd(q, k, v, 1.5, causal)
    assert torch.isfinite(o.float()).all() and torch.isfinite(lse).all()
    ro, rl = OA.attention(f64(q), f64(k), f64(v), 1.5, causal)
    assert max_abs(f64(o), ro) <= O_TOL[torch.bfloat16]
    assert max_abs(lse.double().numpy(), rl) <= LSE_TOL


def test_no_lse_output():
    q, k, v = dense_inputs(B=1, Hq=2, Hkv=1, N=100, d=64, dtype="bf16", seed=2)
    o1, _ = run_fwd(q, k, v, 0.125, True, want_lse=False)
    o2, _ = run_fwd(q, k, v, 0.125, True)
    assert torch.equal(o1, o2)


def test_determinism():
    cfg = DENSE_CONFIGS["gqa_causal_t8192"]
    q, k, v = (t.to(DEV) for t in dense_inputs(cfg))
    outs = []
    for _ in range(3):
        o, lse = attn_fwd(q, k, v, scale=cfg.scale, causal=True)
        torch.cuda.synchronize()
        outs.append((o.cpu(), lse.cpu()))
    for o, lse in outs[1:]:
        assert torch.equal(o, outs[0][0]) and torch.equal(lse, outs[0][1])


def test_forced_foreign_arch_is_rejected(monkeypatch):
    """The architecture check, forced from the host: nothing is launched and
    the output keeps its contents."""
    q, k, v = (t.to(DEV) for t in dense_inputs(B=1, Hq=2, Hkv=1, N=64, d=64, dtype="bf16"))
    o = torch.full_like(q, 5.0)
    monkeypatch.setenv("ATTN_FORCE_ARCH", "gfx942")
    with pytest.raises(AttnError) as ei:
        attn_fwd(q, k, v, o=o, causal=False)
    assert ei.value.status == 2
    torch.cuda.synchronize()
    assert torch.all(o == 5.0)


# ------------------------------------------------- workload configs ----

def test_config_vit_fp32_full():
    cfg = DENSE_CONFIGS["vit_b16_fp32"]
    check_dense_full(*dense_inputs(cfg), cfg.scale, cfg.causal, cfg.name)


@pytest.mark.parametrize("name", ["vit_b16_bf16", "vit_b16_bf16_n577", "gqa_causal_t8192",
                                  "mha_causal_t32768"])
def test_config_full(name):
    """Every output element of each full-size workload (64 images of 196 or
    577 tokens; the 8192-token GQA and 32768-token MHA causal prefills)
    against the oracle."""
    cfg = DENSE_CONFIGS[name]
    check_config_full(*dense_inputs(cfg), cfg.scale, cfg.causal, cfg.name)


def test_long_prefill_allocates_nothing():
    """T = 32768, 16 heads: with o and lse passed in, the call leaves torch's
    peak allocation and the device's free memory where they were (the fp32
    score matrix the tiles avoid would be 16 * 32768^2 * 4 B = 68.7 GB)."""
    from exact_tiled_self_amd import attn_fwd
    cfg = DENSE_CONFIGS["mha_causal_t32768"]
    q, k, v = (t.to(DEV) for t in dense_inputs(cfg))
    o = torch.empty_like(q)
    lse = torch.empty(q.shape[:3], dtype=torch.float32, device=DEV)
    torch.cuda.synchronize()
    torch.cuda.reset_peak_memory_stats()
    peak0 = torch.cuda.max_memory_allocated()
    free0 = torch.cuda.mem_get_info()[0]
    attn_fwd(q, k, v, scale=cfg.scale, causal=True, o=o, lse=lse)
    torch.cuda.synchronize()
    assert torch.cuda.max_memory_allocated() == peak0
    assert abs(torch.cuda.mem_get_info()[0] - free0) < (64 << 20)
    assert torch.isfinite(o[0, :, -1].float()).all()


def staircase_inputs(N, d, step, seed):
    """One head whose scores climb by `step` (natural-log units at scale 1)
    from one 32-key block to the next and are equal inside a block, so that
    every lane's part of a row sum of weights exceeds 2^7 while the running
    maximum rises by less or more than 2^8 in weight from tile to tile."""
    g = torch.Generator().manual_seed(seed)
    q = torch.zeros(1, 1, N, d)
    k = torch.zeros(1, 1, N, d)
    q[..., 0] = 1.0
    k[0, 0, :, 0] = step * (torch.arange(N) // 32).float()
    v = torch.randn(1, 1, N, d, generator=g)
    return tuple(t.to(torch.bfloat16) for t in (q, k, v))


@pytest.mark.parametrize("d,bn", [(64, "32"), (64, "64"), (128, "32"), (128, "64")])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("step", [4.5, 7.0, -3.0])
def test_rescale_quick_test_fallback(monkeypatch, d, bn, causal, step):
    """The tile step first takes a tile's weights against the running maximum
    and forms the tile maximum only when a row-sum part exceeds 2^7; these
    inputs make that happen on every tile (steps of 4.5 and 7 in natural
    units: growths of 6.5 and 10 in base 2, below and above the lazy
    threshold of 8), or never after the first (falling scores), on both tile
    sizes of the plain kernel; every element against the oracle."""
    monkeypatch.setenv("ATTN_PREFILL_BN", bn)
    q, k, v = staircase_inputs(300, d, step, seed=int(10 * step) + d)
    o, lse = run_fwd(q, k, v, 1.0, causal)
    assert torch.isfinite(o.float()).all() and torch.isfinite(lse).all()
    ro, rl = OA.attention(f64(q), f64(k), f64(v), 1.0, causal)
    assert max_abs(f64(o), ro) <= O_TOL[torch.bfloat16]
    assert max_abs(lse.double().numpy(), rl) <= LSE_TOL

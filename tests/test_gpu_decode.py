"""GPU parity of attn_paged_decode against the float64 oracle: the full
64-sequence workload, ragged lengths, NaN poison in every slot that must not
be read, a spike key located through the block table, an identity table
against dense attention, empty contexts, bad device-resident lengths and
table entries, many sequences, more than 16 query heads per kv head, the
wave count forced down (long pieces, several pieces per wave, wide merges)
and determinism."""

import math
import os

import numpy as np
import pytest
import torch

from exact_tiled_self_amd import attn_fwd, attn_paged_decode
from exact_tiled_self_amd.inputs import PAGED_CONFIG, PagedConfig, paged_inputs
from oracle import exact as OA
from tests.gpu_util import DEV, LSE_TOL, O_TOL, announce, f64, max_abs

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _name_case(request):
    announce(request.node.nodeid)
    yield


def _dev(p):
    return {k: (v.to(DEV) if isinstance(v, torch.Tensor) else v) for k, v in p.items()}


def run_decode(p, scale, **kw):
    d = _dev(p)
    o, lse = attn_paged_decode(d["q"], d["k_cache"], d["v_cache"], d["block_table"],
                               d["ctx_lens"], d["block_size"], scale, **kw)
    torch.cuda.synchronize()
    return o.cpu(), lse.cpu()


def oracle_decode(p, scale):
    return OA.paged_decode(f64(p["q"]), f64(p["k_cache"]), f64(p["v_cache"]),
                           p["block_table"].numpy(), p["ctx_lens"].numpy(), p["block_size"], scale)


def check(p, scale, name):
    announce(f"decode {name} S={p['q'].shape[0]} nb={p['num_blocks']}")
    o, lse = run_decode(p, scale)
    ro, rl = oracle_decode(p, scale)
    ctx = p["ctx_lens"].numpy()
    live = ctx > 0
    assert torch.isfinite(o.float()).all(), name
    eo = max_abs(f64(o)[live], ro[live])
    el = max_abs(lse.double().numpy()[live], rl[live])
    assert eo <= O_TOL[torch.bfloat16], f"{name}: o max-abs {eo}"
    assert el <= LSE_TOL, f"{name}: lse max-abs {el}"
    if (~live).any():
        assert torch.all(o[torch.from_numpy(~live)] == 0)
        assert torch.all(torch.isneginf(lse[torch.from_numpy(~live)]))
    return eo, el


def small_cfg(Hq=12, Hkv=2, d=128):
    return PagedConfig("small", S=1, Hq=Hq, Hkv=Hkv, d=d, block_size=16, ctx_lo=1, ctx_hi=1,
                       max_blocks=1, dtype="bf16", seed=0)


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("Hq,Hkv", [(12, 2), (8, 8), (16, 1), (6, 3)])
def test_ragged_lengths_with_poison(d, Hq, Hkv):
    ctx = [1, 2, 15, 16, 17, 63, 64, 65, 255, 256, 257, 511, 700, 1024, 2000]
    p = paged_inputs(small_cfg(Hq, Hkv, d), S=len(ctx), ctx_lens=ctx, poison=True,
                     extra_blocks=5, max_blocks=130, seed=d + Hq)
    check(p, 1.0 / math.sqrt(d), f"ragged d{d} {Hq}/{Hkv}")


def test_empty_contexts():
    ctx = [0, 5, 0, 300, 0]
    p = paged_inputs(small_cfg(), S=5, ctx_lens=ctx, poison=True, extra_blocks=2, max_blocks=20, seed=3)
    check(p, 0.0884, "empty")


@pytest.mark.parametrize("scale", [-0.2, 0.0, 1.7])
def test_unusual_scales(scale):
    p = paged_inputs(small_cfg(), S=4, ctx_lens=[3, 40, 290, 513], poison=True, max_blocks=40, seed=9)
    check(p, scale, f"scale={scale}")


def test_spike_through_block_table():
    """One key per sequence scores far above the rest at a random logical
    position p*; the output must be the value at the physical slot that the
    table maps p* to."""
    cfg = small_cfg(Hq=12, Hkv=2, d=128)
    ctx = [17, 100, 513, 1500, 4000, 8192]
    rng = np.random.default_rng(17)
    for rep in range(3):
        p = paged_inputs(cfg, S=len(ctx), ctx_lens=ctx, poison=True, extra_blocks=3,
                         max_blocks=512, seed=100 + rep)
        q = torch.zeros_like(p["q"], dtype=torch.float32)
        q[..., 0] = 1.0
        kc = p["k_cache"].float()
        kc[..., 0] = torch.where(torch.isnan(kc[..., 0]), kc[..., 0],
                                 torch.from_numpy(rng.uniform(-1, 1, kc.shape[:-1]).astype(np.float32)))
        t = p["block_table"].numpy()
        targets = []
        for s, n in enumerate(ctx):
            ps = int(rng.integers(0, n))
            blk, slot = int(t[s, ps // 16]), ps % 16
            kc[blk, :, slot, 0] = 40.0
            targets.append(p["v_cache"][blk, :, slot].double())
        p["q"] = q.to(torch.bfloat16)
        p["k_cache"] = kc.to(torch.bfloat16)
        o, _ = run_decode(p, 1.0)
        for s in range(len(ctx)):
            for h in range(12):
                g = h // 6
                err = (o[s, h].double() - targets[s][g]).abs().max().item()
                assert err <= 1e-2, (rep, s, h, err)


def test_row_max_spans_all_lane_groups():
    """The decode's row maximum combines four 16-lane groups, each holding 4
    of a block's 16 keys.  Put the only large score of a sequence in each group
    in turn (slot 1, 6, 9, 14, ...), so far above the rest (c s ~ 277) that a
    maximum missing that group would overflow 2^(c (s - m)); the output must
    be exactly that key's value row."""
    cfg = small_cfg(Hq=12, Hkv=2, d=128)
    ctx = [16, 16, 16, 16, 40, 700]
    spikes = [1, 6, 9, 14, 36, 699]            # slots 1, 6, 9, 14, 4, 11: every lane group
    p = paged_inputs(cfg, S=len(ctx), ctx_lens=ctx, poison=True, extra_blocks=2,
                     max_blocks=64, seed=21)
    q = torch.zeros_like(p["q"], dtype=torch.float32)
    q[..., 0] = 8.0
    kc = p["k_cache"].float()
    kc[..., 0] = torch.where(torch.isnan(kc[..., 0]), kc[..., 0], torch.zeros_like(kc[..., 0]))
    t = p["block_table"].numpy()
    targets = []
    for s, ps in enumerate(spikes):
        blk, slot = int(t[s, ps // 16]), ps % 16
        kc[blk, :, slot, 0] = 16.0
        targets.append(p["v_cache"][blk, :, slot].double())
    p["q"] = q.to(torch.bfloat16)
    p["k_cache"] = kc.to(torch.bfloat16)
    o, lse = run_decode(p, 1.5)
    assert torch.isfinite(o.float()).all() and torch.isfinite(lse).all()
    for s in range(len(ctx)):
        for h in range(12):
            err = (o[s, h].double() - targets[s][h // 6]).abs().max().item()
            assert err <= 1e-2, (s, h, err)
    assert (lse.double() - 192.0).abs().max().item() <= LSE_TOL


def test_identity_table_matches_dense():
    """A contiguous cache with an identity table is ordinary single-query
    attention: compare with the dense kernel on the same keys."""
    S, Hq, Hkv, d, n = 3, 12, 2, 128, 1000
    nb = (n + 15) // 16
    gen = torch.Generator().manual_seed(5)
    K = torch.randn(S, Hkv, nb * 16, d, generator=gen).to(torch.bfloat16)
    V = torch.randn(S, Hkv, nb * 16, d, generator=gen).to(torch.bfloat16)
    q = torch.randn(S, Hq, d, generator=gen).to(torch.bfloat16)
    kc = K.view(S, Hkv, nb, 16, d).permute(0, 2, 1, 3, 4).reshape(S * nb, Hkv, 16, d).contiguous()
    vc = V.view(S, Hkv, nb, 16, d).permute(0, 2, 1, 3, 4).reshape(S * nb, Hkv, 16, d).contiguous()
    table = torch.arange(S * nb, dtype=torch.int32).view(S, nb)
    ctx = torch.full((S,), n, dtype=torch.int32)
    p = dict(q=q, k_cache=kc, v_cache=vc, block_table=table, ctx_lens=ctx, block_size=16,
             num_blocks=S * nb, max_blocks=nb)
    o, lse = run_decode(p, 0.0884)
    for s in range(S):
        # dense kernel: the decode query as row n-1 of a causal prefill over n keys
        qd = torch.zeros(1, Hq, n, d, dtype=torch.bfloat16)
        qd[0, :, n - 1] = q[s]
        od, ld = attn_fwd(qd.to(DEV), K[s:s + 1, :, :n].contiguous().to(DEV),
                          V[s:s + 1, :, :n].contiguous().to(DEV), scale=0.0884, causal=True)
        torch.cuda.synchronize()
        assert max_abs(f64(o[s]), f64(od[0, :, n - 1])) <= 1e-2
        assert max_abs(lse[s].double().numpy(), ld[0, :, n - 1].double().cpu().numpy()) <= 1e-4


def test_full_workload_with_poison():
    p = paged_inputs(PAGED_CONFIG, poison=True, extra_blocks=64)
    check(p, PAGED_CONFIG.scale, "paged_decode_s64 poison")


def test_full_workload_and_determinism():
    p = paged_inputs(PAGED_CONFIG)
    eo, el = check(p, PAGED_CONFIG.scale, "paged_decode_s64")
    o1, l1 = run_decode(p, PAGED_CONFIG.scale)
    o2, l2 = run_decode(p, PAGED_CONFIG.scale)
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


@pytest.mark.parametrize("waves", [4, 12, 36, 2048])
def test_wave_counts(monkeypatch, waves):
    """Few waves give long pieces (several 64-block table chunks), waves that
    cross many (sequence, kv head) pairs, and pairs merged from many waves."""
    rng = np.random.default_rng(41)
    ctx = rng.integers(0, 3000, 70)
    ctx[[3, 10, 11, 50]] = 0
    ctx[5] = 4096
    p = paged_inputs(small_cfg(), S=70, ctx_lens=ctx.tolist(), poison=True, extra_blocks=4,
                     max_blocks=256, seed=42)
    monkeypatch.setenv("ATTN_DECODE_WAVES", str(waves))
    o, lse = run_decode(p, 0.0884)
    check(p, 0.0884, f"waves={waves}")
    o2, lse2 = run_decode(p, 0.0884)
    assert torch.equal(o, o2) and torch.equal(lse, lse2)


def test_many_short_sequences():
    rng = np.random.default_rng(43)
    ctx = rng.integers(0, 40, 200)
    p = paged_inputs(small_cfg(Hq=8, Hkv=2, d=64), S=200, ctx_lens=ctx.tolist(), poison=True,
                     max_blocks=3, seed=44)
    check(p, 0.125, "S=200 short")


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("Hq,Hkv", [(17, 1), (40, 2), (32, 1), (48, 1), (64, 1), (71, 1)])
def test_more_than_16_heads_per_kv_head(d, Hq, Hkv):
    """More than 16 query heads per kv head (multi-query models) run as groups
    of at most 16 rows: 17 heads as 9 + 8, 20 as 10 + 10, 32 as 16 + 16 (teams
    of two waves), 48 as three groups of 16 (teams of three, the fourth wave
    of each workgroup idle), 64 as four of 16 (teams of four), 71 as four
    groups of 15 and one of 11 (five groups: no teams, each group a kv head
    of its own)."""
    ctx = [1, 16, 17, 300, 0, 1000, 2000, 64]
    p = paged_inputs(small_cfg(Hq, Hkv, d), S=len(ctx), ctx_lens=ctx, poison=True, extra_blocks=4,
                     max_blocks=130, seed=Hq + d)
    check(p, 1.0 / math.sqrt(d), f"groups d{d} {Hq}/{Hkv}")


@pytest.mark.parametrize("waves", [4, 36])
@pytest.mark.parametrize("Hq,Hkv", [(48, 2), (48, 1), (128, 2), (144, 2)])
def test_head_groups_with_few_waves(monkeypatch, waves, Hq, Hkv):
    """Head groups with long pieces: a team's (or, beyond four groups, a
    wave's) units run across kv heads and sequences, and pairs are merged
    from many teams: 24 heads per kv head in teams of two, 48 in teams of
    three, 64 in teams of four, 72 as five groups without teams."""
    rng = np.random.default_rng(47)
    ctx = rng.integers(0, 2500, 20)
    ctx[[2, 9]] = 0
    p = paged_inputs(small_cfg(Hq, Hkv, 128), S=20, ctx_lens=ctx.tolist(), poison=True, extra_blocks=4,
                     max_blocks=160, seed=48)
    monkeypatch.setenv("ATTN_DECODE_WAVES", str(waves))
    o, lse = run_decode(p, 0.0884)
    check(p, 0.0884, f"groups {Hq}/{Hkv} waves={waves}")
    o2, lse2 = run_decode(p, 0.0884)
    assert torch.equal(o, o2) and torch.equal(lse, lse2)


@pytest.mark.parametrize("waves", [4, 2048])
@pytest.mark.parametrize("Hq,Hkv", [(12, 2), (64, 2)])
def test_bad_device_inputs_give_nan(monkeypatch, waves, Hq, Hkv):
    """Lengths outside [0, max_blocks*16] and needed table entries outside
    [0, num_blocks) make that sequence's outputs NaN, touch nothing out of
    bounds, and leave the other sequences exact (also with 32 query heads
    per kv head, read by teams of two waves)."""
    ctx = [100, 300, 200, 50, 700, 33]
    p = paged_inputs(small_cfg(Hq, Hkv), S=6, ctx_lens=ctx, poison=True, max_blocks=48, seed=45)
    ref_o, ref_l = oracle_decode(p, 0.0884)
    cap = 48 * 16
    p["ctx_lens"] = p["ctx_lens"].clone()
    p["ctx_lens"][1] = -3
    p["ctx_lens"][3] = cap + 5
    p["block_table"] = p["block_table"].clone()
    p["block_table"][4, 20] = p["num_blocks"]       # inside sequence 4's 44 blocks
    p["block_table"][5, 1] = -7                      # inside sequence 5's 3 blocks
    monkeypatch.setenv("ATTN_DECODE_WAVES", str(waves))
    o, lse = run_decode(p, 0.0884)
    for s in (1, 3, 4, 5):
        assert torch.isnan(o[s].float()).all(), s
        assert torch.isnan(lse[s]).all(), s
    for s in (0, 2):
        assert max_abs(f64(o[s]), ref_o[s]) <= O_TOL[torch.bfloat16]
        assert max_abs(lse[s].double().numpy(), ref_l[s]) <= LSE_TOL


@pytest.mark.parametrize("Hq", [12, 64])
def test_graph_replay_matches_eager(Hq):
    """The decode step captured in a HIP graph: replayed several times, with
    eager library calls in between and the inputs rewritten in place between
    replays (new queries, one more token per sequence written into its block),
    every replay equals an eager call on the same buffers bit for bit (also
    with 32 query heads per kv head, read by teams of two waves)."""
    from exact_tiled_self_amd.graph import DecodeGraph
    rng = np.random.default_rng(71)
    ctx = rng.integers(100, 3000, 16)
    p = paged_inputs(small_cfg(Hq, 2), S=16, ctx_lens=ctx.tolist(), extra_blocks=40, max_blocks=200, seed=72)
    d = _dev(p)
    # free pool blocks (never referenced) to grow into
    used = set(p["block_table"].numpy()[p["block_table"].numpy() >= 0].tolist())
    free = [b for b in range(p["num_blocks"]) if b not in used]
    g = DecodeGraph(d["q"], d["k_cache"], d["v_cache"], d["block_table"], d["ctx_lens"], 16, 0.0884,
                    calls=2)
    for rep in range(4):
        o_g, l_g = g.replay()
        torch.cuda.synchronize()
        o_e, l_e = attn_paged_decode(d["q"], d["k_cache"], d["v_cache"], d["block_table"],
                                     d["ctx_lens"], 16, 0.0884)
        torch.cuda.synchronize()
        assert torch.equal(o_g, o_e) and torch.equal(l_g, l_e), rep
        # next step: new queries, and one more token appended to every sequence
        d["q"].copy_(torch.randn(d["q"].shape, generator=torch.Generator().manual_seed(rep)).to(d["q"]))
        lens = d["ctx_lens"].cpu()
        table = d["block_table"].cpu()
        for s in range(16):
            pos = int(lens[s])
            if pos % 16 == 0:
                table[s, pos // 16] = free.pop()
            blk = int(table[s, pos // 16])
            d["k_cache"][blk, :, pos % 16] = torch.randn(2, 128, generator=torch.Generator().manual_seed(s)).to(d["k_cache"])
            d["v_cache"][blk, :, pos % 16] = torch.randn(2, 128, generator=torch.Generator().manual_seed(99 + s)).to(d["v_cache"])
        d["block_table"].copy_(table)
        d["ctx_lens"].copy_(lens + 1)
    # the final state against the oracle
    o_g, l_g = g.replay()
    torch.cuda.synchronize()
    host = {k: (v.cpu() if isinstance(v, torch.Tensor) else v) for k, v in d.items()}
    ro, rl = oracle_decode(host, 0.0884)
    assert max_abs(f64(o_g), ro) <= O_TOL[torch.bfloat16]
    assert max_abs(l_g.cpu().double().numpy(), rl) <= LSE_TOL

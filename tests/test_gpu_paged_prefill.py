"""GPU parity of the steps either side of decode: attn_kv_append (bit-exact
against the oracle's token-by-token scatter, whole caches compared byte for
byte) and attn_paged_prefill (chunked prefill over the paged cache, against
the float64 oracle): ragged lengths and chunk sizes, NaN poison in every
slot that must not be read, agreement with decode (one new row) and with
dense causal prefill (no earlier context), bad device-resident values, the
full 64-sequence cache with 256-row chunks at sampled sequences, an
append -> prefill -> decode chain, and determinism."""

import math

import numpy as np
import pytest
import torch

from exact_tiled_self_amd import attn_fwd, attn_kv_append, attn_paged_decode, attn_paged_prefill
from exact_tiled_self_amd.inputs import CHUNK_NEW, PAGED_CONFIG, PagedConfig, chunked_inputs
from oracle import exact as OA
from oracle.kvcache import append_paged
from tests.gpu_util import DEV, LSE_TOL, O_TOL, announce, f64, max_abs

pytestmark = pytest.mark.gpu

BF16_TOL = O_TOL[torch.bfloat16]


@pytest.fixture(autouse=True)
def _name_case(request):
    announce(request.node.nodeid)
    yield


def cfg(Hq=12, Hkv=2, d=128, dtype="bf16", bs=16):
    return PagedConfig("t", S=1, Hq=Hq, Hkv=Hkv, d=d, block_size=bs, ctx_lo=1, ctx_hi=1,
                       max_blocks=1, dtype=dtype, seed=0)


def to_dev(p):
    return {k: (v.to(DEV) if isinstance(v, torch.Tensor) else v) for k, v in p.items()}


def bits(t):
    """Raw integer view of a CPU tensor (exact comparison, NaN included)."""
    return t.view({2: torch.int16, 4: torch.int32}[t.element_size()]).numpy()


# -------------------------------------------------------------- append ----

def gpu_append(p, ctx=None, max_new=None):
    d = to_dev(p)
    kc, vc = d["k_cache"].clone(), d["v_cache"].clone()
    lens = d["ctx_lens"] if ctx is None else torch.as_tensor(ctx, dtype=torch.int32, device=DEV)
    attn_kv_append(d["k_new"], d["v_new"], kc, vc, d["block_table"], lens, d["starts"],
                   p["block_size"], max_new=p["max_new"] if max_new is None else max_new)
    torch.cuda.synchronize()
    return kc.cpu(), vc.cpu()


def oracle_append(p, ctx=None):
    ctx = p["ctx_lens"].numpy() if ctx is None else np.asarray(ctx)
    return append_paged(bits(p["k_cache"]), bits(p["v_cache"]), p["block_table"].numpy(), ctx,
                        p["starts"].numpy(), bits(p["k_new"]), bits(p["v_new"]), p["block_size"])


@pytest.mark.parametrize("dtype,d,bs", [("bf16", 128, 16), ("bf16", 64, 16), ("f32", 128, 16),
                                        ("bf16", 128, 1), ("f32", 64, 5)])
def test_append_bit_exact(dtype, d, bs):
    ctx = [1, 15, 16, 17, 40, 100, 300, 33, 5]
    new = [1, 1, 16, 2, 0, 100, 37, 18, 5]
    p = chunked_inputs(cfg(d=d, dtype=dtype, bs=bs), S=len(ctx), ctx_lens=ctx, new_lens=new,
                       poison=True, extra_blocks=4, max_blocks=(300 + bs - 1) // bs + 2, seed=d + bs)
    kc, vc = gpu_append(p)
    ek, ev = oracle_append(p)
    assert np.array_equal(bits(kc), ek) and np.array_equal(bits(vc), ev)


def test_append_device_values_that_write_nothing():
    ctx = [20, 20, 20, 20, 20, 20]
    new = [4, 4, 4, 4, 4, 4]
    p = chunked_inputs(cfg(), S=6, ctx_lens=ctx, new_lens=new, extra_blocks=3, max_blocks=3, seed=9)
    p["block_table"][1, 1] = 10 ** 6          # seq 1: positions 16..19 -> bad entry
    p["block_table"][2, 1] = -7               # seq 2: negative entry
    lens = np.array(ctx)
    lens[3] = 3                               # seq 3: shorter than its new rows
    starts = p["starts"].clone()
    starts[4] = 17                            # seq 3 rows 12..16 (5 rows > its length 3), seq 4 rows 17..19
    starts[6] = 30                            # seq 5 rows 20..29 run past T = 24
    p["starts"] = starts
    kc, vc = gpu_append(p, ctx=lens, max_new=8)
    ek, ev = oracle_append(p, ctx=lens)
    assert np.array_equal(bits(kc), ek) and np.array_equal(bits(vc), ev)
    # max_new below a sequence's row count: that sequence is skipped whole
    p2 = chunked_inputs(cfg(), S=3, ctx_lens=[20, 20, 20], new_lens=[2, 6, 2], max_blocks=3, seed=10)
    kc2, vc2 = gpu_append(p2, max_new=4)
    lens2 = np.array([20, -1, 20])            # the oracle's "skip" for sequence 1
    ek2, ev2 = oracle_append(p2, ctx=lens2)
    assert np.array_equal(bits(kc2), ek2) and np.array_equal(bits(vc2), ev2)


@pytest.mark.parametrize("new", [1, CHUNK_NEW])
def test_append_full_cache(new):
    p = chunked_inputs(PAGED_CONFIG, new_lens=new)
    kc, vc = gpu_append(p)
    ek, ev = oracle_append(p)
    assert np.array_equal(bits(kc), ek) and np.array_equal(bits(vc), ev)


# ------------------------------------------------------- chunked prefill ----

def gpu_prefill(p, scale, max_new=None, o=None, lse=None, ctx=None):
    d = to_dev(p)
    lens = d["ctx_lens"] if ctx is None else torch.as_tensor(ctx, dtype=torch.int32, device=DEV)
    o_, l_ = attn_paged_prefill(d["q_new"], d["k_cache"], d["v_cache"], d["block_table"], lens,
                                d["starts"], p["block_size"], scale,
                                max_new=p["max_new"] if max_new is None else max_new,
                                o=None if o is None else o.to(DEV),
                                lse=None if lse is None else lse.to(DEV))
    torch.cuda.synchronize()
    return o_.cpu(), l_.cpu()


def oracle_prefill(p, scale, seqs=None, ctx=None):
    """The oracle on all sequences, or on a subset (rows re-packed)."""
    st = p["starts"].numpy().astype(np.int64)
    ctx = p["ctx_lens"].numpy() if ctx is None else np.asarray(ctx)
    table = p["block_table"].numpy()
    q = p["q_new"]
    if seqs is not None:
        rows = np.concatenate([np.arange(st[s], st[s + 1]) for s in seqs])
        n = np.array([st[s + 1] - st[s] for s in seqs])
        q = q[torch.from_numpy(rows)]
        table, ctx = table[seqs], ctx[seqs]
        st = np.concatenate([[0], np.cumsum(n)])
    return OA.paged_prefill(f64(q), f64(p["k_cache"]), f64(p["v_cache"]), table, ctx, st,
                            p["block_size"], scale)


def assert_close(o, lse, ro, rl, rows=None, name=""):
    go, gl = f64(o), lse.double().numpy()
    if rows is not None:
        go, gl = go[rows], gl[rows]
    assert np.isfinite(go).all() and np.isfinite(gl).all(), name
    eo, el = max_abs(go, ro), max_abs(gl, rl)
    assert eo <= BF16_TOL, f"{name}: o max-abs {eo}"
    assert el <= LSE_TOL, f"{name}: lse max-abs {el}"
    return eo, el


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("Hq,Hkv", [(12, 2), (8, 8), (16, 1)])
def test_ragged_chunks_with_poison(d, Hq, Hkv):
    ctx = [1, 16, 17, 100, 129, 300, 700, 1000, 64, 5]
    new = [1, 16, 5, 100, 129, 37, 256, 1, 64, 0]
    p = chunked_inputs(cfg(Hq, Hkv, d), S=len(ctx), ctx_lens=ctx, new_lens=new, poison=True,
                       extra_blocks=3, max_blocks=64, seed=d * Hq)
    sc = 1.0 / math.sqrt(d)
    o, lse = gpu_prefill(p, sc)
    ro, rl = oracle_prefill(p, sc)
    assert_close(o, lse, ro, rl, name=f"ragged d{d} {Hq}/{Hkv}")


@pytest.mark.parametrize("scale", [0.0, -0.3, 0.9])
def test_scales(scale):
    p = chunked_inputs(cfg(), S=3, ctx_lens=[50, 200, 130], new_lens=[50, 70, 129], poison=True,
                       max_blocks=16, seed=21)
    o, lse = gpu_prefill(p, scale)
    ro, rl = oracle_prefill(p, scale)
    assert_close(o, lse, ro, rl, name=f"scale {scale}")


def test_one_new_row_is_decode():
    ctx = [1, 17, 64, 500, 1111]
    p = chunked_inputs(cfg(), S=5, ctx_lens=ctx, new_lens=1, poison=True, max_blocks=80, seed=31)
    sc = 0.0884
    o, lse = gpu_prefill(p, sc)
    d = to_dev(p)
    od, ld = attn_paged_decode(d["q_new"], d["k_cache"], d["v_cache"], d["block_table"],
                               d["ctx_lens"], 16, sc)
    torch.cuda.synchronize()
    assert max_abs(f64(o), f64(od.cpu())) <= BF16_TOL
    assert max_abs(lse.double().numpy(), ld.cpu().double().numpy()) <= LSE_TOL
    ro, rl = oracle_prefill(p, sc)
    assert_close(o, lse, ro, rl, name="decode-like")


def test_no_context_is_dense_causal():
    """Every sequence's rows are its whole context: causal attn_fwd per sequence."""
    lens = [300, 129, 64]
    p = chunked_inputs(cfg(), S=3, ctx_lens=lens, new_lens=lens, poison=True, max_blocks=20, seed=41)
    sc = 0.0884
    o, lse = gpu_prefill(p, sc)
    st = p["starts"].numpy()
    for s, n in enumerate(lens):
        # the same keys, gathered densely on the CPU, through attn_fwd
        K = torch.stack([p["k_cache"][p["block_table"][s, t // 16], :, t % 16] for t in range(n)], 1)
        V = torch.stack([p["v_cache"][p["block_table"][s, t // 16], :, t % 16] for t in range(n)], 1)
        Q = p["q_new"][st[s]:st[s + 1]].transpose(0, 1)
        od, ld = attn_fwd(Q[None].contiguous().to(DEV), K[None].contiguous().to(DEV),
                          V[None].contiguous().to(DEV), scale=sc, causal=True)
        torch.cuda.synchronize()
        assert max_abs(f64(o[st[s]:st[s + 1]]), f64(od[0].transpose(0, 1).cpu())) <= BF16_TOL
        assert max_abs(lse[st[s]:st[s + 1]].double().numpy(),
                       ld[0].transpose(0, 1).cpu().double().numpy()) <= LSE_TOL
    ro, rl = oracle_prefill(p, sc)
    assert_close(o, lse, ro, rl, name="no context")


def test_bad_device_values():
    ctx = [40, 40, 40, 40, 40, 40]
    new = [4, 30, 4, 4, 4, 4]
    p = chunked_inputs(cfg(), S=6, ctx_lens=ctx, new_lens=new, max_blocks=3, seed=51)
    p["block_table"][1, 1] = 10 ** 6          # seq 1: block 1 (positions 16..31) bad
    lens = np.array(ctx)
    lens[2] = 3                               # seq 2: shorter than its rows -> NaN rows
    lens[3] = 3 * 16 + 1                      # seq 3: longer than the table -> NaN rows
    starts = p["starts"].clone()
    starts[6] = starts[6] + 5                 # seq 5's rows run past T -> left unwritten
    p["starts"] = starts
    T = p["q_new"].shape[0]
    sentinel = torch.full((T, 12, 128), 7.0, dtype=torch.bfloat16)
    sentinel_l = torch.full((T, 12), 7.0)
    o, lse = gpu_prefill(p, 0.0884, o=sentinel, lse=sentinel_l, ctx=lens)
    st = p["starts"].numpy()
    ro, rl = oracle_prefill(p, 0.0884, ctx=lens)
    ok = np.isfinite(rl).all(axis=1)
    # rows the oracle computes: within tolerance
    assert max_abs(f64(o)[ok], ro[ok]) <= BF16_TOL and max_abs(lse.double().numpy()[ok], rl[ok]) <= LSE_TOL
    # seq 1: rows at positions 10..15 fine, 16..39 NaN
    assert np.isfinite(f64(o[st[1]:st[1] + 6])).all()
    assert torch.isnan(o[st[1] + 6:st[2]].float()).all() and torch.isnan(lse[st[1] + 6:st[2]]).all()
    # seq 2 and 3: NaN rows
    assert torch.isnan(o[st[2]:st[4]].float()).all() and torch.isnan(lse[st[2]:st[4]]).all()
    # seq 4 is computed; seq 5 keeps the sentinel
    assert np.isfinite(f64(o[st[4]:st[5]])).all()
    assert torch.all(o[st[5]:] == 7) and torch.all(lse[st[5]:] == 7)
    # max_new below a row count: that sequence is left unwritten
    p2 = chunked_inputs(cfg(), S=2, ctx_lens=[40, 40], new_lens=[10, 3], max_blocks=3, seed=52)
    o2, l2 = gpu_prefill(p2, 0.0884, max_new=5,
                         o=torch.full((13, 12, 128), 7.0, dtype=torch.bfloat16),
                         lse=torch.full((13, 12), 7.0))
    assert torch.all(o2[:10] == 7) and torch.all(l2[:10] == 7)
    ro2, rl2 = oracle_prefill(p2, 0.0884, seqs=[1])
    assert_close(o2[10:], l2[10:], ro2, rl2, name="max_new skip")


def test_full_cache_chunks_sampled():
    """The 64-sequence cache with 256 new rows each, in the launch the bench
    times; four sequences (shortest, longest, two more) checked in full."""
    p = chunked_inputs(PAGED_CONFIG, new_lens=CHUNK_NEW)
    sc = PAGED_CONFIG.scale
    o, lse = gpu_prefill(p, sc)
    ctx = p["ctx_lens"].numpy()
    seqs = sorted({int(ctx.argmin()), int(ctx.argmax()), 7, 40})
    ro, rl = oracle_prefill(p, sc, seqs=seqs)
    st = p["starts"].numpy()
    rows = np.concatenate([np.arange(st[s], st[s + 1]) for s in seqs])
    assert_close(o, lse, ro, rl, rows=rows, name="full cache")
    assert torch.isfinite(o.float()).all() and torch.isfinite(lse).all()


def test_append_prefill_decode_chain():
    """One serving step per sequence: append the chunk's K/V, prefill its
    rows, then decode one more token - each against the oracle chain."""
    ctx = [20, 100, 257]
    new = [20, 37, 64]
    p = chunked_inputs(cfg(), S=3, ctx_lens=ctx, new_lens=new, poison=True, max_blocks=20, seed=61)
    sc = 0.0884
    d = to_dev(p)
    kc, vc = d["k_cache"].clone(), d["v_cache"].clone()
    attn_kv_append(d["k_new"], d["v_new"], kc, vc, d["block_table"], d["ctx_lens"], d["starts"],
                   max_new=p["max_new"])
    o, lse = attn_paged_prefill(d["q_new"], kc, vc, d["block_table"], d["ctx_lens"], d["starts"],
                                scale=sc, max_new=p["max_new"])
    # one more token each: append it, then decode
    rng = np.random.default_rng(62)
    k1 = torch.from_numpy(rng.standard_normal((3, 2, 128), dtype=np.float32)).to(torch.bfloat16)
    v1 = torch.from_numpy(rng.standard_normal((3, 2, 128), dtype=np.float32)).to(torch.bfloat16)
    q1 = torch.from_numpy(rng.standard_normal((3, 12, 128), dtype=np.float32)).to(torch.bfloat16)
    lens1 = torch.tensor([c + 1 for c in ctx], dtype=torch.int32)
    st1 = torch.arange(4, dtype=torch.int32)
    attn_kv_append(k1.to(DEV), v1.to(DEV), kc, vc, d["block_table"], lens1.to(DEV), st1.to(DEV), max_new=1)
    od, ld = attn_paged_decode(q1.to(DEV), kc, vc, d["block_table"], lens1.to(DEV), 16, sc)
    torch.cuda.synchronize()

    ek, ev = append_paged(f64(p["k_cache"]), f64(p["v_cache"]), p["block_table"].numpy(),
                          p["ctx_lens"].numpy(), p["starts"].numpy(), f64(p["k_new"]), f64(p["v_new"]), 16)
    ro, rl = OA.paged_prefill(f64(p["q_new"]), ek, ev, p["block_table"].numpy(), p["ctx_lens"].numpy(),
                              p["starts"].numpy(), 16, sc)
    assert_close(o.cpu(), lse.cpu(), ro, rl, name="chain prefill")
    ek, ev = append_paged(ek, ev, p["block_table"].numpy(), lens1.numpy(), st1.numpy(), f64(k1), f64(v1), 16)
    # the device caches equal the oracle chain's exactly (values are bf16)
    assert np.array_equal(f64(kc.cpu()), ek, equal_nan=True) and np.array_equal(f64(vc.cpu()), ev, equal_nan=True)
    rod, rld = OA.paged_decode(f64(q1), ek, ev, p["block_table"].numpy(), lens1.numpy(), 16, sc)
    assert max_abs(f64(od.cpu()), rod) <= BF16_TOL and max_abs(ld.cpu().double().numpy(), rld) <= LSE_TOL


def test_deterministic():
    p = chunked_inputs(cfg(), S=4, ctx_lens=[300, 50, 129, 1000], new_lens=[300, 1, 100, 200],
                       max_blocks=70, seed=71)
    o1, l1 = gpu_prefill(p, 0.0884)
    o2, l2 = gpu_prefill(p, 0.0884)
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16)) and torch.equal(l1, l2)


def _lens(seed, S, new_hi, extra_hi):
    rng = np.random.default_rng(seed)
    new = rng.integers(1, new_hi + 1, S)
    return [int(n + e) for n, e in zip(new, rng.integers(0, extra_hi + 1, S))], [int(n) for n in new]


# (d, Hq, Hkv, S, most new rows, most earlier context): the automatic cut puts
# 3 query tiles in an item for the first three, 2 for the fourth; the last
# has more than 512 chunks (no cost ranking: later chunks first).
CUT_CASES = [(128, 8, 8, 10, 300, 400), (128, 12, 2, 40, 300, 300), (64, 16, 1, 70, 300, 200),
             (128, 12, 2, 33, 256, 500), (64, 12, 2, 520, 2, 40)]


@pytest.mark.parametrize("d,Hq,Hkv,S,new_hi,extra_hi", CUT_CASES)
def test_item_cuts(monkeypatch, d, Hq, Hkv, S, new_hi, extra_hi):
    """The work is cut into items of up to cq query tiles of one sequence and
    kv head, each item on one XCD: every cut (ATTN_PAGED_CQ) gives the same
    bits, and the automatic one matches the oracle."""
    ctx, new = _lens(S * Hq + d, S, new_hi, extra_hi)
    p = chunked_inputs(cfg(Hq, Hkv, d), S=S, ctx_lens=ctx, new_lens=new, poison=True,
                       max_blocks=(max(ctx) + 15) // 16 + 1, seed=S + d)
    sc = 1.0 / math.sqrt(d)
    o, lse = gpu_prefill(p, sc)
    n_qt = (p["max_new"] + 127) // 128
    for cq in sorted({1, 2, n_qt} & set(range(1, n_qt + 1))):
        monkeypatch.setenv("ATTN_PAGED_CQ", str(cq))
        o2, l2 = gpu_prefill(p, sc)
        assert torch.equal(o.view(torch.int16), o2.view(torch.int16)), f"o differs at cq={cq}"
        assert torch.equal(lse.view(torch.int32), l2.view(torch.int32)), f"lse differs at cq={cq}"
    monkeypatch.delenv("ATTN_PAGED_CQ")
    ro, rl = oracle_prefill(p, sc)
    assert_close(o, lse, ro, rl, name=f"cuts d{d} {Hq}/{Hkv} S={S}")


@pytest.mark.parametrize("step", [4.5, 7.0, -3.0])
def test_rescale_quick_test_fallback(step):
    """Scores that climb (or fall) from one 32-position block of the context
    to the next and are equal inside a block: the tile step's quick row-sum
    test fails on every tile (or never after the first), so the exact-maximum
    path runs after it; every row against the oracle."""
    ctx = [300, 130, 64, 200]
    new = [300, 40, 64, 1]
    p = chunked_inputs(cfg(), S=len(ctx), ctx_lens=ctx, new_lens=new, poison=True, max_blocks=20,
                       seed=int(10 * abs(step)) + (7 if step < 0 else 5))
    p["q_new"].zero_()
    p["q_new"][..., 0] = 1.0
    kc = p["k_cache"]
    table = p["block_table"].numpy()
    for s, n in enumerate(ctx):
        for t in range(n):
            blk, slot = int(table[s, t // 16]), t % 16
            kc[blk, :, slot, :] = 0.0
            kc[blk, :, slot, 0] = step * (t // 32)
    o, lse = gpu_prefill(p, 1.0)
    ro, rl = oracle_prefill(p, 1.0)
    assert_close(o, lse, ro, rl, name=f"staircase step {step}")

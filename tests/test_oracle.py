"""Pins of the CPU oracle against facts fixed outside it.

Every check here compares the oracle with something it does not compute
itself: the worked example printed on the pages, closed forms, invariants,
PyTorch's scaled_dot_product_attention on float64 CPU tensors, and 40-digit
brute force.  test_mutants_are_caught plants plausible mistakes in the
oracle (on the CPU) and shows that each one fails at least one pin.
"""

import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
from oracle import exact as OA
from oracle import recurrence as R
from tests.bruteforce import bf_attention, bf_paged

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rand(shape, seed, amp=1.0):
    return amp * np.random.default_rng(seed).standard_normal(shape)


def _golden():
    with open(os.path.join(GOLDEN, "worked_example.json")) as f:
        g = json.load(f)
    scores = [math.log(3.0) if s == "ln(3)" else float(s) for s in g["scores"]]
    return g, np.array(scores), np.array(g["values"])


# ---------------------------------------------------------------- pins ----

def pin_worked_example_recurrence():
    g, s, v = _golden()
    out, st = R.online_aggregate(s, v, g["partition"])
    assert abs(out[0] - g["expected_output"]) < 1e-15
    num, den = g["expected_output_fraction"]
    assert abs(st.l * math.exp(st.m) - den) < 1e-12       # 1 + 1 + 3 + 3
    blocks = [R.online_aggregate(s[a:b], v[a:b], [b - a])[0][0]
              for a, b in R.blocks_of(len(s), g["partition"])]
    assert np.allclose(blocks, g["block_results"], atol=1e-15)
    naive = R.naive_block_average(s, v, g["partition"])[0]
    assert abs(naive - g["naive_block_average"]) < 1e-15


def pin_worked_example_dense():
    """The same example through the dense oracle, as a 4-token head."""
    g, s, v = _golden()
    d = 64
    q = np.zeros((1, 1, 4, d)); q[..., 0] = 1.0                 # q = e0 for every row
    k = np.zeros((1, 1, 4, d)); k[0, 0, :, 0] = s               # k_j = s_j e0
    vv = np.zeros((1, 1, 4, d)); vv[0, 0, :, 0] = v
    o, lse = OA.attention(q, k, vv, 1.0, causal=False, workers=1)
    assert np.all(np.abs(o[0, 0, :, 0] - g["expected_output"]) < 1e-15)
    assert np.all(o[0, 0, :, 1:] == 0.0)
    assert np.allclose(lse[0, 0], math.log(8.0), atol=1e-15)
    # bf16-exact variant used on the GPU: k in {0, 1}, scale = float32(ln 3)
    k2 = np.zeros((1, 1, 4, d)); k2[0, 0, :, 0] = [0, 0, 1, 1]
    o2, _ = OA.attention(q, k2, vv, math.log(3.0), causal=False, workers=1)
    w = math.exp(float(np.float32(math.log(3.0))))
    assert abs(o2[0, 0, 0, 0] - 2 * w / (2 + 2 * w)) < 1e-15
    assert abs(o2[0, 0, 0, 0] - 0.75) < 1e-7


def pin_uniform_scores(causal):
    """scale 0 (or q = 0): every allowed key has weight 1 / #allowed."""
    B, Hq, Hkv, N, d = 2, 4, 2, 37, 16
    q, k, v = _rand((B, Hq, N, d), 1), _rand((B, Hkv, N, d), 2), _rand((B, Hkv, N, d), 3)
    for qq, sc in ((q, 0.0), (np.zeros_like(q), 0.7)):
        o, lse = OA.attention(qq, k, v, sc, causal=causal, workers=2)
        for b in range(B):
            for h in range(Hq):
                g = h // (Hq // Hkv)
                if causal:
                    expect = np.cumsum(v[b, g], axis=0) / np.arange(1, N + 1)[:, None]
                    expect_lse = np.log(np.arange(1, N + 1))
                else:
                    expect = np.broadcast_to(v[b, g].mean(axis=0), (N, d))
                    expect_lse = np.full(N, math.log(N))
                assert np.allclose(o[b, h], expect, atol=1e-13)
                assert np.allclose(lse[b, h], expect_lse, atol=1e-13)


def pin_constant_values(causal):
    B, Hq, Hkv, N, d = 1, 3, 3, 29, 8
    q, k = _rand((B, Hq, N, d), 4, 3.0), _rand((B, Hkv, N, d), 5, 3.0)
    c = _rand((d,), 6)
    v = np.broadcast_to(c, (B, Hkv, N, d)).copy()
    o, _ = OA.attention(q, k, v, 0.3, causal=causal, workers=1)
    assert np.allclose(o, np.broadcast_to(c, o.shape), atol=1e-13)


def pin_identity_values(causal):
    """V = I makes O the probability matrix: rows sum to 1, matches the
    library softmax of the masked scaled scores, and the causal upper
    triangle is exactly zero."""
    from scipy.special import softmax
    N = d = 32
    q, k = _rand((1, 1, N, d), 7), _rand((1, 1, N, d), 8)
    v = np.eye(N)[None, None]
    sc = 0.25
    o, _ = OA.attention(q, k, v, sc, causal=causal, workers=1)
    P = o[0, 0]
    assert np.allclose(P.sum(axis=1), 1.0, atol=1e-14)
    sg = float(np.float32(sc))
    S = sg * q[0, 0] @ k[0, 0].T
    if causal:
        S = np.where(np.tril(np.ones((N, N), bool)), S, -np.inf)
        assert np.all(P[np.triu_indices(N, 1)] == 0.0)
    assert np.allclose(P, softmax(S, axis=1), atol=1e-14)


def pin_spike():
    """One key scoring 40 above the rest: o equals its value to ~N e^-40."""
    N, d = 50, 16
    rng = np.random.default_rng(9)
    q = np.zeros((1, 1, N, d)); q[..., 0] = 1.0
    k = rng.uniform(-1, 1, (1, 1, N, d)); k[..., 0] = rng.uniform(-1, 1, N)
    j = 17
    k[0, 0, j, 0] = 41.0
    v = rng.standard_normal((1, 1, N, d))
    o, lse = OA.attention(q, k, v, 1.0, causal=False, workers=1)
    assert np.allclose(o[0, 0], np.broadcast_to(v[0, 0, j], (N, d)), atol=N * math.exp(-39))
    assert np.allclose(lse[0, 0], 41.0, atol=1e-10)


def pin_bruteforce_dense():
    cases = [(1, 1, 1, 1, 1, False), (1, 2, 1, 5, 3, True), (2, 4, 2, 17, 8, True),
             (1, 4, 2, 17, 8, False), (1, 3, 3, 9, 4, True), (1, 4, 1, 6, 2, False)]
    for i, (B, Hq, Hkv, N, d, causal) in enumerate(cases):
        q, k, v = (_rand((B, Hq, N, d), 10 + i, 2.0), _rand((B, Hkv, N, d), 20 + i, 2.0),
                   _rand((B, Hkv, N, d), 30 + i))
        sc = 0.7 + 0.1 * i
        o, lse = OA.attention(q, k, v, sc, causal=causal, workers=2, chunk=4)
        ob, lb = bf_attention(q, k, v, sc, causal)
        assert np.allclose(o, ob, atol=1e-14, rtol=0), (B, Hq, Hkv, N, d, causal)
        assert np.allclose(lse, lb, atol=1e-13, rtol=0), (B, Hq, Hkv, N, d, causal)


def _small_paged(seed, S=3, Hq=4, Hkv=2, d=4, bs=16, ctx=(1, 16, 37), max_blocks=4):
    rng = np.random.default_rng(seed)
    ctx = np.array(ctx, dtype=np.int32)
    nblk = (ctx + bs - 1) // bs
    nb = int(nblk.sum()) + 2
    perm = rng.permutation(nb)
    table = np.full((S, max_blocks), -1, np.int32)
    off = 0
    for s in range(S):
        table[s, :nblk[s]] = perm[off:off + nblk[s]]
        off += nblk[s]
    q = rng.standard_normal((S, Hq, d))
    kc = rng.standard_normal((nb, Hkv, bs, d))
    vc = rng.standard_normal((nb, Hkv, bs, d))
    return q, kc, vc, table, ctx, bs


def pin_bruteforce_paged():
    q, kc, vc, table, ctx, bs = _small_paged(40)
    o, lse = OA.paged_decode(q, kc, vc, table, ctx, bs, 0.5, workers=1)
    ob, lb = bf_paged(q, kc, vc, table, ctx, bs, 0.5)
    assert np.allclose(o, ob, atol=1e-14, rtol=0)
    assert np.allclose(lse, lb, atol=1e-13, rtol=0)


def pin_sdpa_crosscheck():
    """PyTorch's SDPA on float64 CPU tensors (GQA by repeat_interleave)."""
    B, Hq, Hkv, N, d = 2, 6, 2, 70, 32
    q, k, v = _rand((B, Hq, N, d), 50), _rand((B, Hkv, N, d), 51), _rand((B, Hkv, N, d), 52)
    sc = 1.0 / math.sqrt(d)
    for causal in (False, True):
        o, _ = OA.attention(q, k, v, sc, causal=causal, workers=2, chunk=32)
        ref = torch.nn.functional.scaled_dot_product_attention(
            torch.from_numpy(q), torch.from_numpy(k), torch.from_numpy(v),
            is_causal=causal, scale=float(np.float32(sc)), enable_gqa=True).numpy()
        assert np.allclose(o, ref, atol=1e-12, rtol=0)


def pin_permutation():
    B, Hq, Hkv, N, d = 1, 2, 1, 40, 8
    q, k, v = _rand((B, Hq, N, d), 60), _rand((B, Hkv, N, d), 61), _rand((B, Hkv, N, d), 62)
    o, lse = OA.attention(q, k, v, 0.4, causal=False, workers=1)
    pk = np.random.default_rng(63).permutation(N)
    pq = np.random.default_rng(64).permutation(N)
    o2, lse2 = OA.attention(q[:, :, pq], k[:, :, pk], v[:, :, pk], 0.4, causal=False, workers=1)
    assert np.allclose(o2, o[:, :, pq], atol=1e-14)
    assert np.allclose(lse2, lse[:, :, pq], atol=1e-14)


def pin_paged_spike():
    """A spike key at a random logical position p*: the output must be the
    value stored at the physical slot the table maps p* to."""
    q, kc, vc, table, ctx, bs = _small_paged(70, S=4, Hq=2, Hkv=1, d=8, ctx=(5, 16, 33, 64), max_blocks=4)
    rng = np.random.default_rng(71)
    q[:] = 0.0
    q[:, :, 0] = 1.0
    kc[..., 0] = rng.uniform(-1, 1, kc.shape[:-1])
    targets = []
    for s in range(len(ctx)):
        p = int(rng.integers(0, ctx[s]))
        blk, slot = table[s, p // bs], p % bs
        kc[blk, 0, slot, 0] = 60.0
        targets.append(vc[blk, 0, slot].copy())
    o, _ = OA.paged_decode(q, kc, vc, table, ctx, bs, 1.0, workers=1)
    for s, t in enumerate(targets):
        assert np.allclose(o[s], np.broadcast_to(t, o[s].shape), atol=1e-20 + 70 * math.exp(-58))


def pin_paged_equals_dense():
    """Identity table over a contiguous cache equals dense single-row attention."""
    S, Hq, Hkv, d, bs = 2, 4, 2, 8, 16
    n = 45
    rng = np.random.default_rng(80)
    K = rng.standard_normal((S, Hkv, 48, d)); V = rng.standard_normal((S, Hkv, 48, d))
    q = rng.standard_normal((S, Hq, d))
    kc = K.reshape(S, Hkv, 3, bs, d).transpose(0, 2, 1, 3, 4).reshape(S * 3, Hkv, bs, d)
    vc = V.reshape(S, Hkv, 3, bs, d).transpose(0, 2, 1, 3, 4).reshape(S * 3, Hkv, bs, d)
    table = np.arange(S * 3, dtype=np.int32).reshape(S, 3)
    ctx = np.array([n, 48], dtype=np.int32)
    o, lse = OA.paged_decode(q, kc, vc, table, ctx, bs, 0.35, workers=1)
    for s in range(S):
        nn = int(ctx[s])
        for h in range(Hq):
            g = h // (Hq // Hkv)
            Qd = np.zeros((1, 1, nn, d))
            Qd[0, 0, 0] = q[s, h]                   # the decode query as row 0
            od, ld = OA.attention(Qd, K[s, g, :nn][None, None], V[s, g, :nn][None, None],
                                  0.35, workers=1)
            assert np.allclose(o[s, h], od[0, 0, 0], atol=1e-14)
            assert np.allclose(lse[s, h], ld[0, 0, 0], atol=1e-14)


def pin_recurrence_partitions():
    """Any block partition of the keys gives the oracle's row (block size is
    not a parameter of the result)."""
    N, d = 97, 5
    q, k, v = _rand((1, 1, N, d), 90), _rand((1, 1, N, d), 91, 2.0), _rand((1, 1, N, d), 92)
    o, lse = OA.attention(q, k, v, 0.9, causal=False, workers=1)
    sg = float(np.float32(0.9))
    i = 13
    scores = sg * (k[0, 0] @ q[0, 0, i])
    for part in (1, 2, 3, 16, 64, N, [1, 50, 46]):
        out, st = R.online_aggregate(scores, v[0, 0], part)
        assert np.allclose(out, o[0, 0, i], atol=1e-13)
        assert abs(st.m + math.log(st.l) - lse[0, 0, i]) < 1e-13


def pin_merge():
    """Merging split states (in any grouping) equals the whole row."""
    N, d = 64, 6
    rng = np.random.default_rng(95)
    s = 3.0 * rng.standard_normal(N)
    v = rng.standard_normal((N, d))
    whole, _ = R.online_aggregate(s, v, [N])
    parts = [(0, 10), (10, 11), (11, 40), (40, 64)]
    states = [R.online_aggregate(s[a:b], v[a:b], [b - a])[1] for a, b in parts]
    acc = R.OnlineState(u=np.zeros(d))
    for st in states:
        acc = R.merge_states(acc, st)
    assert np.allclose(acc.result(), whole, atol=1e-14)
    # empty state is the identity of the merge
    e = R.OnlineState(u=np.zeros(d))
    assert np.allclose(R.merge_states(e, states[0]).result(), states[0].result(), atol=0)


def pin_empty_context():
    q, kc, vc, table, ctx, bs = _small_paged(99, ctx=(0, 3, 16))
    o, lse = OA.paged_decode(q, kc, vc, table, ctx, bs, 0.5, workers=1)
    assert np.all(o[0] == 0.0) and np.all(np.isneginf(lse[0]))
    assert np.all(np.isfinite(o[1:])) and np.all(np.isfinite(lse[1:]))


ALL_PINS = [
    pin_worked_example_recurrence, pin_worked_example_dense,
    lambda: pin_uniform_scores(False), lambda: pin_uniform_scores(True),
    lambda: pin_constant_values(False), lambda: pin_constant_values(True),
    lambda: pin_identity_values(False), lambda: pin_identity_values(True),
    pin_spike, pin_bruteforce_dense, pin_bruteforce_paged, pin_sdpa_crosscheck,
    pin_permutation, pin_paged_spike, pin_paged_equals_dense,
    pin_recurrence_partitions, pin_merge, pin_empty_context,
]


# --------------------------------------------------------------- tests ----

def test_worked_example_recurrence():
    pin_worked_example_recurrence()


def test_worked_example_dense():
    pin_worked_example_dense()


@pytest.mark.parametrize("causal", [False, True])
def test_uniform_scores(causal):
    pin_uniform_scores(causal)


@pytest.mark.parametrize("causal", [False, True])
def test_constant_values(causal):
    pin_constant_values(causal)


@pytest.mark.parametrize("causal", [False, True])
def test_identity_values(causal):
    pin_identity_values(causal)


def test_spike():
    pin_spike()


def test_bruteforce_dense():
    pin_bruteforce_dense()


def test_bruteforce_paged():
    pin_bruteforce_paged()


def test_sdpa_crosscheck():
    pin_sdpa_crosscheck()


def test_permutation():
    pin_permutation()


def test_paged_spike():
    pin_paged_spike()


def test_paged_equals_dense():
    pin_paged_equals_dense()


def test_recurrence_partitions():
    pin_recurrence_partitions()


def test_merge():
    pin_merge()


def test_empty_context():
    pin_empty_context()


def test_attention_rows_matches_full():
    B, Hq, Hkv, N, d = 1, 4, 2, 300, 16
    q, k, v = _rand((B, Hq, N, d), 100), _rand((B, Hkv, N, d), 101), _rand((B, Hkv, N, d), 102)
    for causal in (False, True):
        o, lse = OA.attention(q, k, v, 0.25, causal=causal, workers=2, chunk=64)
        rows = np.array([0, 1, 63, 64, 150, 299])
        for h in range(Hq):
            orr, lr = OA.attention_rows(q, k, v, 0.25, causal, 0, h, rows)
            assert np.allclose(orr, o[0, h, rows], atol=1e-14)
            assert np.allclose(lr, lse[0, h, rows], atol=1e-14)


# ------------------------------------------------------ planted mistakes ----

def _make_mutant(strict=False, use_sigma=True, lse_max=True, normalise=True, kv=False):
    """A copy of the oracle's row computation with one plausible mistake."""
    def rows(q_rows, k, v, sigma, row_ids, causal):
        s = (sigma if use_sigma else 1.0) * (q_rows @ k.T)
        if causal:
            j = np.arange(k.shape[0])
            allowed = (j[None, :] < row_ids[:, None]) if strict else (j[None, :] <= row_ids[:, None])
            if strict:
                allowed[:, 0] = True                 # keep every row non-empty
            s = np.where(allowed, s, -np.inf)
        m = s.max(axis=1)
        w = np.exp(s - m[:, None])
        l = w.sum(axis=1)
        o = w @ (k if kv else v)
        if normalise:
            o = o / l[:, None]
        return o, (m if lse_max else 0.0) + np.log(l)
    return rows


def _mut_gqa_modulo(h, Hq, Hkv):
    return h % Hkv


@pytest.mark.parametrize("name,target,mutant", [
    ("causal diagonal dropped", "_complete_rows", _make_mutant(strict=True)),
    ("scale ignored", "_complete_rows", _make_mutant(use_sigma=False)),
    ("lse missing the max", "_complete_rows", _make_mutant(lse_max=False)),
    ("output not divided by l", "_complete_rows", _make_mutant(normalise=False)),
    ("keys used as values", "_complete_rows", _make_mutant(kv=True)),
    ("GQA heads interleaved", "kv_head_of", _mut_gqa_modulo),
])
def test_mutants_are_caught(monkeypatch, name, target, mutant):
    """Each planted mistake in the oracle must make some pin fail."""
    monkeypatch.setattr(OA, target, mutant)
    failed = []
    for pin in ALL_PINS:
        try:
            pin()
        except (AssertionError, ValueError):
            failed.append(pin)
    assert failed, f"no pin catches: {name}"


def test_unmutated_oracle_passes_every_pin():
    for pin in ALL_PINS:
        pin()


def test_package_exports():
    assert oracle.attention is OA.attention
    assert callable(oracle.paged_decode) and callable(oracle.online_aggregate)

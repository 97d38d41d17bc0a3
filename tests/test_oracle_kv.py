"""Pins of the paged-cache oracles that serve the steps either side of decode:
appending new tokens (oracle/kvcache.py) and chunked prefill over the paged
cache (oracle.exact.paged_prefill).

Each is checked against things it does not compute itself: reading back
through the already-pinned gather, literal worked cases, counts of changed
elements, dense causal attention (pinned against PyTorch's SDPA and 40-digit
brute force in test_oracle.py), the pinned decode, and brute force."""

import numpy as np
import pytest

from oracle import exact as OA
from oracle.kvcache import append_paged
from tests.bruteforce import bf_rows

BS = 16


def _pool(num_blocks, Hkv, d, fill=np.nan):
    return np.full((num_blocks, Hkv, BS, d), fill, dtype=np.float64)


def _starts(ns):
    return np.concatenate([[0], np.cumsum(ns)]).astype(np.int64)


# ------------------------------------------------------------- append ----

def test_literal_case_crosses_a_block_boundary():
    # one sequence growing from 15 to 18 positions: the three new tokens go to
    # block 7 slot 15, then block 2 slots 0 and 1
    kc, vc = _pool(9, 1, 2), _pool(9, 1, 2)
    table = np.array([[7, 2, -1]])
    kn = np.array([[[1.0, 2.0]], [[3.0, 4.0]], [[5.0, 6.0]]])
    k2, v2 = append_paged(kc, vc, table, [18], [0, 3], kn, -kn, BS)
    assert list(k2[7, 0, 15]) == [1.0, 2.0]
    assert list(k2[2, 0, 0]) == [3.0, 4.0]
    assert list(k2[2, 0, 1]) == [5.0, 6.0]
    assert list(v2[2, 0, 1]) == [-5.0, -6.0]
    assert np.isnan(k2[7, 0, 14]).all() and np.isnan(k2[2, 0, 2]).all()
    assert np.isnan(k2[[0, 1, 3, 4, 5, 6, 8]]).all()


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_chunks_read_back_through_the_table(seed):
    """Appending chunks of random sizes (some empty), starting from empty
    sequences, and reading back with the gather gives the chunks concatenated
    in order, for every sequence and kv head."""
    rng = np.random.default_rng(seed)
    S, Hkv, d, max_blocks = 4, 2, 8, 12
    num_blocks = S * max_blocks + 3
    table = rng.permutation(num_blocks)[:S * max_blocks].reshape(S, max_blocks)
    kc, vc = _pool(num_blocks, Hkv, d), _pool(num_blocks, Hkv, d)
    lens = np.zeros(S, dtype=np.int64)
    hist_k = [[] for _ in range(S)]
    hist_v = [[] for _ in range(S)]
    for _ in range(5):
        ns = rng.integers(0, 30, S)
        T = int(ns.sum())
        kn = rng.standard_normal((T, Hkv, d))
        vn = rng.standard_normal((T, Hkv, d))
        st = _starts(ns)
        lens = lens + ns
        kc, vc = append_paged(kc, vc, table, lens, st, kn, vn, BS)
        for s in range(S):
            hist_k[s].append(kn[st[s]:st[s + 1]])
            hist_v[s].append(vn[st[s]:st[s + 1]])
    for s in range(S):
        want_k = np.concatenate(hist_k[s], axis=0)   # [len, Hkv, d]
        want_v = np.concatenate(hist_v[s], axis=0)
        for g in range(Hkv):
            kk, vv = OA.gather_paged_kv(kc, vc, table, lens[s], s, g, BS)
            assert np.array_equal(kk, want_k[:, g, :])
            assert np.array_equal(vv, want_v[:, g, :])
    # nothing else changed: exactly the appended elements differ from NaN
    assert int(np.count_nonzero(~np.isnan(kc))) == int(lens.sum()) * Hkv * d


def test_decode_after_append_is_dense_attention():
    rng = np.random.default_rng(5)
    S, Hq, Hkv, d, max_blocks = 3, 4, 2, 16, 6
    num_blocks = S * max_blocks
    table = rng.permutation(num_blocks).reshape(S, max_blocks)
    lens0 = np.array([0, 17, 40])
    k_old = rng.standard_normal((S, 40, Hkv, d))
    v_old = rng.standard_normal((S, 40, Hkv, d))
    kc, vc = _pool(num_blocks, Hkv, d), _pool(num_blocks, Hkv, d)
    # the old positions as one packed append, then 9 more tokens each
    rows = np.concatenate([k_old[s, :lens0[s]] for s in range(S)])
    rows_v = np.concatenate([v_old[s, :lens0[s]] for s in range(S)])
    kc, vc = append_paged(kc, vc, table, lens0, _starts(lens0), rows, rows_v, BS)
    kn = rng.standard_normal((S * 9, Hkv, d))
    vn = rng.standard_normal((S * 9, Hkv, d))
    kc, vc = append_paged(kc, vc, table, lens0 + 9, _starts([9] * S), kn, vn, BS)
    q = rng.standard_normal((S, Hq, d))
    o, lse = OA.paged_decode(q, kc, vc, table, lens0 + 9, BS, 0.25)
    for s in range(S):
        K = np.concatenate([k_old[s, :lens0[s]], kn[9 * s:9 * s + 9]], axis=0).transpose(1, 0, 2)[None]
        V = np.concatenate([v_old[s, :lens0[s]], vn[9 * s:9 * s + 9]], axis=0).transpose(1, 0, 2)[None]
        for h in range(Hq):
            ro, rl = OA.attention_rows(q[s][None, :, None, :], K, V, 0.25, False, 0, h, [0])
            assert np.allclose(o[s, h], ro[0], rtol=0, atol=1e-12)
            assert np.allclose(lse[s, h], rl[0], rtol=0, atol=1e-12)


def test_out_of_range_tokens_are_not_written():
    rng = np.random.default_rng(7)
    Hkv, d = 1, 4
    kc, vc = _pool(5, Hkv, d), _pool(5, Hkv, d)
    table = np.array([[0, -1], [9, 1], [2, 3], [4, 4]])   # -1 and 9 are not blocks
    lens = np.array([18, 4, 34, 2])
    st = np.array([0, 4, 8, 12, 16])                      # 4 new tokens each
    kn = rng.standard_normal((16, Hkv, d))
    k2, _ = append_paged(kc, vc, table, lens, st, kn, kn, BS)
    # seq 0: positions 14, 15 land in block 0; 16, 17 need entry -1 -> dropped
    assert np.array_equal(k2[0, 0, 14], kn[0, 0]) and np.array_equal(k2[0, 0, 15], kn[1, 0])
    # seq 1: entry 9 is not a block -> nothing
    # seq 2: 30, 31 in block 3; 32, 33 are past the table's width -> dropped
    assert np.array_equal(k2[3, 0, 14], kn[8, 0]) and np.array_equal(k2[3, 0, 15], kn[9, 0])
    # seq 3: length 2 < 4 new tokens -> nothing; every other slot untouched
    assert int(np.count_nonzero(~np.isnan(k2))) == 4 * d
    # decreasing offsets: seq 0 (rows 0..3, positions 0..3 of block 0) is
    # written, seq 1 (rows 4..2) is skipped
    k3, _ = append_paged(kc, vc, table[:2], [4, 4], [0, 4, 2], kn[:4], kn[:4], BS)
    assert np.array_equal(k3[0, 0, :4], kn[:4, 0])
    assert int(np.count_nonzero(~np.isnan(k3))) == 4 * d
    # offsets past the last row -> skipped
    k4, _ = append_paged(kc, vc, table[:1], [5], [0, 5], kn[:4], kn[:4], BS)
    assert int(np.count_nonzero(~np.isnan(k4))) == 0


# ----------------------------------------------------- chunked prefill ----

def _paged_from_dense(K, V, rng, max_blocks, spare=3):
    """Scatter dense per-sequence K, V ([S][n_s, Hkv, d]) into a shuffled
    pool; returns (kc, vc, table)."""
    S = len(K)
    Hkv, d = K[0].shape[1], K[0].shape[2]
    nblk = [(k.shape[0] + BS - 1) // BS for k in K]
    num_blocks = sum(nblk) + spare
    perm = rng.permutation(num_blocks)
    table = np.full((S, max_blocks), -1, dtype=np.int64)
    kc = rng.standard_normal((num_blocks, Hkv, BS, d))     # garbage everywhere else
    vc = rng.standard_normal((num_blocks, Hkv, BS, d))
    off = 0
    for s in range(S):
        table[s, :nblk[s]] = perm[off:off + nblk[s]]
        off += nblk[s]
        for p in range(K[s].shape[0]):
            kc[table[s, p // BS], :, p % BS] = K[s][p]
            vc[table[s, p // BS], :, p % BS] = V[s][p]
    return kc, vc, table


def test_chunked_prefill_is_the_tail_of_dense_causal_attention():
    """The n_s new rows of a sequence of length L are rows L-n_s..L-1 of dense
    causal attention over the whole sequence."""
    rng = np.random.default_rng(11)
    Hq, Hkv, d = 6, 2, 16
    L = [37, 16, 70, 5]
    ns = [37, 3, 20, 1]          # a fresh prompt, a short chunk, a long chunk, a decode-like row
    K = [rng.standard_normal((n, Hkv, d)) for n in L]
    V = [rng.standard_normal((n, Hkv, d)) for n in L]
    Qfull = [rng.standard_normal((n, Hq, d)) for n in L]
    kc, vc, table = _paged_from_dense(K, V, rng, max_blocks=6)
    q = np.concatenate([Qfull[s][L[s] - ns[s]:] for s in range(4)])
    o, lse = OA.paged_prefill(q, kc, vc, table, L, _starts(ns), BS, 0.3, workers=2)
    st = _starts(ns)
    for s in range(4):
        Qd = Qfull[s].transpose(1, 0, 2)[None]
        Kd = K[s].transpose(1, 0, 2)[None]
        Vd = V[s].transpose(1, 0, 2)[None]
        od, ld = OA.attention(Qd, Kd, Vd, 0.3, causal=True, workers=1)
        tail = slice(L[s] - ns[s], L[s])
        assert np.allclose(o[st[s]:st[s + 1]], od[0][:, tail].transpose(1, 0, 2), atol=1e-13, rtol=0)
        assert np.allclose(lse[st[s]:st[s + 1]], ld[0][:, tail].T, atol=1e-13, rtol=0)


def test_single_new_row_is_decode():
    rng = np.random.default_rng(12)
    S, Hq, Hkv, d = 3, 4, 1, 8
    L = [1, 33, 64]
    K = [rng.standard_normal((n, Hkv, d)) for n in L]
    V = [rng.standard_normal((n, Hkv, d)) for n in L]
    kc, vc, table = _paged_from_dense(K, V, rng, max_blocks=5)
    q = rng.standard_normal((S, Hq, d))
    o, lse = OA.paged_prefill(q, kc, vc, table, L, np.arange(S + 1), BS, 0.7, workers=1)
    od, ld = OA.paged_decode(q, kc, vc, table, L, BS, 0.7, workers=1)
    assert np.allclose(o, od, atol=1e-14, rtol=0) and np.allclose(lse, ld, atol=1e-14, rtol=0)


def test_chunked_prefill_bruteforce():
    """40-digit brute force over explicitly enumerated key positions."""
    rng = np.random.default_rng(13)
    Hq, Hkv, d = 2, 1, 3
    L, ns = [19, 6], [4, 6]
    K = [rng.standard_normal((n, Hkv, d)) for n in L]
    V = [rng.standard_normal((n, Hkv, d)) for n in L]
    kc, vc, table = _paged_from_dense(K, V, rng, max_blocks=2)
    q = rng.standard_normal((sum(ns), Hq, d))
    o, lse = OA.paged_prefill(q, kc, vc, table, L, _starts(ns), BS, 0.9, workers=1)
    st = _starts(ns)
    for s in range(2):
        first = L[s] - ns[s]
        sets = [list(range(first + t + 1)) for t in range(ns[s])]
        for h in range(Hq):
            ob, lb = bf_rows(q[st[s]:st[s + 1], h], K[s][:, 0], V[s][:, 0], float(np.float32(0.9)), sets)
            assert np.allclose(o[st[s]:st[s + 1], h], ob, atol=1e-14, rtol=0)
            assert np.allclose(lse[st[s]:st[s + 1], h], lb, atol=1e-13, rtol=0)


def test_chunked_prefill_bad_inputs_give_nan():
    rng = np.random.default_rng(14)
    Hq, Hkv, d = 2, 1, 4
    L = [40, 40, 40]
    K = [rng.standard_normal((n, Hkv, d)) for n in L]
    kc, vc, table = _paged_from_dense(K, K, rng, max_blocks=3)
    table[1, 1] = 10 ** 6                # block 1 (positions 16..31) of seq 1 is bad
    q = rng.standard_normal((12, Hq, d))
    lens = np.array([40, 40, 3])         # seq 2: 4 new rows but length 3
    o, lse = OA.paged_prefill(q, kc, vc, table, lens, [0, 4, 8, 12], BS, 0.5, workers=1)
    assert np.isfinite(o[0:4]).all()
    assert np.isnan(o[4:8]).all()        # rows at 36..39 all read block 1
    assert np.isnan(o[8:12]).all() and np.isnan(lse[8:12]).all()
    # with 30 new rows in seq 1, rows at positions 10..15 only need block 0
    q2 = rng.standard_normal((30, Hq, d))
    o2, _ = OA.paged_prefill(q2, kc, vc, table[1:2], [40], [0, 30], BS, 0.5, workers=1)
    assert np.isfinite(o2[:6]).all() and np.isnan(o2[6:]).all()

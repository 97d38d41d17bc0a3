"""Pins of the paged KV-append oracle (oracle/kvcache.py) against things it
does not compute itself: reading back through the block table with the
already-pinned gather, a literal worked case, the count of changed elements,
and decode after append against dense attention."""

import numpy as np
import pytest

from oracle import exact as OA
from oracle.kvcache import append_paged

BS = 16


def _pool(num_blocks, Hkv, d, fill=np.nan):
    return np.full((num_blocks, Hkv, BS, d), fill, dtype=np.float64)


def test_literal_case_crosses_a_block_boundary():
    # one sequence holding 15 positions in block 7; three new tokens go to
    # block 7 slot 15, then block 2 slots 0 and 1
    kc, vc = _pool(9, 1, 2), _pool(9, 1, 2)
    table = np.array([[7, 2, -1]])
    kn = np.array([[[[1.0, 2.0]], [[3.0, 4.0]], [[5.0, 6.0]]]])
    k2, v2 = append_paged(kc, vc, table, [15], kn, -kn, BS)
    assert list(k2[7, 0, 15]) == [1.0, 2.0]
    assert list(k2[2, 0, 0]) == [3.0, 4.0]
    assert list(k2[2, 0, 1]) == [5.0, 6.0]
    assert list(v2[2, 0, 1]) == [-5.0, -6.0]
    assert np.isnan(k2[7, 0, 14]).all() and np.isnan(k2[2, 0, 2]).all()
    assert np.isnan(k2[[0, 1, 3, 4, 5, 6, 8]]).all()


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_chunks_read_back_through_the_table(seed):
    """Appending chunks of random sizes, starting from empty sequences, and
    reading back with the (separately pinned) gather gives the chunks
    concatenated in order, for every sequence and kv head."""
    rng = np.random.default_rng(seed)
    S, Hkv, d, max_blocks = 4, 2, 8, 12
    num_blocks = S * max_blocks + 3
    perm = rng.permutation(num_blocks)
    table = perm[:S * max_blocks].reshape(S, max_blocks)
    kc, vc = _pool(num_blocks, Hkv, d), _pool(num_blocks, Hkv, d)
    lens = np.zeros(S, dtype=np.int64)
    hist_k = [[] for _ in range(S)]
    hist_v = [[] for _ in range(S)]
    for _ in range(5):
        n_new = int(rng.integers(1, 30))
        kn = rng.standard_normal((S, n_new, Hkv, d))
        vn = rng.standard_normal((S, n_new, Hkv, d))
        kc, vc = append_paged(kc, vc, table, lens, kn, vn, BS)
        for s in range(S):
            hist_k[s].append(kn[s])
            hist_v[s].append(vn[s])
        lens = lens + n_new
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
    # fill the old positions, then append 9 more
    for s in range(S):
        kc, vc = append_paged(kc, vc, table[s:s + 1], [0], k_old[s:s + 1, :lens0[s]],
                              v_old[s:s + 1, :lens0[s]], BS) if lens0[s] else (kc, vc)
    kn = rng.standard_normal((S, 9, Hkv, d))
    vn = rng.standard_normal((S, 9, Hkv, d))
    kc, vc = append_paged(kc, vc, table, lens0, kn, vn, BS)
    q = rng.standard_normal((S, Hq, d))
    o, lse = OA.paged_decode(q, kc, vc, table, lens0 + 9, BS, 0.25)
    for s in range(S):
        K = np.concatenate([k_old[s, :lens0[s]], kn[s]], axis=0).transpose(1, 0, 2)[None]   # [1,Hkv,n,d]
        V = np.concatenate([v_old[s, :lens0[s]], vn[s]], axis=0).transpose(1, 0, 2)[None]
        for h in range(Hq):
            ro, rl = OA.attention_rows(q[s][None, :, None, :], K, V, 0.25, False, 0, h, [0])
            assert np.allclose(o[s, h], ro[0], rtol=0, atol=1e-12)
            assert np.allclose(lse[s, h], rl[0], rtol=0, atol=1e-12)


def test_out_of_range_tokens_are_not_written():
    rng = np.random.default_rng(7)
    Hkv, d = 1, 4
    kc, vc = _pool(5, Hkv, d), _pool(5, Hkv, d)
    table = np.array([[0, -1], [9, 1], [2, 3], [4, 4]])     # -1 and 9 are not blocks
    lens = np.array([14, 0, 30, -2])                          # seq 2 runs past 2 blocks; seq 3 invalid
    kn = rng.standard_normal((4, 4, Hkv, d))
    k2, _ = append_paged(kc, vc, table, lens, kn, kn, BS)
    # seq 0: positions 14, 15 land in block 0; 16, 17 need entry -1 -> dropped
    assert np.array_equal(k2[0, 0, 14], kn[0, 0, 0]) and np.array_equal(k2[0, 0, 15], kn[0, 1, 0])
    # seq 1: block 9 does not exist -> nothing; seq 2: 30, 31 in block 3, 32, 33 past max_blocks
    assert np.array_equal(k2[3, 0, 14], kn[2, 0, 0]) and np.array_equal(k2[3, 0, 15], kn[2, 1, 0])
    # seq 3: negative length -> nothing; every other slot untouched
    assert int(np.count_nonzero(~np.isnan(k2))) == 4 * d

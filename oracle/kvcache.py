"""Appending new tokens' keys and values to a paged KV cache, plainly.

TEST INFRASTRUCTURE ONLY (see the package docstring): never imported by the
product path.

What is computed ([KR] "Atención tipo FlashAttention y atención paginada"):
the KV cache keeps the keys and values already computed and grows one token
(or one chunk of tokens) at a time; it is stored as a pool of fixed-size
blocks, and a block table maps each sequence's logical positions to physical
blocks.  Logical position p of sequence s lives in physical block
block_table[s, p // block_size], slot p % block_size, for every kv head.

Readings (listed with their reasons in the design notes):
  * the new tokens of all sequences are packed row after row: k_new, v_new
    are [T, Hkv, d] and the n_s = starts[s+1] - starts[s] new tokens of
    sequence s are rows starts[s] .. starts[s+1]-1 (n_s may be 0)
  * ctx_lens[s] is the length AFTER the append, the same length the decode
    and the chunked prefill read: the new tokens take positions
    ctx_lens[s] - n_s .. ctx_lens[s] - 1, in row order
  * the caller has already placed table entries for the blocks those
    positions fall in; nothing here changes the table or the lengths
  * a sequence whose rows or lengths are malformed (starts decreasing or
    outside [0, T], or ctx_lens[s] < n_s) is not written at all; a single
    token whose block index is past the table's width, or whose table entry
    is outside [0, num_blocks), is not written
"""

from __future__ import annotations

import numpy as np


def append_paged(k_cache, v_cache, block_table, ctx_lens, starts, k_new, v_new, block_size):
    """Return copies of (k_cache, v_cache) with the new tokens written in.

    One token at a time, straight from the definition above.
    k_cache, v_cache: [num_blocks, Hkv, block_size, d]; block_table:
    [S, max_blocks]; ctx_lens: [S]; starts: [S + 1]; k_new, v_new: [T, Hkv, d].
    """
    kc = np.array(k_cache, copy=True)
    vc = np.array(v_cache, copy=True)
    table = np.asarray(block_table)
    lens = np.asarray(ctx_lens)
    starts = np.asarray(starts)
    kn = np.asarray(k_new)
    vn = np.asarray(v_new)
    T, Hkv, d = kn.shape
    S = table.shape[0]
    num_blocks = kc.shape[0]
    max_blocks = table.shape[1]
    for s in range(S):
        a, b = int(starts[s]), int(starts[s + 1])
        n = b - a
        if a < 0 or b > T or n < 0 or int(lens[s]) < n:
            continue
        first = int(lens[s]) - n
        for t in range(n):
            p = first + t
            blk = p // block_size
            if blk >= max_blocks:
                continue
            phys = int(table[s, blk])
            if phys < 0 or phys >= num_blocks:
                continue
            for g in range(Hkv):
                kc[phys, g, p % block_size, :] = kn[a + t, g, :]
                vc[phys, g, p % block_size, :] = vn[a + t, g, :]
    return kc, vc

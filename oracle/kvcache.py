"""Appending new tokens' keys and values to a paged KV cache, plainly.

TEST INFRASTRUCTURE ONLY (see the package docstring): never imported by the
product path.

What is computed ([KR] "Atención tipo FlashAttention y atención paginada"):
the KV cache keeps the keys and values already computed and grows one token
(or one chunk of tokens) at a time; it is stored as a pool of fixed-size
blocks, and a block table maps each sequence's logical positions to physical
blocks.  Appending n_new tokens to sequence s whose cache already holds
ctx_lens[s] positions writes token t at logical position p = ctx_lens[s] + t,
i.e. into physical block block_table[s, p // block_size], slot
p % block_size, for every kv head.

Readings (listed with their reasons in the design notes):
  * layout  k_new, v_new: [S, n_new, Hkv, d] (token-major, as a projection
            emits them); caches [num_blocks, Hkv, block_size, d]
  * the caller has already placed table entries for the blocks the new
            positions fall in; ctx_lens is the length before the append and
            is not modified
  * a token whose block index p // block_size is outside [0, max_blocks), or
            whose table entry is outside [0, num_blocks), or whose sequence
            has a negative length, is not written anywhere
"""

from __future__ import annotations

import numpy as np


def append_paged(k_cache, v_cache, block_table, ctx_lens, k_new, v_new, block_size):
    """Return copies of (k_cache, v_cache) with the new tokens written in.

    One token at a time, straight from the definition above.
    """
    kc = np.array(k_cache, copy=True)
    vc = np.array(v_cache, copy=True)
    table = np.asarray(block_table)
    lens = np.asarray(ctx_lens)
    kn = np.asarray(k_new)
    vn = np.asarray(v_new)
    S, n_new, Hkv, d = kn.shape
    num_blocks = kc.shape[0]
    max_blocks = table.shape[1]
    for s in range(S):
        if int(lens[s]) < 0:
            continue
        for t in range(n_new):
            p = int(lens[s]) + t
            b = p // block_size
            if b >= max_blocks:
                continue
            phys = int(table[s, b])
            if phys < 0 or phys >= num_blocks:
                continue
            for g in range(Hkv):
                kc[phys, g, p % block_size, :] = kn[s, t, g, :]
                vc[phys, g, p % block_size, :] = vn[s, t, g, :]
    return kc, vc

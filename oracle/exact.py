"""The definition of exact scaled-dot-product attention, in float64 on the CPU.

TEST INFRASTRUCTURE ONLY (see the package docstring): never imported by the
product path.

What is computed (page [AT] section 1; page [FA] "No basta con promediar..."):
for a query row q_i and the keys k_j / values v_j it may attend to,

    s_ij  = sigma * <q_i, k_j>                       (scaled score)
    m_i   = max_j s_ij
    l_i   = sum_j exp(s_ij - m_i)                    (sum of weights)
    o_i   = sum_j exp(s_ij - m_i) v_j / l_i          (u / l)
    lse_i = m_i + ln l_i                             (saved statistic)

Every score row is materialised in full: this is the "standard" attention the
pages contrast FlashAttention with ([AT] section 3), which is exactly what
the tiled method must reproduce up to floating-point order ([FA] "Mecanismo
y detalles").  Subtracting m_i before exp is the textbook stable softmax: it
changes no value of the weights, only avoids overflow.

Readings where the pages are silent (listed with their reasons in the design
notes):
  * layout  q, o: [B, Hq, N, d];  k, v: [B, Hkv, N, d];  lse: [B, Hq, N]
  * sigma   the scale is carried as a 32-bit float by the library ABI, so the
            oracle uses float64(float32(scale))
  * causal  key j is allowed for query i iff j <= i (one N for queries and
            keys, diagonal included)
  * GQA     Hq % Hkv == 0; query head h reads kv head h // (Hq // Hkv)
            (contiguous groups; [FA] last section only says K/V heads are fewer)
  * paged   k_cache, v_cache: [num_blocks, Hkv, block_size, d]; logical
            position p of sequence s lives in physical block
            block_table[s, p // block_size], slot p % block_size ([KR]
            "Atención tipo FlashAttention y atención paginada"); the single
            decode query attends to all ctx_lens[s] positions; an empty
            context gives o = 0 and lse = -inf.
  * chunked the new query rows of all sequences are packed: q, o [T, Hq, d],
            lse [T, Hq]; rows starts[s] .. starts[s+1]-1 belong to sequence
            s, whose ctx_lens[s] positions already include them, so its
            t-th new row sits at position ctx_lens[s] - n_s + t and attends
            to positions 0 .. that one (causal, diagonal included).
"""

from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

__all__ = ["sigma_of", "kv_head_of", "attention", "attention_rows",
           "gather_paged_kv", "paged_decode", "paged_prefill", "default_workers"]


def sigma_of(scale: float) -> float:
    """The scale as the kernel receives it: a float32, widened to float64."""
    return float(np.float32(scale))


def kv_head_of(h: int, Hq: int, Hkv: int) -> int:
    """GQA head sharing: contiguous groups of G = Hq // Hkv query heads."""
    if Hq % Hkv:
        raise ValueError("Hq must be a multiple of Hkv")
    return h // (Hq // Hkv)


def _complete_rows(q_rows, k, v, sigma, row_ids, causal):
    """o, lse for complete score rows.

    q_rows: [R, d] queries at positions row_ids; k, v: [Nk, d] keys/values at
    positions 0..Nk-1, which must include every key the rows may attend to.
    """
    s = sigma * (q_rows @ k.T)                       # [R, Nk] scaled scores
    if causal:
        j = np.arange(k.shape[0])
        s = np.where(j[None, :] <= row_ids[:, None], s, -np.inf)
    m = s.max(axis=1)
    w = np.exp(s - m[:, None])                       # unnormalised weights
    l = w.sum(axis=1)
    o = (w @ v) / l[:, None]
    lse = m + np.log(l)
    return o, lse


def default_workers() -> int:
    try:
        return max(1, len(os.sched_getaffinity(0)))
    except AttributeError:  # pragma: no cover - non-Linux
        return max(1, os.cpu_count() or 1)


def _run_items(fn, items, workers):
    """Map fn over items, in a thread pool with single-threaded BLAS."""
    if workers <= 1 or len(items) <= 1:
        return [fn(it) for it in items]
    try:
        from threadpoolctl import threadpool_limits
        limiter = threadpool_limits(limits=1)
    except Exception:  # pragma: no cover - threadpoolctl missing
        limiter = None
    try:
        with ThreadPoolExecutor(max_workers=workers) as ex:
            return list(ex.map(fn, items))
    finally:
        if limiter is not None:
            limiter.restore_original_limits()


def attention(q, k, v, scale, causal=False, *, workers=None, chunk=512):
    """Dense attention forward, the plain definition in float64.

    q: [B, Hq, N, d]; k, v: [B, Hkv, N, d] (any real dtype; widened to
    float64).  Returns (o [B, Hq, N, d], lse [B, Hq, N]) as float64.

    Rows are processed in chunks of complete rows (each chunk still sees its
    whole score rows), so this is the definition, not a recurrence.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    B, Hq, N, d = q.shape
    Hkv = k.shape[1]
    if k.shape != (B, Hkv, N, d) or v.shape != k.shape:
        raise ValueError("k and v must be [B, Hkv, N, d] matching q")
    sigma = sigma_of(scale)
    o = np.empty_like(q)
    lse = np.empty((B, Hq, N), dtype=np.float64)

    items = [(b, h, r0, min(N, r0 + chunk))
             for b in range(B) for h in range(Hq) for r0 in range(0, N, chunk)]

    def work(item):
        b, h, r0, r1 = item
        g = kv_head_of(h, Hq, Hkv)
        nk = r1 if causal else N                  # every allowed key of rows r0..r1-1
        rows = np.arange(r0, r1)
        ob, lb = _complete_rows(q[b, h, r0:r1], k[b, g, :nk], v[b, g, :nk],
                                sigma, rows, causal)
        o[b, h, r0:r1] = ob
        lse[b, h, r0:r1] = lb

    _run_items(work, items, default_workers() if workers is None else workers)
    return o, lse


def attention_rows(q, k, v, scale, causal, b, h, rows):
    """Selected query rows of one (batch, query head): the same definition.

    Used to check full-size runs at sampled outputs.  q: [B, Hq, N, d] or the
    single row block q[b, h] is read; k, v as in `attention`.
    Returns (o [len(rows), d], lse [len(rows)]) in float64.
    """
    rows = np.asarray(rows, dtype=np.int64)
    Hq, Hkv = q.shape[1], k.shape[1]
    g = kv_head_of(h, Hq, Hkv)
    N = k.shape[2]
    nk = int(rows.max()) + 1 if causal else N
    qr = np.asarray(q[b, h][rows], dtype=np.float64)
    kk = np.asarray(k[b, g, :nk], dtype=np.float64)
    vv = np.asarray(v[b, g, :nk], dtype=np.float64)
    return _complete_rows(qr, kk, vv, sigma_of(scale), rows, causal)


def gather_paged_kv(k_cache, v_cache, block_table, ctx_len, s, g, block_size):
    """Logical K, V [ctx_len, d] of sequence s, kv head g, read through the
    block table: position p -> (block_table[s, p // bs], g, p % bs)."""
    p = np.arange(int(ctx_len))
    blocks = np.asarray(block_table)[s, p // block_size]
    slots = p % block_size
    kk = np.asarray(k_cache)[blocks, g, slots, :]
    vv = np.asarray(v_cache)[blocks, g, slots, :]
    return kk.astype(np.float64), vv.astype(np.float64)


def paged_decode(q, k_cache, v_cache, block_table, ctx_lens, block_size, scale,
                 *, workers=None):
    """Single-token decode over a paged KV cache, the plain definition.

    q: [S, Hq, d]; k_cache, v_cache: [num_blocks, Hkv, block_size, d];
    block_table: int [S, max_blocks]; ctx_lens: int [S].
    Returns (o [S, Hq, d], lse [S, Hq]) as float64.  A sequence with
    ctx_len 0 gives o = 0 and lse = -inf.
    """
    q = np.asarray(q, dtype=np.float64)
    S, Hq, d = q.shape
    Hkv = np.asarray(k_cache).shape[1]
    sigma = sigma_of(scale)
    o = np.zeros((S, Hq, d), dtype=np.float64)
    lse = np.full((S, Hq), -np.inf, dtype=np.float64)
    ctx_lens = np.asarray(ctx_lens)

    def work(item):
        s, g = item
        n = int(ctx_lens[s])
        if n == 0:
            return
        kk, vv = gather_paged_kv(k_cache, v_cache, block_table, n, s, g, block_size)
        heads = [h for h in range(Hq) if kv_head_of(h, Hq, Hkv) == g]
        ob, lb = _complete_rows(q[s, heads], kk, vv, sigma,
                                np.zeros(len(heads), dtype=np.int64), False)
        o[s, heads] = ob
        lse[s, heads] = lb

    items = [(s, g) for s in range(S) for g in range(Hkv)]
    _run_items(work, items, default_workers() if workers is None else workers)
    return o, lse


def paged_prefill(q, k_cache, v_cache, block_table, ctx_lens, starts, block_size, scale,
                  *, workers=None):
    """Chunked prefill over a paged KV cache, the plain definition.

    q: [T, Hq, d] packed new rows; k_cache, v_cache: [num_blocks, Hkv,
    block_size, d]; block_table: int [S, max_blocks]; ctx_lens: int [S]
    (lengths including the new rows); starts: int [S + 1].
    Returns (o [T, Hq, d], lse [T, Hq]) as float64.  Row t of sequence s is
    query position ctx_lens[s] - n_s + t, which sees keys 0 .. that position
    gathered through the table.  Rows that belong to no sequence are NaN.

    The library's contract for inputs it cannot check before launch is
    modelled too: a sequence with ctx_lens[s] < n_s or ctx_lens[s] >
    max_blocks * block_size gets NaN rows, and so does every row whose keys
    include a block with a table entry outside [0, num_blocks).
    """
    q = np.asarray(q, dtype=np.float64)
    T, Hq, d = q.shape
    kc, vc = np.asarray(k_cache), np.asarray(v_cache)
    num_blocks, Hkv = kc.shape[0], kc.shape[1]
    table = np.asarray(block_table)
    max_blocks = table.shape[1]
    ctx_lens, starts = np.asarray(ctx_lens), np.asarray(starts)
    S = table.shape[0]
    sigma = sigma_of(scale)
    o = np.full((T, Hq, d), np.nan)
    lse = np.full((T, Hq), np.nan)

    def work(item):
        s, g = item
        a, b = int(starts[s]), int(starts[s + 1])
        n, ctx = b - a, int(ctx_lens[s])
        if n <= 0 or ctx < n or ctx > max_blocks * block_size:
            return
        first = ctx - n
        pos = first + np.arange(n)
        entries = table[s, :(ctx + block_size - 1) // block_size]
        bad = np.nonzero((entries < 0) | (entries >= num_blocks))[0]
        ok = pos < (bad[0] * block_size if len(bad) else ctx)   # rows that read only good blocks
        if not ok.any():
            return
        nk = int(pos[ok].max()) + 1
        kk, vv = gather_paged_kv(kc, vc, table, nk, s, g, block_size)
        heads = [h for h in range(Hq) if kv_head_of(h, Hq, Hkv) == g]
        rows = np.nonzero(ok)[0]
        for h in heads:
            ob, lb = _complete_rows(q[a + rows, h], kk, vv, sigma, pos[rows], True)
            o[a + rows, h] = ob
            lse[a + rows, h] = lb

    items = [(s, g) for s in range(S) for g in range(Hkv)
             if 0 <= int(starts[s]) <= int(starts[s + 1]) <= T]
    _run_items(work, items, default_workers() if workers is None else workers)
    return o, lse

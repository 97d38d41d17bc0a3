"""Gradients of exact scaled-dot-product attention, in float64 on the CPU.

TEST INFRASTRUCTURE ONLY (see the package docstring): never imported by the
product path.

What is computed.  The forward pass keeps only o and the per-row statistic
lse, and the backward pass recomputes the attention weights from q, k and
lse instead of storing them ([AT] section 3, "Recálculo durante la
retropropagación"; [FA] "Mecanismo y detalles": the result is exact, so its
gradient is the gradient of the plain definition).  For one head, with the
allowed keys of row i as in the forward (causal or not) and sigma the scale:

    s_ij  = sigma * <q_i, k_j>
    p_ij  = exp(s_ij - lse_i)                     (= softmax_j, 0 if masked)
    o_i   = sum_j p_ij v_j
    dv_j  = sum_i p_ij do_i
    dp_ij = <do_i, v_j>
    D_i   = sum_j p_ij dp_ij  (= <do_i, o_i>)
    ds_ij = p_ij (dp_ij - D_i)
    dq_i  = sigma * sum_j ds_ij k_j
    dk_j  = sigma * sum_i ds_ij q_i

These are the chain rule through o = P V and the softmax Jacobian
(d p_ij / d s_il = p_ij (delta_jl - p_il)), written out.  With grouped K/V
heads, dk and dv of a kv head are the sums over the query heads that read it.

Readings (listed with their reasons in the design notes):
  * the gradient is taken of the loss whose gradient with respect to o is
    `do` (the caller's upstream gradient), for the exact forward, so it needs
    neither the forward's rounded o nor its lse: they are recomputed here in
    float64 from q, k, v
  * layout and GQA mapping as in the forward (exact.py)
"""

from __future__ import annotations

import numpy as np

from .exact import _run_items, default_workers, kv_head_of, sigma_of

__all__ = ["attention_bwd"]


def _head_bwd(q, k, v, do, sigma, causal, chunk):
    """dq [N, d], dk [N, d], dv [N, d] of one query head against its kv head.

    Query rows are processed in chunks of complete rows: each chunk's weight
    rows are whole, so this is the definition, chunk by chunk.
    """
    N = q.shape[0]
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    for r0 in range(0, N, chunk):
        r1 = min(N, r0 + chunk)
        s = sigma * (q[r0:r1] @ k.T)                          # [R, N]
        if causal:
            j = np.arange(N)
            i = np.arange(r0, r1)
            s = np.where(j[None, :] <= i[:, None], s, -np.inf)
        m = s.max(axis=1, keepdims=True)
        w = np.exp(s - m)
        p = w / w.sum(axis=1, keepdims=True)                  # softmax rows
        g = do[r0:r1]
        dv += p.T @ g
        dp = g @ v.T
        D = (p * dp).sum(axis=1, keepdims=True)
        ds = p * (dp - D)
        dq[r0:r1] = sigma * (ds @ k)
        dk += sigma * (ds.T @ q[r0:r1])
    return dq, dk, dv


def attention_bwd(q, k, v, do, scale, causal=False, *, workers=None, chunk=512):
    """Gradients (dq, dk, dv) of exact attention, float64.

    q, do: [B, Hq, N, d]; k, v: [B, Hkv, N, d].  Returns dq [B, Hq, N, d] and
    dk, dv [B, Hkv, N, d] (summed over each kv head's query heads).
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    do = np.asarray(do, dtype=np.float64)
    B, Hq, N, d = q.shape
    Hkv = k.shape[1]
    if k.shape != (B, Hkv, N, d) or v.shape != k.shape or do.shape != q.shape:
        raise ValueError("q, do must be [B, Hq, N, d] and k, v [B, Hkv, N, d]")
    sigma = sigma_of(scale)
    dq = np.empty_like(q)
    per_head = {}

    def work(item):
        b, h = item
        g = kv_head_of(h, Hq, Hkv)
        dqh, dkh, dvh = _head_bwd(q[b, h], k[b, g], v[b, g], do[b, h], sigma, causal, chunk)
        dq[b, h] = dqh
        per_head[(b, h)] = (dkh, dvh)

    items = [(b, h) for b in range(B) for h in range(Hq)]
    _run_items(work, items, default_workers() if workers is None else workers)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    for b in range(B):
        for h in range(Hq):                                   # fixed order: deterministic sums
            g = kv_head_of(h, Hq, Hkv)
            dk[b, g] += per_head[(b, h)][0]
            dv[b, g] += per_head[(b, h)][1]
    return dq, dk, dv

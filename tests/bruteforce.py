"""40-digit brute force of attention on tiny inputs (Python decimal, loops).

Independent of the float64 oracle: no BLAS, no vectorised masking, every
allowed key enumerated explicitly, exp and ln at 40 significant digits.
Float inputs are converted to Decimal exactly.
"""

from decimal import Decimal, localcontext

import numpy as np


def _dec(x):
    return Decimal(float(x))


def bf_rows(qrows, keys, vals, sigma, allowed_sets, digits=40):
    """Outputs and log-sum-exps for query rows with explicit allowed key sets."""
    outs, lses = [], []
    with localcontext() as ctx:
        ctx.prec = digits
        sg = _dec(sigma)
        for qi, allowed in zip(qrows, allowed_sets):
            if not allowed:
                outs.append([0.0] * vals.shape[1])
                lses.append(float("-inf"))
                continue
            s = []
            for j in allowed:
                acc = Decimal(0)
                for c in range(len(qi)):
                    acc += _dec(qi[c]) * _dec(keys[j][c])
                s.append(sg * acc)
            m = max(s)
            w = [(sj - m).exp() for sj in s]
            l = sum(w, Decimal(0))
            o = []
            for c in range(vals.shape[1]):
                num = Decimal(0)
                for wj, j in zip(w, allowed):
                    num += wj * _dec(vals[j][c])
                o.append(float(num / l))
            outs.append(o)
            lses.append(float(m + l.ln()))
    return np.array(outs, dtype=np.float64), np.array(lses, dtype=np.float64)


def bf_attention(q, k, v, scale, causal):
    """Dense case: q [B,Hq,N,d], k, v [B,Hkv,N,d]."""
    B, Hq, N, d = q.shape
    Hkv = k.shape[1]
    G = Hq // Hkv
    sigma = float(np.float32(scale))
    o = np.zeros((B, Hq, N, d))
    lse = np.zeros((B, Hq, N))
    for b in range(B):
        for h in range(Hq):
            g = h // G
            sets = [[j for j in range(N) if (not causal) or j <= i] for i in range(N)]
            ob, lb = bf_rows(q[b, h], k[b, g], v[b, g], sigma, sets)
            o[b, h], lse[b, h] = ob, lb
    return o, lse


def bf_paged(q, k_cache, v_cache, table, ctx_lens, bs, scale):
    """Paged decode: walk every logical position through the table."""
    S, Hq, d = q.shape
    Hkv = k_cache.shape[1]
    G = Hq // Hkv
    sigma = float(np.float32(scale))
    o = np.zeros((S, Hq, d))
    lse = np.full((S, Hq), -np.inf)
    for s in range(S):
        n = int(ctx_lens[s])
        for h in range(Hq):
            g = h // G
            keys = np.array([k_cache[table[s][p // bs], g, p % bs] for p in range(n)]).reshape(n, d)
            vals = np.array([v_cache[table[s][p // bs], g, p % bs] for p in range(n)]).reshape(n, d)
            ob, lb = bf_rows(q[s, h][None], keys, vals, sigma, [list(range(n))])
            o[s, h], lse[s, h] = ob[0], lb[0]
    return o, lse

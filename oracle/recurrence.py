"""Scalar model of the block-by-block online-softmax recurrence.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Page [FA], section "No basta con promediar los resultados de los bloques",
describes how one query's output is built block by block: keep the running
maximum score m, the sum l of e^(s_j - m) and the numerator u of
e^(s_j - m) v_j; the answer is u / l; when a new block raises the maximum to
m', the earlier l and u are first multiplied by e^(m - m') and only then are
the new block's terms added.  Page [AT] section 3 ("El truco de Softmax en
línea") states the same idea.  The same page [FA] section warns that the mean
of the blocks' separately normalised results is wrong, with a worked example.

This module writes those steps out in float64 for one query with scores s_j
and values v_j (scalars or vectors), for an arbitrary partition of the keys
into blocks.  It is used to pin the worked example (0.75 against the naive
0.5), block-size invariance and the merge of two partial states, which the
split-KV decode uses to combine its partial results.

Initial state (the pages do not state it): m = -inf, l = 0, u = 0.  When the
running maximum is still -inf the rescale factor is taken as 0, which is the
limit of e^(m - m') and avoids the undefined (-inf) - (-inf).
"""

from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import Sequence

import numpy as np

__all__ = ["OnlineState", "add_block", "online_aggregate", "merge_states",
           "naive_block_average", "blocks_of"]


@dataclass
class OnlineState:
    m: float = -math.inf
    l: float = 0.0
    u: np.ndarray = field(default_factory=lambda: np.zeros(1))

    def result(self):
        """u / l (0 for an empty state)."""
        if self.l == 0.0:
            return np.zeros_like(self.u)
        return self.u / self.l


def _factor(m_old: float, m_new: float) -> float:
    """e^(m_old - m_new), with an empty running state contributing 0."""
    if m_old == -math.inf:
        return 0.0
    return math.exp(m_old - m_new)


def add_block(state: OnlineState, scores, values) -> OnlineState:
    """Fold one block of (score, value) pairs into the running state."""
    scores = np.asarray(scores, dtype=np.float64)
    values = np.asarray(values, dtype=np.float64).reshape(len(scores), -1)
    if len(scores) == 0:
        return state
    m_new = max(state.m, float(scores.max()))
    r = _factor(state.m, m_new)                  # rescale of the earlier terms
    w = np.exp(scores - m_new)                    # this block's weights
    l = state.l * r + float(w.sum())
    u = state.u * r + (w[:, None] * values).sum(axis=0)
    return OnlineState(m_new, l, u)


def blocks_of(n: int, partition: Sequence[int] | int):
    """Block boundaries for n keys: an int block size or explicit sizes."""
    if isinstance(partition, int):
        sizes = [partition] * (n // partition) + ([n % partition] if n % partition else [])
    else:
        sizes = list(partition)
    if sum(sizes) != n or any(sz <= 0 for sz in sizes):
        raise ValueError("partition must cover the keys with positive sizes")
    out, start = [], 0
    for sz in sizes:
        out.append((start, start + sz))
        start += sz
    return out


def online_aggregate(scores, values, partition):
    """One query's output u / l built block by block; returns (out, state)."""
    scores = np.asarray(scores, dtype=np.float64)
    values = np.asarray(values, dtype=np.float64).reshape(len(scores), -1)
    st = OnlineState(u=np.zeros(values.shape[1]))
    for a, b in blocks_of(len(scores), partition):
        st = add_block(st, scores[a:b], values[a:b])
    return st.result(), st


def merge_states(a: OnlineState, b: OnlineState) -> OnlineState:
    """Combine two partial states over disjoint key sets.

    Each is a running state in the sense above, so the larger maximum wins
    and the other state's l and u are rescaled by e^(m - M) before adding.
    """
    M = max(a.m, b.m)
    if M == -math.inf:
        return OnlineState(-math.inf, 0.0, np.zeros_like(a.u))
    ra, rb = _factor(a.m, M), _factor(b.m, M)
    return OnlineState(M, a.l * ra + b.l * rb, a.u * ra + b.u * rb)


def naive_block_average(scores, values, partition):
    """The WRONG combination: mean of each block's own softmax average."""
    scores = np.asarray(scores, dtype=np.float64)
    values = np.asarray(values, dtype=np.float64).reshape(len(scores), -1)
    outs = []
    for a, b in blocks_of(len(scores), partition):
        out, _ = online_aggregate(scores[a:b], values[a:b], [b - a])
        outs.append(out)
    return np.mean(outs, axis=0)

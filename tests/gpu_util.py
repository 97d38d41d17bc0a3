"""Helpers for the GPU parity tests: move seeded inputs to the device, run the
library, and compare with the float64 oracle."""

import sys

import numpy as np
import torch

from oracle import exact as OA

DEV = "cuda"
O_TOL = {torch.float32: 1e-5, torch.bfloat16: 2e-2}   # max-abs on o
LSE_TOL = 1e-4                                         # max-abs on lse


def announce(msg: str):
    """Name the case on the real stderr before a GPU step (survives capture)."""
    print(f"[gpu-case] {msg}", file=sys.__stderr__, flush=True)


def f64(t: torch.Tensor) -> np.ndarray:
    return t.detach().to("cpu").to(torch.float64).numpy()


def run_fwd(q, k, v, scale, causal, **kw):
    from exact_tiled_self_amd import attn_fwd
    qd, kd, vd = (t.to(DEV) for t in (q, k, v))
    o, lse = attn_fwd(qd, kd, vd, scale=scale, causal=causal, **kw)
    torch.cuda.synchronize()
    return o.cpu(), (lse.cpu() if lse is not None else None)


def max_abs(a, b) -> float:
    d = np.abs(np.asarray(a, dtype=np.float64) - np.asarray(b, dtype=np.float64))
    return float(d.max()) if d.size else 0.0


def check_dense_full(q, k, v, scale, causal, name=""):
    """Every output element against the oracle."""
    announce(f"dense {name} q={tuple(q.shape)} kv={tuple(k.shape)} {q.dtype} causal={causal}")
    o, lse = run_fwd(q, k, v, scale, causal)
    ro, rl = OA.attention(f64(q), f64(k), f64(v), scale, causal)
    eo, el = max_abs(f64(o), ro), max_abs(lse.numpy(), rl)
    assert np.all(np.isfinite(f64(o))), name
    assert eo <= O_TOL[q.dtype], f"{name}: o max-abs {eo}"
    assert el <= LSE_TOL, f"{name}: lse max-abs {el}"
    return eo, el


def check_config_full(q, k, v, scale, causal, name=""):
    """A full-size workload: the GPU output of the whole call compared with
    the oracle at every element, one (batch, query head) at a time so the
    host holds one head's float64 result at once.  Returns the worst o and
    lse errors."""
    announce(f"dense full {name} q={tuple(q.shape)} kv={tuple(k.shape)} {q.dtype} causal={causal}")
    o, lse = run_fwd(q, k, v, scale, causal)
    assert torch.isfinite(o.float()).all() and torch.isfinite(lse).all(), name
    B, Hq = q.shape[0], q.shape[1]
    G = Hq // k.shape[1]
    worst_o, worst_l = 0.0, 0.0
    for b in range(B):
        for h in range(Hq):
            g = h // G
            ro, rl = OA.attention(f64(q[b:b + 1, h:h + 1]), f64(k[b:b + 1, g:g + 1]), f64(v[b:b + 1, g:g + 1]),
                                  scale, causal)
            worst_o = max(worst_o, max_abs(f64(o[b:b + 1, h:h + 1]), ro))
            worst_l = max(worst_l, max_abs(lse[b:b + 1, h:h + 1].double().numpy(), rl))
    print(f"[parity] {name}: o max-abs {worst_o:.3e}, lse max-abs {worst_l:.3e}", file=sys.__stderr__,
          flush=True)
    assert worst_o <= O_TOL[q.dtype], f"{name}: o max-abs {worst_o}"
    assert worst_l <= LSE_TOL, f"{name}: lse max-abs {worst_l}"
    return worst_o, worst_l


def check_dense_rows(o, lse, q, k, v, scale, causal, samples, name=""):
    """Sampled (b, h, rows) of a large run against the oracle, row by row."""
    worst_o, worst_l = 0.0, 0.0
    for b, h, rows in samples:
        rows = np.asarray(sorted(set(int(r) for r in rows)))
        ro, rl = OA.attention_rows(q, k, v, scale, causal, b, h, rows)
        go = f64(o[b, h, torch.as_tensor(rows)])
        gl = lse[b, h, torch.as_tensor(rows)].double().numpy()
        worst_o = max(worst_o, max_abs(go, ro))
        worst_l = max(worst_l, max_abs(gl, rl))
    assert worst_o <= O_TOL[o.dtype], f"{name}: o max-abs {worst_o}"
    assert worst_l <= LSE_TOL, f"{name}: lse max-abs {worst_l}"
    return worst_o, worst_l

"""The memory-bound fusions around attention in a transformer layer, plainly.

TEST INFRASTRUCTURE ONLY (see the package docstring): never imported by the
product path.

What is computed ([KR] "Kernels de atención rápida y fusión de operadores",
section "Fusión de operadores"): a layer's normalisation, activation and
residual additions would each be a kernel writing its intermediate tensor to
HBM; fused, the same values are produced in one pass.  Two of the fusions
the page names:

  * residual add + RMSNorm: h = x + residual is the new residual stream, and
    y_i = h_i / sqrt(mean_j h_j^2 + eps) * w_i is the normalised input of the
    next sub-layer (RMSNorm, Zhang and Sennrich 2019: no mean subtraction,
    no bias);
  * the SwiGLU block's activation: between the gate/up projections and the
    down projection, a = silu(g) * u with silu(g) = g / (1 + e^-g), in place
    of a SiLU kernel followed by a multiply kernel.

Readings (listed with their reasons in the design notes):
  * the residual stream is stored in the activations' dtype (bf16), and the
    norm reads it as stored: y = RMSNorm(bf16(x + residual)), exactly what the
    unfused pair of kernels (add, then norm) computes; rounding to bf16 (8
    significant bits, nearest, ties to even) is a step of that definition
  * everything else in float64
"""

from __future__ import annotations

import numpy as np

__all__ = ["round_bf16", "add_rmsnorm", "swiglu"]


def round_bf16(x):
    """Round float64 values to the nearest bfloat16 (8 significant bits, ties
    to even), returned as float64.  Normal range only (|x| in [2^-126, 2^127]
    or 0), which is all the tests use."""
    x = np.asarray(x, dtype=np.float64)
    m, e = np.frexp(x)                        # x = m * 2^e, 0.5 <= |m| < 1
    return np.ldexp(np.rint(m * 256.0) / 256.0, e)    # rint: half to even


def add_rmsnorm(x, residual, weight, eps):
    """Returns (h, y): h = bf16(x + residual) [T, D] and y = RMSNorm(h) * weight
    in float64 (y not rounded)."""
    x = np.asarray(x, dtype=np.float64)
    r = np.asarray(residual, dtype=np.float64)
    w = np.asarray(weight, dtype=np.float64)
    h = round_bf16(x + r)                     # x + r of two bf16 values is exact in float64
    ms = np.mean(h * h, axis=-1, keepdims=True)
    y = h / np.sqrt(ms + float(np.float32(eps))) * w
    return h, y


def swiglu(gate, up):
    """silu(gate) * up in float64."""
    g = np.asarray(gate, dtype=np.float64)
    u = np.asarray(up, dtype=np.float64)
    return g / (1.0 + np.exp(-g)) * u

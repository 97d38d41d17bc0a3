"""Seeded synthetic inputs for the attention workloads.

This module only draws and lays out input tensors; it contains none of the
attention arithmetic, and both the oracle-based tests and the HIP path read
what it produces.

Workloads (shapes from the pages' examples):
  * ViT-B/16 self-attention: a 224x224 image in 16x16 patches gives N = 196
    tokens, model width 768 in 12 heads of d = 64 ("Autoatención, kernels
    CUDA y FlashAttention", section 1); N = 577 is the same model on a
    384x384 image (24*24 patches + class token).
  * long causal prefill of a decoder-only model, with grouped K/V heads
    ("FlashAttention" notes, last section; "Kernels de atención rápida...",
    section "Atención tipo FlashAttention y atención paginada").
  * paged-KV decode with 16-token blocks (same section of the last page).
  * chunked prefill over that paged cache: each sequence brings a chunk of
    new rows whose keys and values are appended to the cache and whose
    queries attend to everything cached up to their own position.

Recipe: numpy.random.default_rng(seed).standard_normal(shape, float32) drawn
in the order q, k, v (after the context lengths and the block permutation
for the paged case); an amplitude other than 1 multiplies in float32; bf16
tensors are the float32 draws rounded to nearest-even by torch on the CPU.
Real activations and weights are not available, so N(0, 1) tensors stand in
for them.
"""

from __future__ import annotations

import math
from dataclasses import dataclass, asdict

import numpy as np
import torch

__all__ = ["DenseConfig", "PagedConfig", "DENSE_CONFIGS", "PAGED_CONFIG", "CHUNK_NEW",
           "dense_inputs", "paged_inputs", "chunked_inputs", "torch_dtype"]


@dataclass(frozen=True)
class DenseConfig:
    name: str
    B: int
    Hq: int
    Hkv: int
    N: int
    d: int
    dtype: str          # "f32" or "bf16"
    causal: bool
    amp: float = 1.0
    seed: int = 0

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.d)

    def as_dict(self):
        return asdict(self)


@dataclass(frozen=True)
class PagedConfig:
    name: str
    S: int
    Hq: int
    Hkv: int
    d: int
    block_size: int
    ctx_lo: int
    ctx_hi: int          # inclusive
    max_blocks: int
    dtype: str = "bf16"
    seed: int = 4

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.d)

    def as_dict(self):
        return asdict(self)


DENSE_CONFIGS = {
    "vit_b16_fp32": DenseConfig("vit_b16_fp32", 1, 12, 12, 196, 64, "f32", False, 1.0, 0),
    "vit_b16_bf16": DenseConfig("vit_b16_bf16", 64, 12, 12, 196, 64, "bf16", False, 1.0, 1),
    "vit_b16_bf16_n577": DenseConfig("vit_b16_bf16_n577", 64, 12, 12, 577, 64, "bf16", False, 1.0, 1),
    "gqa_causal_t8192": DenseConfig("gqa_causal_t8192", 1, 12, 2, 8192, 128, "bf16", True, 0.5, 2),
    "mha_causal_t32768": DenseConfig("mha_causal_t32768", 1, 16, 16, 32768, 128, "bf16", True, 1.0, 3),
}

PAGED_CONFIG = PagedConfig("paged_decode_s64", S=64, Hq=12, Hkv=2, d=128, block_size=16,
                           ctx_lo=512, ctx_hi=8192, max_blocks=512, dtype="bf16", seed=4)


# New rows per sequence in the chunked-prefill workload over PAGED_CONFIG's cache.
CHUNK_NEW = 256


def torch_dtype(name: str):
    return {"f32": torch.float32, "bf16": torch.bfloat16}[name]


def _cast(x: np.ndarray, dtype: str) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(x)).to(torch_dtype(dtype))


def dense_inputs(cfg: DenseConfig | None = None, *, B=None, Hq=None, Hkv=None, N=None,
                 d=None, dtype=None, amp=None, seed=None):
    """q [B,Hq,N,d], k, v [B,Hkv,N,d] as CPU torch tensors of the config's dtype.

    Either pass a DenseConfig or the individual fields (keywords override).
    """
    f = cfg.as_dict() if cfg is not None else {}
    for key, val in dict(B=B, Hq=Hq, Hkv=Hkv, N=N, d=d, dtype=dtype, amp=amp, seed=seed).items():
        if val is not None:
            f[key] = val
    f.setdefault("amp", 1.0)
    f.setdefault("seed", 0)
    rng = np.random.default_rng(f["seed"])
    qs = (f["B"], f["Hq"], f["N"], f["d"])
    ks = (f["B"], f["Hkv"], f["N"], f["d"])
    q = rng.standard_normal(qs, dtype=np.float32)
    k = rng.standard_normal(ks, dtype=np.float32)
    v = rng.standard_normal(ks, dtype=np.float32)
    if f["amp"] != 1.0:
        a = np.float32(f["amp"])
        q, k, v = q * a, k * a, v * a
    return _cast(q, f["dtype"]), _cast(k, f["dtype"]), _cast(v, f["dtype"])


def paged_inputs(cfg: PagedConfig = PAGED_CONFIG, *, S=None, ctx_lens=None, seed=None,
                 poison=False, extra_blocks=0, max_blocks=None):
    """A paged KV cache and its block table.

    Returns a dict with q [S,Hq,d], k_cache / v_cache [num_blocks,Hkv,bs,d]
    (torch, cfg dtype), block_table int32 [S,max_blocks] (unused entries -1),
    ctx_lens int32 [S], num_blocks and max_blocks.

    Physical blocks are a seeded random permutation of the pool.  With
    poison=True every slot that must never be read holds NaN: the slots past
    each sequence's length in its last block and `extra_blocks` pool blocks
    that no table entry references.
    """
    S = cfg.S if S is None else S
    seed = cfg.seed if seed is None else seed
    max_blocks = cfg.max_blocks if max_blocks is None else max_blocks
    bs = cfg.block_size
    rng = np.random.default_rng(seed)
    if ctx_lens is None:
        ctx = rng.integers(cfg.ctx_lo, cfg.ctx_hi + 1, S).astype(np.int32)
    else:
        ctx = np.asarray(ctx_lens, dtype=np.int32).copy()
        if len(ctx) != S:
            raise ValueError("ctx_lens must have S entries")
    nblk = (ctx.astype(np.int64) + bs - 1) // bs
    if int(nblk.max(initial=0)) > max_blocks:
        raise ValueError("a context does not fit max_blocks")
    used = int(nblk.sum())
    num_blocks = used + int(extra_blocks)
    perm = rng.permutation(num_blocks).astype(np.int32)
    table = np.full((S, max_blocks), -1, dtype=np.int32)
    off = 0
    for s in range(S):
        table[s, :nblk[s]] = perm[off:off + nblk[s]]
        off += int(nblk[s])
    q = rng.standard_normal((S, cfg.Hq, cfg.d), dtype=np.float32)
    kc = rng.standard_normal((num_blocks, cfg.Hkv, bs, cfg.d), dtype=np.float32)
    vc = rng.standard_normal((num_blocks, cfg.Hkv, bs, cfg.d), dtype=np.float32)
    if poison:
        for s in range(S):
            n = int(ctx[s])
            if n % bs:
                last = table[s, n // bs]
                kc[last, :, n % bs:, :] = np.nan
                vc[last, :, n % bs:, :] = np.nan
        for blk in perm[used:]:
            kc[blk] = np.nan
            vc[blk] = np.nan
    return dict(q=_cast(q, cfg.dtype), k_cache=_cast(kc, cfg.dtype), v_cache=_cast(vc, cfg.dtype),
                block_table=torch.from_numpy(table), ctx_lens=torch.from_numpy(ctx),
                num_blocks=num_blocks, max_blocks=max_blocks, block_size=bs)


def chunked_inputs(cfg: PagedConfig = PAGED_CONFIG, *, new_lens, S=None, ctx_lens=None, seed=None,
                   poison=False, extra_blocks=0, max_blocks=None):
    """A paged cache (as paged_inputs) plus a packed chunk of new rows.

    new_lens: the number of new rows of every sequence (an int for all, or
    one per sequence); each must not exceed that sequence's length, which
    counts them.  Adds to paged_inputs' dict: q_new [T,Hq,d], k_new and
    v_new [T,Hkv,d] (cfg dtype), starts int32 [S+1] (row offsets), new_lens
    int32 [S] and max_new.  The new rows are drawn from
    default_rng(seed + 1) in the order q_new, k_new, v_new, after the cache.
    """
    seed = cfg.seed if seed is None else seed
    p = paged_inputs(cfg, S=S, ctx_lens=ctx_lens, seed=seed, poison=poison,
                     extra_blocks=extra_blocks, max_blocks=max_blocks)
    ctx = p["ctx_lens"].numpy().astype(np.int64)
    n = np.broadcast_to(np.asarray(new_lens, dtype=np.int64), ctx.shape).copy()
    if (n < 0).any() or (n > ctx).any():
        raise ValueError("every new_lens entry must lie in [0, ctx_lens]")
    starts = np.concatenate([[0], np.cumsum(n)]).astype(np.int32)
    T = int(starts[-1])
    rng = np.random.default_rng(seed + 1)
    qn = rng.standard_normal((T, cfg.Hq, cfg.d), dtype=np.float32)
    kn = rng.standard_normal((T, cfg.Hkv, cfg.d), dtype=np.float32)
    vn = rng.standard_normal((T, cfg.Hkv, cfg.d), dtype=np.float32)
    p.update(q_new=_cast(qn, cfg.dtype), k_new=_cast(kn, cfg.dtype), v_new=_cast(vn, cfg.dtype),
             starts=torch.from_numpy(starts), new_lens=torch.from_numpy(n.astype(np.int32)),
             max_new=int(n.max(initial=0)))
    return p

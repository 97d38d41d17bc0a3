"""The seeded generators: deterministic, well-formed block tables, poison
only where nothing may be read."""

import hashlib

import numpy as np
import torch

from exact_tiled_self_amd.inputs import (DENSE_CONFIGS, PAGED_CONFIG, dense_inputs,
                                         paged_inputs)


def _digest(*ts):
    h = hashlib.sha256()
    for t in ts:
        h.update(t.contiguous().view(torch.uint8).numpy().tobytes() if t.dtype != torch.int32
                 else t.numpy().tobytes())
    return h.hexdigest()


def test_dense_deterministic_and_dtypes():
    a = dense_inputs(DENSE_CONFIGS["vit_b16_fp32"])
    b = dense_inputs(DENSE_CONFIGS["vit_b16_fp32"])
    assert _digest(*a) == _digest(*b)
    assert a[0].dtype == torch.float32 and tuple(a[0].shape) == (1, 12, 196, 64)
    c = dense_inputs(B=1, Hq=12, Hkv=2, N=64, d=128, dtype="bf16", amp=0.5, seed=2)
    assert c[0].dtype == torch.bfloat16 and tuple(c[1].shape) == (1, 2, 64, 128)
    assert _digest(*dense_inputs(B=1, Hq=2, Hkv=2, N=8, d=64, dtype="bf16", seed=7)) != \
        _digest(*dense_inputs(B=1, Hq=2, Hkv=2, N=8, d=64, dtype="bf16", seed=8))


def test_bf16_is_rne_of_fp32_draw():
    q32, _, _ = dense_inputs(B=1, Hq=1, Hkv=1, N=16, d=64, dtype="f32", seed=3)
    qb, _, _ = dense_inputs(B=1, Hq=1, Hkv=1, N=16, d=64, dtype="bf16", seed=3)
    # bf16 keeps the top 16 bits after round-to-nearest-even of the fp32 bits
    bits = q32.view(torch.int32).numpy().astype(np.int64) & 0xFFFFFFFF
    rne = ((bits + 0x7FFF + ((bits >> 16) & 1)) >> 16) & 0xFFFF
    got = qb.view(torch.int16).numpy().astype(np.int64) & 0xFFFF
    assert np.array_equal(rne, got)


def test_paged_recipe_at_seed4():
    p = paged_inputs(PAGED_CONFIG)
    ctx = p["ctx_lens"].numpy()
    assert ctx.dtype == np.int32 and len(ctx) == 64
    assert ctx.min() >= 512 and ctx.max() <= 8192
    # figures of the decode workload at seed 4 (sum of lengths, pool size)
    assert int(ctx.sum()) == 311415 and p["num_blocks"] == 19492
    t = p["block_table"].numpy()
    nblk = (ctx + 15) // 16
    used = np.concatenate([t[s, :nblk[s]] for s in range(64)])
    assert np.array_equal(np.sort(used), np.arange(p["num_blocks"]))   # a permutation
    for s in range(64):
        assert np.all(t[s, nblk[s]:] == -1)
    assert tuple(p["k_cache"].shape) == (19492, 2, 16, 128)


def test_paged_poison_placement():
    p = paged_inputs(PAGED_CONFIG, S=5, ctx_lens=[1, 16, 17, 100, 0], poison=True,
                     extra_blocks=3, max_blocks=8, seed=11)
    k = p["k_cache"].float().numpy()
    v = p["v_cache"].float().numpy()
    t = p["block_table"].numpy()
    ctx = p["ctx_lens"].numpy()
    readable = np.zeros(k.shape[:3], dtype=bool)       # [block, kvh, slot]
    for s in range(5):
        for pos in range(ctx[s]):
            readable[t[s, pos // 16], :, pos % 16] = True
    assert np.all(np.isfinite(k[readable])) and np.all(np.isfinite(v[readable]))
    assert np.all(np.isnan(k[~readable])) and np.all(np.isnan(v[~readable]))
    assert p["num_blocks"] == 1 + 1 + 2 + 7 + 0 + 3

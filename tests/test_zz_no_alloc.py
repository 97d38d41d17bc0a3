"""attn_paged_decode_noalloc, the decode entry point that allocates nothing
(its partial states live in the library's own per-GPU array): two calls in a
row through the C ABI, the second on a smaller input, each bit-identical to
attn_paged_decode with a caller workspace (the same kernels on the same
partition) and within the tolerances of the oracle; with its outputs passed
in, the call leaves torch's allocations and the device's free memory as
they were."""

import math

import numpy as np
import pytest
import torch

from exact_tiled_self_amd import attn_paged_decode, attn_paged_decode_noalloc
from exact_tiled_self_amd.inputs import PAGED_CONFIG, PagedConfig, paged_inputs
from oracle import exact as OA
from tests.gpu_util import DEV, LSE_TOL, O_TOL, announce, f64, max_abs

pytestmark = pytest.mark.gpu


def _to_dev(p):
    return {k: (v.to(DEV) if isinstance(v, torch.Tensor) else v) for k, v in p.items()}


def _one_call(p, scale, name):
    announce(f"noalloc decode {name} S={p['q'].shape[0]} nb={p['num_blocks']}")
    d = _to_dev(p)
    S, Hq, hd = d["q"].shape
    o_ref, l_ref = attn_paged_decode(d["q"], d["k_cache"], d["v_cache"], d["block_table"], d["ctx_lens"],
                                     d["block_size"], scale)
    o = torch.full((S, Hq, hd), 7.0, dtype=torch.bfloat16, device=DEV)
    lse = torch.full((S, Hq), 7.0, dtype=torch.float32, device=DEV)
    torch.cuda.synchronize()
    torch.cuda.reset_peak_memory_stats()
    alloc0 = torch.cuda.memory_allocated()
    free0 = torch.cuda.mem_get_info()[0]
    attn_paged_decode_noalloc(d["q"], d["k_cache"], d["v_cache"], d["block_table"], d["ctx_lens"],
                              d["block_size"], scale, o=o, lse=lse)
    torch.cuda.synchronize()
    assert torch.cuda.max_memory_allocated() == alloc0
    # nothing the size of the partial states (32 MiB array) was taken from the device
    assert abs(torch.cuda.mem_get_info()[0] - free0) < (2 << 20)
    assert torch.equal(o.view(torch.int16), o_ref.view(torch.int16)), f"{name}: o differs from the workspace call"
    assert torch.equal(lse.view(torch.int32), l_ref.view(torch.int32)), f"{name}: lse differs"
    ro, rl = OA.paged_decode(f64(p["q"]), f64(p["k_cache"]), f64(p["v_cache"]), p["block_table"].numpy(),
                             p["ctx_lens"].numpy(), p["block_size"], scale)
    live = p["ctx_lens"].numpy() > 0
    oc, lc = o.cpu(), lse.cpu()
    assert max_abs(f64(oc)[live], ro[live]) <= O_TOL[torch.bfloat16]
    assert max_abs(lc.double().numpy()[live], rl[live]) <= LSE_TOL
    if (~live).any():
        assert torch.all(oc[torch.from_numpy(~live)] == 0)
        assert torch.all(torch.isneginf(lc[torch.from_numpy(~live)]))


def test_noalloc_matches_workspace_call_twice():
    scale = PAGED_CONFIG.scale
    # first: the full 64-sequence workload, NaN in every slot that must not be read
    big = paged_inputs(PAGED_CONFIG, poison=True, extra_blocks=8)
    _one_call(big, scale, "paged_decode_s64")
    # second, smaller: ragged lengths with an empty context; what the first
    # call left in the shared array must not leak into it
    small_cfg = PagedConfig("small", S=1, Hq=12, Hkv=2, d=128, block_size=16, ctx_lo=1, ctx_hi=1,
                            max_blocks=1, dtype="bf16", seed=0)
    ctx = [1, 0, 17, 300, 1000, 2500, 16]
    small = paged_inputs(small_cfg, S=len(ctx), ctx_lens=ctx, poison=True, extra_blocks=3,
                         max_blocks=160, seed=9)
    _one_call(small, 0.3, "ragged S=7")


def test_noalloc_other_group_sizes():
    """Other head groupings (up to 48 query heads per kv head, run as
    groups of at most 16 by teams of waves) and d = 64 go through the same
    array."""
    for Hq, Hkv, d in ((16, 1, 128), (8, 8, 64), (6, 3, 128), (40, 2, 128), (48, 1, 64)):
        cfg = PagedConfig("g", S=1, Hq=Hq, Hkv=Hkv, d=d, block_size=16, ctx_lo=1, ctx_hi=1, max_blocks=1,
                          dtype="bf16", seed=0)
        ctx = [5, 700, 64, 1300]
        p = paged_inputs(cfg, S=len(ctx), ctx_lens=ctx, poison=True, extra_blocks=2, max_blocks=90,
                         seed=Hq + d)
        _one_call(p, 1.0 / math.sqrt(d), f"{Hq}/{Hkv} d{d}")

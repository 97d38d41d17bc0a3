"""Paged decode captured in a HIP graph.

A graph records a sequence of GPU launches once and replays it with a single
submission, which removes the per-call launch cost; it needs stable buffer
addresses and fixed shapes ("Kernels de atención rápida y fusión de
operadores", section "Fusión y CUDA Graphs con torch.compile").  The decode
call qualifies: its kernels take only device pointers and sizes, allocate
nothing and record no memset, so a graph of `calls` decode launches on fixed
q / cache / table / length / output / workspace buffers can be replayed after
the caller has rewritten those buffers in place (new query, longer lengths,
new table entries).  Shapes (S, Hq, d, max_blocks, num_blocks) are fixed at
capture.

This module is plumbing around the library's own entry point: every replayed
launch is `attn_paged_decode`'s kernels.
"""

from __future__ import annotations

import math

import torch

from ._lib import attn_paged_decode, attn_paged_decode_workspace_size

__all__ = ["DecodeGraph"]


class DecodeGraph:
    """Capture `calls` consecutive paged-decode launches on fixed buffers.

    The constructor keeps references to the given tensors (their addresses are
    baked into the graph), allocates the outputs and the workspace once, runs
    one eager call on a side stream (as graph capture requires) and records the
    graph.  `replay()` re-runs it on the current stream; the results are in
    `o` and `lse` (those of the last recorded call).
    """

    def __init__(self, q, k_cache, v_cache, block_table, ctx_lens, block_size=16, scale=None,
                 calls=1):
        if calls < 1:
            raise ValueError("calls must be >= 1")
        self.q, self.k_cache, self.v_cache = q, k_cache, v_cache
        self.block_table, self.ctx_lens = block_table, ctx_lens
        self.block_size = block_size
        self.scale = 1.0 / math.sqrt(q.shape[-1]) if scale is None else float(scale)
        S, Hq, d = q.shape
        self.o = torch.empty_like(q)
        self.lse = torch.empty((S, Hq), dtype=torch.float32, device=q.device)
        need = attn_paged_decode_workspace_size(S, Hq, d, block_table.shape[1], block_size)
        self.workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=q.device)
        self.calls = calls

        side = torch.cuda.Stream(device=q.device)
        side.wait_stream(torch.cuda.current_stream(q.device))
        with torch.cuda.stream(side):
            self._launch(side)
        torch.cuda.current_stream(q.device).wait_stream(side)
        torch.cuda.synchronize(q.device)

        self.graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(self.graph):
            cap = torch.cuda.current_stream(q.device)
            for _ in range(calls):
                self._launch(cap)

    def _launch(self, stream):
        attn_paged_decode(self.q, self.k_cache, self.v_cache, self.block_table, self.ctx_lens,
                          self.block_size, self.scale, o=self.o, lse=self.lse,
                          workspace=self.workspace, stream=stream)

    def replay(self):
        self.graph.replay()
        return self.o, self.lse

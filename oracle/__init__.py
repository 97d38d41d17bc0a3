"""CPU oracle for exact scaled-dot-product attention (fp64, numpy).

TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
benchmark's CPU-baseline leg may import anything from this package.  The
product path (the HIP library and its Python binding) never imports, calls
or links it, and this package imports nothing from the product path.

Modules
-------
exact       the plain definition, softmax(s * Q K^T) V per head, with every
            score row materialised in float64 (dense prefill, paged decode and
            chunked prefill over a paged cache)
recurrence  a scalar model of the block-by-block online-softmax recurrence
            (running max m, sum l, numerator u, rescale by e^(m - m')), the
            merge of two such states, and the naive block average the pages
            warn against
kvcache     appending new tokens' keys and values to a paged KV cache,
            one token at a time through the block table
backward    the gradients dq, dk, dv of the exact attention (chain rule
            through o = P V and the softmax, weights recomputed from q, k)
fusion      residual add + RMSNorm and the SwiGLU activation (silu(g) * u),
            the memory-bound fusions around attention in a layer

Sources (web pages; cited by title and section):
  [AT]  "Autoatención, kernels CUDA y FlashAttention", section 1 (how
        self-attention works in a vision transformer) and section 3
        (FlashAttention: tiling, online softmax, saved statistics,
        recomputation in the backward pass)
  [FA]  "FlashAttention" (notes page), sections "Mecanismo y detalles" and
        "No basta con promediar los resultados de los bloques"
  [KR]  "Kernels de atención rápida y fusión de operadores" (the-ai.news),
        section "Atención tipo FlashAttention y atención paginada"

Parity pins: every function here is pinned by tests under tests/ that check
it against values printed by the pages (the worked example), closed forms,
invariants, a library routine on float64 CPU tensors and 40-digit brute force
on tiny inputs.  No function is parity-unpinned.
"""

from .exact import attention, attention_rows, paged_decode, paged_prefill, gather_paged_kv  # noqa: F401
from .recurrence import (  # noqa: F401
    OnlineState,
    online_aggregate,
    merge_states,
    naive_block_average,
)
from .kvcache import append_paged  # noqa: F401
from .backward import attention_bwd  # noqa: F401
from .fusion import add_rmsnorm, swiglu  # noqa: F401

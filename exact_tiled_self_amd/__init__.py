"""Exact tiled scaled-dot-product attention forward for MI355X (gfx950).

The compute lives in the HIP library `libattn.so` (sources under csrc/,
C ABI in include/attn.h); this package is a thin ctypes binding over it plus
the seeded input generators.  Importing the package does not load the
library; the first call does, and raises if it is missing.
"""

__all__ = ["attn_fwd", "attn_paged_decode", "attn_paged_decode_workspace_size", "attn_paged_decode_noalloc",
           "attn_kv_append", "attn_paged_prefill", "attn_bwd", "attn_bwd_workspace_size",
           "attn_add_rmsnorm", "attn_swiglu", "attention",
           "AttnError", "library_path", "abi_version"]


def __getattr__(name):
    if name == "attention":
        from .autograd import attention
        return attention
    if name in __all__:
        from . import _lib
        return getattr(_lib, name)
    raise AttributeError(name)

"""ctypes binding of libattn.so: the C ABI's entry points under the same
names, taking torch tensors for device memory and the current torch stream.

Argument marshalling only: shapes are read from the tensors, outputs are
allocated with torch when not given, and every computation happens in the
library's HIP kernels.  Tensors must already be contiguous CUDA (HIP)
tensors of the right dtype; nothing is copied or converted here.  A missing
library or a non-OK status raises; there is no fallback.
"""

from __future__ import annotations

import ctypes
import math
import os

import torch

from .build import LIB_PATH

__all__ = ["AttnError", "attn_fwd", "attn_paged_decode", "attn_paged_decode_workspace_size",
           "attn_paged_decode_noalloc", "DECODE_NOALLOC_SCRATCH_BYTES",
           "attn_kv_append", "attn_paged_prefill", "attn_bwd", "attn_bwd_workspace_size",
           "attn_add_rmsnorm", "attn_swiglu", "library_path", "abi_version", "raw_library", "ATTN_OK", "ATTN_ERR_INVALID_ARG",
           "ATTN_ERR_UNSUPPORTED", "ATTN_ERR_NO_DEVICE", "ATTN_ERR_LAUNCH", "ATTN_F32", "ATTN_BF16"]

ATTN_OK, ATTN_ERR_INVALID_ARG, ATTN_ERR_UNSUPPORTED, ATTN_ERR_NO_DEVICE, ATTN_ERR_LAUNCH = range(5)
ATTN_F32, ATTN_BF16 = 0, 1

_DTYPE = {torch.float32: ATTN_F32, torch.bfloat16: ATTN_BF16}

# ATTN_DECODE_NOALLOC_SCRATCH_BYTES of include/attn.h: the library's own
# per-GPU array that attn_paged_decode_noalloc keeps its partial states in.
DECODE_NOALLOC_SCRATCH_BYTES = 32 << 20


class AttnError(RuntimeError):
    """A non-OK status from the library (or the library is missing)."""

    def __init__(self, status: int, detail: str):
        super().__init__(f"status {status}: {detail}")
        self.status = status
        self.detail = detail


_lib = None

vp, ci, cf, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t


def library_path() -> str:
    return os.environ.get("ATTN_LIBRARY", LIB_PATH)


def raw_library():
    """The loaded CDLL with argument and return types declared."""
    global _lib
    if _lib is None:
        path = library_path()
        if not os.path.exists(path):
            raise AttnError(-1, f"{path} is not built (python -m exact_tiled_self_amd.build)")
        lib = ctypes.CDLL(path)
        lib.attn_fwd.restype = ci
        lib.attn_fwd.argtypes = [vp, vp, vp, vp, vp, ci, ci, ci, ci, ci, cf, ci, ci, vp]
        lib.attn_paged_decode_workspace_size.restype = sz
        lib.attn_paged_decode_workspace_size.argtypes = [ci, ci, ci, ci, ci]
        lib.attn_paged_decode.restype = ci
        lib.attn_paged_decode.argtypes = [vp, vp, vp, vp, vp, ci, vp, vp, ci, ci, ci, ci, ci, ci,
                                          cf, ci, vp, sz, vp]
        lib.attn_paged_decode_noalloc.restype = ci
        lib.attn_paged_decode_noalloc.argtypes = [vp, vp, vp, vp, vp, ci, vp, vp, ci, ci, ci, ci, ci, ci,
                                                  cf, ci, vp]
        lib.attn_kv_append.restype = ci
        lib.attn_kv_append.argtypes = [vp, vp, vp, vp, vp, vp, vp, ci, ci, ci, ci, ci, ci, ci, ci,
                                       ci, vp]
        lib.attn_paged_prefill.restype = ci
        lib.attn_paged_prefill.argtypes = [vp, vp, vp, vp, vp, vp, ci, vp, vp, ci, ci, ci, ci, ci,
                                           ci, ci, ci, cf, ci, vp]
        lib.attn_bwd_workspace_size.restype = sz
        lib.attn_bwd_workspace_size.argtypes = [ci, ci, ci, ci, ci]
        lib.attn_bwd.restype = ci
        lib.attn_bwd.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, ci, ci, ci, ci, ci, cf, ci, ci, vp,
                                 sz, vp]
        lib.attn_add_rmsnorm.restype = ci
        lib.attn_add_rmsnorm.argtypes = [vp, vp, vp, vp, vp, ci, ci, cf, ci, vp]
        lib.attn_swiglu.restype = ci
        lib.attn_swiglu.argtypes = [vp, vp, vp, ci, ci, ci, ci, ci, vp]
        lib.attn_status_string.restype = ctypes.c_char_p
        lib.attn_status_string.argtypes = [ci]
        lib.attn_last_error.restype = ctypes.c_char_p
        lib.attn_last_error.argtypes = []
        lib.attn_abi_version.restype = ci
        lib.attn_abi_version.argtypes = []
        _lib = lib
    return _lib


def abi_version() -> int:
    return raw_library().attn_abi_version()


def _check(status: int):
    if status != ATTN_OK:
        lib = raw_library()
        raise AttnError(status, f"{lib.attn_status_string(status).decode()}: "
                                f"{lib.attn_last_error().decode()}")


def _dev(t: torch.Tensor, name: str):
    if not isinstance(t, torch.Tensor) or t.device.type != "cuda":
        raise ValueError(f"{name} must be a device (cuda/HIP) tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t.data_ptr()


def _check_out(t, name: str, shape, dtype, ref: torch.Tensor):
    """A caller-supplied output must be exactly what the kernels write: the
    library receives only its pointer, so a smaller or differently typed
    buffer would be written past its end."""
    if not isinstance(t, torch.Tensor):
        raise ValueError(f"{name} must be a tensor")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if t.dtype != dtype:
        raise ValueError(f"{name} must have dtype {dtype}, got {t.dtype}")
    if t.device != ref.device:
        raise ValueError(f"{name} must be on {ref.device}, got {t.device}")


def _same_device(ref: torch.Tensor, **tensors):
    for name, t in tensors.items():
        if t is not None and t.device != ref.device:
            raise ValueError(f"{name} must be on {ref.device}, got {t.device}")


def _stream_ptr(device, stream):
    if stream is None:
        stream = torch.cuda.current_stream(device)
    return ctypes.c_void_p(stream.cuda_stream if isinstance(stream, torch.cuda.Stream) else int(stream))


def attn_fwd(q, k, v, scale=None, causal=False, *, o=None, lse=None, want_lse=True, stream=None):
    """Dense attention forward: returns (o, lse) (lse is None if not wanted).

    q: [B, Hq, N, d]; k, v: [B, Hkv, N, d]; float32 or bfloat16.
    """
    if q.dim() != 4 or k.dim() != 4 or v.dim() != 4:
        raise ValueError("q, k, v must be 4-D [B, H, N, d]")
    if not (q.dtype == k.dtype == v.dtype) or q.dtype not in _DTYPE:
        raise ValueError("q, k, v must share dtype float32 or bfloat16")
    B, Hq, N, d = q.shape
    Hkv = k.shape[1]
    if tuple(k.shape) != (B, Hkv, N, d) or tuple(v.shape) != tuple(k.shape):
        raise ValueError("k and v must be [B, Hkv, N, d] matching q")
    _same_device(q, k=k, v=v)
    if o is None:
        o = torch.empty_like(q)
    else:
        _check_out(o, "o", (B, Hq, N, d), q.dtype, q)
    if lse is None and want_lse:
        lse = torch.empty((B, Hq, N), dtype=torch.float32, device=q.device)
    elif lse is not None:
        _check_out(lse, "lse", (B, Hq, N), torch.float32, q)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    ptrs = [_dev(q, "q"), _dev(k, "k"), _dev(v, "v"), _dev(o, "o"),
            _dev(lse, "lse") if lse is not None else None]
    st = raw_library().attn_fwd(*ptrs, B, Hq, Hkv, N, d, float(scale), int(bool(causal)),
                                _DTYPE[q.dtype], _stream_ptr(q.device, stream))
    _check(st)
    return o, lse


def attn_paged_decode_workspace_size(S, Hq, d, max_blocks, block_size=16) -> int:
    return int(raw_library().attn_paged_decode_workspace_size(S, Hq, d, max_blocks, block_size))


def attn_paged_decode(q, k_cache, v_cache, block_table, ctx_lens, block_size=16, scale=None, *,
                      o=None, lse=None, want_lse=True, workspace=None, stream=None):
    """Paged single-token decode: returns (o, lse).

    q: [S, Hq, d]; k_cache, v_cache: [num_blocks, Hkv, block_size, d];
    block_table: int32 [S, max_blocks]; ctx_lens: int32 [S].
    """
    if q.dim() != 3 or k_cache.dim() != 4 or v_cache.shape != k_cache.shape:
        raise ValueError("q must be [S, Hq, d] and the caches [num_blocks, Hkv, block_size, d]")
    if block_table.dtype != torch.int32 or ctx_lens.dtype != torch.int32:
        raise ValueError("block_table and ctx_lens must be int32")
    if q.dtype not in _DTYPE or k_cache.dtype != q.dtype or v_cache.dtype != q.dtype:
        raise ValueError("q and the caches must share dtype")
    S, Hq, d = q.shape
    num_blocks, Hkv, bs, d2 = k_cache.shape
    if d2 != d or bs != block_size or block_table.dim() != 2 or block_table.shape[0] != S \
            or tuple(ctx_lens.shape) != (S,):
        raise ValueError("inconsistent decode shapes")
    max_blocks = block_table.shape[1]
    _same_device(q, k_cache=k_cache, v_cache=v_cache, block_table=block_table, ctx_lens=ctx_lens,
                 workspace=workspace)
    if o is None:
        o = torch.empty_like(q)
    else:
        _check_out(o, "o", (S, Hq, d), q.dtype, q)
    if lse is None and want_lse:
        lse = torch.empty((S, Hq), dtype=torch.float32, device=q.device)
    elif lse is not None:
        _check_out(lse, "lse", (S, Hq), torch.float32, q)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    need = attn_paged_decode_workspace_size(S, Hq, d, max_blocks, block_size)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=q.device)
    ws_bytes = workspace.numel() * workspace.element_size()
    st = raw_library().attn_paged_decode(
        _dev(q, "q"), _dev(k_cache, "k_cache"), _dev(v_cache, "v_cache"),
        _dev(block_table, "block_table"), _dev(ctx_lens, "ctx_lens"), int(block_size),
        _dev(o, "o"), _dev(lse, "lse") if lse is not None else None, S, Hq, Hkv, d, max_blocks,
        num_blocks, float(scale), _DTYPE[q.dtype], _dev(workspace, "workspace"), ws_bytes,
        _stream_ptr(q.device, stream))
    _check(st)
    return o, lse


def attn_paged_decode_noalloc(q, k_cache, v_cache, block_table, ctx_lens, block_size=16, scale=None, *,
                              o=None, lse=None, want_lse=True, stream=None):
    """attn_paged_decode with no workspace: the partial states live in the
    library's own per-GPU array (DECODE_NOALLOC_SCRATCH_BYTES), so with o
    (and lse, or want_lse=False) passed in, the call allocates nothing.
    Calls that may overlap on one GPU race on that array."""
    if q.dim() != 3 or k_cache.dim() != 4 or v_cache.shape != k_cache.shape:
        raise ValueError("q must be [S, Hq, d] and the caches [num_blocks, Hkv, block_size, d]")
    if block_table.dtype != torch.int32 or ctx_lens.dtype != torch.int32:
        raise ValueError("block_table and ctx_lens must be int32")
    if q.dtype not in _DTYPE or k_cache.dtype != q.dtype or v_cache.dtype != q.dtype:
        raise ValueError("q and the caches must share dtype")
    S, Hq, d = q.shape
    num_blocks, Hkv, bs, d2 = k_cache.shape
    if d2 != d or bs != block_size or block_table.dim() != 2 or block_table.shape[0] != S \
            or tuple(ctx_lens.shape) != (S,):
        raise ValueError("inconsistent decode shapes")
    max_blocks = block_table.shape[1]
    _same_device(q, k_cache=k_cache, v_cache=v_cache, block_table=block_table, ctx_lens=ctx_lens)
    if o is None:
        o = torch.empty_like(q)
    else:
        _check_out(o, "o", (S, Hq, d), q.dtype, q)
    if lse is None and want_lse:
        lse = torch.empty((S, Hq), dtype=torch.float32, device=q.device)
    elif lse is not None:
        _check_out(lse, "lse", (S, Hq), torch.float32, q)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    st = raw_library().attn_paged_decode_noalloc(
        _dev(q, "q"), _dev(k_cache, "k_cache"), _dev(v_cache, "v_cache"),
        _dev(block_table, "block_table"), _dev(ctx_lens, "ctx_lens"), int(block_size),
        _dev(o, "o"), _dev(lse, "lse") if lse is not None else None, S, Hq, Hkv, d, max_blocks,
        num_blocks, float(scale), _DTYPE[q.dtype], _stream_ptr(q.device, stream))
    _check(st)
    return o, lse


def _paged_meta(k_cache, v_cache, block_table, ctx_lens, starts, block_size):
    if k_cache.dim() != 4 or v_cache.shape != k_cache.shape or k_cache.dtype != v_cache.dtype:
        raise ValueError("the caches must both be [num_blocks, Hkv, block_size, d] of one dtype")
    if block_table.dtype != torch.int32 or ctx_lens.dtype != torch.int32 or starts.dtype != torch.int32:
        raise ValueError("block_table, ctx_lens and starts must be int32")
    S = ctx_lens.shape[0]
    if ctx_lens.dim() != 1 or block_table.dim() != 2 or block_table.shape[0] != S \
            or tuple(starts.shape) != (S + 1,) or k_cache.shape[2] != block_size:
        raise ValueError("inconsistent paged-cache shapes")
    return S, k_cache.shape[0], k_cache.shape[1], k_cache.shape[3], block_table.shape[1]


def attn_kv_append(k_new, v_new, k_cache, v_cache, block_table, ctx_lens, starts, block_size=16, *,
                   max_new=None, stream=None):
    """Write packed new tokens k_new, v_new [T, Hkv, d] into the paged caches
    in place.  starts: int32 [S + 1] row offsets; ctx_lens: int32 [S], the
    lengths after the append.  max_new bounds every sequence's new-token
    count and sizes the launch (default T, always safe)."""
    S, num_blocks, Hkv, d, max_blocks = _paged_meta(k_cache, v_cache, block_table, ctx_lens, starts,
                                                    block_size)
    if k_new.dim() != 3 or v_new.shape != k_new.shape or tuple(k_new.shape[1:]) != (Hkv, d):
        raise ValueError("k_new and v_new must be [T, Hkv, d] matching the caches")
    if k_new.dtype != k_cache.dtype or v_new.dtype != k_cache.dtype or k_cache.dtype not in _DTYPE:
        raise ValueError("new rows and caches must share dtype float32 or bfloat16")
    _same_device(k_cache, k_new=k_new, v_new=v_new, v_cache=v_cache, block_table=block_table,
                 ctx_lens=ctx_lens, starts=starts)
    T = k_new.shape[0]
    st = raw_library().attn_kv_append(
        _dev(k_new, "k_new"), _dev(v_new, "v_new"), _dev(k_cache, "k_cache"), _dev(v_cache, "v_cache"),
        _dev(block_table, "block_table"), _dev(ctx_lens, "ctx_lens"), _dev(starts, "starts"),
        int(block_size), S, T, T if max_new is None else int(max_new), Hkv, d, max_blocks, num_blocks,
        _DTYPE[k_cache.dtype], _stream_ptr(k_cache.device, stream))
    _check(st)


def attn_paged_prefill(q, k_cache, v_cache, block_table, ctx_lens, starts, block_size=16, scale=None,
                       *, max_new=None, o=None, lse=None, want_lse=True, stream=None):
    """Chunked prefill of packed query rows q [T, Hq, d] against the paged
    cache (their own keys already appended): returns (o [T, Hq, d], lse
    [T, Hq]).  Rows of no sequence are left as allocated."""
    S, num_blocks, Hkv, d, max_blocks = _paged_meta(k_cache, v_cache, block_table, ctx_lens, starts,
                                                    block_size)
    if q.dim() != 3 or q.shape[2] != d or q.dtype != k_cache.dtype or q.dtype not in _DTYPE:
        raise ValueError("q must be [T, Hq, d] with the caches' d and dtype")
    T, Hq = q.shape[0], q.shape[1]
    _same_device(q, k_cache=k_cache, v_cache=v_cache, block_table=block_table, ctx_lens=ctx_lens,
                 starts=starts)
    if o is None:
        o = torch.empty_like(q)
    else:
        _check_out(o, "o", (T, Hq, d), q.dtype, q)
    if lse is None and want_lse:
        lse = torch.empty((T, Hq), dtype=torch.float32, device=q.device)
    elif lse is not None:
        _check_out(lse, "lse", (T, Hq), torch.float32, q)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    st = raw_library().attn_paged_prefill(
        _dev(q, "q"), _dev(k_cache, "k_cache"), _dev(v_cache, "v_cache"),
        _dev(block_table, "block_table"), _dev(ctx_lens, "ctx_lens"), _dev(starts, "starts"),
        int(block_size), _dev(o, "o"), _dev(lse, "lse") if lse is not None else None, S, T,
        T if max_new is None else int(max_new), Hq, Hkv, d, max_blocks, num_blocks, float(scale),
        _DTYPE[q.dtype], _stream_ptr(q.device, stream))
    _check(st)
    return o, lse


def attn_bwd_workspace_size(B, Hq, Hkv, N, d) -> int:
    return int(raw_library().attn_bwd_workspace_size(B, Hq, Hkv, N, d))


def attn_bwd(q, k, v, o, lse, dout, scale=None, causal=False, *, dq=None, dk=None, dv=None,
             workspace=None, stream=None):
    """Gradients (dq, dk, dv) of attn_fwd, recomputing the weights from q, k
    and the forward's lse.  q, o, dout: [B, Hq, N, d] bf16; k, v: [B, Hkv, N, d]
    bf16; lse: [B, Hq, N] float32 (as attn_fwd returned it)."""
    if q.dim() != 4 or k.dim() != 4 or v.shape != k.shape or o.shape != q.shape or dout.shape != q.shape:
        raise ValueError("q, o, dout must be [B, Hq, N, d] and k, v [B, Hkv, N, d]")
    if not (q.dtype == k.dtype == v.dtype == o.dtype == dout.dtype) or q.dtype not in _DTYPE:
        raise ValueError("q, k, v, o and dout must share dtype")
    B, Hq, N, d = q.shape
    Hkv = k.shape[1]
    if tuple(k.shape) != (B, Hkv, N, d) or tuple(lse.shape) != (B, Hq, N) or lse.dtype != torch.float32:
        raise ValueError("inconsistent shapes, or lse not float32 [B, Hq, N]")
    _same_device(q, k=k, v=v, o=o, lse=lse, dout=dout, workspace=workspace)
    for t, name, ref in ((dq, "dq", q), (dk, "dk", k), (dv, "dv", v)):
        if t is not None:
            _check_out(t, name, ref.shape, ref.dtype, q)
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(v) if dv is None else dv
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    need = attn_bwd_workspace_size(B, Hq, Hkv, N, d)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=q.device)
    st = raw_library().attn_bwd(
        _dev(q, "q"), _dev(k, "k"), _dev(v, "v"), _dev(o, "o"), _dev(lse, "lse"), _dev(dout, "dout"),
        _dev(dq, "dq"), _dev(dk, "dk"), _dev(dv, "dv"), B, Hq, Hkv, N, d, float(scale),
        int(bool(causal)), _DTYPE[q.dtype], _dev(workspace, "workspace"),
        workspace.numel() * workspace.element_size(), _stream_ptr(q.device, stream))
    _check(st)
    return dq, dk, dv


def attn_add_rmsnorm(x, residual, weight, eps=1e-6, *, out=None, residual_out=None, stream=None):
    """Returns (out, residual_out): residual_out = bf16(x + residual) and
    out = RMSNorm(residual_out) * weight.  x, residual: [T, D] bf16; weight
    [D].  Pass residual_out=residual to update the residual in place."""
    if x.dim() != 2 or residual.shape != x.shape or weight.dim() != 1 or weight.shape[0] != x.shape[1]:
        raise ValueError("x, residual must be [T, D] and weight [D]")
    if not (x.dtype == residual.dtype == weight.dtype) or x.dtype not in _DTYPE:
        raise ValueError("x, residual and weight must share dtype")
    _same_device(x, residual=residual, weight=weight)
    for t, name in ((out, "out"), (residual_out, "residual_out")):
        if t is not None:
            _check_out(t, name, x.shape, x.dtype, x)
    out = torch.empty_like(x) if out is None else out
    residual_out = torch.empty_like(x) if residual_out is None else residual_out
    T, D = x.shape
    st = raw_library().attn_add_rmsnorm(_dev(x, "x"), _dev(residual, "residual"), _dev(weight, "weight"),
                                        _dev(out, "out"), _dev(residual_out, "residual_out"), T, D,
                                        float(eps), _DTYPE[x.dtype], _stream_ptr(x.device, stream))
    _check(st)
    return out, residual_out


def attn_swiglu(gate, up=None, *, out=None, stream=None):
    """silu(gate) * up.  With up=None, gate is one merged [T, 2F] projection
    output whose first F columns are the gate and last F the up half."""
    if gate.dim() != 2 or gate.dtype not in _DTYPE:
        raise ValueError("gate must be a 2-D tensor")
    if up is None:
        T, F2 = gate.shape
        if F2 % 2:
            raise ValueError("a merged gate/up tensor needs an even width")
        F, ld_in = F2 // 2, F2
    else:
        if up.shape != gate.shape or up.dtype != gate.dtype:
            raise ValueError("gate and up must match")
        _same_device(gate, up=up)
        T, F = gate.shape
        ld_in = F
    if out is not None:
        _check_out(out, "out", (T, F), gate.dtype, gate)
    out = torch.empty((T, F), dtype=gate.dtype, device=gate.device) if out is None else out
    g_ptr = _dev(gate, "gate")
    u_ptr = g_ptr + F * gate.element_size() if up is None else _dev(up, "up")
    st = raw_library().attn_swiglu(g_ptr, u_ptr, _dev(out, "out"), T, F, ld_in, F, _DTYPE[gate.dtype],
                                   _stream_ptr(gate.device, stream))
    _check(st)
    return out

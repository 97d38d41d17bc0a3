"""The C ABI on the CPU: the library loads, exports every function the header
declares, and rejects every host-checkable bad argument before touching the
HIP runtime (so these run without a GPU).  No kernel is launched here: each
call below fails validation, except the no-device check, which only runs
where no GPU is present."""

import ctypes
import math
import os
import re
import subprocess

import pytest
import torch

from exact_tiled_self_amd import _lib
from exact_tiled_self_amd.build import LIB_PATH, build

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "attn.h")

OK, INVALID, UNSUPPORTED, NO_DEVICE = 0, 1, 2, 3
F32, BF16 = 0, 1
A = 0x100000          # fake, 16-byte aligned addresses: never dereferenced
MB = 1 << 20


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(LIB_PATH):
        build()
    return _lib.raw_library()


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(attn_[a-z_]+)\s*\(", text)))


def test_header_declares_the_entry_points():
    names = _declared_functions()
    assert names == sorted(["attn_fwd", "attn_paged_decode", "attn_paged_decode_workspace_size",
                            "attn_paged_decode_noalloc",
                            "attn_kv_append", "attn_paged_prefill", "attn_bwd",
                            "attn_bwd_workspace_size", "attn_add_rmsnorm", "attn_swiglu",
                            "attn_status_string", "attn_last_error", "attn_abi_version"])


def test_library_exports_every_declared_symbol(lib):
    out = subprocess.run(["nm", "-D", "--defined-only", LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = set(re.findall(r"\bT (attn_\w+)", out))
    for name in _declared_functions():
        assert name in exported, name
        assert hasattr(lib, name)
    assert lib.attn_abi_version() == 2


def test_status_strings(lib):
    for code, name in enumerate(["ATTN_OK", "ATTN_ERR_INVALID_ARG", "ATTN_ERR_UNSUPPORTED",
                                 "ATTN_ERR_NO_DEVICE", "ATTN_ERR_LAUNCH"]):
        assert lib.attn_status_string(code).decode() == name


def fwd(lib, q=A, k=A + 64 * MB, v=A + 128 * MB, o=A + 192 * MB, lse=A + 256 * MB, B=1, Hq=4,
        Hkv=2, N=128, d=128, scale=0.125, causal=0, dtype=BF16):
    return lib.attn_fwd(q, k, v, o, lse, B, Hq, Hkv, N, d, scale, causal, dtype, None)


@pytest.mark.parametrize("kw,status", [
    (dict(q=0), INVALID), (dict(k=0), INVALID), (dict(v=0), INVALID), (dict(o=0), INVALID),
    (dict(B=0), INVALID), (dict(Hq=0), INVALID), (dict(Hkv=0), INVALID), (dict(N=0), INVALID),
    (dict(N=-5), INVALID), (dict(Hq=6, Hkv=4), INVALID), (dict(causal=2), INVALID),
    (dict(scale=math.inf), INVALID), (dict(scale=math.nan), INVALID),
    (dict(d=96), UNSUPPORTED), (dict(d=256), UNSUPPORTED), (dict(dtype=7), UNSUPPORTED),
    (dict(q=A + 8), INVALID), (dict(o=A + 192 * MB + 4), INVALID), (dict(lse=A + 256 * MB + 2), INVALID),
    (dict(o=A), INVALID), (dict(lse=A + 64 * MB + 4096), INVALID), (dict(lse=A + 192 * MB), INVALID),
    (dict(N=1 << 24, d=128), UNSUPPORTED), (dict(N=(1 << 22) + 1, d=128, dtype=F32), UNSUPPORTED),
])
def test_fwd_rejects_before_any_launch(lib, kw, status):
    assert fwd(lib, **kw) == status
    assert lib.attn_last_error().decode() != ""


def dec(lib, q=A, kc=A + 64 * MB, vc=A + 128 * MB, table=A + 192 * MB, ctx=A + 200 * MB, bs=16,
        o=A + 208 * MB, lse=A + 216 * MB, S=4, Hq=12, Hkv=2, d=128, max_blocks=8, num_blocks=32,
        scale=0.088, dtype=BF16, ws=A + 256 * MB, ws_bytes=None):
    if ws_bytes is None:
        ws_bytes = lib.attn_paged_decode_workspace_size(S, Hq, d, max_blocks, bs)
    return lib.attn_paged_decode(q, kc, vc, table, ctx, bs, o, lse, S, Hq, Hkv, d, max_blocks,
                                 num_blocks, scale, dtype, ws, ws_bytes, None)


@pytest.mark.parametrize("kw,status", [
    (dict(q=0), INVALID), (dict(kc=0), INVALID), (dict(table=0), INVALID), (dict(ctx=0), INVALID),
    (dict(o=0), INVALID), (dict(S=0), INVALID), (dict(max_blocks=0), INVALID),
    (dict(num_blocks=0), INVALID), (dict(Hq=12, Hkv=5), INVALID), (dict(scale=math.inf), INVALID),
    (dict(dtype=F32), UNSUPPORTED), (dict(d=80), UNSUPPORTED), (dict(bs=32), UNSUPPORTED),
    (dict(ws=0), INVALID), (dict(ws_bytes=16), INVALID),
    # 32 query heads per kv head run as two groups of 16: twice the units
    # (17 * 2 * (2^26 - 1) >= 2^31, while 17 * (2^26 - 1) alone would fit)
    (dict(S=17, Hq=32, Hkv=1, max_blocks=(1 << 26) - 1), UNSUPPORTED),
    (dict(q=A + 4), INVALID), (dict(table=A + 192 * MB + 2), INVALID), (dict(ws=A + 256 * MB + 8), INVALID),
    (dict(o=A + 64 * MB), INVALID), (dict(ws=A + 200 * MB), INVALID),
])
def test_decode_rejects_before_any_launch(lib, kw, status):
    assert dec(lib, **kw) == status
    assert lib.attn_last_error().decode() != ""


def dec_na(lib, q=A, kc=A + 64 * MB, vc=A + 128 * MB, table=A + 192 * MB, ctx=A + 200 * MB, bs=16,
           o=A + 208 * MB, lse=A + 216 * MB, S=4, Hq=12, Hkv=2, d=128, max_blocks=8, num_blocks=32,
           scale=0.088, dtype=BF16):
    return lib.attn_paged_decode_noalloc(q, kc, vc, table, ctx, bs, o, lse, S, Hq, Hkv, d, max_blocks,
                                         num_blocks, scale, dtype, None)


@pytest.mark.parametrize("kw,status", [
    (dict(q=0), INVALID), (dict(kc=0), INVALID), (dict(table=0), INVALID), (dict(ctx=0), INVALID),
    (dict(o=0), INVALID), (dict(S=0), INVALID), (dict(max_blocks=0), INVALID),
    (dict(num_blocks=0), INVALID), (dict(Hq=12, Hkv=5), INVALID), (dict(scale=math.inf), INVALID),
    (dict(dtype=F32), UNSUPPORTED), (dict(d=80), UNSUPPORTED), (dict(bs=32), UNSUPPORTED),
    (dict(q=A + 4), INVALID), (dict(table=A + 192 * MB + 2), INVALID), (dict(o=A + 64 * MB), INVALID),
    (dict(lse=A + 208 * MB), INVALID),
    # partial states of 2048 + S * Hkv pieces beyond the 32 MiB static array
    (dict(S=9000, Hq=12, Hkv=2, max_blocks=1, o=A + 512 * MB, lse=A + 1024 * MB), UNSUPPORTED),
    (dict(S=3000, Hq=16, Hkv=1, max_blocks=1, o=A + 512 * MB, lse=A + 1024 * MB), UNSUPPORTED),
    # 32 heads per kv head: two groups, so 1000 sequences no longer fit
    (dict(S=1000, Hq=32, Hkv=1, max_blocks=1, o=A + 512 * MB, lse=A + 1024 * MB), UNSUPPORTED),
])
def test_decode_noalloc_rejects_before_any_launch(lib, kw, status):
    assert dec_na(lib, **kw) == status
    assert lib.attn_last_error().decode() != ""


def test_decode_noalloc_capacity_bound():
    """The documented fit rule against the header's constant: the full
    64-sequence workload (12/2 heads, d = 128) fits, with room to spare."""
    def need(S, Hq, Hkv, d):
        G = Hq // Hkv
        n = -(-G // 16)
        H, r = n * Hkv, -(-G // n)
        rec = (8 * S * H + 255) // 256 * 256
        return rec + 4 * (2048 + S * H) * (((2 * r + 3) // 4 * 4) + r * d)
    cap = _lib.DECODE_NOALLOC_SCRATCH_BYTES
    assert need(64, 12, 2, 128) < cap // 4
    assert need(4300, 12, 2, 128) <= cap < need(4400, 12, 2, 128)
    assert need(1900, 16, 1, 128) <= cap < need(2000, 16, 1, 128)
    assert need(9000, 12, 2, 128) > cap and need(3000, 16, 1, 128) > cap
    # 32 heads per kv head: two groups of 16, so half the sequences fit
    assert need(900, 32, 1, 128) <= cap < need(1000, 32, 1, 128)


def test_workspace_size(lib):
    # documented bound: 8*S*Hq bytes of pair records rounded up to 256, then
    # fp32 partial states for up to 2048 + S*Hq wave pieces, whose rows number
    # at most 2048*Hq + S*Hq + ceil(S*Hq/16) (groups of at most 16 heads)
    def expect(S, Hq, d):
        rec = (8 * S * Hq + 255) // 256 * 256
        return rec + 4 * ((2048 * Hq + S * Hq + -(-S * Hq // 16)) * (d + 2) + 3 * (2048 + S * Hq))
    assert lib.attn_paged_decode_workspace_size(64, 12, 128, 512, 16) == expect(64, 12, 128)
    assert lib.attn_paged_decode_workspace_size(1, 1, 64, 1, 16) == expect(1, 1, 64)
    assert lib.attn_paged_decode_workspace_size(3, 8, 64, 7, 16) == expect(3, 8, 64)
    assert lib.attn_paged_decode_workspace_size(5, 71, 128, 9, 16) == expect(5, 71, 128)
    assert lib.attn_paged_decode_workspace_size(1, 1, 64, 1, 32) == 0
    assert lib.attn_paged_decode_workspace_size(0, 1, 64, 1, 16) == 0


def app(lib, kn=A, vn=A + 16 * MB, kc=A + 64 * MB, vc=A + 128 * MB, table=A + 192 * MB,
        ctx=A + 200 * MB, starts=A + 201 * MB, bs=16, S=4, T=40, max_new=10, Hkv=2, d=128,
        max_blocks=8, num_blocks=32, dtype=BF16):
    return lib.attn_kv_append(kn, vn, kc, vc, table, ctx, starts, bs, S, T, max_new, Hkv, d,
                              max_blocks, num_blocks, dtype, None)


@pytest.mark.parametrize("kw,status", [
    (dict(kn=0), INVALID), (dict(vc=0), INVALID), (dict(starts=0), INVALID), (dict(S=0), INVALID),
    (dict(Hkv=0), INVALID), (dict(num_blocks=0), INVALID), (dict(T=-1), INVALID),
    (dict(max_new=-1), INVALID), (dict(dtype=5), UNSUPPORTED), (dict(d=4), UNSUPPORTED),
    (dict(d=4096), UNSUPPORTED), (dict(bs=0), UNSUPPORTED), (dict(bs=2048), UNSUPPORTED),
    (dict(S=70000), UNSUPPORTED), (dict(kn=A + 8), INVALID), (dict(kc=A + 64 * MB + 4), INVALID),
    (dict(ctx=A + 200 * MB + 2), INVALID), (dict(vc=A + 64 * MB + 1024), INVALID),
    (dict(kc=A), INVALID), (dict(vc=A + 200 * MB - 4096), INVALID),
])
def test_append_rejects_before_any_launch(lib, kw, status):
    assert app(lib, **kw) == status
    assert lib.attn_last_error().decode() != ""


def test_append_with_nothing_to_write_launches_nothing(lib):
    # valid arguments with T = 0 or max_new = 0 return OK without any HIP call
    assert app(lib, T=0) == OK and app(lib, max_new=0) == OK
    assert app(lib, dtype=F32, d=64, T=0) == OK


def ppf(lib, q=A, kc=A + 64 * MB, vc=A + 128 * MB, table=A + 192 * MB, ctx=A + 200 * MB,
        starts=A + 201 * MB, bs=16, o=A + 208 * MB, lse=A + 216 * MB, S=4, T=40, max_new=10, Hq=12,
        Hkv=2, d=128, max_blocks=8, num_blocks=32, scale=0.088, dtype=BF16):
    return lib.attn_paged_prefill(q, kc, vc, table, ctx, starts, bs, o, lse, S, T, max_new, Hq,
                                  Hkv, d, max_blocks, num_blocks, scale, dtype, None)


@pytest.mark.parametrize("kw,status", [
    (dict(q=0), INVALID), (dict(starts=0), INVALID), (dict(o=0), INVALID), (dict(S=0), INVALID),
    (dict(Hq=12, Hkv=5), INVALID), (dict(T=-3), INVALID), (dict(max_new=-1), INVALID),
    (dict(scale=math.nan), INVALID), (dict(dtype=F32), UNSUPPORTED), (dict(d=96), UNSUPPORTED),
    (dict(bs=8), UNSUPPORTED), (dict(max_new=1 << 20, Hq=64), UNSUPPORTED),
    (dict(q=A + 4), INVALID), (dict(starts=A + 201 * MB + 1), INVALID), (dict(lse=A + 216 * MB + 2), INVALID),
    (dict(o=A + 64 * MB), INVALID), (dict(lse=A + 200 * MB), INVALID), (dict(lse=A + 208 * MB), INVALID),
])
def test_paged_prefill_rejects_before_any_launch(lib, kw, status):
    assert ppf(lib, **kw) == status
    assert lib.attn_last_error().decode() != ""


def test_paged_prefill_with_no_rows_launches_nothing(lib):
    assert ppf(lib, T=0) == OK and ppf(lib, max_new=0) == OK


def bwd(lib, q=A, k=A + 16 * MB, v=A + 32 * MB, o=A + 48 * MB, lse=A + 64 * MB, do=A + 80 * MB,
        dq=A + 96 * MB, dk=A + 112 * MB, dv=A + 128 * MB, B=1, Hq=4, Hkv=2, N=128, d=128, scale=0.1,
        causal=1, dtype=BF16, ws=A + 144 * MB, ws_bytes=None):
    if ws_bytes is None:
        ws_bytes = lib.attn_bwd_workspace_size(B, Hq, Hkv, N, d)
    return lib.attn_bwd(q, k, v, o, lse, do, dq, dk, dv, B, Hq, Hkv, N, d, scale, causal, dtype, ws,
                        ws_bytes, None)


@pytest.mark.parametrize("kw,status", [
    (dict(q=0), INVALID), (dict(lse=0), INVALID), (dict(do=0), INVALID), (dict(dv=0), INVALID),
    (dict(B=0), INVALID), (dict(N=0), INVALID), (dict(Hq=6, Hkv=4), INVALID), (dict(causal=3), INVALID),
    (dict(scale=math.inf), INVALID), (dict(dtype=F32), UNSUPPORTED), (dict(d=96), UNSUPPORTED),
    (dict(N=1 << 24), UNSUPPORTED), (dict(ws=0), INVALID), (dict(ws_bytes=64), INVALID),
    (dict(q=A + 8), INVALID), (dict(lse=A + 64 * MB + 2), INVALID), (dict(ws=A + 144 * MB + 4), INVALID),
    (dict(dq=A), INVALID), (dict(dk=A + 96 * MB), INVALID), (dict(ws=A + 128 * MB), INVALID),
])
def test_bwd_rejects_before_any_launch(lib, kw, status):
    assert bwd(lib, **kw) == status
    assert lib.attn_last_error().decode() != ""


def test_bwd_workspace_size(lib):
    # per-row D (rounded up to 64 floats), plus fp32 dk, dv per query head when grouped
    assert lib.attn_bwd_workspace_size(1, 4, 4, 100, 128) == 4 * 448      # 400 rows -> 448
    assert lib.attn_bwd_workspace_size(2, 12, 2, 8192, 128) == 4 * (2 * 12 * 8192 + 2 * 2 * 12 * 8192 * 128)
    assert lib.attn_bwd_workspace_size(1, 6, 4, 10, 64) == 0


def rms(lib, x=A, r=A + 16 * MB, w=A + 32 * MB, out=A + 48 * MB, rout=A + 64 * MB, T=100, D=1536,
        eps=1e-6, dtype=BF16):
    return lib.attn_add_rmsnorm(x, r, w, out, rout, T, D, eps, dtype, None)


@pytest.mark.parametrize("kw,status", [
    (dict(x=0), INVALID), (dict(w=0), INVALID), (dict(rout=0), INVALID), (dict(T=-1), INVALID),
    (dict(D=0), INVALID), (dict(eps=-1.0), INVALID), (dict(eps=math.nan), INVALID),
    (dict(dtype=F32), UNSUPPORTED), (dict(D=1540), UNSUPPORTED), (dict(D=8200), UNSUPPORTED),
    (dict(x=A + 8), INVALID), (dict(out=A + 48 * MB + 2), INVALID), (dict(out=A), INVALID),
    (dict(out=A + 64 * MB), INVALID), (dict(rout=A + 16 * MB + 1024), INVALID), (dict(rout=A + 100), INVALID),
])
def test_add_rmsnorm_rejects_before_any_launch(lib, kw, status):
    assert rms(lib, **kw) == status
    assert lib.attn_last_error().decode() != ""


def test_add_rmsnorm_in_place_and_empty(lib):
    # residual_out == residual is allowed; T = 0 returns OK without a launch
    assert rms(lib, rout=A + 16 * MB, T=0) == OK
    assert rms(lib, T=0) == OK


def swi(lib, g=A, u=A + 32 * MB, out=A + 64 * MB, T=100, F=8960, ld_in=8960, ld_out=8960, dtype=BF16):
    return lib.attn_swiglu(g, u, out, T, F, ld_in, ld_out, dtype, None)


@pytest.mark.parametrize("kw,status", [
    (dict(g=0), INVALID), (dict(out=0), INVALID), (dict(T=-2), INVALID), (dict(F=0), INVALID),
    (dict(ld_in=100), INVALID), (dict(ld_out=8952), INVALID), (dict(dtype=F32), UNSUPPORTED),
    (dict(F=8962, ld_in=8968, ld_out=8968), UNSUPPORTED), (dict(ld_in=8964), UNSUPPORTED),
    (dict(g=A + 4), INVALID), (dict(out=A + 64 * MB + 8), INVALID), (dict(out=A + 1024), INVALID),
    (dict(out=A + 32 * MB + 4096), INVALID),
])
def test_swiglu_rejects_before_any_launch(lib, kw, status):
    assert swi(lib, **kw) == status
    assert lib.attn_last_error().decode() != ""


def _gpu_present():
    return os.path.exists("/dev/kfd") or torch.cuda.is_available()


@pytest.mark.skipif(_gpu_present(), reason="valid arguments would launch on a GPU")
def test_no_device_status(lib):
    assert fwd(lib) == NO_DEVICE
    assert dec(lib) == NO_DEVICE
    assert dec_na(lib) == NO_DEVICE
    assert app(lib) == NO_DEVICE
    assert ppf(lib) == NO_DEVICE
    assert bwd(lib) == NO_DEVICE
    assert rms(lib) == NO_DEVICE and rms(lib, rout=A + 16 * MB) == NO_DEVICE
    assert swi(lib) == NO_DEVICE


def test_binding_rejects_host_tensors():
    q = torch.zeros(1, 2, 8, 64)
    with pytest.raises(ValueError):
        _lib.attn_fwd(q, q[:, :1], q[:, :1])
    with pytest.raises(ValueError):
        _lib.attn_fwd(q.to(torch.float16), q[:, :1], q[:, :1])


# ---------------------------------------- binding: caller-supplied outputs ----
# The C ABI receives only pointers, so the binding checks every output it is
# handed against the shape and dtype the kernels write.  These checks run
# before any pointer is taken, so host tensors show them without a GPU.

def _expect_bad_output(fn, match):
    with pytest.raises(ValueError, match=match):
        fn()


def test_binding_rejects_wrong_fwd_outputs():
    q = torch.zeros(1, 4, 8, 64, dtype=torch.bfloat16)
    k = torch.zeros(1, 2, 8, 64, dtype=torch.bfloat16)
    _expect_bad_output(lambda: _lib.attn_fwd(q, k, k, o=torch.zeros(1, 4, 7, 64, dtype=torch.bfloat16)),
                       "o must have shape")
    _expect_bad_output(lambda: _lib.attn_fwd(q, k, k, o=torch.zeros(1, 4, 8, 64)), "o must have dtype")
    _expect_bad_output(lambda: _lib.attn_fwd(q, k, k, lse=torch.zeros(1, 4, 8, dtype=torch.bfloat16)),
                       "lse must have dtype")
    _expect_bad_output(lambda: _lib.attn_fwd(q, k, k, lse=torch.zeros(1, 4, 9)), "lse must have shape")


def test_binding_rejects_wrong_decode_outputs():
    q = torch.zeros(3, 12, 128, dtype=torch.bfloat16)
    kc = torch.zeros(10, 2, 16, 128, dtype=torch.bfloat16)
    tab = torch.zeros(3, 4, dtype=torch.int32)
    ctx = torch.zeros(3, dtype=torch.int32)
    _expect_bad_output(lambda: _lib.attn_paged_decode(q, kc, kc, tab, ctx, o=torch.zeros(3, 12, 64,
                                                                                          dtype=torch.bfloat16)),
                       "o must have shape")
    _expect_bad_output(lambda: _lib.attn_paged_decode(q, kc, kc, tab, ctx, lse=torch.zeros(3, 12,
                                                                                            dtype=torch.float64)),
                       "lse must have dtype")


def test_binding_rejects_wrong_paged_prefill_outputs():
    q = torch.zeros(5, 12, 128, dtype=torch.bfloat16)
    kc = torch.zeros(10, 2, 16, 128, dtype=torch.bfloat16)
    tab = torch.zeros(2, 4, dtype=torch.int32)
    ctx = torch.zeros(2, dtype=torch.int32)
    starts = torch.zeros(3, dtype=torch.int32)
    _expect_bad_output(lambda: _lib.attn_paged_prefill(q, kc, kc, tab, ctx, starts,
                                                       o=torch.zeros(4, 12, 128, dtype=torch.bfloat16)),
                       "o must have shape")
    _expect_bad_output(lambda: _lib.attn_paged_prefill(q, kc, kc, tab, ctx, starts,
                                                       lse=torch.zeros(5, 12, dtype=torch.bfloat16)),
                       "lse must have dtype")


def test_binding_rejects_wrong_bwd_outputs():
    q = torch.zeros(1, 4, 8, 64, dtype=torch.bfloat16)
    k = torch.zeros(1, 2, 8, 64, dtype=torch.bfloat16)
    lse = torch.zeros(1, 4, 8)
    _expect_bad_output(lambda: _lib.attn_bwd(q, k, k, q, lse, q, dq=torch.zeros(1, 4, 8, 32, dtype=torch.bfloat16)),
                       "dq must have shape")
    _expect_bad_output(lambda: _lib.attn_bwd(q, k, k, q, lse, q, dk=torch.zeros_like(q)), "dk must have shape")
    _expect_bad_output(lambda: _lib.attn_bwd(q, k, k, q, lse, q, dv=torch.zeros(1, 2, 8, 64)), "dv must have dtype")


def test_binding_rejects_wrong_fusion_outputs():
    x = torch.zeros(4, 256, dtype=torch.bfloat16)
    w = torch.zeros(256, dtype=torch.bfloat16)
    _expect_bad_output(lambda: _lib.attn_add_rmsnorm(x, x, w, out=torch.zeros(4, 128, dtype=torch.bfloat16)),
                       "out must have shape")
    _expect_bad_output(lambda: _lib.attn_add_rmsnorm(x, x, w, residual_out=torch.zeros(4, 256)),
                       "residual_out must have dtype")
    gu = torch.zeros(4, 512, dtype=torch.bfloat16)
    _expect_bad_output(lambda: _lib.attn_swiglu(gu, out=torch.zeros(4, 512, dtype=torch.bfloat16)),
                       "out must have shape")
    _expect_bad_output(lambda: _lib.attn_swiglu(x, x, out=torch.zeros(4, 256)), "out must have dtype")


def test_autograd_wrapper_has_no_cpu_path():
    """attention() (the autograd function over attn_fwd and attn_bwd) passes
    host tensors to the binding, which refuses them: there is no CPU
    fallback."""
    from exact_tiled_self_amd import attention
    q = torch.zeros(1, 2, 8, 64, dtype=torch.bfloat16, requires_grad=True)
    k = torch.zeros(1, 2, 8, 64, dtype=torch.bfloat16, requires_grad=True)
    with pytest.raises(ValueError, match="device"):
        attention(q, k, k, causal=True)

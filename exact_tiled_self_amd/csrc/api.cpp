// C ABI of libattn.so: argument validation, device check and dispatch.
//
// Order of checks: every argument check first (no HIP runtime call, so the
// same errors come back on a machine without a GPU), then the device check,
// then the launch.  On any error nothing is enqueued.

#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <atomic>

#include "../../include/attn.h"
#include "internal.h"

namespace {

thread_local char g_err[256] = "";

attn_status fail(attn_status st, const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof(g_err), fmt, ap);
    va_end(ap);
    return st;
}

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

bool overlap(const void* a, size_t na, const void* b, size_t nb) {
    if (!a || !b || na == 0 || nb == 0) return false;
    const uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
    return x < y + nb && y < x + na;
}

// Architecture check, cached per device: 0 unknown, 1 gfx950, 2 other.
constexpr int kMaxDevices = 64;
std::atomic<int> g_arch[kMaxDevices];

attn_status check_device() {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0) {
        (void)hipGetLastError();
        return fail(ATTN_ERR_NO_DEVICE, "no HIP device is available");
    }
    const char* forced = getenv("ATTN_FORCE_ARCH");   // test hook: pretend another architecture
    if (forced && *forced) {
        if (strncmp(forced, "gfx950", 6) != 0)
            return fail(ATTN_ERR_UNSUPPORTED, "device architecture %s is not gfx950", forced);
        return ATTN_OK;
    }
    int st = dev < kMaxDevices ? g_arch[dev].load(std::memory_order_relaxed) : 0;
    if (st == 0) {
        hipDeviceProp_t prop;
        if (hipGetDeviceProperties(&prop, dev) != hipSuccess) {
            (void)hipGetLastError();
            return fail(ATTN_ERR_NO_DEVICE, "cannot query device %d", dev);
        }
        st = strncmp(prop.gcnArchName, "gfx950", 6) == 0 ? 1 : 2;
        if (dev < kMaxDevices) g_arch[dev].store(st, std::memory_order_relaxed);
        if (st == 2) return fail(ATTN_ERR_UNSUPPORTED, "device architecture %s is not gfx950", prop.gcnArchName);
    }
    if (st == 2) return fail(ATTN_ERR_UNSUPPORTED, "device architecture is not gfx950");
    return ATTN_OK;
}

attn_status launch_status(hipError_t e) {
    if (e == hipSuccess) return ATTN_OK;
    return fail(ATTN_ERR_LAUNCH, "kernel launch failed: %s", hipGetErrorString(e));
}

size_t elem_size(attn_dtype dt) { return dt == ATTN_F32 ? 4 : 2; }

}  // namespace

extern "C" {

int attn_abi_version(void) { return ATTN_ABI_VERSION; }

const char* attn_last_error(void) { return g_err; }

const char* attn_status_string(attn_status s) {
    switch (s) {
        case ATTN_OK: return "ATTN_OK";
        case ATTN_ERR_INVALID_ARG: return "ATTN_ERR_INVALID_ARG";
        case ATTN_ERR_UNSUPPORTED: return "ATTN_ERR_UNSUPPORTED";
        case ATTN_ERR_NO_DEVICE: return "ATTN_ERR_NO_DEVICE";
        case ATTN_ERR_LAUNCH: return "ATTN_ERR_LAUNCH";
    }
    return "ATTN_STATUS_UNKNOWN";
}

attn_status attn_fwd(const void* q, const void* k, const void* v, void* o, float* lse, int B, int Hq,
                     int Hkv, int N, int d, float scale, int causal, attn_dtype dtype, void* stream) {
    g_err[0] = '\0';
    if (!q || !k || !v || !o) return fail(ATTN_ERR_INVALID_ARG, "q, k, v and o must be non-null");
    if (B < 1 || Hq < 1 || Hkv < 1 || N < 1)
        return fail(ATTN_ERR_INVALID_ARG, "B, Hq, Hkv and N must be >= 1 (got %d, %d, %d, %d)", B, Hq, Hkv, N);
    if (Hq % Hkv != 0) return fail(ATTN_ERR_INVALID_ARG, "Hq (%d) must be a multiple of Hkv (%d)", Hq, Hkv);
    if (causal != 0 && causal != 1) return fail(ATTN_ERR_INVALID_ARG, "causal must be 0 or 1");
    if (!isfinite(scale)) return fail(ATTN_ERR_INVALID_ARG, "scale must be finite");
    if (dtype != ATTN_F32 && dtype != ATTN_BF16) return fail(ATTN_ERR_UNSUPPORTED, "dtype %d is not supported", (int)dtype);
    if (d != 64 && d != 128) return fail(ATTN_ERR_UNSUPPORTED, "head dim %d is not supported (64 or 128)", d);
    // per-head byte offsets (plus one tile of look-ahead) must fit 32 bits
    if ((long long)N * d > (1LL << 31) - (1LL << 16))
        return fail(ATTN_ERR_UNSUPPORTED, "N * d must be at most 2^31 - 2^16");
    // fp32: a head's bytes (4 per element) are addressed with 32-bit offsets
    if (dtype == ATTN_F32 && (long long)N * d > (1LL << 29))
        return fail(ATTN_ERR_UNSUPPORTED, "fp32: N * d must be at most 2^29");
    const int rows_per_wg = dtype == ATTN_F32 ? 16 : 64;   // the smallest row tile of either kernel
    const long long grid = (long long)B * Hq * ((N + rows_per_wg - 1) / rows_per_wg);
    if (grid >= (1LL << 31)) return fail(ATTN_ERR_UNSUPPORTED, "problem too large for one launch");
    if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(o, 16))
        return fail(ATTN_ERR_INVALID_ARG, "q, k, v and o must be 16-byte aligned");
    if (lse && !aligned(lse, 4)) return fail(ATTN_ERR_INVALID_ARG, "lse must be 4-byte aligned");
    const size_t es = elem_size(dtype);
    const size_t qbytes = (size_t)B * Hq * N * d * es, kvbytes = (size_t)B * Hkv * N * d * es;
    const size_t lbytes = lse ? (size_t)B * Hq * N * 4 : 0;
    if (overlap(o, qbytes, q, qbytes) || overlap(o, qbytes, k, kvbytes) || overlap(o, qbytes, v, kvbytes) ||
        overlap(lse, lbytes, q, qbytes) || overlap(lse, lbytes, k, kvbytes) ||
        overlap(lse, lbytes, v, kvbytes) || overlap(lse, lbytes, o, qbytes))
        return fail(ATTN_ERR_INVALID_ARG, "outputs must not overlap inputs or each other");

    attn_status st = check_device();
    if (st != ATTN_OK) return st;

    attn::PrefillArgs a;
    a.q = q; a.k = k; a.v = v; a.o = o; a.lse = lse;
    a.B = B; a.Hq = Hq; a.Hkv = Hkv; a.N = N; a.d = d;
    a.c = (float)(fabs((double)scale) * 1.4426950408889634);
    a.negate = scale < 0.f ? 1 : 0;
    a.causal = causal;
    hipStream_t s = static_cast<hipStream_t>(stream);
    return launch_status(dtype == ATTN_BF16 ? attn::launch_prefill_bf16(a, s) : attn::launch_prefill_f32(a, s));
}

size_t attn_paged_decode_workspace_size(int S, int Hq, int d, int max_blocks, int block_size) {
    if (S < 1 || Hq < 1 || d < 1 || max_blocks < 1 || block_size != attn::kDecodeBlock) return 0;
    return attn::decode_workspace_bound(S, Hq, d);
}

}  // extern "C"

namespace {

static_assert(ATTN_DECODE_NOALLOC_SCRATCH_BYTES == attn::kDecodeScratchBytes, "scratch size");

// Checks shared by both decode entry points (everything but the workspace).
attn_status check_decode_args(const void* q, const void* k_cache, const void* v_cache,
                              const int32_t* block_table, const int32_t* ctx_lens, int block_size,
                              void* o, float* lse, int S, int Hq, int Hkv, int d, int max_blocks,
                              int num_blocks, float scale, attn_dtype dtype) {
    if (!q || !k_cache || !v_cache || !block_table || !ctx_lens || !o)
        return fail(ATTN_ERR_INVALID_ARG, "q, k_cache, v_cache, block_table, ctx_lens and o must be non-null");
    if (S < 1 || Hq < 1 || Hkv < 1 || max_blocks < 1 || num_blocks < 1)
        return fail(ATTN_ERR_INVALID_ARG, "S, Hq, Hkv, max_blocks and num_blocks must be >= 1");
    if (Hq % Hkv != 0) return fail(ATTN_ERR_INVALID_ARG, "Hq (%d) must be a multiple of Hkv (%d)", Hq, Hkv);
    if (!isfinite(scale)) return fail(ATTN_ERR_INVALID_ARG, "scale must be finite");
    if (dtype != ATTN_BF16) return fail(ATTN_ERR_UNSUPPORTED, "paged decode supports bf16 only");
    if (d != 64 && d != 128) return fail(ATTN_ERR_UNSUPPORTED, "head dim %d is not supported (64 or 128)", d);
    if (block_size != attn::kDecodeBlock)
        return fail(ATTN_ERR_UNSUPPORTED, "block_size %d is not supported (16)", block_size);
    if ((long long)max_blocks * block_size >= (1LL << 30)) return fail(ATTN_ERR_UNSUPPORTED, "max_blocks too large");
    if ((long long)num_blocks * Hkv * block_size * d >= (1LL << 40))
        return fail(ATTN_ERR_UNSUPPORTED, "KV pool too large");
    // (pairs of sequence and virtual kv head: at most 16 query heads each)
    const long long hv = (long long)Hkv * attn::decode_groups(Hq / Hkv);
    if ((long long)S * hv * max_blocks >= (1LL << 31) || S > 65535 || Hkv > 65535)
        return fail(ATTN_ERR_UNSUPPORTED, "too many sequences or blocks for one launch");
    if (!aligned(q, 16) || !aligned(k_cache, 16) || !aligned(v_cache, 16) || !aligned(o, 16))
        return fail(ATTN_ERR_INVALID_ARG, "q, k_cache, v_cache and o must be 16-byte aligned");
    if (!aligned(block_table, 4) || !aligned(ctx_lens, 4) || (lse && !aligned(lse, 4)))
        return fail(ATTN_ERR_INVALID_ARG, "block_table, ctx_lens and lse must be 4-byte aligned");
    const size_t es = 2;
    const size_t qb = (size_t)S * Hq * d * es, cb = (size_t)num_blocks * Hkv * block_size * d * es;
    const size_t tb = (size_t)S * max_blocks * 4, lb = (size_t)S * 4, lsb = lse ? (size_t)S * Hq * 4 : 0;
    const void* ins[5] = {q, k_cache, v_cache, block_table, ctx_lens};
    const size_t insz[5] = {qb, cb, cb, tb, lb};
    for (int i = 0; i < 5; ++i)
        if (overlap(o, qb, ins[i], insz[i]) || overlap(lse, lsb, ins[i], insz[i]))
            return fail(ATTN_ERR_INVALID_ARG, "outputs must not overlap the inputs");
    if (overlap(o, qb, lse, lsb)) return fail(ATTN_ERR_INVALID_ARG, "o and lse must not overlap");
    return ATTN_OK;
}

attn::DecodeArgs decode_args(const void* q, const void* k_cache, const void* v_cache,
                             const int32_t* block_table, const int32_t* ctx_lens, void* o, float* lse,
                             int S, int Hq, int Hkv, int d, int max_blocks, int num_blocks, float scale,
                             void* workspace) {
    attn::DecodeArgs a;
    a.q = q; a.k_cache = k_cache; a.v_cache = v_cache; a.block_table = block_table; a.ctx_lens = ctx_lens;
    a.o = o; a.lse = lse; a.S = S; a.Hq = Hq; a.Hkv = Hkv; a.d = d;
    a.max_blocks = max_blocks; a.num_blocks = num_blocks;
    a.c = (float)(fabs((double)scale) * 1.4426950408889634);
    a.negate = scale < 0.f ? 1 : 0;
    a.workspace = static_cast<float*>(workspace);
    return a;
}

}  // namespace

extern "C" {

attn_status attn_paged_decode(const void* q, const void* k_cache, const void* v_cache,
                              const int32_t* block_table, const int32_t* ctx_lens, int block_size,
                              void* o, float* lse, int S, int Hq, int Hkv, int d, int max_blocks,
                              int num_blocks, float scale, attn_dtype dtype, void* workspace,
                              size_t workspace_bytes, void* stream) {
    g_err[0] = '\0';
    attn_status st = check_decode_args(q, k_cache, v_cache, block_table, ctx_lens, block_size, o, lse, S, Hq,
                                       Hkv, d, max_blocks, num_blocks, scale, dtype);
    if (st != ATTN_OK) return st;
    const size_t need = attn_paged_decode_workspace_size(S, Hq, d, max_blocks, block_size);
    if (!workspace || workspace_bytes < need)
        return fail(ATTN_ERR_INVALID_ARG, "workspace needs %zu bytes (got %zu)", need, workspace ? workspace_bytes : (size_t)0);
    if (!aligned(workspace, 16)) return fail(ATTN_ERR_INVALID_ARG, "workspace must be 16-byte aligned");
    const size_t es = 2;
    const size_t qb = (size_t)S * Hq * d * es, cb = (size_t)num_blocks * Hkv * block_size * d * es;
    const size_t tb = (size_t)S * max_blocks * 4, lb = (size_t)S * 4, lsb = lse ? (size_t)S * Hq * 4 : 0;
    const void* others[7] = {q, k_cache, v_cache, block_table, ctx_lens, o, lse};
    const size_t osz[7] = {qb, cb, cb, tb, lb, qb, lsb};
    for (int i = 0; i < 7; ++i)
        if (overlap(workspace, need, others[i], osz[i]))
            return fail(ATTN_ERR_INVALID_ARG, "the workspace must not overlap the inputs or outputs");

    st = check_device();
    if (st != ATTN_OK) return st;
    const attn::DecodeArgs a = decode_args(q, k_cache, v_cache, block_table, ctx_lens, o, lse, S, Hq, Hkv, d,
                                           max_blocks, num_blocks, scale, workspace);
    return launch_status(attn::launch_paged_decode_bf16(a, static_cast<hipStream_t>(stream)));
}

attn_status attn_paged_decode_noalloc(const void* q, const void* k_cache, const void* v_cache,
                                      const int32_t* block_table, const int32_t* ctx_lens, int block_size,
                                      void* o, float* lse, int S, int Hq, int Hkv, int d, int max_blocks,
                                      int num_blocks, float scale, attn_dtype dtype, void* stream) {
    g_err[0] = '\0';
    attn_status st = check_decode_args(q, k_cache, v_cache, block_table, ctx_lens, block_size, o, lse, S, Hq,
                                       Hkv, d, max_blocks, num_blocks, scale, dtype);
    if (st != ATTN_OK) return st;
    const size_t need = attn::decode_workspace_exact(S, Hq, Hkv, d);
    if (need > attn::kDecodeScratchBytes)
        return fail(ATTN_ERR_UNSUPPORTED, "this decode needs %zu bytes of partial states; the library's static "
                    "scratch holds %zu (use attn_paged_decode with a workspace)", need, attn::kDecodeScratchBytes);

    st = check_device();
    if (st != ATTN_OK) return st;
    const attn::DecodeArgs a = decode_args(q, k_cache, v_cache, block_table, ctx_lens, o, lse, S, Hq, Hkv, d,
                                           max_blocks, num_blocks, scale, nullptr);
    return launch_status(attn::launch_paged_decode_bf16_noalloc(a, static_cast<hipStream_t>(stream)));
}

attn_status attn_kv_append(const void* k_new, const void* v_new, void* k_cache, void* v_cache,
                           const int32_t* block_table, const int32_t* ctx_lens, const int32_t* starts,
                           int block_size, int S, int T, int max_new, int Hkv, int d, int max_blocks,
                           int num_blocks, attn_dtype dtype, void* stream) {
    g_err[0] = '\0';
    if (!k_new || !v_new || !k_cache || !v_cache || !block_table || !ctx_lens || !starts)
        return fail(ATTN_ERR_INVALID_ARG, "k_new, v_new, k_cache, v_cache, block_table, ctx_lens and starts must be non-null");
    if (S < 1 || Hkv < 1 || d < 1 || max_blocks < 1 || num_blocks < 1)
        return fail(ATTN_ERR_INVALID_ARG, "S, Hkv, d, max_blocks and num_blocks must be >= 1");
    if (T < 0 || max_new < 0) return fail(ATTN_ERR_INVALID_ARG, "T and max_new must be >= 0");
    if (dtype != ATTN_F32 && dtype != ATTN_BF16) return fail(ATTN_ERR_UNSUPPORTED, "dtype %d is not supported", (int)dtype);
    const size_t es = elem_size(dtype);
    const size_t row = (size_t)d * es;
    if (row % 16 != 0 || row > 4096)
        return fail(ATTN_ERR_UNSUPPORTED, "d * element size must be a multiple of 16 bytes, at most 4096");
    if (block_size < 1 || block_size > 1024)
        return fail(ATTN_ERR_UNSUPPORTED, "block_size %d is not supported (1 .. 1024)", block_size);
    if (S > 65535) return fail(ATTN_ERR_UNSUPPORTED, "at most 65535 sequences per call");
    if ((long long)max_blocks * block_size >= (1LL << 30)) return fail(ATTN_ERR_UNSUPPORTED, "max_blocks too large");
    const int cpr = (int)(row / 16);
    if ((long long)max_new * Hkv * cpr >= (1LL << 31) - 256)
        return fail(ATTN_ERR_UNSUPPORTED, "max_new too large for one launch");
    if ((long long)num_blocks * Hkv * block_size * (long long)row >= (1LL << 48))
        return fail(ATTN_ERR_UNSUPPORTED, "KV pool too large");
    if (!aligned(k_new, 16) || !aligned(v_new, 16) || !aligned(k_cache, 16) || !aligned(v_cache, 16))
        return fail(ATTN_ERR_INVALID_ARG, "k_new, v_new, k_cache and v_cache must be 16-byte aligned");
    if (!aligned(block_table, 4) || !aligned(ctx_lens, 4) || !aligned(starts, 4))
        return fail(ATTN_ERR_INVALID_ARG, "block_table, ctx_lens and starts must be 4-byte aligned");
    const size_t nb = (size_t)T * Hkv * row, cb = (size_t)num_blocks * Hkv * block_size * row;
    const void* ins[5] = {k_new, v_new, block_table, ctx_lens, starts};
    const size_t insz[5] = {nb, nb, (size_t)S * max_blocks * 4, (size_t)S * 4, (size_t)(S + 1) * 4};
    for (int i = 0; i < 5; ++i)
        if (overlap(k_cache, cb, ins[i], insz[i]) || overlap(v_cache, cb, ins[i], insz[i]))
            return fail(ATTN_ERR_INVALID_ARG, "the caches must not overlap the inputs");
    if (overlap(k_cache, cb, v_cache, cb)) return fail(ATTN_ERR_INVALID_ARG, "k_cache and v_cache must not overlap");
    if (T == 0 || max_new == 0) return ATTN_OK;

    attn_status st = check_device();
    if (st != ATTN_OK) return st;

    attn::KvAppendArgs a;
    a.k_new = k_new; a.v_new = v_new; a.k_cache = k_cache; a.v_cache = v_cache;
    a.block_table = block_table; a.ctx_lens = ctx_lens; a.starts = starts;
    a.S = S; a.T = T; a.max_new = max_new; a.Hkv = Hkv; a.block_size = block_size;
    a.max_blocks = max_blocks; a.num_blocks = num_blocks; a.cpr = cpr;
    return launch_status(attn::launch_kv_append(a, static_cast<hipStream_t>(stream)));
}

attn_status attn_paged_prefill(const void* q, const void* k_cache, const void* v_cache,
                               const int32_t* block_table, const int32_t* ctx_lens, const int32_t* starts,
                               int block_size, void* o, float* lse, int S, int T, int max_new, int Hq,
                               int Hkv, int d, int max_blocks, int num_blocks, float scale,
                               attn_dtype dtype, void* stream) {
    g_err[0] = '\0';
    if (!q || !k_cache || !v_cache || !block_table || !ctx_lens || !starts || !o)
        return fail(ATTN_ERR_INVALID_ARG, "q, k_cache, v_cache, block_table, ctx_lens, starts and o must be non-null");
    if (S < 1 || Hq < 1 || Hkv < 1 || max_blocks < 1 || num_blocks < 1)
        return fail(ATTN_ERR_INVALID_ARG, "S, Hq, Hkv, max_blocks and num_blocks must be >= 1");
    if (T < 0 || max_new < 0) return fail(ATTN_ERR_INVALID_ARG, "T and max_new must be >= 0");
    if (Hq % Hkv != 0) return fail(ATTN_ERR_INVALID_ARG, "Hq (%d) must be a multiple of Hkv (%d)", Hq, Hkv);
    if (!isfinite(scale)) return fail(ATTN_ERR_INVALID_ARG, "scale must be finite");
    if (dtype != ATTN_BF16) return fail(ATTN_ERR_UNSUPPORTED, "paged prefill supports bf16 only");
    if (d != 64 && d != 128) return fail(ATTN_ERR_UNSUPPORTED, "head dim %d is not supported (64 or 128)", d);
    if (block_size != attn::kDecodeBlock)
        return fail(ATTN_ERR_UNSUPPORTED, "block_size %d is not supported (16)", block_size);
    if ((long long)max_blocks * block_size >= (1LL << 30)) return fail(ATTN_ERR_UNSUPPORTED, "max_blocks too large");
    if ((long long)max_new * Hq * d * 2 >= (1LL << 31))
        return fail(ATTN_ERR_UNSUPPORTED, "max_new * Hq * d * 2 must be below 2^31");
    if ((long long)((max_new + 127) / 128) * S * Hq + 8LL * Hq >= (1LL << 31))
        return fail(ATTN_ERR_UNSUPPORTED, "problem too large for one launch");
    if ((long long)num_blocks * Hkv * block_size * d >= (1LL << 40))
        return fail(ATTN_ERR_UNSUPPORTED, "KV pool too large");
    if (!aligned(q, 16) || !aligned(k_cache, 16) || !aligned(v_cache, 16) || !aligned(o, 16))
        return fail(ATTN_ERR_INVALID_ARG, "q, k_cache, v_cache and o must be 16-byte aligned");
    if (!aligned(block_table, 4) || !aligned(ctx_lens, 4) || !aligned(starts, 4) || (lse && !aligned(lse, 4)))
        return fail(ATTN_ERR_INVALID_ARG, "block_table, ctx_lens, starts and lse must be 4-byte aligned");
    const size_t qb = (size_t)T * Hq * d * 2, cb = (size_t)num_blocks * Hkv * block_size * d * 2;
    const size_t lsb = lse ? (size_t)T * Hq * 4 : 0;
    const void* ins[6] = {q, k_cache, v_cache, block_table, ctx_lens, starts};
    const size_t insz[6] = {qb, cb, cb, (size_t)S * max_blocks * 4, (size_t)S * 4, (size_t)(S + 1) * 4};
    for (int i = 0; i < 6; ++i)
        if (overlap(o, qb, ins[i], insz[i]) || overlap(lse, lsb, ins[i], insz[i]))
            return fail(ATTN_ERR_INVALID_ARG, "outputs must not overlap the inputs");
    if (overlap(o, qb, lse, lsb)) return fail(ATTN_ERR_INVALID_ARG, "o and lse must not overlap");
    if (T == 0 || max_new == 0) return ATTN_OK;

    attn_status st = check_device();
    if (st != ATTN_OK) return st;

    attn::PagedPrefillArgs a;
    a.q = q; a.k_cache = k_cache; a.v_cache = v_cache; a.block_table = block_table;
    a.ctx_lens = ctx_lens; a.starts = starts; a.o = o; a.lse = lse;
    a.S = S; a.T = T; a.max_new = max_new; a.Hq = Hq; a.Hkv = Hkv; a.d = d;
    a.max_blocks = max_blocks; a.num_blocks = num_blocks;
    a.c = (float)(fabs((double)scale) * 1.4426950408889634);
    a.negate = scale < 0.f ? 1 : 0;
    return launch_status(attn::launch_paged_prefill_bf16(a, static_cast<hipStream_t>(stream)));
}

size_t attn_bwd_workspace_size(int B, int Hq, int Hkv, int N, int d) {
    if (B < 1 || Hq < 1 || Hkv < 1 || N < 1 || d < 1 || Hq % Hkv != 0) return 0;
    return attn::bwd_workspace_bytes(B, Hq, Hkv, N, d);
}

attn_status attn_bwd(const void* q, const void* k, const void* v, const void* o, const float* lse,
                     const void* dout, void* dq, void* dk, void* dv, int B, int Hq, int Hkv, int N, int d,
                     float scale, int causal, attn_dtype dtype, void* workspace, size_t workspace_bytes,
                     void* stream) {
    g_err[0] = '\0';
    if (!q || !k || !v || !o || !lse || !dout || !dq || !dk || !dv)
        return fail(ATTN_ERR_INVALID_ARG, "q, k, v, o, lse, dout, dq, dk and dv must be non-null");
    if (B < 1 || Hq < 1 || Hkv < 1 || N < 1)
        return fail(ATTN_ERR_INVALID_ARG, "B, Hq, Hkv and N must be >= 1 (got %d, %d, %d, %d)", B, Hq, Hkv, N);
    if (Hq % Hkv != 0) return fail(ATTN_ERR_INVALID_ARG, "Hq (%d) must be a multiple of Hkv (%d)", Hq, Hkv);
    if (causal != 0 && causal != 1) return fail(ATTN_ERR_INVALID_ARG, "causal must be 0 or 1");
    if (!isfinite(scale)) return fail(ATTN_ERR_INVALID_ARG, "scale must be finite");
    if (dtype != ATTN_BF16) return fail(ATTN_ERR_UNSUPPORTED, "the backward pass supports bf16 only");
    if (d != 64 && d != 128) return fail(ATTN_ERR_UNSUPPORTED, "head dim %d is not supported (64 or 128)", d);
    if ((long long)N * d > (1LL << 31) - (1LL << 16))
        return fail(ATTN_ERR_UNSUPPORTED, "N * d must be at most 2^31 - 2^16");
    // fp32: a head's bytes (4 per element) are addressed with 32-bit offsets
    if (dtype == ATTN_F32 && (long long)N * d > (1LL << 29))
        return fail(ATTN_ERR_UNSUPPORTED, "fp32: N * d must be at most 2^29");
    const long long grid = (long long)B * Hq * ((N + 127) / 128);
    if (grid >= (1LL << 31) || (long long)B * Hq * N * (d / 8) >= (1LL << 38))
        return fail(ATTN_ERR_UNSUPPORTED, "problem too large for one launch");
    const size_t need = attn_bwd_workspace_size(B, Hq, Hkv, N, d);
    if (!workspace || workspace_bytes < need)
        return fail(ATTN_ERR_INVALID_ARG, "workspace needs %zu bytes (got %zu)", need, workspace ? workspace_bytes : (size_t)0);
    if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(o, 16) || !aligned(dout, 16) ||
        !aligned(dq, 16) || !aligned(dk, 16) || !aligned(dv, 16) || !aligned(workspace, 16))
        return fail(ATTN_ERR_INVALID_ARG, "q, k, v, o, dout, dq, dk, dv and workspace must be 16-byte aligned");
    if (!aligned(lse, 4)) return fail(ATTN_ERR_INVALID_ARG, "lse must be 4-byte aligned");
    const size_t qb = (size_t)B * Hq * N * d * 2, kb = (size_t)B * Hkv * N * d * 2, lb = (size_t)B * Hq * N * 4;
    const void* ins[6] = {q, k, v, o, lse, dout};
    const size_t insz[6] = {qb, kb, kb, qb, lb, qb};
    const void* outs[4] = {dq, dk, dv, workspace};
    const size_t outsz[4] = {qb, kb, kb, need};
    for (int i = 0; i < 4; ++i) {
        for (int j = 0; j < 6; ++j)
            if (overlap(outs[i], outsz[i], ins[j], insz[j]))
                return fail(ATTN_ERR_INVALID_ARG, "outputs and workspace must not overlap the inputs");
        for (int j = i + 1; j < 4; ++j)
            if (overlap(outs[i], outsz[i], outs[j], outsz[j]))
                return fail(ATTN_ERR_INVALID_ARG, "dq, dk, dv and workspace must not overlap");
    }

    attn_status st = check_device();
    if (st != ATTN_OK) return st;

    attn::BackwardArgs a;
    a.q = q; a.k = k; a.v = v; a.o = o; a.lse = lse; a.dout = dout;
    a.dq = dq; a.dk = dk; a.dv = dv;
    a.B = B; a.Hq = Hq; a.Hkv = Hkv; a.N = N; a.d = d;
    a.scale = scale; a.causal = causal;
    a.workspace = static_cast<float*>(workspace);
    return launch_status(attn::launch_backward_bf16(a, static_cast<hipStream_t>(stream)));
}

attn_status attn_add_rmsnorm(const void* x, const void* residual, const void* weight, void* out,
                             void* residual_out, int T, int D, float eps, attn_dtype dtype, void* stream) {
    g_err[0] = '\0';
    if (!x || !residual || !weight || !out || !residual_out)
        return fail(ATTN_ERR_INVALID_ARG, "x, residual, weight, out and residual_out must be non-null");
    if (T < 0 || D < 1) return fail(ATTN_ERR_INVALID_ARG, "T must be >= 0 and D >= 1");
    if (!isfinite(eps) || eps < 0.f) return fail(ATTN_ERR_INVALID_ARG, "eps must be finite and >= 0");
    if (dtype != ATTN_BF16) return fail(ATTN_ERR_UNSUPPORTED, "add_rmsnorm supports bf16 only");
    if (D % 8 != 0 || D > 8192) return fail(ATTN_ERR_UNSUPPORTED, "D must be a multiple of 8, at most 8192");
    if (!aligned(x, 16) || !aligned(residual, 16) || !aligned(weight, 16) || !aligned(out, 16) ||
        !aligned(residual_out, 16))
        return fail(ATTN_ERR_INVALID_ARG, "all pointers must be 16-byte aligned");
    const size_t rb = (size_t)T * D * 2, wb = (size_t)D * 2;
    if (overlap(out, rb, x, rb) || overlap(out, rb, residual, rb) || overlap(out, rb, weight, wb) ||
        overlap(out, rb, residual_out, rb))
        return fail(ATTN_ERR_INVALID_ARG, "out must not overlap the inputs or residual_out");
    if ((residual_out != residual && overlap(residual_out, rb, residual, rb)) ||
        overlap(residual_out, rb, x, rb) || overlap(residual_out, rb, weight, wb))
        return fail(ATTN_ERR_INVALID_ARG, "residual_out must be residual itself or overlap no input");
    if (T == 0) return ATTN_OK;

    attn_status st = check_device();
    if (st != ATTN_OK) return st;
    attn::AddRmsNormArgs a;
    a.x = x; a.residual = residual; a.weight = weight; a.out = out; a.residual_out = residual_out;
    a.T = T; a.D = D; a.eps = eps;
    return launch_status(attn::launch_add_rmsnorm_bf16(a, static_cast<hipStream_t>(stream)));
}

attn_status attn_swiglu(const void* gate, const void* up, void* out, int T, int F, int ld_in, int ld_out,
                        attn_dtype dtype, void* stream) {
    g_err[0] = '\0';
    if (!gate || !up || !out) return fail(ATTN_ERR_INVALID_ARG, "gate, up and out must be non-null");
    if (T < 0 || F < 1) return fail(ATTN_ERR_INVALID_ARG, "T must be >= 0 and F >= 1");
    if (ld_in < F || ld_out < F) return fail(ATTN_ERR_INVALID_ARG, "row strides must be >= F");
    if (dtype != ATTN_BF16) return fail(ATTN_ERR_UNSUPPORTED, "swiglu supports bf16 only");
    if (F % 8 != 0 || ld_in % 8 != 0 || ld_out % 8 != 0)
        return fail(ATTN_ERR_UNSUPPORTED, "F and the row strides must be multiples of 8");
    if ((long long)T * (F / 8) >= (1LL << 38)) return fail(ATTN_ERR_UNSUPPORTED, "problem too large for one launch");
    if (!aligned(gate, 16) || !aligned(up, 16) || !aligned(out, 16))
        return fail(ATTN_ERR_INVALID_ARG, "gate, up and out must be 16-byte aligned");
    const size_t ib = T ? ((size_t)(T - 1) * ld_in + F) * 2 : 0, ob = T ? ((size_t)(T - 1) * ld_out + F) * 2 : 0;
    if (overlap(out, ob, gate, ib) || overlap(out, ob, up, ib))
        return fail(ATTN_ERR_INVALID_ARG, "out must not overlap gate or up");
    if (T == 0) return ATTN_OK;

    attn_status st = check_device();
    if (st != ATTN_OK) return st;
    attn::SwigluArgs a;
    a.gate = gate; a.up = up; a.out = out; a.T = T; a.F = F; a.ld_in = ld_in; a.ld_out = ld_out;
    return launch_status(attn::launch_swiglu_bf16(a, static_cast<hipStream_t>(stream)));
}

}  // extern "C"

/*
 * attn.h - exact tiled scaled-dot-product attention forward on MI355X (gfx950).
 *
 * C ABI of libattn.so.  Every tensor argument is a plain pointer to DEVICE
 * memory owned by the caller; sizes are plain integers; `stream` is a
 * hipStream_t passed as void* (NULL = the default stream).
 *
 * What is computed.  For each query row q_i and the keys k_j / values v_j it
 * may attend to ("Autoatención, kernels CUDA y FlashAttention", section 1):
 *
 *     o_i   = sum_j softmax_j(scale * <q_i, k_j>) v_j
 *     lse_i = ln sum_j exp(scale * <q_i, k_j>)          (natural log)
 *
 * The library evaluates this exactly (up to floating-point order) block by
 * block with the online-softmax recurrence ("FlashAttention" notes, section
 * "No basta con promediar los resultados de los bloques"): a running maximum
 * m, sum l and numerator u per row, earlier l and u rescaled by e^(m - m')
 * when a block raises the maximum, output u / l.  The N x N score matrix is
 * never written to device memory (same page, introduction; first page,
 * section 3).  Only o and the per-row statistic lse leave the chip; lse is
 * the normalisation statistic kept for a backward pass (first page,
 * section 3, "Recálculo durante la retropropagación").
 *
 * Ownership and concurrency.  The caller allocates and frees every buffer,
 * including the decode workspace.  The library allocates no device memory,
 * never synchronises, and never changes the current device: all work is
 * enqueued on `stream` for the current device and runs asynchronously, so
 * buffers must stay alive until that work completes.  Outputs are fully
 * overwritten; inputs are only read and must not overlap the outputs.  The
 * library keeps no state between calls apart from a per-device cache of the
 * architecture check and a per-thread error string, so concurrent calls
 * from several host threads are safe when their buffers are disjoint.
 *
 * Errors.  Every condition the host can check is checked synchronously,
 * before anything is enqueued: on a non-OK return nothing has been launched
 * and the outputs are untouched; attn_last_error() then gives a one-line
 * reason.  There is no fallback path: unsupported shapes, dtypes or devices
 * are errors.  Argument checks come before any HIP runtime call, so they
 * behave the same with no GPU present.
 */
#ifndef ATTN_H
#define ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define ATTN_ABI_VERSION 2

typedef enum {
    ATTN_OK = 0,
    ATTN_ERR_INVALID_ARG = 1,   /* null pointer, bad size, misalignment, overlap,
                                   Hq % Hkv != 0, non-finite scale, small workspace */
    ATTN_ERR_UNSUPPORTED = 2,   /* valid but not implemented: head dim, dtype,
                                   block size, sizes beyond one launch, device
                                   architecture */
    ATTN_ERR_NO_DEVICE = 3,     /* no HIP device is current / visible */
    ATTN_ERR_LAUNCH = 4         /* the HIP runtime rejected a kernel launch */
} attn_status;

typedef enum {
    ATTN_F32 = 0,               /* IEEE binary32 in and out, fp32 arithmetic throughout */
    ATTN_BF16 = 1,              /* bfloat16 in and out, fp32 accumulation */
    /* Not element types: these two bounds make every 32-bit int a valid value
       of attn_dtype, so whatever a caller passes can be read and rejected
       with ATTN_ERR_UNSUPPORTED (in C++ reading a value outside an enum's
       range is undefined).  The type stays int-sized. */
    ATTN_DTYPE_RANGE_MIN_ = -0x7fffffff - 1,
    ATTN_DTYPE_RANGE_MAX_ = 0x7fffffff
} attn_dtype;

/*
 * attn_fwd - dense attention forward (prefill), optionally causal, with
 * grouped K/V heads.
 *
 *   q, o : [B, Hq,  N, d]  contiguous, element type `dtype`
 *   k, v : [B, Hkv, N, d]  contiguous, element type `dtype`
 *   lse  : [B, Hq,  N]     fp32, or NULL to skip it
 *
 * Query head h reads K/V head h / (Hq / Hkv) (contiguous groups; grouped-
 * query attention, "FlashAttention" notes, last section).  With causal = 1,
 * query row i attends to keys j <= i (diagonal included); with causal = 0
 * to all N keys.  `scale` multiplies the dot products before the softmax
 * (1/sqrt(d) in the pages' formula); any finite value is accepted.
 * o is written in `dtype` (round-to-nearest-even for bf16).
 *
 * Supported: dtype F32 or BF16; d = 64 or 128; B, Hq, Hkv, N >= 1;
 * N * d <= 2^31 - 2^16 (2^29 for F32); q, k, v, o 16-byte aligned; lse 4-byte aligned.
 * Returns INVALID_ARG / UNSUPPORTED / NO_DEVICE / LAUNCH as described above.
 */
attn_status attn_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
                     int B, int Hq, int Hkv, int N, int d, float scale, int causal,
                     attn_dtype dtype, void* stream);

/*
 * attn_paged_decode_workspace_size - bytes of device workspace that
 * attn_paged_decode needs for these sizes (0 on invalid sizes).  The
 * workspace holds, per (sequence, kv head) pair, the first and last wave that
 * worked on it, and the fp32 partial states (m, l, u) that waves covering
 * only part of a pair leave for the merge (with more than 16 query heads per
 * kv head, per group of at most 16 of them).  The size is a bound that holds
 * for every Hkv dividing Hq: round_up(8*S*Hq, 256)
 * + 4*((2048*Hq + S*Hq + ceil(S*Hq/16))*(d + 2) + 3*(2048 + S*Hq)) bytes.
 */
size_t attn_paged_decode_workspace_size(int S, int Hq, int d, int max_blocks, int block_size);

/*
 * attn_paged_decode - one new query token per sequence against a paged KV
 * cache ("Kernels de atención rápida y fusión de operadores", section
 * "Atención tipo FlashAttention y atención paginada"): the cache is a pool
 * of fixed-size blocks and a block table maps each sequence's logical
 * positions to physical blocks.
 *
 *   q, o          : [S, Hq, d]                          element type `dtype`
 *   k_cache,
 *   v_cache       : [num_blocks, Hkv, block_size, d]   element type `dtype`
 *   block_table   : int32 [S, max_blocks]; logical position p of sequence s
 *                   lives in block block_table[s][p / block_size], slot
 *                   p % block_size.  Entries at or past
 *                   ceil(ctx_lens[s] / block_size) are never read.
 *   ctx_lens      : int32 [S]; the query attends to positions 0..ctx_lens[s]-1
 *                   (its own K/V already appended).  0 gives o = 0, lse = -inf.
 *   lse           : fp32 [S, Hq], or NULL
 *   workspace     : device scratch of at least
 *                   attn_paged_decode_workspace_size(S, Hq, d, max_blocks,
 *                   block_size) bytes, 16-byte aligned; contents on entry
 *                   are ignored.  Calls that share a workspace must be
 *                   ordered on one stream.
 *
 * Supported: dtype BF16; d = 64 or 128; block_size = 16; Hq % Hkv == 0;
 * S, max_blocks, num_blocks >= 1; S * n * Hkv * max_blocks < 2^31 with n as
 * below.  The G = Hq / Hkv query heads of a kv head share each K/V block
 * read; more than 16 are split into n = ceil(G / 16) groups of at most
 * ceil(G / n) heads, and each group reads the kv head's blocks once.
 *
 * Device-resident values cannot be checked before launch.  A ctx_lens entry
 * outside [0, max_blocks * block_size] or a needed block_table entry outside
 * [0, num_blocks) never causes an out-of-bounds access: that sequence's
 * outputs are set to NaN instead.
 */
attn_status attn_paged_decode(const void* q, const void* k_cache, const void* v_cache,
                              const int32_t* block_table, const int32_t* ctx_lens,
                              int block_size, void* o, float* lse, int S, int Hq, int Hkv,
                              int d, int max_blocks, int num_blocks, float scale,
                              attn_dtype dtype, void* workspace, size_t workspace_bytes,
                              void* stream);

/*
 * attn_paged_decode_noalloc - attn_paged_decode without a workspace
 * argument, for callers that cannot allocate device memory: code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc.
 *
 * Arguments, layouts, results and errors are those of attn_paged_decode
 * (same kernels, bit-identical outputs), minus `workspace` and
 * `workspace_bytes`.  The partial states that attn_paged_decode keeps in the
 * caller's workspace live instead in a device array owned by the library,
 * ATTN_DECODE_NOALLOC_SCRATCH_BYTES per GPU, which each GPU the library
 * runs on holds until the process ends.  A call whose partial states would
 * not fit, i.e. when
 *     256-byte-rounded(8 * S * H) + 4 * (2048 + S * H) * (round4(2 * r) + r * d)
 * exceeds that size, with G = Hq / Hkv, n = ceil(G / 16), H = n * Hkv and
 * r = ceil(G / n), returns ATTN_ERR_UNSUPPORTED before anything is
 * enqueued (S * Hkv up to about 8700 fits at G = 6, d = 128; about 1900 at
 * G = 16).  Nothing is allocated, freed or memset.  Every call on one GPU
 * shares that GPU's array, so calls that may run at the same time on one
 * GPU (different streams, or host threads) race and must be ordered by the
 * caller.
 */
#define ATTN_DECODE_NOALLOC_SCRATCH_BYTES ((size_t)32 << 20)

attn_status attn_paged_decode_noalloc(const void* q, const void* k_cache, const void* v_cache,
                                      const int32_t* block_table, const int32_t* ctx_lens,
                                      int block_size, void* o, float* lse, int S, int Hq, int Hkv,
                                      int d, int max_blocks, int num_blocks, float scale,
                                      attn_dtype dtype, void* stream);

/*
 * attn_kv_append - write new tokens' keys and values into a paged KV cache
 * ("Kernels de atención rápida y fusión de operadores", section "Atención
 * tipo FlashAttention y atención paginada": the cache grows by a token, or a
 * chunk of tokens, per step and is kept as fixed-size blocks reached through
 * a block table).  A pure copy: the bytes land unchanged.
 *
 *   k_new, v_new  : [T, Hkv, d] element type `dtype`; the new tokens of all
 *                   sequences packed row after row
 *   starts        : int32 [S + 1]; rows starts[s] .. starts[s+1]-1 are the
 *                   n_s new tokens of sequence s (n_s may be 0)
 *   ctx_lens      : int32 [S]; lengths AFTER the append (they count the new
 *                   tokens): token t of sequence s goes to position
 *                   p = ctx_lens[s] - n_s + t, i.e. block
 *                   block_table[s][p / block_size], slot p % block_size, for
 *                   every kv head.  Neither lengths nor table are modified.
 *   k_cache,
 *   v_cache       : [num_blocks, Hkv, block_size, d] element type `dtype`,
 *                   written in place; every other slot keeps its bytes
 *   block_table   : int32 [S, max_blocks]
 *   max_new       : host-side upper bound on every n_s; it sizes the launch
 *
 * Supported: dtype F32 or BF16; d * element size a multiple of 16 bytes and
 * at most 4096 bytes; 1 <= block_size <= 1024; 1 <= S <= 65535; T >= 0 and
 * max_new >= 0 (either 0: nothing to write, returns OK without a launch);
 * Hkv, max_blocks, num_blocks >= 1.  k_new, v_new, k_cache, v_cache 16-byte
 * aligned; block_table, ctx_lens, starts 4-byte aligned; the caches must not
 * overlap each other or any input.
 *
 * Device-resident values never cause an out-of-bounds access.  A sequence
 * whose offsets are malformed (starts[s] < 0, starts[s+1] > T or
 * starts[s+1] < starts[s]), with n_s > max_new, or with ctx_lens[s] < n_s
 * writes nothing; a token whose block index is >= max_blocks or whose table
 * entry is outside [0, num_blocks) is not written.  Two new tokens that map
 * to the same slot race (which one lands is unspecified).
 */
attn_status attn_kv_append(const void* k_new, const void* v_new, void* k_cache, void* v_cache,
                           const int32_t* block_table, const int32_t* ctx_lens,
                           const int32_t* starts, int block_size, int S, int T, int max_new,
                           int Hkv, int d, int max_blocks, int num_blocks, attn_dtype dtype,
                           void* stream);

/*
 * attn_paged_prefill - chunked (variable-length) prefill against a paged KV
 * cache: several new query rows per sequence, each attending causally to
 * every cached position up to its own (same page and section as above; the
 * per-row result is the attention definition at the top of this file).
 *
 *   q, o          : [T, Hq, d] bf16; the new query rows of all sequences
 *                   packed row after row
 *   lse           : fp32 [T, Hq], or NULL
 *   starts        : int32 [S + 1]; rows starts[s] .. starts[s+1]-1 belong to
 *                   sequence s (n_s rows, may be 0)
 *   ctx_lens      : int32 [S]; cached length of sequence s, which already
 *                   includes its n_s new tokens (append them first): row t of
 *                   sequence s is position ctx_lens[s] - n_s + t and attends
 *                   to positions 0 .. that one, diagonal included
 *   k_cache,
 *   v_cache       : [num_blocks, Hkv, block_size, d] bf16, as in
 *                   attn_paged_decode
 *   block_table   : int32 [S, max_blocks]
 *   max_new       : host-side upper bound on every n_s; it sizes the launch
 *
 * With n_s = 1 for every sequence this is attn_paged_decode; with no earlier
 * context (ctx_lens[s] = n_s) it is causal attn_fwd over each sequence.
 * Rows that belong to no sequence are not written.
 *
 * Supported: dtype BF16; d = 64 or 128; block_size = 16; Hq % Hkv == 0;
 * S, Hq, Hkv, max_blocks, num_blocks >= 1; T >= 0 and max_new >= 0 (either
 * 0: nothing to do, returns OK without a launch); max_new * Hq * d * 2 <
 * 2^31.  q, o, k_cache, v_cache 16-byte aligned; block_table, ctx_lens,
 * starts, lse 4-byte aligned; o and lse must not overlap the inputs or
 * each other.
 *
 * Device-resident values never cause an out-of-bounds access.  A sequence
 * whose offsets are malformed (as for attn_kv_append) or with n_s > max_new
 * is not written; one with ctx_lens[s] < n_s or ctx_lens[s] > max_blocks *
 * block_size gets NaN in o and lse; a row that attends to a block whose
 * table entry is outside [0, num_blocks) gets NaN.
 */
attn_status attn_paged_prefill(const void* q, const void* k_cache, const void* v_cache,
                               const int32_t* block_table, const int32_t* ctx_lens,
                               const int32_t* starts, int block_size, void* o, float* lse, int S,
                               int T, int max_new, int Hq, int Hkv, int d, int max_blocks,
                               int num_blocks, float scale, attn_dtype dtype, void* stream);

/*
 * attn_bwd_workspace_size - bytes of device workspace attn_bwd needs (0 on
 * invalid sizes): 4 * round_up(B*Hq*N, 64) for the per-row D_i, plus, when
 * Hq > Hkv, 2 * 4 * B*Hq*N*d for one fp32 dk and dv per query head.
 */
size_t attn_bwd_workspace_size(int B, int Hq, int Hkv, int N, int d);

/*
 * attn_bwd - gradients of attn_fwd's output with respect to q, k and v,
 * recomputing the attention weights from q, k and the saved statistic lse
 * instead of storing them ("Autoatención, kernels CUDA y FlashAttention",
 * section 3, recomputation in the backward pass).  For the allowed keys of
 * row i (as in attn_fwd), p_ij = exp(scale <q_i, k_j> - lse_i) and
 * D_i = <dout_i, o_i>:
 *
 *     dv_j = sum_i p_ij dout_i
 *     ds_ij = p_ij (<dout_i, v_j> - D_i)
 *     dq_i = scale sum_j ds_ij k_j,    dk_j = scale sum_i ds_ij q_i
 *
 * with dk, dv of a kv head summed over the query heads that read it.
 *
 *   q, o, dout, dq : [B, Hq, N, d]  bf16 (o as attn_fwd wrote it, dout the
 *                    upstream gradient of o)
 *   k, v, dk, dv   : [B, Hkv, N, d] bf16
 *   lse            : [B, Hq, N] fp32, as attn_fwd wrote it for the same
 *                    q, k, v, scale and causal flag
 *   workspace      : at least attn_bwd_workspace_size(...) bytes, 16-byte
 *                    aligned; contents on entry ignored
 *
 * Accumulation is fp32; the weights and ds enter the matrix products as
 * bf16; outputs are rounded to nearest-even.  No atomics: results are
 * deterministic.  Supported: BF16; d = 64 or 128; the other limits of
 * attn_fwd.  dq, dk, dv and the workspace must not overlap the inputs or
 * each other.  Errors as for attn_fwd.
 */
attn_status attn_bwd(const void* q, const void* k, const void* v, const void* o, const float* lse,
                     const void* dout, void* dq, void* dk, void* dv, int B, int Hq, int Hkv, int N,
                     int d, float scale, int causal, attn_dtype dtype, void* workspace,
                     size_t workspace_bytes, void* stream);

/*
 * attn_add_rmsnorm - residual add fused with RMSNorm ("Kernels de atención
 * rápida y fusión de operadores", section "Fusión de operadores": adding a
 * residual connection followed by an RMSNorm is one of the common fusions).
 * For each of the T rows of D elements:
 *
 *     residual_out = bf16(x + residual)                    (the new residual stream)
 *     out_i = residual_out_i / sqrt(mean_j residual_out_j^2 + eps) * weight_i
 *
 * in fp32, out rounded to nearest-even; the norm reads the residual as
 * stored (bf16), so the result equals an add kernel followed by a norm
 * kernel.  x, residual, out, residual_out: [T, D] bf16 row-major; weight:
 * [D] bf16.  residual_out may be residual itself (in-place update); out
 * overlaps nothing.  Supported: BF16; D a multiple of 8, at most 8192;
 * T >= 0 (0: nothing to do); eps finite and >= 0; 16-byte aligned pointers.
 */
attn_status attn_add_rmsnorm(const void* x, const void* residual, const void* weight, void* out,
                             void* residual_out, int T, int D, float eps, attn_dtype dtype,
                             void* stream);

/*
 * attn_swiglu - the SwiGLU block's activation fused into one pass (same
 * page and section: the block runs a SiLU kernel and an elementwise-multiply
 * kernel between its projections): out[t][f] = silu(gate[t][f]) * up[t][f],
 * silu(g) = g / (1 + e^-g), in fp32, rounded to nearest-even.
 *
 *   gate, up : row t at gate + t * ld_in, up + t * ld_in (F elements each):
 *              two [T, F] tensors (ld_in = F), or the halves of one merged
 *              [T, 2F] projection output (up = gate + F, ld_in = 2F)
 *   out      : row t at out + t * ld_out, F elements
 *
 * Supported: BF16; F and the strides multiples of 8; strides >= F; T >= 0;
 * 16-byte aligned pointers; out overlaps neither input.
 */
attn_status attn_swiglu(const void* gate, const void* up, void* out, int T, int F, int ld_in,
                        int ld_out, attn_dtype dtype, void* stream);

/* Static string naming a status code. */
const char* attn_status_string(attn_status s);

/* Detail of the last non-OK return on the calling thread ("" if none). */
const char* attn_last_error(void);

/* ATTN_ABI_VERSION of the loaded library. */
int attn_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* ATTN_H */

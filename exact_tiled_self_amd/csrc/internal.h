// Launchers shared between the C ABI (api.cpp) and the kernel sources.
// Each enqueues its kernels on `stream` and returns the launch status; the
// arguments have already been validated by the caller.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace attn {

// XCDs of an MI355X: workgroup b of a launch is dispatched to XCD b % kXcds,
// and each XCD has its own L2.
constexpr int kXcds = 8;

struct PrefillArgs {
    const void* q;
    const void* k;
    const void* v;
    void* o;
    float* lse;        // may be null
    int B, Hq, Hkv, N, d;
    float c;           // |scale| * log2(e): scores are handled in base 2
    int negate;        // 1 when scale < 0: q is negated on load (exact)
    int causal;
};

hipError_t launch_prefill_bf16(const PrefillArgs& a, hipStream_t stream);
hipError_t launch_prefill_f32(const PrefillArgs& a, hipStream_t stream);

// Paged decode: the (sequence, kv head, 16-token block) units of a call are
// dealt out to a fixed number of waves in equal contiguous ranges; a wave
// whose range covers only part of a (sequence, kv head) pair leaves an fp32
// partial state (m, l, u) per query head in the workspace, which a second
// kernel merges.
constexpr int kDecodeBlock = 16;   // tokens per KV-cache block
constexpr int kDecodeWaves = 2048; // most waves a split kernel launch uses (sizes the workspace)
// Waves launched by default: one 4-wave workgroup per CU of an MI355X.  Half
// the maximum is faster (67.5 against 71.8 us for the 64-sequence workload,
// cache flushed): each CU then runs a single workgroup, and a pair of
// sequence and kv head is split into fewer pieces, so the merge is shorter.
constexpr int kDecodeWavesDefault = 1024;

// Workspace layout: per-pair records (first and last wave of the pair, two
// int32 each) padded to 256 bytes, then one slot per (wave, pair) touch
// (at most kDecodeWaves + S*Hkv of them) of [m[G], l[G], pad to 4, u[G][d]].
inline size_t decode_rec_bytes(int S, int Hkv) {
    return (((size_t)S * Hkv * 2 * sizeof(int32_t)) + 255) & ~(size_t)255;
}
__host__ __device__ inline int decode_ml_pad(int G) { return (2 * G + 3) & ~3; }
__host__ __device__ inline size_t decode_slot_floats(int G, int d) { return (size_t)decode_ml_pad(G) + (size_t)G * d; }
// The G query heads of a kv head are the rows of one 16-row score tile; more
// than 16 are split into decode_groups(G) groups of at most
// decode_group_rows(G) heads, each a "virtual" kv head of its own (its own
// units, partial states and records; its K/V blocks read once per group).
__host__ __device__ inline int decode_groups(int G) { return (G + 15) / 16; }
__host__ __device__ inline int decode_group_rows(int G) { return (G + decode_groups(G) - 1) / decode_groups(G); }
// Waves that read the same blocks together, one group each: all the groups
// when they fit in one 4-wave workgroup, else 1 (each group on its own).
__host__ __device__ inline int decode_team(int G) { return decode_groups(G) <= 4 ? decode_groups(G) : 1; }
// Upper bound over every Hkv dividing Hq (the size query does not take Hkv).
// With n = decode_groups(G) virtual heads per kv head of r rows each,
// n * r <= G + n - 1 <= G + G / 16, so the rows of all pairs' slots are at
// most S*Hq + S*Hq/16, and the waves' slots at most 2048 rows of <= Hq.
inline size_t decode_workspace_bound(int S, int Hq, int d) {
    const size_t rec = (((size_t)S * Hq * 2 * sizeof(int32_t)) + 255) & ~(size_t)255;
    const size_t sq = (size_t)S * Hq;
    const size_t slots_times_g = (size_t)kDecodeWaves * Hq + sq + (sq + 15) / 16;   // >= (W + S*Hkv') * G'
    const size_t slots = (size_t)kDecodeWaves + sq;                                  // >= W + S*Hkv'
    return rec + (slots_times_g * (size_t)(d + 2) + slots * 3) * sizeof(float);
}

struct DecodeArgs {
    const void* q;
    const void* k_cache;
    const void* v_cache;
    const int32_t* block_table;
    const int32_t* ctx_lens;
    void* o;
    float* lse;        // may be null
    int S, Hq, Hkv, d, max_blocks, num_blocks;
    float c;
    int negate;
    float* workspace;
};

hipError_t launch_paged_decode_bf16(const DecodeArgs& a, hipStream_t stream);

// Bytes of workspace a decode launch uses when Hkv is known (the size query
// above bounds it over every Hkv instead).
inline size_t decode_workspace_exact(int S, int Hq, int Hkv, int d) {
    const int G = Hq / Hkv;
    const int hv = Hkv * decode_groups(G);   // virtual kv heads
    return decode_rec_bytes(S, hv) +
           ((size_t)kDecodeWaves + (size_t)S * hv) * decode_slot_floats(decode_group_rows(G), d) * sizeof(float);
}

// The same decode with its partial states in the library's own per-device
// scratch array (decode_paged.hip) instead of a caller workspace; the caller
// has checked that decode_workspace_exact() fits kDecodeScratchBytes.
constexpr size_t kDecodeScratchBytes = (size_t)32 << 20;
hipError_t launch_paged_decode_bf16_noalloc(DecodeArgs a, hipStream_t stream);

// Packed new tokens [T, Hkv, d] written into the paged cache.
struct KvAppendArgs {
    const void* k_new;
    const void* v_new;
    void* k_cache;
    void* v_cache;
    const int32_t* block_table;
    const int32_t* ctx_lens;
    const int32_t* starts;
    int S, T, max_new, Hkv, block_size, max_blocks, num_blocks;
    int cpr;           // 16-byte chunks per (token, kv head) row
};

hipError_t launch_kv_append(const KvAppendArgs& a, hipStream_t stream);

// Chunked prefill: packed new query rows [T, Hq, d] against the paged cache.
struct PagedPrefillArgs {
    const void* q;
    const void* k_cache;
    const void* v_cache;
    const int32_t* block_table;
    const int32_t* ctx_lens;
    const int32_t* starts;
    void* o;
    float* lse;        // may be null
    int S, T, max_new, Hq, Hkv, d, max_blocks, num_blocks;
    float c;
    int negate;
};

hipError_t launch_paged_prefill_bf16(const PagedPrefillArgs& a, hipStream_t stream);

// Backward pass.  Workspace: D_i = <do_i, o_i> for every row (fp32, padded to
// 256 bytes), then, with grouped K/V heads (Hq > Hkv), one fp32 dk and one
// fp32 dv per query head ([B, Hq, N, d] each) that a last kernel sums per
// group.
inline size_t bwd_delta_floats(int B, int Hq, int N) {
    return (((size_t)B * Hq * N) + 63) & ~(size_t)63;
}
inline size_t bwd_workspace_bytes(int B, int Hq, int Hkv, int N, int d) {
    size_t f = bwd_delta_floats(B, Hq, N);
    if (Hq != Hkv) f += 2 * (size_t)B * Hq * N * d;
    return f * sizeof(float);
}

struct BackwardArgs {
    const void* q;
    const void* k;
    const void* v;
    const void* o;
    const float* lse;
    const void* dout;
    void* dq;
    void* dk;
    void* dv;
    int B, Hq, Hkv, N, d;
    float scale;
    int causal;
    float* workspace;
};

hipError_t launch_backward_bf16(const BackwardArgs& a, hipStream_t stream);

// Residual add + RMSNorm over [T, D] rows (bf16).
struct AddRmsNormArgs {
    const void* x;
    const void* residual;
    const void* weight;
    void* out;
    void* residual_out;   // may be residual itself
    int T, D;
    float eps;
};

hipError_t launch_add_rmsnorm_bf16(const AddRmsNormArgs& a, hipStream_t stream);

// silu(gate) * up over [T, F] (bf16), rows of gate and up ld_in apart.
struct SwigluArgs {
    const void* gate;
    const void* up;
    void* out;
    int T, F, ld_in, ld_out;
};

hipError_t launch_swiglu_bf16(const SwigluArgs& a, hipStream_t stream);

}  // namespace attn

// Launchers shared between the C ABI (api.cpp) and the kernel sources.
// Each enqueues its kernels on `stream` and returns the launch status; the
// arguments have already been validated by the caller.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace attn {

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

// Paged decode: keys are processed in splits of kDecodeSplit tokens, each
// producing an fp32 partial state (m, l, u) per query head in the workspace,
// which a second kernel merges.
constexpr int kDecodeSplit = 512;
constexpr int kDecodeBlock = 16;   // tokens per KV-cache block

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

inline int decode_num_splits(int max_blocks) {
    return (int)(((long long)max_blocks * kDecodeBlock + kDecodeSplit - 1) / kDecodeSplit);
}

hipError_t launch_paged_decode_bf16(const DecodeArgs& a, hipStream_t stream);

}  // namespace attn

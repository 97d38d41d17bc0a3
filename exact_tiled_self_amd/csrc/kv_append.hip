// Appending new tokens' keys and values to a paged KV cache, for gfx950.
//
// The cache is a pool of fixed-size blocks and a block table maps each
// sequence's logical positions to physical blocks ("Kernels de atención
// rápida y fusión de operadores", section "Atención tipo FlashAttention y
// atención paginada"); it grows by one token, or one chunk of tokens, per
// step.  The new tokens of all sequences arrive packed, row after row
// ([T, Hkv, d]); sequence s owns rows starts[s] .. starts[s+1]-1 and, since
// ctx_lens[s] already counts them, its t-th new row goes to position
// ctx_lens[s] - n_s + t: block block_table[s][p / block_size], slot
// p % block_size, for every kv head.
//
// This is a pure copy, bound by HBM: every thread moves one 16-byte chunk of
// K and the same chunk of V.  Grid y is the sequence (so its offsets and
// length are uniform, scalar loads), grid x walks its (token, kv head,
// chunk) triples in source order, so reads are fully coalesced and writes
// are contiguous runs of one row (d * element size bytes).  Every device-
// resident value is checked before it forms an address; a token that fails
// a check is simply not written.

#include "common.h"
#include "internal.h"

namespace attn {
namespace {

constexpr int KA_THREADS = 256;

__global__ void __launch_bounds__(KA_THREADS)
kv_append_kernel(const u32x4* __restrict__ kn, const u32x4* __restrict__ vn, u32x4* __restrict__ kc,
                 u32x4* __restrict__ vc, const int32_t* __restrict__ table,
                 const int32_t* __restrict__ ctx_lens, const int32_t* __restrict__ starts, int T,
                 int max_new, int Hkv, int cpr, int block_size, int max_blocks, int num_blocks) {
    const int s = blockIdx.y;
    const int a = starts[s], b = starts[s + 1], ctx = ctx_lens[s];
    const int n = b - a;
    // Malformed offsets or lengths: the whole sequence is left alone.
    if (a < 0 || b > T || n < 0 || n > max_new || ctx < n) return;

    const int idx = blockIdx.x * KA_THREADS + threadIdx.x;   // < max_new * Hkv * cpr < 2^31
    const int row = idx / cpr, c = idx - row * cpr;
    const int t = row / Hkv, g = row - t * Hkv;
    if (t >= n) return;
    const int p = ctx - n + t;                                 // 0 <= p < ctx
    const int blk = p / block_size;
    if (blk >= max_blocks) return;
    const int phys = table[(size_t)s * max_blocks + blk];
    if (phys < 0 || phys >= num_blocks) return;
    const int slot = p - blk * block_size;
    const size_t src = ((size_t)(a + t) * Hkv + g) * cpr + c;
    const size_t dst = (((size_t)phys * Hkv + g) * block_size + slot) * cpr + c;
    kc[dst] = kn[src];
    vc[dst] = vn[src];
}

}  // namespace

hipError_t launch_kv_append(const KvAppendArgs& a, hipStream_t stream) {
    const long long per_seq = (long long)a.max_new * a.Hkv * a.cpr;
    const dim3 grid((unsigned)((per_seq + KA_THREADS - 1) / KA_THREADS), (unsigned)a.S), block(KA_THREADS);
    hipLaunchKernelGGL(kv_append_kernel, grid, block, 0, stream,
                       static_cast<const u32x4*>(a.k_new), static_cast<const u32x4*>(a.v_new),
                       static_cast<u32x4*>(a.k_cache), static_cast<u32x4*>(a.v_cache), a.block_table,
                       a.ctx_lens, a.starts, a.T, a.max_new, a.Hkv, a.cpr, a.block_size,
                       a.max_blocks, a.num_blocks);
    return hipGetLastError();
}

}  // namespace attn

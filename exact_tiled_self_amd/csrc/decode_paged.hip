// Paged-KV single-token decode for gfx950.
//
// The cache is a pool of 16-token blocks; logical position p of sequence s
// lives in block block_table[s][p / 16], slot p % 16 ("Kernels de atención
// rápida y fusión de operadores", section "Atención tipo FlashAttention y
// atención paginada").  Every key position is translated through the table.
//
// Work split.  One workgroup per (sequence, kv head, 256-token split); each
// of its 4 waves takes 4 consecutive logical blocks (64 tokens).  The G query
// heads that share the kv head (grouped-query attention) form the rows of
// the score tile, so the two products are genuine small matrix products and
// run on MFMA (v_mfma_f32_16x16x32_bf16, G <= 16 rows):
//   * S^T = K Q^T: the lane's A operand is 8 dims of one key, loaded straight
//     from the block in HBM; each lane ends up owning one query row
//     (lane % 16) and 4 keys of each block.
//   * O = P V: P comes from the lane's own score registers (keys 4g..4g+3 of
//     two blocks); the V operand needs 8 keys of one dim per lane, so each
//     lane loads a 16-byte row slice of 8 keys (coalesced: 16 lanes cover one
//     256-byte row) and transposes the 8x8 block in registers with v_perm.
//     Output dims are permuted (lane column n holds dims 8n..8n+7 across the
//     8 MFMAs) so that those slices are contiguous.
// Each wave's running state (m, l, u) is merged with the other waves' in
// LDS by the rescale rule of the online softmax, and the workgroup writes one
// fp32 partial state per query head to the workspace.  A second kernel
// merges the partial states of a sequence in split order (deterministic):
// M = max m_k, L = sum l_k e^(m_k - M), O = sum u_k e^(m_k - M) / L
// ("FlashAttention" notes, section "No basta con promediar los resultados de
// los bloques": each part enters with its own weight, not as an average).
//
// Slots past a sequence's length inside its last block are loaded (they are
// inside the block) but their V rows are zeroed and their scores excluded
// before any arithmetic, so stale or NaN contents cannot leak in.  Table
// entries past the length are never read.

#include "common.h"
#include "internal.h"

namespace attn {
namespace {

constexpr int DC_THREADS = 256;
constexpr int DC_BLOCKS_PER_WAVE = 4;
static_assert(4 * DC_BLOCKS_PER_WAVE * kDecodeBlock == kDecodeSplit, "split = 4 waves x 4 blocks");

template <int D>
struct VRow;
template <>
struct VRow<128> { typedef u32x4 T; static constexpr int WORDS = 4; };
template <>
struct VRow<64> { typedef u32x2 T; static constexpr int WORDS = 2; };

template <int D>
__device__ __forceinline__ typename VRow<D>::T ld_vrow(const uint16_t* p) {
    return *reinterpret_cast<const typename VRow<D>::T*>(p);
}

template <int D>
__global__ void __launch_bounds__(DC_THREADS)
decode_partial_kernel(const uint16_t* __restrict__ q, const uint16_t* __restrict__ kc,
                      const uint16_t* __restrict__ vc, const int32_t* __restrict__ table,
                      const int32_t* __restrict__ ctx_lens, float* __restrict__ ws, int Hq,
                      int Hkv, int max_blocks, int num_blocks, int nsplit, float c, int negate) {
    constexpr int KS = D / 32;              // MFMA k-steps over the head dim
    constexpr int DPL = D / 16;             // output dims per lane column
    using VT = typename VRow<D>::T;

    __shared__ float sm_m[4][16];
    __shared__ float sm_l[4][16];
    __shared__ __attribute__((aligned(16))) float sm_o[4][16][D];

    const int split = blockIdx.x, g = blockIdx.y, s = blockIdx.z;
    const int G = Hq / Hkv;
    const int cap = max_blocks * kDecodeBlock;
    int ctx = ctx_lens[s];
    ctx = ctx < 0 ? 0 : (ctx > cap ? cap : ctx);     // out-of-range lengths: see combine
    const int nsplit_s = (ctx + kDecodeSplit - 1) / kDecodeSplit;
    if (split >= nsplit_s) return;

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int l16 = lane & 15, grp = lane >> 4;
    const int nblk = (ctx + kDecodeBlock - 1) / kDecodeBlock;
    const int fb = split * (kDecodeSplit / kDecodeBlock) + wave * DC_BLOCKS_PER_WAVE;

    // Physical blocks of this wave (wave-uniform).
    int phys[DC_BLOCKS_PER_WAVE];
    bool valid[DC_BLOCKS_PER_WAVE];
    bool bad = false;
#pragma unroll
    for (int i = 0; i < DC_BLOCKS_PER_WAVE; ++i) {
        const int lb = fb + i;
        valid[i] = lb < nblk;
        int p = valid[i] ? table[(size_t)s * max_blocks + lb] : 0;
        if (valid[i] && (p < 0 || p >= num_blocks)) {
            bad = true;
            valid[i] = false;
            p = 0;
        }
        phys[i] = p;
    }

    // K operand loads: key l16 of block i, dims 8*(4ks + grp) .. +7.
    u32x4 kr[DC_BLOCKS_PER_WAVE][KS];
#pragma unroll
    for (int i = 0; i < DC_BLOCKS_PER_WAVE; ++i)
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
            kr[i][ks] = valid[i] ? ld16(kc + (((size_t)phys[i] * Hkv + g) * kDecodeBlock + l16) * D +
                                        8 * (4 * ks + grp))
                                 : u32x4{0u, 0u, 0u, 0u};
    // V operand loads: for block pair bp, entry i8 -> block 2bp + i8/4, key
    // 4*grp + i8%4, dims DPL*l16 .. +DPL-1.
    VT vr[2][8];
#pragma unroll
    for (int bp = 0; bp < 2; ++bp)
#pragma unroll
        for (int i8 = 0; i8 < 8; ++i8) {
            const int blk = 2 * bp + (i8 >> 2);
            const int key = 4 * grp + (i8 & 3);
            VT w = {};
            if (valid[blk])
                w = ld_vrow<D>(vc + (((size_t)phys[blk] * Hkv + g) * kDecodeBlock + key) * D + DPL * l16);
            vr[bp][i8] = w;
        }

    // Q operand: query row l16 (head g*G + l16 when l16 < G), same dims as K.
    bf16x8 qf[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
        u32x4 w = {0u, 0u, 0u, 0u};
        if (l16 < G) w = ld16(q + ((size_t)s * Hq + g * G + l16) * D + 8 * (4 * ks + grp));
        if (negate) w = neg_bf16x8(w);
        qf[ks] = __builtin_bit_cast(bf16x8, w);
    }

    // Scores.
    f32x4 sacc[DC_BLOCKS_PER_WAVE];
#pragma unroll
    for (int i = 0; i < DC_BLOCKS_PER_WAVE; ++i) {
        sacc[i] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
            sacc[i] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, kr[i][ks]),
                                                              qf[ks], sacc[i], 0, 0, 0);
    }
    float mx = kNegInf;
#pragma unroll
    for (int i = 0; i < DC_BLOCKS_PER_WAVE; ++i)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int tok = (fb + i) * kDecodeBlock + 4 * grp + r;
            const bool ok = valid[i] && tok < ctx;
            sacc[i][r] = ok ? sacc[i][r] : kNegInf;
            mx = fmaxf(mx, sacc[i][r]);
        }
    mx = fmaxf(mx, xor_shfl(mx, 16));
    mx = fmaxf(mx, xor_shfl(mx, 32));
    const float m_use = (mx == kNegInf) ? 0.f : mx;
    const float mc = m_use * c;
    float lsum = 0.f;
#pragma unroll
    for (int i = 0; i < DC_BLOCKS_PER_WAVE; ++i)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const float sv = sacc[i][r];
            const float p = (sv == kNegInf) ? 0.f : fast_exp2(fmaf(sv, c, -mc));
            sacc[i][r] = p;
            lsum += p;
        }
    lsum += xor_shfl(lsum, 16);
    lsum += xor_shfl(lsum, 32);

    // O = P V over the two block pairs.
    f32x4 oacc[DPL];
#pragma unroll
    for (int j = 0; j < DPL; ++j) oacc[j] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int bp = 0; bp < 2; ++bp) {
        // zero the V rows of positions past the length (NaN-safe)
#pragma unroll
        for (int i8 = 0; i8 < 8; ++i8) {
            const int blk = 2 * bp + (i8 >> 2);
            const int tok = (fb + blk) * kDecodeBlock + 4 * grp + (i8 & 3);
            if (tok >= ctx) vr[bp][i8] = VT{};
        }
        bf16x8 pa;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            pa[i] = (__bf16)sacc[2 * bp][i];
            pa[4 + i] = (__bf16)sacc[2 * bp + 1][i];
        }
#pragma unroll
        for (int j = 0; j < DPL; ++j) {
            const int w = j >> 1;
            const uint32_t sel = (j & 1) ? 0x07060302u : 0x05040100u;
            u32x4 t;
            t.x = __builtin_amdgcn_perm(vr[bp][1][w], vr[bp][0][w], sel);
            t.y = __builtin_amdgcn_perm(vr[bp][3][w], vr[bp][2][w], sel);
            t.z = __builtin_amdgcn_perm(vr[bp][5][w], vr[bp][4][w], sel);
            t.w = __builtin_amdgcn_perm(vr[bp][7][w], vr[bp][6][w], sel);
            oacc[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pa, __builtin_bit_cast(bf16x8, t),
                                                              oacc[j], 0, 0, 0);
        }
    }

    // Merge the four waves' states in LDS.
    if (grp == 0) {
        sm_m[wave][l16] = mx;
        sm_l[wave][l16] = bad ? __builtin_nanf("") : lsum;
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        const int row = 4 * grp + r;
        if (row < G)
#pragma unroll
            for (int j = 0; j < DPL; ++j) sm_o[wave][row][DPL * l16 + j] = oacc[j][r];
    }
    __syncthreads();

    float* part = ws + ((size_t)(s * Hkv + g) * nsplit + split) * (size_t)G * (D + 2);
    for (int e = tid; e < G * D; e += DC_THREADS) {
        const int row = e / D, dim = e - row * D;
        float M = kNegInf;
#pragma unroll
        for (int w = 0; w < 4; ++w) M = fmaxf(M, sm_m[w][row]);
        float U = 0.f, Lw = 0.f;
#pragma unroll
        for (int w = 0; w < 4; ++w) {
            const float mw = sm_m[w][row];
            const float f = (mw == kNegInf) ? 0.f : fast_exp2((mw - M) * c);
            U = fmaf(f, sm_o[w][row][dim], U);
            Lw = fmaf(f, sm_l[w][row], Lw);
        }
        part[2 * G + e] = U;
        if (dim == 0) {
            part[row] = M;
            part[G + row] = Lw;
        }
    }
}

// One wave per (sequence, query head): merge the sequence's split states in
// split order.
template <int D>
__global__ void __launch_bounds__(256)
decode_combine_kernel(const float* __restrict__ ws, const int32_t* __restrict__ ctx_lens,
                      uint16_t* __restrict__ o, float* __restrict__ lse, int S, int Hq, int Hkv,
                      int max_blocks, int nsplit, float c) {
    constexpr int DPT = D / 64;             // dims per lane
    const int lane = threadIdx.x & 63;
    const int sh = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (sh >= S * Hq) return;
    const int s = sh / Hq, h = sh - s * Hq;
    const int G = Hq / Hkv;
    const int g = h / G, n = h - g * G;
    const int cap = max_blocks * kDecodeBlock;
    int ctx = ctx_lens[s];
    const bool bad = ctx < 0 || ctx > cap;
    ctx = ctx < 0 ? 0 : (ctx > cap ? cap : ctx);
    const int nsp = (ctx + kDecodeSplit - 1) / kDecodeSplit;
    const size_t stride = (size_t)G * (D + 2);
    const float* base = ws + (size_t)(s * Hkv + g) * nsplit * stride;

    float M = kNegInf;
    for (int kk = 0; kk < nsp; ++kk) M = fmaxf(M, base[kk * stride + n]);
    float L = 0.f, U[DPT];
#pragma unroll
    for (int t = 0; t < DPT; ++t) U[t] = 0.f;
    for (int kk = 0; kk < nsp; ++kk) {
        const float* p = base + kk * stride;
        const float mk = p[n];
        const float f = (mk == kNegInf) ? 0.f : fast_exp2((mk - M) * c);
        L = fmaf(f, p[G + n], L);
#pragma unroll
        for (int t = 0; t < DPT; ++t) U[t] = fmaf(f, p[2 * G + n * D + lane * DPT + t], U[t]);
    }
    const float nan = __builtin_nanf("");
    const float inv = (L > 0.f) ? 1.f / L : (L == 0.f ? 0.f : nan);
    uint16_t* orow = o + ((size_t)s * Hq + h) * D + lane * DPT;
    if constexpr (DPT == 2) {
        const float a = bad ? nan : U[0] * inv, b2 = bad ? nan : U[1] * inv;
        *reinterpret_cast<uint32_t*>(orow) = pack_bf16x2(a, b2);
    } else {
        const float a = bad ? nan : U[0] * inv;
        typedef __bf16 bf1;
        bf1 x = (bf1)a;
        *orow = __builtin_bit_cast(uint16_t, x);
    }
    if (lse != nullptr && lane == 0) {
        float lv = (M == kNegInf) ? kNegInf : (M * c + log2f(L)) * kLn2;
        if (bad || L != L) lv = nan;
        lse[(size_t)s * Hq + h] = lv;
    }
}

template <int D>
hipError_t launch_decode_t(const DecodeArgs& a, hipStream_t stream) {
    const int nsplit = decode_num_splits(a.max_blocks);
    const dim3 g1((unsigned)nsplit, (unsigned)a.Hkv, (unsigned)a.S), b1(DC_THREADS);
    hipLaunchKernelGGL((decode_partial_kernel<D>), g1, b1, 0, stream,
                       static_cast<const uint16_t*>(a.q), static_cast<const uint16_t*>(a.k_cache),
                       static_cast<const uint16_t*>(a.v_cache), a.block_table, a.ctx_lens,
                       a.workspace, a.Hq, a.Hkv, a.max_blocks, a.num_blocks, nsplit, a.c, a.negate);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const dim3 g2((unsigned)((a.S * a.Hq + 3) / 4)), b2(256);
    hipLaunchKernelGGL((decode_combine_kernel<D>), g2, b2, 0, stream, a.workspace, a.ctx_lens,
                       static_cast<uint16_t*>(a.o), a.lse, a.S, a.Hq, a.Hkv, a.max_blocks, nsplit, a.c);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_paged_decode_bf16(const DecodeArgs& a, hipStream_t stream) {
    return a.d == 128 ? launch_decode_t<128>(a, stream) : launch_decode_t<64>(a, stream);
}

}  // namespace attn

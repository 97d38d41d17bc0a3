// Dense attention forward (prefill), bf16 in / bf16 out, fp32 accumulation,
// for gfx950.
//
// Method ("FlashAttention" notes, section "No basta con promediar los
// resultados de los bloques"; "Autoatención, kernels CUDA y FlashAttention",
// section 3): each workgroup owns a tile of query rows and walks the key
// tiles once, keeping per row a running maximum m, sum l and numerator u;
// when a tile raises the maximum to m', l and u are first scaled by
// e^(m - m').  The score tile exists only in registers; only O = u / l and
// lse = m + ln l are written.  Scores are handled in base 2: with
// c = scale * log2(e), e^(scale*(s - m)) = 2^(c*(s - m)).
//
// MFMA v_mfma_f32_32x32x16_bf16:
//   * 4 waves x 32 query rows = 128 rows per workgroup; key tiles of 64.
//   * The wave computes the TRANSPOSED score tile S^T = K * Q^T, so that each
//     lane owns one query row (lane % 32) and 16 of its keys per 32-key
//     block: the row maximum is an in-lane max plus one exchange with lane
//     ^ 32, the row sum needs no exchange until the epilogue, and the
//     rescale of u by e^(m - m') is lane-local.
//   * O^T = V^T * P^T: P^T comes straight from the score accumulators
//     (converted to bf16); V^T is read from LDS, where the staging code
//     stores V transposed with keys 4..7 and 8..11 of every 16-key group
//     swapped, which is exactly the key order of the accumulator lanes.
//   * K/V tiles are double-buffered in LDS; the loads of tile j+1 are issued
//     before the MFMA work on tile j.  K goes straight from memory into LDS
//     (buffer_load ... lds, 16-byte chunks of each row XOR-swizzled so the
//     operand fetches are free of bank conflicts); V passes through registers
//     to be stored transposed.  Buffer resources bound every load by the
//     head's extent, so rows past N read as zero without branches.
//   * The running maximum is raised lazily: only when a tile's maximum
//     exceeds it by more than 2^8 in weight does the wave rescale l and u.
//   * Causal: tiles entirely above the diagonal are never visited, the q
//     tiles are dispatched heaviest first, and a wave whose rows all lie
//     before a tile skips its arithmetic for it.

#include "common.h"
#include "internal.h"

namespace attn {
namespace {

constexpr int PF_WAVES = 4;
constexpr int PF_BM = 32 * PF_WAVES;   // query rows per workgroup
constexpr int PF_BN = 64;              // keys per tile
constexpr int PF_THREADS = 64 * PF_WAVES;

template <int D>
struct PfLayout {
    static constexpr int CPR = D / 8;           // 16-byte chunks per K row
    static constexpr int VSTR = PF_BN + 8;      // bf16 per V^T row in LDS (16-B pad)
    static constexpr int KELEMS = PF_BN * D;    // K tile, rows XOR-swizzled, no pad
    static constexpr int VELEMS = D * VSTR;
    static constexpr int BUF = KELEMS + VELEMS; // one pipeline stage (bf16 elements)
    static constexpr int KINST = PF_BN * CPR / PF_THREADS;     // K load-to-LDS per thread
    static constexpr int VKPT = PF_BN * D / 8 / PF_THREADS;     // keys per thread (V)
    static constexpr int VKGROUPS = PF_BN / VKPT;
    static_assert(KINST * PF_THREADS == PF_BN * CPR, "K tile split");
    static_assert(VKPT == 2 || VKPT == 4, "V staging handles 2 or 4 keys per thread");
};

// XOR swizzle of the 16-byte chunks of K row r, so that the 16 rows read by
// one MFMA operand fetch hit 16 different bank groups.
template <int CPR>
__device__ __forceinline__ int kswz(int r) {
    return CPR == 16 ? (r & 15) : ((r >> 1) & 7);
}

// Position of key x (within a 16-key group) in the V^T layout: bits 2 and 3
// exchanged.  It is its own inverse.
__device__ __forceinline__ int swap23(int x) {
    return (x & ~0xC) | ((x & 4) << 1) | ((x & 8) >> 1);
}

// A tile raises the running maximum only when some row's new maximum exceeds
// it by more than 2^8 in weight: below that the old maximum stays the
// reference (weights up to 256 are exact in fp32 and bf16 range) and the
// numerator needs no rescale.  u / l is unchanged by the choice of reference.
constexpr float kLazyLog2 = 8.0f;

template <int D, bool CAUSAL>
__global__ void __launch_bounds__(PF_THREADS) __attribute__((amdgpu_waves_per_eu(2, 2)))
prefill_bf16_kernel(const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
                    const uint16_t* __restrict__ v, uint16_t* __restrict__ o,
                    float* __restrict__ lse, int Hq, int Hkv, int N, int BH, int n_qtiles,
                    float c, int negate) {
    using L = PfLayout<D>;
    __shared__ __attribute__((aligned(16))) uint16_t smem[2 * L::BUF];

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int hi = lane >> 5, l32 = lane & 31;

    // Work unit: (b, h, q tile); heaviest q tiles first when causal.
    const int wg = blockIdx.x;
    const int qt = CAUSAL ? (n_qtiles - 1 - wg / BH) : (wg / BH);
    const int bh = wg % BH;
    const int b = bh / Hq, h = bh - b * Hq;
    const int g = h / (Hq / Hkv);
    const uint32_t head_bytes = (uint32_t)N * D * 2;
    const __amdgpu_buffer_rsrc_t qrs = make_rsrc(q + (size_t)bh * N * D, head_bytes);
    const __amdgpu_buffer_rsrc_t krs = make_rsrc(k + ((size_t)b * Hkv + g) * N * D, head_bytes);
    const __amdgpu_buffer_rsrc_t vrs = make_rsrc(v + ((size_t)b * Hkv + g) * N * D, head_bytes);

    const int q0 = qt * PF_BM;
    const int wrow0 = q0 + wave * 32;
    const int myrow = wrow0 + l32;
    const bool wave_active = wrow0 < N;

    // Q as the B operand of S^T = K Q^T: row `myrow`, dims 16*ks + 8*hi .. +7
    // (rows past N read as zero).
    bf16x8 qf[D / 16];
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks) {
        u32x4 w = buf_ld16(qrs, (uint32_t)(myrow * D + ks * 16 + hi * 8) * 2);
        if (negate) w = neg_bf16x8(w);
        qf[ks] = __builtin_bit_cast(bf16x8, w);
    }

    const int row_end = min(q0 + PF_BM, N);
    const int n_kt = CAUSAL ? (row_end + PF_BN - 1) / PF_BN : (N + PF_BN - 1) / PF_BN;

    // K staging: load-to-LDS unit p = (i * waves + wave) * 64 + lane holds the
    // 16-byte chunk (row p / CPR, chunk (p % CPR) ^ swz(row)) of the tile.
    uint32_t koff[L::KINST];
#pragma unroll
    for (int i = 0; i < L::KINST; ++i) {
        const int p = (i * PF_WAVES + wave) * 64 + lane;
        const int r = p / L::CPR;
        const int cc = (p % L::CPR) ^ kswz<L::CPR>(r);
        koff[i] = (uint32_t)(r * D + cc * 8) * 2;
    }
    // V staging through registers (stored transposed): keys vkg*VKPT + i, dims vdc*8 .. +7.
    const int vkg = tid % L::VKGROUPS;
    const int vdc = tid / L::VKGROUPS;
    const uint32_t voff = (uint32_t)((vkg * L::VKPT) * D + vdc * 8) * 2;
    u32x4 vreg[L::VKPT];

    auto issue_loads = [&](int kt, int buf) {
        const uint32_t t0 = (uint32_t)kt * PF_BN * D * 2;
        uint16_t* Ks = smem + buf * L::BUF;
#pragma unroll
        for (int i = 0; i < L::KINST; ++i)
            buf_ld16_lds(krs, Ks + (i * PF_WAVES + wave) * 64 * 8, t0 + koff[i]);
#pragma unroll
        for (int i = 0; i < L::VKPT; ++i) vreg[i] = buf_ld16(vrs, t0 + voff + (uint32_t)(i * D * 2));
    };

    auto store_v = [&](int buf) {
        uint16_t* Vt = smem + buf * L::BUF + L::KELEMS;
        const int pos = swap23(vkg * L::VKPT);
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const int w = j >> 1;
            const uint32_t sel = (j & 1) ? 0x07060302u : 0x05040100u;
            uint16_t* dst = Vt + (vdc * 8 + j) * L::VSTR + pos;
            if constexpr (L::VKPT == 4) {
                const uint32_t lo = __builtin_amdgcn_perm(vreg[1][w], vreg[0][w], sel);
                const uint32_t hi2 = __builtin_amdgcn_perm(vreg[3][w], vreg[2][w], sel);
                *reinterpret_cast<u32x2*>(dst) = u32x2{lo, hi2};
            } else {
                *reinterpret_cast<uint32_t*>(dst) = __builtin_amdgcn_perm(vreg[1][w], vreg[0][w], sel);
            }
        }
    };

    f32x16 oacc[D / 32];
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[db][r] = 0.f;
    float m_run = kNegInf, l_run = 0.f;

    issue_loads(0, 0);
    __builtin_amdgcn_s_waitcnt(0);
    store_v(0);
    __syncthreads();

    for (int kt = 0; kt < n_kt; ++kt) {
        const int buf = kt & 1;
        const bool more = kt + 1 < n_kt;
        if (more) issue_loads(kt + 1, buf ^ 1);
        const int k0 = kt * PF_BN;
        const bool compute = wave_active && (!CAUSAL || k0 <= wrow0 + 31);
        if (compute) {
            const uint16_t* Ks = smem + buf * L::BUF;
            const uint16_t* Vt = Ks + L::KELEMS;

            // S^T = K Q^T for the 64 keys of this tile (two 32-key blocks).
            f32x16 sacc[PF_BN / 32];
#pragma unroll
            for (int kb = 0; kb < PF_BN / 32; ++kb)
#pragma unroll
                for (int r = 0; r < 16; ++r) sacc[kb][r] = 0.f;
#pragma unroll
            for (int ks = 0; ks < D / 16; ++ks) {
#pragma unroll
                for (int kb = 0; kb < PF_BN / 32; ++kb) {
                    const int r = kb * 32 + l32;
                    const int cc = (ks * 2 + hi) ^ kswz<L::CPR>(r);
                    const bf16x8 a = *reinterpret_cast<const bf16x8*>(Ks + r * D + cc * 8);
                    sacc[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[ks], sacc[kb], 0, 0, 0);
                }
            }

            // Lane key of accumulator entry r in block kb: k0 + 32kb + 8(r/4) + 4hi + r%4.
            const bool need_mask = (k0 + PF_BN > N) || (CAUSAL && k0 + PF_BN - 1 > wrow0);
            float mx = kNegInf;
            if (need_mask) {
#pragma unroll
                for (int kb = 0; kb < PF_BN / 32; ++kb)
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        const int key = k0 + kb * 32 + 8 * (r >> 2) + 4 * hi + (r & 3);
                        const bool ok = key < N && (!CAUSAL || key <= myrow);
                        sacc[kb][r] = ok ? sacc[kb][r] : kNegInf;
                        mx = fmaxf(mx, sacc[kb][r]);
                    }
            } else {
#pragma unroll
                for (int kb = 0; kb < PF_BN / 32; ++kb)
#pragma unroll
                    for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sacc[kb][r]);
            }
            mx = fmaxf(mx, xor_shfl(mx, 32));

            // Lazy rescale: a wave-uniform branch taken only when some row's
            // maximum grew by more than 2^kLazyLog2 (always on the first tile).
            const bool grow = (m_run == kNegInf) ? (mx != kNegInf) : ((mx - m_run) * c > kLazyLog2);
            if (__builtin_amdgcn_ballot_w64(grow) != 0) {
                const float m_new = grow ? mx : m_run;
                const float alpha = (m_run == kNegInf) ? 0.f : fast_exp2((m_run - m_new) * c);
                l_run *= alpha;
#pragma unroll
                for (int db = 0; db < D / 32; ++db)
#pragma unroll
                    for (int r = 0; r < 16; ++r) oacc[db][r] *= alpha;
                m_run = m_new;
            }
            const float mc = (m_run == kNegInf) ? 0.f : m_run * c;
            float lsum = 0.f;
            if (need_mask) {
#pragma unroll
                for (int kb = 0; kb < PF_BN / 32; ++kb)
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        const float sv = sacc[kb][r];
                        const float p = (sv == kNegInf) ? 0.f : fast_exp2(fmaf(sv, c, -mc));
                        sacc[kb][r] = p;
                        lsum += p;
                    }
            } else {
#pragma unroll
                for (int kb = 0; kb < PF_BN / 32; ++kb)
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        const float p = fast_exp2(fmaf(sacc[kb][r], c, -mc));
                        sacc[kb][r] = p;
                        lsum += p;
                    }
            }
            l_run += lsum;

            // O^T += V^T P^T, 16 keys per MFMA.
#pragma unroll
            for (int c16 = 0; c16 < PF_BN / 16; ++c16) {
                const int kb = c16 >> 1, sh = (c16 & 1) * 8;
                bf16x8 pb;
#pragma unroll
                for (int i = 0; i < 8; ++i) pb[i] = (__bf16)sacc[kb][sh + i];
#pragma unroll
                for (int db = 0; db < D / 32; ++db) {
                    const bf16x8 a = *reinterpret_cast<const bf16x8*>(
                        Vt + (db * 32 + l32) * L::VSTR + c16 * 16 + hi * 8);
                    oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pb, oacc[db], 0, 0, 0);
                }
            }
        }
        if (more) {
            __builtin_amdgcn_s_waitcnt(0);     // tile kt+1: K in LDS, V in registers
            store_v(buf ^ 1);
        }
        __syncthreads();
    }

    // Epilogue: o = u / l, lse = m + ln l (natural log).
    const float l_tot = l_run + xor_shfl(l_run, 32);
    if (wave_active && myrow < N) {
        const float inv = (l_tot > 0.f) ? 1.f / l_tot : 0.f;
        uint16_t* orow = o + ((size_t)bh * N + myrow) * D;
#pragma unroll
        for (int db = 0; db < D / 32; ++db)
#pragma unroll
            for (int rg = 0; rg < 4; ++rg) {
                const int dim0 = db * 32 + rg * 8 + hi * 4;
                const u32x2 w = {pack_bf16x2(oacc[db][rg * 4 + 0] * inv, oacc[db][rg * 4 + 1] * inv),
                                 pack_bf16x2(oacc[db][rg * 4 + 2] * inv, oacc[db][rg * 4 + 3] * inv)};
                *reinterpret_cast<u32x2*>(orow + dim0) = w;
            }
        if (lse != nullptr && hi == 0)
            lse[(size_t)bh * N + myrow] = (m_run * c + log2f(l_tot)) * kLn2;
    }
}

template <int D, bool CAUSAL>
hipError_t launch_bf16_t(const PrefillArgs& a, hipStream_t stream) {
    const int BH = a.B * a.Hq;
    const int n_qt = (a.N + PF_BM - 1) / PF_BM;
    const dim3 grid((unsigned)(BH * n_qt)), block(PF_THREADS);
    hipLaunchKernelGGL((prefill_bf16_kernel<D, CAUSAL>), grid, block, 0, stream,
                       static_cast<const uint16_t*>(a.q), static_cast<const uint16_t*>(a.k),
                       static_cast<const uint16_t*>(a.v), static_cast<uint16_t*>(a.o), a.lse,
                       a.Hq, a.Hkv, a.N, BH, n_qt, a.c, a.negate);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_prefill_bf16(const PrefillArgs& a, hipStream_t stream) {
    if (a.d == 128) return a.causal ? launch_bf16_t<128, true>(a, stream) : launch_bf16_t<128, false>(a, stream);
    return a.causal ? launch_bf16_t<64, true>(a, stream) : launch_bf16_t<64, false>(a, stream);
}

}  // namespace attn

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
//     (converted to bf16); V^T comes from the row-major V tile through LDS
//     transpose loads (two per MFMA), which deliver 8 keys of one dim per
//     lane in the key order of the accumulator lanes.
//   * K/V tiles are double-buffered in LDS (two separate arrays, the loop
//     unrolled by two); the loads of tile j+1 are issued before the MFMA work
//     on tile j.  K and V go straight from memory into
//     LDS (buffer_load ... lds), their 16-byte chunks XOR-swizzled per row so
//     the operand fetches of each are free of bank conflicts.  Buffer
//     resources bound every load by the head's extent, so rows past N read
//     as zero without branches.
//   * The running maximum is raised lazily: only when a tile's maximum
//     exceeds it by more than 2^8 in weight does the wave rescale l and u.
//   * Causal: tiles entirely above the diagonal are never visited, the q
//     tiles are dispatched heaviest first, and a wave whose rows all lie
//     before a tile skips its arithmetic for it.

#include "internal.h"
#include "prefill_tile.h"

namespace attn {
namespace {

template <int D, bool CAUSAL>
__global__ void __launch_bounds__(PF_THREADS) __attribute__((amdgpu_waves_per_eu(2, 2)))
prefill_bf16_kernel(const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
                    const uint16_t* __restrict__ v, uint16_t* __restrict__ o,
                    float* __restrict__ lse, int Hq, int Hkv, int N, int BH, int n_qtiles,
                    float c, int negate) {
    using L = PfLayout<D>;
    __shared__ __attribute__((aligned(16))) uint16_t smem0[L::BUF];
    __shared__ __attribute__((aligned(16))) uint16_t smem1[L::BUF];

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
    // V staging: the same chunks, straight to LDS, with V's own swizzle.
    uint32_t voff[L::KINST];
#pragma unroll
    for (int i = 0; i < L::KINST; ++i) {
        const int p = (i * PF_WAVES + wave) * 64 + lane;
        const int r = p / L::CPR;
        const int cc = (p % L::CPR) ^ vswz<L::CPR>(r);
        voff[i] = (uint32_t)(r * D + cc * 8) * 2;
    }

    auto issue_loads = [&](int kt, uint16_t* Ks) {
        const uint32_t t0 = (uint32_t)kt * PF_BN * D * 2;
        uint16_t* Vs = Ks + L::KELEMS;
#pragma unroll
        for (int i = 0; i < L::KINST; ++i)
            buf_ld16_lds(krs, Ks + (i * PF_WAVES + wave) * 64 * 8, t0 + koff[i]);
#pragma unroll
        for (int i = 0; i < L::KINST; ++i)
            buf_ld16_lds(vrs, Vs + (i * PF_WAVES + wave) * 64 * 8, t0 + voff[i]);
    };

    f32x16 oacc[D / 32];
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[db][r] = 0.f;
    float m_run = kNegInf, l_run = 0.f;

    issue_loads(0, smem0);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();

    // One key tile: compute from `cur` while the next one loads into `nxt`.
    // The two buffers are separate LDS arrays and the loop is unrolled by two,
    // so every access names its buffer: the compiler can then tell that the
    // transpose loads of `cur` do not read what the loads into `nxt` write,
    // and does not drain those loads before them.
    auto step = [&](int kt, const uint16_t* cur, uint16_t* nxt) {
        const bool more = kt + 1 < n_kt;
        if (more) issue_loads(kt + 1, nxt);
        const int k0 = kt * PF_BN;
        const bool compute = wave_active && (!CAUSAL || k0 <= wrow0 + 31);
        if (compute) {
            const bool need_mask = (k0 + PF_BN > N) || (CAUSAL && k0 + PF_BN - 1 > wrow0);
            pf_tile_step<D, CAUSAL>(cur, cur + L::KELEMS, qf, oacc, m_run, l_run, k0, N, myrow,
                                    need_mask, c, hi, l32);
        }
        if (more) __builtin_amdgcn_s_waitcnt(0);     // tile kt+1 in LDS
        __syncthreads();
    };
    for (int kt = 0; kt < n_kt; kt += 2) {
        step(kt, smem0, smem1);
        if (kt + 1 < n_kt) step(kt + 1, smem1, smem0);
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

// Dense attention forward (prefill) for fp32 inputs and outputs, gfx950.
//
// Method ("FlashAttention" notes, section "No basta con promediar los
// resultados de los bloques"; "Autoatención, kernels CUDA y FlashAttention",
// section 3): each workgroup owns a tile of query rows and walks the key
// tiles once, keeping per row a running maximum m, sum l and numerator u;
// when a tile raises the maximum to m', l and u are first scaled by
// e^(m - m').  Only O = u / l and lse = m + ln l are written.  Scores are
// handled in base 2 with c = scale * log2(e).
//
// fp32 throughout: FMA on the vector ALU, no reduced-precision step, so the
// result stays within a few fp32 ulps of the exact one.

#include "common.h"
#include "internal.h"

namespace attn {
namespace {

// ---------------------------------------------------------------- fp32 ----
// One query row per 64-dim slice held by a thread (D / 64 threads per row),
// 64 rows per workgroup, key tiles of 32 staged in LDS.  Exponent arguments
// are formed as (s - m) * c to keep the rounding of the largest weights at
// one ulp.

constexpr int F32_ROWS = 64;
constexpr int F32_BN = 32;

template <int D, bool CAUSAL>
__global__ void __launch_bounds__(F32_ROWS * (D / 64))
prefill_f32_kernel(const float* __restrict__ q, const float* __restrict__ k,
                   const float* __restrict__ v, float* __restrict__ o, float* __restrict__ lse,
                   int Hq, int Hkv, int N, int BH, int n_qtiles, float c, int negate) {
    constexpr int TPR = D / 64;
    constexpr int THREADS = F32_ROWS * TPR;
    __shared__ __attribute__((aligned(16))) float Ks[F32_BN * D];
    __shared__ __attribute__((aligned(16))) float Vs[F32_BN * D];

    const int tid = threadIdx.x;
    const int rl = tid / TPR, part = tid % TPR;
    const int wg = blockIdx.x;
    const int qt = CAUSAL ? (n_qtiles - 1 - wg / BH) : (wg / BH);
    const int bh = wg % BH;
    const int b = bh / Hq, h = bh - b * Hq;
    const int g = h / (Hq / Hkv);
    const float* qh = q + (size_t)bh * N * D;
    const float* kh = k + ((size_t)b * Hkv + g) * N * D;
    const float* vh = v + ((size_t)b * Hkv + g) * N * D;
    const int q0 = qt * F32_ROWS;
    const int myrow = q0 + rl;

    float qr[64], acc[64];
#pragma unroll
    for (int i = 0; i < 64; ++i) {
        const float x = (myrow < N) ? qh[(size_t)myrow * D + part * 64 + i] : 0.f;
        qr[i] = negate ? -x : x;
        acc[i] = 0.f;
    }
    float m_run = kNegInf, l_run = 0.f;
    const int row_end = min(q0 + F32_ROWS, N);
    const int n_kt = CAUSAL ? (row_end + F32_BN - 1) / F32_BN : (N + F32_BN - 1) / F32_BN;

    for (int kt = 0; kt < n_kt; ++kt) {
        const int k0 = kt * F32_BN;
        __syncthreads();
        for (int e = tid * 4; e < F32_BN * D; e += THREADS * 4) {
            const int r = e / D, cc = e % D;
            const int key = k0 + r;
            f32x4 kk = {0.f, 0.f, 0.f, 0.f}, vv = {0.f, 0.f, 0.f, 0.f};
            if (key < N) {
                kk = *reinterpret_cast<const f32x4*>(kh + (size_t)key * D + cc);
                vv = *reinterpret_cast<const f32x4*>(vh + (size_t)key * D + cc);
            }
            *reinterpret_cast<f32x4*>(Ks + e) = kk;
            *reinterpret_cast<f32x4*>(Vs + e) = vv;
        }
        __syncthreads();

        float s[F32_BN];
        float mx = kNegInf;
#pragma unroll
        for (int j = 0; j < F32_BN; ++j) {
            float dot = 0.f;
#pragma unroll
            for (int i = 0; i < 64; ++i) dot = fmaf(qr[i], Ks[j * D + part * 64 + i], dot);
            if constexpr (TPR == 2) dot += __shfl_xor(dot, 1, 64);
            const int key = k0 + j;
            const bool ok = key < N && (!CAUSAL || key <= myrow);
            s[j] = ok ? dot : kNegInf;
            mx = fmaxf(mx, s[j]);
        }
        const float m_new = fmaxf(m_run, mx);
        const float m_use = (m_new == kNegInf) ? 0.f : m_new;
        const float alpha = (m_run == kNegInf) ? 0.f : fast_exp2((m_run - m_use) * c);
        float lsum = 0.f;
#pragma unroll
        for (int j = 0; j < F32_BN; ++j) {
            const float p = (s[j] == kNegInf) ? 0.f : fast_exp2((s[j] - m_use) * c);
            s[j] = p;
            lsum += p;
        }
        l_run = l_run * alpha + lsum;
#pragma unroll
        for (int i = 0; i < 64; ++i) acc[i] *= alpha;
#pragma unroll
        for (int j = 0; j < F32_BN; ++j)
#pragma unroll
            for (int i = 0; i < 64; ++i) acc[i] = fmaf(s[j], Vs[j * D + part * 64 + i], acc[i]);
        m_run = m_new;
    }

    if (myrow < N) {
        const float inv = (l_run > 0.f) ? 1.f / l_run : 0.f;
        float* orow = o + ((size_t)bh * N + myrow) * D + part * 64;
#pragma unroll
        for (int i = 0; i < 64; i += 4)
            *reinterpret_cast<f32x4*>(orow + i) =
                f32x4{acc[i] * inv, acc[i + 1] * inv, acc[i + 2] * inv, acc[i + 3] * inv};
        if (lse != nullptr && part == 0)
            lse[(size_t)bh * N + myrow] = (m_run * c + log2f(l_run)) * kLn2;
    }
}

template <int D, bool CAUSAL>
hipError_t launch_f32_t(const PrefillArgs& a, hipStream_t stream) {
    const int BH = a.B * a.Hq;
    const int n_qt = (a.N + F32_ROWS - 1) / F32_ROWS;
    const dim3 grid((unsigned)(BH * n_qt)), block(F32_ROWS * (D / 64));
    hipLaunchKernelGGL((prefill_f32_kernel<D, CAUSAL>), grid, block, 0, stream,
                       static_cast<const float*>(a.q), static_cast<const float*>(a.k),
                       static_cast<const float*>(a.v), static_cast<float*>(a.o), a.lse,
                       a.Hq, a.Hkv, a.N, BH, n_qt, a.c, a.negate);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_prefill_f32(const PrefillArgs& a, hipStream_t stream) {
    if (a.d == 128) return a.causal ? launch_f32_t<128, true>(a, stream) : launch_f32_t<128, false>(a, stream);
    return a.causal ? launch_f32_t<64, true>(a, stream) : launch_f32_t<64, false>(a, stream);
}

}  // namespace attn

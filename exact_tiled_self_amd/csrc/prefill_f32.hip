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
// 16 query rows per workgroup, 4 lanes per row (a quarter of the dims each),
// so a wave holds all 16 rows; the 4 waves split every 32-key tile staged in
// LDS (8 keys each), each keeping its own running (m, l, u) per row.  At the
// end the 4 partial states of a row are merged with the same rule: M = max
// m_w, L = sum l_w e^(m_w - M), U = sum u_w e^(m_w - M), o = U / L.  The
// problems that come in fp32 are small (a ViT image: 12 heads of 196 rows),
// so the split keeps enough waves in flight.  Exponent arguments are formed
// as (s - m) * c to keep the rounding of the largest weights at one ulp.

constexpr int F32_ROWS = 16;
constexpr int F32_BN = 32;
constexpr int F32_THREADS = 256;
constexpr int F32_KPW = F32_BN / 4;          // keys of a tile per wave

template <int D, bool CAUSAL>
__global__ void __launch_bounds__(F32_THREADS)
prefill_f32_kernel(const float* __restrict__ q, const float* __restrict__ k,
                   const float* __restrict__ v, float* __restrict__ o, float* __restrict__ lse,
                   int Hq, int Hkv, int N, int BH, int n_qtiles, float c, int negate) {
    constexpr int DPL = D / 4;               // dims per lane
    constexpr int KV = 2 * F32_BN * D;       // staged K and V (floats)
    constexpr int MERGE = 4 * 64 * (DPL + 2);
    __shared__ __attribute__((aligned(16))) float smem[KV > MERGE ? KV : MERGE];
    float* Ks = smem;
    float* Vs = smem + F32_BN * D;

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int rr = lane >> 2, part = lane & 3;
    const int wg = blockIdx.x;
    const int qt = CAUSAL ? (n_qtiles - 1 - wg / BH) : (wg / BH);
    const int bh = wg % BH;
    const int b = bh / Hq, h = bh - b * Hq;
    const int g = h / (Hq / Hkv);
    const float* qh = q + (size_t)bh * N * D;
    const float* kh = k + ((size_t)b * Hkv + g) * N * D;
    const float* vh = v + ((size_t)b * Hkv + g) * N * D;
    const int q0 = qt * F32_ROWS;
    const int myrow = q0 + rr;

    float qr[DPL], acc[DPL];
#pragma unroll
    for (int i = 0; i < DPL; i += 4) {
        f32x4 x = {0.f, 0.f, 0.f, 0.f};
        if (myrow < N) x = *reinterpret_cast<const f32x4*>(qh + (size_t)myrow * D + part * DPL + i);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            qr[i + j] = negate ? -x[j] : x[j];
            acc[i + j] = 0.f;
        }
    }
    float m_run = kNegInf, l_run = 0.f;
    const int row_end = min(q0 + F32_ROWS, N);
    const int n_kt = CAUSAL ? (row_end + F32_BN - 1) / F32_BN : (N + F32_BN - 1) / F32_BN;

    for (int kt = 0; kt < n_kt; ++kt) {
        const int k0 = kt * F32_BN;
        __syncthreads();
        for (int e = tid * 4; e < F32_BN * D; e += F32_THREADS * 4) {
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

        // this wave's 8 keys of the tile
        float s[F32_KPW];
        float mx = kNegInf;
#pragma unroll
        for (int jj = 0; jj < F32_KPW; ++jj) {
            const int j = wave * F32_KPW + jj;
            float dot = 0.f;
#pragma unroll
            for (int i = 0; i < DPL; ++i) dot = fmaf(qr[i], Ks[j * D + part * DPL + i], dot);
            dot += __shfl_xor(dot, 1, 64);
            dot += __shfl_xor(dot, 2, 64);
            const int key = k0 + j;
            const bool ok = key < N && (!CAUSAL || key <= myrow);
            s[jj] = ok ? dot : kNegInf;
            mx = fmaxf(mx, s[jj]);
        }
        const float m_new = fmaxf(m_run, mx);
        const float m_use = (m_new == kNegInf) ? 0.f : m_new;
        const float alpha = (m_run == kNegInf) ? 0.f : fast_exp2((m_run - m_use) * c);
        float lsum = 0.f;
#pragma unroll
        for (int jj = 0; jj < F32_KPW; ++jj) {
            const float p = (s[jj] == kNegInf) ? 0.f : fast_exp2((s[jj] - m_use) * c);
            s[jj] = p;
            lsum += p;
        }
        l_run = l_run * alpha + lsum;
#pragma unroll
        for (int i = 0; i < DPL; ++i) acc[i] *= alpha;
#pragma unroll
        for (int jj = 0; jj < F32_KPW; ++jj) {
            const int j = wave * F32_KPW + jj;
#pragma unroll
            for (int i = 0; i < DPL; ++i) acc[i] = fmaf(s[jj], Vs[j * D + part * DPL + i], acc[i]);
        }
        m_run = m_new;
    }

    // Merge the 4 waves' partial states of every (row, dim slice).
    __syncthreads();
    float* ua = smem;                                   // [wave][lane][DPL]
    float* ml = smem + 4 * 64 * DPL;                    // [wave][lane][2]
#pragma unroll
    for (int i = 0; i < DPL; i += 4)
        *reinterpret_cast<f32x4*>(ua + (wave * 64 + lane) * DPL + i) = f32x4{acc[i], acc[i + 1], acc[i + 2], acc[i + 3]};
    ml[(wave * 64 + lane) * 2] = m_run;
    ml[(wave * 64 + lane) * 2 + 1] = l_run;
    __syncthreads();
    if (wave == 0 && myrow < N) {
        float M = kNegInf;
#pragma unroll
        for (int w = 0; w < 4; ++w) M = fmaxf(M, ml[(w * 64 + lane) * 2]);
        float f[4], L = 0.f;
#pragma unroll
        for (int w = 0; w < 4; ++w) {
            const float mw = ml[(w * 64 + lane) * 2];
            f[w] = (mw == kNegInf) ? 0.f : fast_exp2((mw - M) * c);
            L = fmaf(f[w], ml[(w * 64 + lane) * 2 + 1], L);
        }
        const float inv = (L > 0.f) ? 1.f / L : 0.f;
        float* orow = o + ((size_t)bh * N + myrow) * D + part * DPL;
#pragma unroll
        for (int i = 0; i < DPL; i += 4) {
            f32x4 u = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int w = 0; w < 4; ++w) {
                const f32x4 x = *reinterpret_cast<const f32x4*>(ua + (w * 64 + lane) * DPL + i);
                u += f[w] * x;
            }
            *reinterpret_cast<f32x4*>(orow + i) = u * inv;
        }
        if (lse != nullptr && part == 0)
            lse[(size_t)bh * N + myrow] = (M * c + log2f(L)) * kLn2;
    }
}

template <int D, bool CAUSAL>
hipError_t launch_f32_t(const PrefillArgs& a, hipStream_t stream) {
    const int BH = a.B * a.Hq;
    const int n_qt = (a.N + F32_ROWS - 1) / F32_ROWS;
    const dim3 grid((unsigned)(BH * n_qt)), block(F32_THREADS);
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

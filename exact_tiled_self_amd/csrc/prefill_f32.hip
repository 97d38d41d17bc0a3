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
// fp32 throughout: fp32 products and sums (fp32 matrix cores at d = 64, FMA
// on the vector ALU at d = 128), no reduced-precision step, so the result
// stays within a few fp32 ulps of the exact one.

#include "common.h"
#include <stdlib.h>

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

// ------------------------------------------------------- fp32 on MFMA ----
// d = 64 on the fp32 matrix cores (v_mfma_f32_32x32x2_f32: fp32 operands,
// fp32 accumulation; no reduced-precision step).  A workgroup owns one 32-row
// query block of one head; its W waves (at most 8) take the head's 32-key
// blocks in turn (wave w: blocks w, w + W, ...), each with its own running
// (m, l, u) per row, and the W partial states of a row are merged through LDS
// at the end with M = max m_w, L = sum l_w e^(m_w - M), U = sum u_w
// e^(m_w - M), o = U / L.  The operands come straight from memory into
// registers, so a key block costs one memory round trip and the matrix
// cores, not LDS traffic:
//   * S^T = K Q^T: lane l gives K[key l % 32][dim 32 (l / 32) + s] and
//     Q[row l % 32][the same dim] at step s (the dims are split between the
//     two lane halves, each half walking its 32 in order: 32 steps of 2);
//     lane l gets back the scores of row l % 32 with keys
//     8 (r / 4) + 4 (l / 32) + r % 4, r = 0..15.
//   * O^T += V^T P^T: step s pairs key 8 (s / 4) + 4 h + s % 4 with lane half
//     h, which is exactly the lane's own score entry r = s, so P^T is the
//     lane's weights in order and V^T is V[that key][dim 32 db + l % 32].
constexpr int F32M_MAXW = 8;

template <bool CAUSAL>
__global__ void __launch_bounds__(64 * F32M_MAXW)
prefill_f32_mfma_kernel(const float* __restrict__ q, const float* __restrict__ k, const float* __restrict__ v,
                        float* __restrict__ o, float* __restrict__ lse, int Hq, int Hkv, int N, int BH,
                        int n_qb, float c, int negate) {
    constexpr int D = 64;
    // partial states: u[w][entry][lane] (lane fastest: no bank conflicts),
    // then m and l per (w, row); the merged output tile, [32 rows][65] (one
    // float of padding per row), reuses the u area
    constexpr int OS = D + 1;
    __shared__ __attribute__((aligned(16))) float su[F32M_MAXW * 32 * 64];
    __shared__ float sm[F32M_MAXW * 32], sl[F32M_MAXW * 32];

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int W = blockDim.x >> 6;
    const int h2 = lane >> 5, l32 = lane & 31;
    const int wg = blockIdx.x;
    const int qb = CAUSAL ? (n_qb - 1 - wg / BH) : (wg / BH);
    const int bh = wg % BH;
    const int b = bh / Hq, h = bh - b * Hq;
    const int g = h / (Hq / Hkv);
    const uint32_t head_bytes = (uint32_t)N * D * 4;
    const __amdgpu_buffer_rsrc_t qrs = make_rsrc(q + (size_t)bh * N * D, head_bytes);
    const __amdgpu_buffer_rsrc_t krs = make_rsrc(k + ((size_t)b * Hkv + g) * N * D, head_bytes);
    const __amdgpu_buffer_rsrc_t vrs = make_rsrc(v + ((size_t)b * Hkv + g) * N * D, head_bytes);
    const int q0 = qb * 32;
    const int myrow = q0 + l32;
    const int n_kb = CAUSAL ? min(qb + 1, (N + 31) / 32) : (N + 31) / 32;

    // q: row l32, dims 32 h2 .. 32 h2 + 31 (zero past N).  A negative scale
    // negates the scores after the product instead of q, so nothing waits for
    // these loads before the key blocks' loads are issued.
    float qv[32];
#pragma unroll
    for (int i = 0; i < 32; i += 4) {
        const f32x4 x = __builtin_bit_cast(f32x4, buf_ld16(qrs, (uint32_t)(myrow * D + 32 * h2 + i) * 4));
#pragma unroll
        for (int j = 0; j < 4; ++j) qv[i + j] = x[j];
    }

    f32x16 oacc[2];
#pragma unroll
    for (int db = 0; db < 2; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[db][r] = 0.f;
    float m_run = kNegInf, l_run = 0.f;

    for (int kb = wave; kb < n_kb; kb += W) {
        const int k0 = kb * 32;
        // K row k0 + l32, dims 32 h2 ..; V rows of the pairing, dims 32 db + l32
        float kv[32], vv[2][16];
#pragma unroll
        for (int i = 0; i < 32; i += 4) {
            const f32x4 x = __builtin_bit_cast(f32x4, buf_ld16(krs, (uint32_t)((k0 + l32) * D + 32 * h2 + i) * 4));
#pragma unroll
            for (int j = 0; j < 4; ++j) kv[i + j] = x[j];
        }
#pragma unroll
        for (int db = 0; db < 2; ++db)
#pragma unroll
            for (int st = 0; st < 16; ++st) {
                const int key = k0 + 8 * (st >> 2) + 4 * h2 + (st & 3);
                vv[db][st] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(
                                                            vrs, (uint32_t)(key * D + 32 * db + l32) * 4, 0, 0));
            }
        // every load of the block is issued before the first product uses
        // one (otherwise the compiler interleaves them with the products and
        // each K load becomes its own round trip)
        __builtin_amdgcn_sched_barrier(0);

        // two accumulators (even and odd k-steps), so that consecutive
        // products do not wait for each other's results
        f32x16 sacc, sacc1;
#pragma unroll
        for (int r = 0; r < 16; ++r) sacc[r] = sacc1[r] = 0.f;
#pragma unroll
        for (int st = 0; st < 32; st += 2) {
            sacc = __builtin_amdgcn_mfma_f32_32x32x2f32(kv[st], qv[st], sacc, 0, 0, 0);
            sacc1 = __builtin_amdgcn_mfma_f32_32x32x2f32(kv[st + 1], qv[st + 1], sacc1, 0, 0, 0);
        }
        sacc += sacc1;
        if (negate) sacc = -sacc;   // (-q).k, exactly

        // mask, row maximum (the row's 32 keys: 16 in this lane, 16 in lane ^ 32)
        float mx = kNegInf;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int key = k0 + 8 * (r >> 2) + 4 * h2 + (r & 3);
            const bool ok = key < N && (!CAUSAL || key <= myrow);
            sacc[r] = ok ? sacc[r] : kNegInf;
            mx = fmaxf(mx, sacc[r]);
        }
        mx = max_halves(mx);
        const float m_new = fmaxf(m_run, mx);
        const float m_use = (m_new == kNegInf) ? 0.f : m_new;
        const float alpha = (m_run == kNegInf) ? 0.f : fast_exp2((m_run - m_use) * c);
        float lsum = 0.f;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const float p = (sacc[r] == kNegInf) ? 0.f : fast_exp2((sacc[r] - m_use) * c);
            sacc[r] = p;
            lsum += p;
        }
        l_run = l_run * alpha + lsum;
        oacc[0] *= alpha;
        oacc[1] *= alpha;
#pragma unroll
        for (int st = 0; st < 16; ++st)
#pragma unroll
            for (int db = 0; db < 2; ++db)
                oacc[db] = __builtin_amdgcn_mfma_f32_32x32x2f32(vv[db][st], sacc[st], oacc[db], 0, 0, 0);
        m_run = m_new;
    }
    // the row's sum over both lane halves
    l_run += __shfl_xor(l_run, 32, 64);

    // merge the W partial states of each row through LDS
#pragma unroll
    for (int db = 0; db < 2; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) su[(wave * 32 + db * 16 + r) * 64 + lane] = oacc[db][r];
    if (h2 == 0) {
        sm[wave * 32 + l32] = m_run;
        sl[wave * 32 + l32] = l_run;
    }
    __syncthreads();
    // Every wave forms the weights e^(m_w - M) of the W states of its lanes'
    // rows and merges the groups of 4 entries wave, wave + W, ... of the
    // numerator (W-fold fewer LDS reads per wave than one wave merging all
    // 32).
    // (Branch-free: state w >= W reads state W - 1 with weight 0, so that
    // all of a group's LDS reads issue together.)
    float M = kNegInf, L = 0.f;
    float f[F32M_MAXW], mw[F32M_MAXW], lw[F32M_MAXW];
#pragma unroll
    for (int w = 0; w < F32M_MAXW; ++w) {
        const int wc = min(w, W - 1);
        mw[w] = sm[wc * 32 + l32];
        lw[w] = sl[wc * 32 + l32];
        M = fmaxf(M, mw[w]);
    }
#pragma unroll
    for (int w = 0; w < F32M_MAXW; ++w) {
        f[w] = (w >= W || mw[w] == kNegInf) ? 0.f : fast_exp2((mw[w] - M) * c);
        L = fmaf(f[w], lw[w], L);
    }
    const float inv = (L > 0.f) ? 1.f / L : 0.f;
    // entries in groups of 4: group gi = wave, wave + W, ... (8 groups)
    float res[32];
#pragma unroll
    for (int gk = 0; gk < 8; ++gk) {
        const int gi = wave + gk * W;
        if (gi < 8) {
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int i = 4 * gi + j;
                float u = 0.f;
#pragma unroll
                for (int w = 0; w < F32M_MAXW; ++w) u = fmaf(f[w], su[(min(w, W - 1) * 32 + i) * 64 + lane], u);
                res[4 * gk + j] = u * inv;
            }
        }
    }
    __syncthreads();
    // transpose through LDS into [row][dim] and store whole rows: entry
    // i = 16 db + r of lane (l32, h2) is dim 32 db + 8 (r / 4) + 4 h2 + r % 4
    float* so = su;   // [32 rows][OS]
#pragma unroll
    for (int gk = 0; gk < 8; ++gk) {
        const int gi = wave + gk * W;
        if (gi < 8) {
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int i = 4 * gi + j;
                so[l32 * OS + 32 * (i >> 4) + 8 * ((i & 15) >> 2) + 4 * h2 + (i & 3)] = res[4 * gk + j];
            }
        }
    }
    if (wave == 0 && lse != nullptr && h2 == 0 && myrow < N) lse[(size_t)bh * N + myrow] = (M * c + log2f(L)) * kLn2;
    __syncthreads();
    for (int e = tid * 4; e < 32 * D; e += blockDim.x * 4) {
        const int row = e / D, col = e % D;
        if (q0 + row < N) {
            const float* src = &so[row * OS + col];
            *reinterpret_cast<f32x4*>(o + ((size_t)bh * N + q0 + row) * D + col) =
                f32x4{src[0], src[1], src[2], src[3]};
        }
    }
}

// The same on 16-row query blocks (v_mfma_f32_16x16x4f32: twice the
// workgroups, each wave's products half as long).  A workgroup owns one
// 16-row block of one head; its W waves take the head's 32-key blocks in turn
// and the partial states are merged through LDS as above.  Per 32-key block,
// two 16-key halves h:
//   * S^T = K Q^T: at step s lane l gives K[key 16h + l % 16][dim 16 (l / 16)
//     + s] and Q[row l % 16][the same dim] (each lane group walks its own 16
//     dims); lane l gets back the scores of row l % 16 with keys
//     16h + 4 (l / 16) + r, r = 0..3.
//   * O^T += V^T P^T, one product per (h, r) and 16-dim block db: step (h, r)
//     pairs key 16h + 4 (l / 16) + r with lane group l / 16, which is the
//     lane's own score entry, so P^T is the lane's weights in order and V^T is
//     V[that key][dim 16 db + l % 16]; lane l gets back dims
//     16 db + 4 (l / 16) + r' of row l % 16.
template <bool CAUSAL>
__global__ void __launch_bounds__(64 * F32M_MAXW)
prefill_f32_mfma16_kernel(const float* __restrict__ q, const float* __restrict__ k, const float* __restrict__ v,
                          float* __restrict__ o, float* __restrict__ lse, int Hq, int Hkv, int N, int BH,
                          int n_qb, float c, int negate) {
    constexpr int D = 64;
    // partial states: u[w][entry][lane] (lane fastest: no bank conflicts),
    // then m and l per (w, row)
    __shared__ __attribute__((aligned(16))) float su[F32M_MAXW * 16 * 64];
    __shared__ float sm[F32M_MAXW * 16], sl[F32M_MAXW * 16];

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int W = blockDim.x >> 6;
    const int grp = lane >> 4, l16 = lane & 15;
    const int wg = blockIdx.x;
    const int qb = CAUSAL ? (n_qb - 1 - wg / BH) : (wg / BH);
    const int bh = wg % BH;
    const int b = bh / Hq, h = bh - b * Hq;
    const int g = h / (Hq / Hkv);
    const uint32_t head_bytes = (uint32_t)N * D * 4;
    const __amdgpu_buffer_rsrc_t qrs = make_rsrc(q + (size_t)bh * N * D, head_bytes);
    const __amdgpu_buffer_rsrc_t krs = make_rsrc(k + ((size_t)b * Hkv + g) * N * D, head_bytes);
    const __amdgpu_buffer_rsrc_t vrs = make_rsrc(v + ((size_t)b * Hkv + g) * N * D, head_bytes);
    const int q0 = qb * 16;
    const int myrow = q0 + l16;
    const int n_kb = CAUSAL ? min((q0 + 15) / 32 + 1, (N + 31) / 32) : (N + 31) / 32;

    // q: row l16, dims 16 grp .. 16 grp + 15 (zero past N)
    float qv[16];
#pragma unroll
    for (int i = 0; i < 16; i += 4) {
        const f32x4 x = __builtin_bit_cast(f32x4, buf_ld16(qrs, (uint32_t)(myrow * D + 16 * grp + i) * 4));
#pragma unroll
        for (int j = 0; j < 4; ++j) qv[i + j] = x[j];
    }

    f32x4 oacc[4];
#pragma unroll
    for (int db = 0; db < 4; ++db) oacc[db] = f32x4{0.f, 0.f, 0.f, 0.f};
    float m_run = kNegInf, l_run = 0.f;

    for (int kb = wave; kb < n_kb; kb += W) {
        const int k0 = kb * 32;
        // K rows k0 + 16 hh + l16, dims 16 grp ..; V of the pairing, dims 16 db + l16
        float kv[2][16], vv[2][4][4];
#pragma unroll
        for (int hh = 0; hh < 2; ++hh)
#pragma unroll
            for (int i = 0; i < 16; i += 4) {
                const f32x4 x = __builtin_bit_cast(
                    f32x4, buf_ld16(krs, (uint32_t)((k0 + 16 * hh + l16) * D + 16 * grp + i) * 4));
#pragma unroll
                for (int j = 0; j < 4; ++j) kv[hh][i + j] = x[j];
            }
#pragma unroll
        for (int hh = 0; hh < 2; ++hh)
#pragma unroll
            for (int r = 0; r < 4; ++r)
#pragma unroll
                for (int db = 0; db < 4; ++db) {
                    const int key = k0 + 16 * hh + 4 * grp + r;
                    vv[hh][r][db] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(
                                                                  vrs, (uint32_t)(key * D + 16 * db + l16) * 4, 0, 0));
                }
        // every load of the block is issued before the first product uses one
        __builtin_amdgcn_sched_barrier(0);

        // the two halves are independent accumulator chains
        f32x4 sacc[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
#pragma unroll
        for (int st = 0; st < 16; ++st)
#pragma unroll
            for (int hh = 0; hh < 2; ++hh)
                sacc[hh] = __builtin_amdgcn_mfma_f32_16x16x4f32(kv[hh][st], qv[st], sacc[hh], 0, 0, 0);
        if (negate) {
            sacc[0] = -sacc[0];   // (-q).k, exactly
            sacc[1] = -sacc[1];
        }

        // mask, row maximum (the row's 32 keys: 8 in each of lanes l16 + 16 grp)
        float mx = kNegInf;
#pragma unroll
        for (int hh = 0; hh < 2; ++hh)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int key = k0 + 16 * hh + 4 * grp + r;
                const bool ok = key < N && (!CAUSAL || key <= myrow);
                sacc[hh][r] = ok ? sacc[hh][r] : kNegInf;
                mx = fmaxf(mx, sacc[hh][r]);
            }
        mx = fmaxf(mx, xor_shfl(mx, 16));
        mx = fmaxf(mx, xor_shfl(mx, 32));
        const float m_new = fmaxf(m_run, mx);
        const float m_use = (m_new == kNegInf) ? 0.f : m_new;
        const float alpha = (m_run == kNegInf) ? 0.f : fast_exp2((m_run - m_use) * c);
        float lsum = 0.f;
#pragma unroll
        for (int hh = 0; hh < 2; ++hh)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const float p = (sacc[hh][r] == kNegInf) ? 0.f : fast_exp2((sacc[hh][r] - m_use) * c);
                sacc[hh][r] = p;
                lsum += p;
            }
        l_run = l_run * alpha + lsum;
#pragma unroll
        for (int db = 0; db < 4; ++db) oacc[db] *= alpha;
#pragma unroll
        for (int hh = 0; hh < 2; ++hh)
#pragma unroll
            for (int r = 0; r < 4; ++r)
#pragma unroll
                for (int db = 0; db < 4; ++db)
                    oacc[db] = __builtin_amdgcn_mfma_f32_16x16x4f32(vv[hh][r][db], sacc[hh][r], oacc[db], 0, 0, 0);
        m_run = m_new;
    }
    // the row's sum over its four lane groups
    l_run += xor_shfl(l_run, 16);
    l_run += xor_shfl(l_run, 32);

    // merge the W partial states of each row through LDS
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
        for (int r = 0; r < 4; ++r) su[(wave * 16 + db * 4 + r) * 64 + lane] = oacc[db][r];
    if (grp == 0) {
        sm[wave * 16 + l16] = m_run;
        sl[wave * 16 + l16] = l_run;
    }
    __syncthreads();
    // Every wave forms the weights e^(m_w - M) of its lanes' rows; wave db
    // (< 4) merges the four entries of dims block db and stores them as one
    // 16-byte run per lane.  (Branch-free: state w >= W reads state W - 1 with
    // weight 0.)
    float M = kNegInf, L = 0.f;
    float f[F32M_MAXW], mw[F32M_MAXW], lw[F32M_MAXW];
#pragma unroll
    for (int w = 0; w < F32M_MAXW; ++w) {
        const int wc = min(w, W - 1);
        mw[w] = sm[wc * 16 + l16];
        lw[w] = sl[wc * 16 + l16];
        M = fmaxf(M, mw[w]);
    }
#pragma unroll
    for (int w = 0; w < F32M_MAXW; ++w) {
        f[w] = (w >= W || mw[w] == kNegInf) ? 0.f : fast_exp2((mw[w] - M) * c);
        L = fmaf(f[w], lw[w], L);
    }
    const float inv = (L > 0.f) ? 1.f / L : 0.f;
    for (int db = wave; db < 4; db += W) {
        f32x4 u = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int r = 0; r < 4; ++r)
#pragma unroll
            for (int w = 0; w < F32M_MAXW; ++w) u[r] = fmaf(f[w], su[(min(w, W - 1) * 16 + db * 4 + r) * 64 + lane], u[r]);
        if (myrow < N)
            *reinterpret_cast<f32x4*>(o + ((size_t)bh * N + myrow) * D + 16 * db + 4 * grp) = u * inv;
    }
    if (wave == 0 && lse != nullptr && grp == 0 && myrow < N) lse[(size_t)bh * N + myrow] = (M * c + log2f(L)) * kLn2;
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
    // d = 64: the matrix-core kernel, one 16-row block per workgroup and at
    // most 8 waves over the 32-key blocks (ATTN_F32_ROWS=32, a test hook: the
    // 32-row kernel, another partition of the rows and keys)
    const int BH = a.B * a.Hq;
    const int n_kb = (a.N + 31) / 32;
    const int W = min(F32M_MAXW, n_kb);
    const char* rows_env = getenv("ATTN_F32_ROWS");
    if (!(rows_env != nullptr && rows_env[0] == '3' && rows_env[1] == '2')) {
        const int n_qb16 = (a.N + 15) / 16;
        const dim3 grid16((unsigned)(BH * n_qb16)), block16((unsigned)(64 * W));
        if (a.causal)
            hipLaunchKernelGGL((prefill_f32_mfma16_kernel<true>), grid16, block16, 0, stream,
                               static_cast<const float*>(a.q), static_cast<const float*>(a.k),
                               static_cast<const float*>(a.v), static_cast<float*>(a.o), a.lse, a.Hq, a.Hkv, a.N,
                               BH, n_qb16, a.c, a.negate);
        else
            hipLaunchKernelGGL((prefill_f32_mfma16_kernel<false>), grid16, block16, 0, stream,
                               static_cast<const float*>(a.q), static_cast<const float*>(a.k),
                               static_cast<const float*>(a.v), static_cast<float*>(a.o), a.lse, a.Hq, a.Hkv, a.N,
                               BH, n_qb16, a.c, a.negate);
        return hipGetLastError();
    }
    const int n_qb = n_kb;
    const dim3 grid((unsigned)(BH * n_qb)), block((unsigned)(64 * W));
    if (a.causal)
        hipLaunchKernelGGL((prefill_f32_mfma_kernel<true>), grid, block, 0, stream, static_cast<const float*>(a.q),
                           static_cast<const float*>(a.k), static_cast<const float*>(a.v), static_cast<float*>(a.o),
                           a.lse, a.Hq, a.Hkv, a.N, BH, n_qb, a.c, a.negate);
    else
        hipLaunchKernelGGL((prefill_f32_mfma_kernel<false>), grid, block, 0, stream, static_cast<const float*>(a.q),
                           static_cast<const float*>(a.k), static_cast<const float*>(a.v), static_cast<float*>(a.o),
                           a.lse, a.Hq, a.Hkv, a.N, BH, n_qb, a.c, a.negate);
    return hipGetLastError();
}

}  // namespace attn

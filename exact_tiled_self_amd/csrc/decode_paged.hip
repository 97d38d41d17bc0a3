// Paged-KV single-token decode for gfx950.
//
// The cache is a pool of 16-token blocks; logical position p of sequence s
// lives in block block_table[s][p / 16], slot p % 16 ("Kernels de atención
// rápida y fusión de operadores", section "Atención tipo FlashAttention y
// atención paginada").  Every key position is translated through the table.
//
// Work split.  One workgroup per (sequence, kv head, 512-token split); each
// of its 4 waves streams 8 consecutive logical blocks (128 tokens) in steps
// of two blocks, with two register sets so that the loads of step j+1 are in
// flight while step j computes, and keeps its own running state (m, l, u).
// The G query heads that share the kv head (grouped-query attention) form
// the rows of the score tile, so the two products are genuine small matrix
// products and run on MFMA (v_mfma_f32_16x16x32_bf16, G <= 16 rows):
//   * S^T = K Q^T: the lane's A operand is 8 dims of one key, loaded straight
//     from the block; each lane ends up owning one query row (lane % 16) and
//     4 keys of each block.
//   * O^T = V^T P^T: P^T comes from the lane's own score registers (keys
//     4g..4g+3 of both blocks); the V^T operand needs 8 keys of one dim per
//     lane, so each lane loads 16-byte row slices of its 8 keys (coalesced:
//     16 lanes cover one 256-byte row) and transposes the 8x8 block in
//     registers with v_perm.  The output again has one query row per lane,
//     so the rescale by e^(m - m') is lane-local.
// The four waves' states are merged in LDS by the rescale rule of the online
// softmax, and the workgroup writes one fp32 partial state per query head to
// the workspace.  A second kernel merges the partial states of a sequence in
// split order (deterministic): M = max m_k, L = sum l_k e^(m_k - M),
// O = sum u_k e^(m_k - M) / L ("FlashAttention" notes, section "No basta con
// promediar los resultados de los bloques": each part enters with its own
// weight, not as an average).
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
constexpr int DC_WAVE_BLOCKS = 8;        // 128 tokens per wave
constexpr int DC_STEP_BLOCKS = 2;        // 32 tokens per pipeline step
constexpr int DC_STEPS = DC_WAVE_BLOCKS / DC_STEP_BLOCKS;
static_assert(4 * DC_WAVE_BLOCKS * kDecodeBlock == kDecodeSplit, "split = 4 waves x 8 blocks");

template <int D>
struct VRow;
template <>
struct VRow<128> { typedef u32x4 T; };
template <>
struct VRow<64> { typedef u32x2 T; };

// Registers of one pipeline step (two blocks): K operands and V row slices.
template <int D>
struct StepRegs {
    u32x4 k[DC_STEP_BLOCKS][D / 32];
    typename VRow<D>::T v[8];
    int phys[DC_STEP_BLOCKS];
    bool valid[DC_STEP_BLOCKS];
};

template <int D>
__global__ void __launch_bounds__(DC_THREADS)
decode_partial_kernel(const uint16_t* __restrict__ q, const uint16_t* __restrict__ kc,
                      const uint16_t* __restrict__ vc, const int32_t* __restrict__ table,
                      const int32_t* __restrict__ ctx_lens, float* __restrict__ ws, int Hq,
                      int Hkv, int max_blocks, int num_blocks, int nsplit, float c, int negate) {
    constexpr int KS = D / 32;              // MFMA k-steps over the head dim
    constexpr int DPL = D / 16;             // dims per lane column of an MFMA
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

    // the wave index is uniform: keep the block-table walk in scalar registers
    const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l16 = lane & 15, grp = lane >> 4;
    const int nblk = (ctx + kDecodeBlock - 1) / kDecodeBlock;
    const int fb = split * (kDecodeSplit / kDecodeBlock) + wave * DC_WAVE_BLOCKS;
    const int wblocks = min(max(nblk - fb, 0), DC_WAVE_BLOCKS);
    const int nsteps = (wblocks + DC_STEP_BLOCKS - 1) / DC_STEP_BLOCKS;

    // The wave's table entries, fetched once up front (lane j holds entry
    // fb + j), so that no K/V load waits behind a table read; entries outside
    // [0, num_blocks) are not followed (the sequence's output becomes NaN).
    int tab = 0;
    if (lane < wblocks) tab = table[(size_t)s * max_blocks + fb + lane];
    const bool tab_ok = lane < wblocks && tab >= 0 && tab < num_blocks;
    const uint64_t valid_mask = __builtin_amdgcn_ballot_w64(tab_ok);
    const bool bad = __builtin_amdgcn_ballot_w64(lane < wblocks && !tab_ok) != 0;

    // Q operand (B of S^T = K Q^T): query row l16 (head g*G + l16 when l16 < G),
    // dims 8*(4ks + grp) .. +7.
    bf16x8 qf[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
        u32x4 w = {0u, 0u, 0u, 0u};
        if (l16 < G) w = ld16(q + ((size_t)s * Hq + g * G + l16) * D + 8 * (4 * ks + grp));
        if (negate) w = neg_bf16x8(w);
        qf[ks] = __builtin_bit_cast(bf16x8, w);
    }

    auto load_step = [&](StepRegs<D>& R, int st) {
#pragma unroll
        for (int bi = 0; bi < DC_STEP_BLOCKS; ++bi) {
            const int j = st * DC_STEP_BLOCKS + bi;            // block index within the wave
            const bool ok = (valid_mask >> j) & 1;
            R.phys[bi] = ok ? __builtin_amdgcn_readlane(tab, j) : 0;
            R.valid[bi] = ok;
        }
#pragma unroll
        for (int bi = 0; bi < DC_STEP_BLOCKS; ++bi) {
            const uint16_t* kb = kc + (((size_t)R.phys[bi] * Hkv + g) * kDecodeBlock + l16) * D;
#pragma unroll
            for (int ks = 0; ks < KS; ++ks)
                R.k[bi][ks] = R.valid[bi] ? ld16(kb + 8 * (4 * ks + grp)) : u32x4{0u, 0u, 0u, 0u};
        }
#pragma unroll
        for (int i8 = 0; i8 < 8; ++i8) {
            const int bi = i8 >> 2;
            const uint16_t* vr = vc + (((size_t)R.phys[bi] * Hkv + g) * kDecodeBlock + 4 * grp + (i8 & 3)) * D;
            R.v[i8] = R.valid[bi] ? *reinterpret_cast<const VT*>(vr + DPL * l16) : VT{};
        }
    };

    float m_run = kNegInf, l_run = 0.f;
    f32x4 oacc[DPL];
#pragma unroll
    for (int j = 0; j < DPL; ++j) oacc[j] = f32x4{0.f, 0.f, 0.f, 0.f};

    auto compute_step = [&](StepRegs<D>& R, int st) {
        const int tok0 = (fb + st * DC_STEP_BLOCKS) * kDecodeBlock;
        f32x4 sacc[DC_STEP_BLOCKS];
#pragma unroll
        for (int bi = 0; bi < DC_STEP_BLOCKS; ++bi) {
            sacc[bi] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < KS; ++ks)
                sacc[bi] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, R.k[bi][ks]),
                                                                   qf[ks], sacc[bi], 0, 0, 0);
        }
        // lane: query row l16, keys 4*grp + r of each block
        float mx = kNegInf;
#pragma unroll
        for (int bi = 0; bi < DC_STEP_BLOCKS; ++bi)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const bool ok = R.valid[bi] && (tok0 + bi * kDecodeBlock + 4 * grp + r) < ctx;
                sacc[bi][r] = ok ? sacc[bi][r] : kNegInf;
                mx = fmaxf(mx, sacc[bi][r]);
            }
        mx = fmaxf(mx, xor_shfl(mx, 16));
        mx = fmaxf(mx, xor_shfl(mx, 32));
        const float m_new = fmaxf(m_run, mx);
        const float m_use = (m_new == kNegInf) ? 0.f : m_new;
        const float alpha = (m_run == kNegInf) ? 0.f : fast_exp2((m_run - m_use) * c);
        const float mc = m_use * c;
        float lsum = 0.f;
#pragma unroll
        for (int bi = 0; bi < DC_STEP_BLOCKS; ++bi)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const float sv = sacc[bi][r];
                const float p = (sv == kNegInf) ? 0.f : fast_exp2(fmaf(sv, c, -mc));
                sacc[bi][r] = p;
                lsum += p;
            }
        l_run = l_run * alpha + lsum;
        m_run = m_new;
        // P^T operand: row l16, keys (4grp..4grp+3) of block 0 then of block 1
        bf16x8 pb;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            pb[i] = (__bf16)sacc[0][i];
            pb[4 + i] = (__bf16)sacc[1][i];
        }
        // V rows of positions past the length are zeroed (NaN-safe)
#pragma unroll
        for (int i8 = 0; i8 < 8; ++i8)
            if (!(R.valid[i8 >> 2] && (tok0 + (i8 >> 2) * kDecodeBlock + 4 * grp + (i8 & 3)) < ctx))
                R.v[i8] = VT{};
        // O^T += V^T P^T: A operand = 8 keys of dim DPL*l16 + j (8x8 register transpose)
#pragma unroll
        for (int j = 0; j < DPL; ++j) {
            const int w = j >> 1;
            const uint32_t sel = (j & 1) ? 0x07060302u : 0x05040100u;
            u32x4 t;
            t.x = __builtin_amdgcn_perm(R.v[1][w], R.v[0][w], sel);
            t.y = __builtin_amdgcn_perm(R.v[3][w], R.v[2][w], sel);
            t.z = __builtin_amdgcn_perm(R.v[5][w], R.v[4][w], sel);
            t.w = __builtin_amdgcn_perm(R.v[7][w], R.v[6][w], sel);
            oacc[j] *= alpha;
            oacc[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, t), pb,
                                                              oacc[j], 0, 0, 0);
        }
    };

    // Two register sets, ping-pong: the loads of step st+1 are in flight
    // while step st computes.
    StepRegs<D> ra, rb;
    if (nsteps > 0) load_step(ra, 0);
#pragma unroll 1
    for (int st = 0; st < nsteps; st += 2) {
        if (st + 1 < nsteps) load_step(rb, st + 1);
        compute_step(ra, st);
        if (st + 1 < nsteps) {
            if (st + 2 < nsteps) load_step(ra, st + 2);
            compute_step(rb, st + 1);
        }
    }

    // lane: row l16, dims DPL*(4grp + r) + j.  Merge the four waves in LDS.
    l_run += xor_shfl(l_run, 16);
    l_run += xor_shfl(l_run, 32);
    if (grp == 0) {
        sm_m[wave][l16] = m_run;
        sm_l[wave][l16] = bad ? __builtin_nanf("") : l_run;
    }
    if (l16 < G) {
#pragma unroll
        for (int r = 0; r < 4; ++r)
#pragma unroll
            for (int j = 0; j < DPL; ++j) sm_o[wave][l16][DPL * (4 * grp + r) + j] = oacc[j][r];
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

// One workgroup per (query head, sequence), one thread per output dim:
// merge the sequence's split states for that head in split order (fixed
// order, so the result is deterministic):  M = max m_k,
// L = sum l_k e^(m_k - M), O = sum u_k e^(m_k - M) / L, lse = M + ln L.
// Each wave reads the splits' (m_k, l_k) with one load per lane (split k in
// lane k), reduces them across lanes, and then issues all the u_k loads of
// its dim at once.
template <int D>
__global__ void __launch_bounds__(D)
decode_combine_kernel(const float* __restrict__ ws, const int32_t* __restrict__ ctx_lens,
                      uint16_t* __restrict__ o, float* __restrict__ lse, int S, int Hq, int Hkv,
                      int max_blocks, int nsplit, float c) {
    const int h = blockIdx.x, s = blockIdx.y, dim = threadIdx.x, lane = dim & 63;
    const int G = Hq / Hkv, g = h / G, row = h - g * G;
    const int cap = max_blocks * kDecodeBlock;
    int ctx = ctx_lens[s];
    const bool bad = ctx < 0 || ctx > cap;
    ctx = ctx < 0 ? 0 : (ctx > cap ? cap : ctx);
    const int nsp = (ctx + kDecodeSplit - 1) / kDecodeSplit;
    const size_t stride = (size_t)G * (D + 2);
    const float* base = ws + (size_t)(s * Hkv + g) * nsplit * stride;

    // M over all splits, 64 per pass
    float M = kNegInf;
    for (int k0 = 0; k0 < nsp; k0 += 64) {
        const float mk = (k0 + lane < nsp) ? base[(k0 + lane) * stride + row] : kNegInf;
        float mx = mk;
#pragma unroll
        for (int off = 32; off >= 1; off >>= 1) mx = fmaxf(mx, __shfl_xor(mx, off, 64));
        M = fmaxf(M, mx);
    }
    float L = 0.f, U = 0.f;
    for (int k0 = 0; k0 < nsp; k0 += 64) {
        const bool in = k0 + lane < nsp;
        const float mk = in ? base[(k0 + lane) * stride + row] : kNegInf;
        const float lk = in ? base[(k0 + lane) * stride + G + row] : 0.f;
        const float fk = (mk == kNegInf) ? 0.f : fast_exp2((mk - M) * c);
        float lw = fk * lk;
#pragma unroll
        for (int off = 32; off >= 1; off >>= 1) lw += __shfl_xor(lw, off, 64);
        L += lw;
        const int nk = min(64, nsp - k0);
        // u loads in groups of 16, all issued before they are summed (in split order)
        for (int j0 = 0; j0 < nk; j0 += 16) {
            float uv[16], fw[16];
#pragma unroll
            for (int j = 0; j < 16; ++j) {
                const int kk = min(j0 + j, nk - 1);
                fw[j] = (j0 + j < nk) ? __shfl(fk, kk, 64) : 0.f;
                uv[j] = base[(k0 + kk) * stride + 2 * G + row * D + dim];
            }
#pragma unroll
            for (int j = 0; j < 16; ++j) U = fmaf(fw[j], uv[j], U);
        }
    }
    const float nan = __builtin_nanf("");
    const float inv = (L > 0.f) ? 1.f / L : (L == 0.f ? 0.f : nan);
    const float val = bad ? nan : U * inv;
    const __bf16 bv = (__bf16)val;
    o[((size_t)s * Hq + h) * D + dim] = __builtin_bit_cast(uint16_t, bv);
    if (lse != nullptr && dim == 0) {
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
    const dim3 g2((unsigned)a.Hq, (unsigned)a.S), b2(D);
    hipLaunchKernelGGL((decode_combine_kernel<D>), g2, b2, 0, stream, a.workspace, a.ctx_lens,
                       static_cast<uint16_t*>(a.o), a.lse, a.S, a.Hq, a.Hkv, a.max_blocks, nsplit, a.c);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_paged_decode_bf16(const DecodeArgs& a, hipStream_t stream) {
    return a.d == 128 ? launch_decode_t<128>(a, stream) : launch_decode_t<64>(a, stream);
}

}  // namespace attn

// One key tile of the bf16 prefill recurrence, shared by the dense prefill
// and the chunked prefill over a paged cache.
//
// A workgroup of 4 waves owns 128 query rows (32 per wave); key tiles of 64
// keys are staged in LDS: K row-major with 16-byte chunks XOR-swizzled, V
// transposed.  One call of pf_tile_step advances one wave's 32 rows over one
// staged tile with the online-softmax recurrence ("FlashAttention" notes,
// section "No basta con promediar los resultados de los bloques"): scores of
// the tile, new running maximum, rescale of l and u by e^(m - m') when it
// rises, P = e^(s - m), l += rowsum P, u += P V.  Scores are in base 2 with
// c = |scale| * log2(e).
//
// MFMA v_mfma_f32_32x32x16_bf16 on the TRANSPOSED products: S^T = K Q^T puts
// one query row per lane (lane % 32) with 16 of its keys per 32-key block,
// so the row maximum is an in-lane max plus one exchange with lane ^ 32, and
// the rescale of u is lane-local; O^T += V^T P^T takes P^T straight from the
// score accumulators.  The V^T layout in LDS stores keys 4..7 and 8..11 of
// every 16-key group swapped, which is the key order of the accumulator
// lanes.
#pragma once

#include "common.h"

namespace attn {

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

// Store the V rows one thread loaded (VKPT keys from key0, dims 8*vdc ..
// 8*vdc + 7) transposed into the V^T area of an LDS stage; pos = swap23(key0).
template <int D>
__device__ __forceinline__ void pf_store_vt(uint16_t* Vt, const u32x4* vreg, int pos, int vdc) {
    using L = PfLayout<D>;
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
}

// Advance one wave's rows over the tile of keys k0 .. k0 + 63 staged at Ks
// (K) and Vt (V^T).  Key position `key` is allowed for this lane's row iff
// key < kend and (when CAUSAL) key <= mypos; `need_mask` must be true
// whenever some key of the tile fails that test for some row of the wave.
template <int D, bool CAUSAL>
__device__ __forceinline__ void pf_tile_step(const uint16_t* Ks, const uint16_t* Vt, const bf16x8* qf,
                                             f32x16* oacc, float& m_run, float& l_run, int k0,
                                             int kend, int mypos, bool need_mask, float c, int hi,
                                             int l32) {
    using L = PfLayout<D>;
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
            const bf16x8 a = *reinterpret_cast<const bf16x8*>(Ks + (r * D + cc * 8));
            sacc[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[ks], sacc[kb], 0, 0, 0);
        }
    }

    // Lane key of accumulator entry r in block kb: k0 + 32kb + 8(r/4) + 4hi + r%4.
    float mx = kNegInf;
    if (need_mask) {
#pragma unroll
        for (int kb = 0; kb < PF_BN / 32; ++kb)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int key = k0 + kb * 32 + 8 * (r >> 2) + 4 * hi + (r & 3);
                const bool ok = key < kend && (!CAUSAL || key <= mypos);
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

}  // namespace attn

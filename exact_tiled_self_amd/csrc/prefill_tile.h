// One key tile of the bf16 prefill recurrence, shared by the dense prefill
// and the chunked prefill over a paged cache.
//
// A workgroup of 4 waves owns 128 query rows (32 per wave); key tiles of 64
// keys are staged in LDS, K and V both row-major with their 16-byte chunks
// XOR-swizzled (straight from memory, no register staging).  One call of pf_tile_step advances one wave's 32 rows over one
// staged tile with the online-softmax recurrence ("FlashAttention" notes,
// section "No basta con promediar los resultados de los bloques"): scores of
// the tile, new running maximum, rescale of l and u by e^(m - m') when it
// rises, P = e^(s - m), l += rowsum P, u += P V.  Scores are in base 2 with
// c = |scale| * log2(e).  The maximum moves lazily (only by more than 2^8 in
// weight), and the tile's weights, taken against the running maximum first,
// show through their row sums whether it could move at all: only then is the
// tile's maximum formed.
//
// MFMA v_mfma_f32_32x32x16_bf16 on the TRANSPOSED products: S^T = K Q^T puts
// one query row per lane (lane % 32) with 16 of its keys per 32-key block,
// so the row maximum is an in-lane max plus one exchange with lane ^ 32, and
// the rescale of u is lane-local; O^T += V^T P^T takes P^T straight from the
// score accumulators.  The V^T operand is read from the row-major V tile with
// the LDS transpose load (ds_read_b64_tr_b16): within each 16-lane group it
// hands lane i the element (i mod 4) of the 8 bytes that lanes i/4, 4 + i/4,
// 8 + i/4 and 12 + i/4 addressed, i.e. it transposes a 4-row x 16-column
// block; two of them give a lane 8 keys of one dim, in the key order of the
// score accumulators.
#pragma once

#include "common.h"

namespace attn {

constexpr int PF_WAVES = 4;
constexpr int PF_BM = 32 * PF_WAVES;   // query rows per workgroup
constexpr int PF_BN = 64;              // keys per tile
constexpr int PF_THREADS = 64 * PF_WAVES;

template <int D, int BN = PF_BN>
struct PfLayout {
    static_assert(BN == 32 || BN == 64, "key tiles of 32 or 64 keys");
    static constexpr int CPR = D / 8;           // 16-byte chunks per row
    static constexpr int KELEMS = BN * D;       // K tile, rows XOR-swizzled, no pad
    static constexpr int VELEMS = BN * D;       // V tile, the same shape
    static constexpr int BUF = KELEMS + VELEMS; // one pipeline stage (bf16 elements)
    static constexpr int KINST = BN * CPR / PF_THREADS;     // load-to-LDS per thread per tile
    static_assert(KINST * PF_THREADS == BN * CPR, "tile split");
};

// XOR swizzle of the 16-byte chunks of K row r, so that the 16 rows read by
// one MFMA operand fetch hit 16 different bank groups.
template <int CPR>
__device__ __forceinline__ int kswz(int r) {
    return CPR == 16 ? (r & 15) : ((r >> 1) & 7);
}

// XOR swizzle of the 16-byte chunks of V row r.  A transpose load reads 4
// consecutive rows x 32 bytes per 16 lanes (and 2 such groups per 32 lanes);
// shifting rows r..r+3 by 0, 6, 12, 10 chunks puts those reads on distinct
// banks.
template <int CPR>
__device__ __forceinline__ int vswz(int r) {
    return (0xAC60 >> (4 * (r & 3))) & 15 & (CPR - 1);
}

typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;

// Per-lane element offsets (inside a V tile, before the key-block term) of
// the two transpose loads that give dims 32*db + (lane % 32), keys
// 16*c16 + 4*hi + {0..3} and {8..11}; the key-block term (16*c16)*D is added
// by the caller.  db-dependent: the swizzle mixes the chunk index.
template <int D>
__device__ __forceinline__ int pf_vtr_offset(int lane, int db) {
    constexpr int CPR = D / 8;
    const int gi = lane >> 4, a = lane & 15;
    const int row = 4 * (gi >> 1) + (a >> 2);                 // + 16*c16 + 8*rd (multiples of 4)
    const int chunk = db * 4 + 2 * (gi & 1) + ((a & 3) >> 1);
    return row * D + ((chunk ^ vswz<CPR>(row)) * 8) + 4 * (a & 1);
}

// A tile raises the running maximum only when some row's new maximum exceeds
// it by more than 2^8 in weight: below that the old maximum stays the
// reference (weights up to 256 are exact in fp32 and bf16 range) and the
// numerator needs no rescale.  u / l is unchanged by the choice of reference.
constexpr float kLazyLog2 = 8.0f;
// The quick form of that test (one lane's part of a row sum of weights at
// most 2^7): it implies the full test's answer with a margin of one in the
// exponent, far above the rounding of either side.
constexpr float kLazyCheck = 128.0f;

// Advance one wave's rows over the tile of keys k0 .. k0 + BN - 1 staged at
// Ks (K) and Vs (V, row-major).  BN (keys per tile) is 64, or 32 for a
// second tile configuration (any partition of the keys gives the same u / l).  Key position `key` is allowed for this lane's row iff
// key < kend and (when CAUSAL) key <= mypos; `need_mask` must be true
// whenever some key of the tile fails that test for some row of the wave.
//
// VB (default all) is the number of 16-key blocks of V the tile holds: a
// last tile of 32 keys whose second 16 lie wholly past kend may be staged
// with only its first 16 V rows (VB = 1); those keys are masked, so their
// weights are 0 and their V rows are never read.
template <int D, bool CAUSAL, int BN = PF_BN, int VB = BN / 16>
__device__ __forceinline__ void pf_tile_step(const uint16_t* Ks, const uint16_t* Vs, const bf16x8* qf,
                                             f32x16* oacc, float& m_run, float& l_run, int k0,
                                             int kend, int mypos, bool need_mask, float c, int hi,
                                             int l32) {
    using L = PfLayout<D, BN>;
    constexpr int KS = D / 16;           // k-steps of the score product
    constexpr int KPF = KS < 4 ? KS : 4; // K operand pairs read ahead of their MFMAs
    const int lane = hi * 32 + l32;

    // Operand reads are issued ahead of the MFMAs that consume them (the
    // scheduling barriers keep the compiler from sinking them back to their
    // uses), so an LDS round trip overlaps the matrix work instead of
    // preceding every MFMA.
    bf16x8 ka[KS][BN / 32];
    auto kread = [&](int ks) {
#pragma unroll
        for (int kb = 0; kb < BN / 32; ++kb) {
            const int r = kb * 32 + l32;
            const int cc = (ks * 2 + hi) ^ kswz<L::CPR>(r);
            ka[ks][kb] = *reinterpret_cast<const bf16x8*>(Ks + (r * D + cc * 8));
        }
    };
    // V^T operand of key block c16 (16 keys), dims block db: two transpose
    // loads.  Each per-lane base is one opaque element offset from Vs, so
    // every read's address stays a short chain from the LDS array: the
    // compiler can then see that these reads do not touch the other buffer,
    // which the next tile's loads are filling, and does not wait for them.
    const uint16_t* vbase[D / 32];
#pragma unroll
    for (int db = 0; db < D / 32; ++db) {
        int off = pf_vtr_offset<D>(lane, db);
        asm("" : "+v"(off));
        vbase[db] = Vs + off;
    }
    auto vread = [&](int c16, bf16x8* dst) {
#pragma unroll
        for (int db = 0; db < D / 32; ++db) {
            const bf16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(vbase[db] + c16 * 16 * D));
            const bf16x4 hi4 = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(vbase[db] + c16 * 16 * D + 8 * D));
            dst[db] = __builtin_shufflevector(lo, hi4, 0, 1, 2, 3, 4, 5, 6, 7);
        }
    };

    // S^T = K Q^T for the keys of this tile (32-key blocks).
    f32x16 sacc[BN / 32];
    auto scores = [&]() {
#pragma unroll
        for (int kb = 0; kb < BN / 32; ++kb)
#pragma unroll
            for (int r = 0; r < 16; ++r) sacc[kb][r] = 0.f;
#pragma unroll
        for (int ks = 0; ks < KPF; ++ks) kread(ks);
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            if (ks + KPF < KS) kread(ks + KPF);
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int kb = 0; kb < BN / 32; ++kb)
                sacc[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka[ks][kb], qf[ks], sacc[kb], 0, 0, 0);
            __builtin_amdgcn_sched_barrier(0);
        }
        // Lane key of accumulator entry r in block kb: k0 + 32kb + 8(r/4) + 4hi + r%4.
        if (need_mask) {
#pragma unroll
            for (int kb = 0; kb < BN / 32; ++kb)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int key = k0 + kb * 32 + 8 * (r >> 2) + 4 * hi + (r & 3);
                    const bool ok = key < kend && (!CAUSAL || key <= mypos);
                    sacc[kb][r] = ok ? sacc[kb][r] : kNegInf;
                }
        }
    };
    // P = 2^(c s - mc) in place, and this lane's part of the row sum.
    auto weights = [&](float mc) {
        float lsum = 0.f;
        if (need_mask) {
#pragma unroll
            for (int kb = 0; kb < BN / 32; ++kb)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const float sv = sacc[kb][r];
                    const float p = (sv == kNegInf) ? 0.f : fast_exp2(fmaf(sv, c, -mc));
                    sacc[kb][r] = p;
                    lsum += p;
                }
        } else {
#pragma unroll
            for (int kb = 0; kb < BN / 32; ++kb)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const float p = fast_exp2(fmaf(sacc[kb][r], c, -mc));
                    sacc[kb][r] = p;
                    lsum += p;
                }
        }
        return lsum;
    };
    scores();

    // The first V^T operands are read now; the softmax below hides them.
    bf16x8 va[2][D / 32];
    vread(0, va[0]);
    __builtin_amdgcn_sched_barrier(0);

    // Once every row has a running maximum, the weights are taken against it
    // directly.  A lane's part of a row sum bounds each of its weights, so
    // when no part exceeds kLazyCheck (2^7) no score rose above the running
    // maximum by more than 2^7 in weight, less than the 2^kLazyLog2 that
    // would move it: the tile keeps the maximum, exactly as the full test
    // below decides.  Otherwise (rare after the first tile: a part that
    // large) the scores are computed again and take the full test.
    bool full = __builtin_amdgcn_ballot_w64(m_run == kNegInf) != 0;
    float lsum = 0.f;
    if (!full) {
        lsum = weights(m_run * c);
        full = __builtin_amdgcn_ballot_w64(!(lsum <= kLazyCheck)) != 0;
        if (full) scores();
    }
    if (full) {
        float mx = kNegInf;
#pragma unroll
        for (int kb = 0; kb < BN / 32; ++kb)
#pragma unroll
            for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sacc[kb][r]);
        mx = max_halves(mx);

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
        lsum = weights((m_run == kNegInf) ? 0.f : m_run * c);
    }
    l_run += lsum;
    __builtin_amdgcn_sched_barrier(0);

    // O^T += V^T P^T, 16 keys per MFMA; the operands of the next key block
    // are read while the current one's MFMAs run.
    static_assert(VB >= 1 && VB <= BN / 16, "V blocks");
#pragma unroll
    for (int c16 = 0; c16 < VB; ++c16) {
        if (c16 + 1 < VB) vread(c16 + 1, va[(c16 + 1) & 1]);
        const int kb = c16 >> 1, sh = (c16 & 1) * 8;
        bf16x8 pb;
#pragma unroll
        for (int i = 0; i < 8; ++i) pb[i] = (__bf16)sacc[kb][sh + i];
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int db = 0; db < D / 32; ++db)
            oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va[c16 & 1][db], pb, oacc[db], 0, 0, 0);
        __builtin_amdgcn_sched_barrier(0);
    }
}

// Pieces of the software-pipelined tile loop (prefill_sp_kernel, the dense
// causal d = 128 prefill): one wave's 32 rows in the same layout as
// pf_tile_step, with the wave's state held by reference.  Key `key` of a tile
// is allowed for this lane's row iff key < kend and (when CAUSAL) key <= mypos.
// The caller places the pieces so that the vector work of one tile sits
// between the MFMAs of another (pf_interleave), because a wave's own
// independent VALU instructions issue while its MFMAs execute.
template <int D, bool CAUSAL>
struct PfPipe {
    static constexpr int KS = D / 16, NDB = D / 32;
    const bf16x8 (&qf)[KS];
    const int (&kofs)[KS];     // K operand offsets (rows l32, per k-step) inside a K tile
    const int (&vofs)[NDB];    // V^T transpose-load offsets per dims block inside a V tile
    f32x16 (&oacc)[NDB];
    float& m_run;
    float& l_run;
    float c;
    int hi, kend, mypos;

    // S^T = K Q^T of one tile (K operands three k-steps ahead of their MFMAs).
    __device__ __forceinline__ void scores(const uint16_t* Kb, f32x16 (&sacc)[2]) const {
        bf16x8 ka[KS][2];
        auto kread = [&](int ks) {
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
                ka[ks][kb] = *reinterpret_cast<const bf16x8*>(Kb + kofs[ks] + kb * 32 * D);
        };
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int r = 0; r < 16; ++r) sacc[kb][r] = 0.f;
        kread(0);
        kread(1);
        kread(2);
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            if (ks + 3 < KS) kread(ks + 3);
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
                sacc[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka[ks][kb], qf[ks], sacc[kb], 0, 0, 0);
        }
    }
    // Mask only (keys of tile k0 .. not allowed -> -inf).
    template <bool MASK>
    __device__ __forceinline__ void mask(f32x16 (&sacc)[2], int k0) const {
        if (MASK) {
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int key = k0 + kb * 32 + 8 * (r >> 2) + 4 * hi + (r & 3);
                    const bool ok = key < kend && (!CAUSAL || key <= mypos);
                    sacc[kb][r] = ok ? sacc[kb][r] : kNegInf;
                }
        }
    }
    // Row maximum of an already masked tile.
    __device__ __forceinline__ float rowmax_masked(const f32x16 (&sacc)[2]) const {
        float mx = kNegInf;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sacc[kb][r]);
        return max_halves(mx);
    }
    // P = 2^(c s - c m) in bf16 and this lane's part of the row sum (not yet
    // added to l).  Masked scores are -inf and give exactly 0 only for c > 0:
    // callers send c = 0 elsewhere.
    __device__ __forceinline__ float probs_part(const f32x16 (&sacc)[2], bf16x8 (&pb)[4]) const {
        const float mc = (m_run == kNegInf) ? 0.f : m_run * c;
        float lsum = 0.f;
#pragma unroll
        for (int c16 = 0; c16 < 4; ++c16)
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const float p = fast_exp2(fmaf(sacc[c16 >> 1][(c16 & 1) * 8 + i], c, -mc));
                lsum += p;
                pb[c16][i] = (__bf16)p;
            }
        return lsum;
    }
    // Lazy rescale (as in pf_tile_step): only when some row's maximum grew by
    // more than 2^kLazyLog2, or on the first tile.
    __device__ __forceinline__ void rescale(float mx) const {
        const bool grow = (m_run == kNegInf) ? (mx != kNegInf) : ((mx - m_run) * c > kLazyLog2);
        if (__builtin_amdgcn_ballot_w64(grow) != 0) {
            const float m_new = grow ? mx : m_run;
            const float alpha = (m_run == kNegInf) ? 0.f : fast_exp2((m_run - m_new) * c);
            l_run *= alpha;
#pragma unroll
            for (int db = 0; db < NDB; ++db)
#pragma unroll
                for (int r = 0; r < 16; ++r) oacc[db][r] *= alpha;
            m_run = m_new;
        }
    }
    // O^T += V^T P^T of one tile (V^T operands one key block ahead).
    __device__ __forceinline__ void pv(const uint16_t* Vb, const bf16x8 (&pb)[4]) const {
        bf16x8 va[2][NDB];
        auto vread = [&](int c16, bf16x8* dst) {
#pragma unroll
            for (int db = 0; db < NDB; ++db) {
                const bf16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
                    (lds_bf16x4*)(Vb + vofs[db] + c16 * 16 * D));
                const bf16x4 hi4 = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
                    (lds_bf16x4*)(Vb + vofs[db] + c16 * 16 * D + 8 * D));
                dst[db] = __builtin_shufflevector(lo, hi4, 0, 1, 2, 3, 4, 5, 6, 7);
            }
        };
        vread(0, va[0]);
#pragma unroll
        for (int c16 = 0; c16 < 4; ++c16) {
            if (c16 + 1 < 4) vread(c16 + 1, va[(c16 + 1) & 1]);
#pragma unroll
            for (int db = 0; db < NDB; ++db)
                oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va[c16 & 1][db], pb[c16], oacc[db], 0, 0, 0);
        }
    }
};

// Interleaving request for the scheduler over the current region: D0 LDS
// reads up front, then NM times one MFMA, NV VALU instructions (trans
// included) and DP LDS reads, so each read is issued several MFMAs before its
// use and the vector work fills the MFMAs' shadow.
template <int NM, int NV, int D0, int DP>
__device__ __forceinline__ void pf_interleave() {
    __builtin_amdgcn_sched_group_barrier(0x100, D0, 0);
#pragma unroll
    for (int i = 0; i < NM; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);    // MFMA
        __builtin_amdgcn_sched_group_barrier(0x402, NV, 0);   // VALU + trans
        __builtin_amdgcn_sched_group_barrier(0x100, DP, 0);   // LDS reads
    }
}

}  // namespace attn

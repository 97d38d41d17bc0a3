// Paged-KV single-token decode for gfx950.
//
// The cache is a pool of 16-token blocks; logical position p of sequence s
// lives in block block_table[s][p / 16], slot p % 16 ("Kernels de atención
// rápida y fusión de operadores", section "Atención tipo FlashAttention y
// atención paginada").  Every key position is translated through the table.
//
// Work split.  The units of a call are the (sequence, kv head, block)
// triples, ordered by sequence, then kv head, then block.  A fixed number of
// waves W (4 independent waves per workgroup) each take one contiguous range
// of floor(U / W) or ceil(U / W) units, so every wave streams the same number
// of bytes whatever the mix of lengths, and no wave waits on another.  Each
// wave first sums the block counts of all sequences (a wave-wide scan of the
// lengths) to find where its range starts.  A wave's range crosses into at
// most a few (sequence, kv head) pairs; for each piece it runs the online
// softmax over its blocks and then either writes the final output (it
// covered the whole pair) or leaves an fp32 partial state (m, l, u) per
// query head in the workspace.  A second kernel merges the partial states of
// a pair in wave order (deterministic): M = max m_k, L = sum l_k e^(m_k - M),
// O = sum u_k e^(m_k - M) / L ("FlashAttention" notes, section "No basta con
// promediar los resultados de los bloques": each part enters with its own
// weight, not as an average).
//
// Inside a piece the wave keeps four register buffers of one block each
// (K and V, 8 KB at d = 128): the loads of the next three blocks are in
// flight while one block computes.  Every load goes through a buffer
// resource sized to the block's valid rows, so slots past the sequence's
// length and blocks with an out-of-range table entry read as zeros without
// a branch; scores of such slots are excluded before any arithmetic.  The G
// query heads that share the kv head (grouped-query attention) form the rows
// of the score tile, so both products run on MFMA:
//   * S^T = K Q^T (v_mfma_f32_16x16x32_bf16): lane (l16, grp) holds key l16's
//     dims D/4*grp .. D/4*grp + D/4 - 1 (one contiguous run per lane; Q uses
//     the same dim order), and gets back the scores of keys 4grp..4grp+3 for
//     query row l16.
//   * O^T += V^T P^T (v_mfma_f32_16x16x16_bf16, one tile per 16 output
//     dims): the P^T operand is exactly the lane's four scores; the V^T
//     operand wants 4 keys of one dim, so each lane loads D/16 consecutive
//     dims of keys 4grp..4grp+3 (4 whole rows per load instruction) and
//     packs key pairs with v_perm; tile j holds dims D/16*m + j.  The output
//     comes back as one query row per lane with D/4 consecutive dims, so the
//     rescale by e^(m - m') is lane-local.
//
// More than 16 query heads per kv head are split into equal groups of at
// most 16.  Up to 4 groups, the waves of one workgroup form a team that
// takes the kv head's units together, one group per wave, so that a block
// the first wave reads is in the CU's caches for the others; beyond 4, each
// group is a kv head of its own in the unit order.  Units are then dealt to
// teams (a lone wave is a team of one), and the partial states and records
// above are per (team, member).

#include <stdlib.h>

#include <atomic>

#include "common.h"
#include "internal.h"

namespace attn {
namespace {

constexpr int DS_THREADS = 256;   // 4 independent waves
constexpr int DS_NBUF = 4;        // one block computing, three in flight

template <int D>
struct VRow;
template <>
struct VRow<128> { typedef u32x4 T; };
template <>
struct VRow<64> { typedef u32x2 T; };

template <int D>
__device__ __forceinline__ typename VRow<D>::T buf_ld_vrow(__amdgpu_buffer_rsrc_t r, uint32_t off);
template <>
__device__ __forceinline__ u32x4 buf_ld_vrow<128>(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    return buf_ld16(r, off);
}
template <>
__device__ __forceinline__ u32x2 buf_ld_vrow<64>(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    return __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, 0));
}

// K operands and V row slices of one 16-token block.
template <int D>
struct KVBuf {
    u32x4 k[D / 32];
    typename VRow<D>::T v[4];
};

typedef short s16x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ int nblocks_of(int ctx, int cap) {
    ctx = ctx < 0 ? 0 : (ctx > cap ? cap : ctx);
    return (ctx + kDecodeBlock - 1) / kDecodeBlock;
}

__device__ __forceinline__ int wave_sum_i(int x) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) x += __shfl_xor(x, off, 64);
    return x;
}

__device__ __forceinline__ int wave_incl_scan(int x, int lane) {
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
        const int y = __shfl_up(x, d, 64);
        if (lane >= d) x += y;
    }
    return x;
}

// With U units dealt to W waves (or teams) as [floor(wU/W), floor((w+1)U/W)),
// the one that covers unit u.
__device__ __forceinline__ int wave_of_unit(long long u, long long U, int W) {
    return (int)(((u + 1) * (long long)W - 1) / U);
}

template <int D, int MODE>
__global__ void __launch_bounds__(DS_THREADS)
decode_split_kernel(const uint16_t* __restrict__ q, const uint16_t* __restrict__ kc,
                    const uint16_t* __restrict__ vc, const int32_t* __restrict__ table,
                    const int32_t* __restrict__ ctx_lens, int32_t* __restrict__ recs,
                    float* __restrict__ slots, uint16_t* __restrict__ o, float* __restrict__ lse,
                    int S, int Hq, int Hkv, int max_blocks, int num_blocks, float c, int negate) {
    // (sequence, virtual kv head) pairs: the G query heads of kv head gp in
    // NG groups of at most GV rows; virtual head v = gp * NG + group.  With
    // NL = NG <= 4 groups, the NL waves of a team (one workgroup) take the
    // same units of kv head gp, one group each, so that their reads of a
    // block meet in the CU's caches; otherwise (NL = 1) every virtual head
    // has units of its own.  HU: heads in the unit order.
    // MODE (compile time): 0 one group (G <= 16), 1 groups without teams,
    // 2 teams.
    const int G = Hq / Hkv, NG = MODE ? decode_groups(G) : 1, GV = MODE ? decode_group_rows(G) : G;
    const int HV = Hkv * NG, NL = MODE == 2 ? decode_team(G) : 1, HU = HV / NL;
    constexpr int KS = D / 32;     // MFMA k-steps over the head dim
    constexpr int DPL = D / 16;    // output tiles; V dims per lane per key
    constexpr int QW = D / 4;      // dims per lane group in the score product
    constexpr int NB = DS_NBUF, LA = DS_NBUF - 1;

    const int lane = threadIdx.x & 63, l16 = lane & 15, grp = lane >> 4;
    // team wt (4 / NL teams per workgroup), member jm; a wave past the last
    // team of its workgroup (NL = 3) has nothing to do
    const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int tpw = 4 / NL;
    if (wv >= tpw * NL) return;
    const int wt = blockIdx.x * tpw + wv / NL, jm = wv - (wv / NL) * NL;
    const int cap = max_blocks * kDecodeBlock;
    const int mlp = decode_ml_pad(GV);
    const size_t sf = decode_slot_floats(GV, D);

    // Total block count over the sequences.
    int n_first = 0, tot = 0;
    for (int s0 = 0; s0 < S; s0 += 64) {
        const int n = (s0 + lane < S) ? nblocks_of(ctx_lens[s0 + lane], cap) : 0;
        if (s0 == 0) n_first = n;
        tot += wave_sum_i(n);
    }
    tot = __builtin_amdgcn_readfirstlane(tot);
    // Units are dealt to W = min(teams launched, U) teams, so that every
    // team in [0, W) has at least one unit (the merge relies on it).
    const long long U = (long long)tot * HU;
    const int W = (int)min((long long)gridDim.x * tpw, U);
    if (wt >= W) return;
    const long long u0 = (long long)wt * U / W, u1 = (long long)(wt + 1) * U / W;

    // The sequence holding unit u0 (unit of (s, gu, b) = HU*P_s + gu*n_s + b,
    // P_s = blocks of the sequences before s).
    int s = 0, Ps = 0, ns = 0;
    {
        int P = 0;
        for (int s0 = 0; s0 < S; s0 += 64) {
            const int n = (s0 == 0) ? n_first : ((s0 + lane < S) ? nblocks_of(ctx_lens[s0 + lane], cap) : 0);
            const int incl = wave_incl_scan(n, lane);
            const long long lo = (long long)HU * (P + incl - n), hi = (long long)HU * (P + incl);
            const uint64_t hit = __builtin_amdgcn_ballot_w64(u0 >= lo && u0 < hi);
            if (hit) {
                const int j = (int)__builtin_ctzll(hit);
                const int nj = __builtin_amdgcn_readlane(n, j);
                s = s0 + j;
                Ps = P + __builtin_amdgcn_readlane(incl, j) - nj;
                ns = nj;
                break;
            }
            P += __builtin_amdgcn_readlane(incl, 63);
        }
    }

    const float nanv = __builtin_nanf("");
    long long u = u0;
    while (true) {
        // ---- one piece: blocks [b0, b1) of pair (s, g) ----
        const long long base = (long long)HU * Ps;
        const int r0 = (int)(u - base);
        const int gu = r0 / ns, b0 = r0 - gu * ns;     // gu: head of the unit order
        const long long pbeg = base + (long long)gu * ns, pend = pbeg + ns;
        const long long send = pend < u1 ? pend : u1;
        const int b1 = b0 + (int)(send - u), nb = b1 - b0;
        const int g = gu * NL + jm;                    // virtual kv head
        const int p = s * HV + g;
        const int gp = g / NG, grp_i = g - gp * NG;    // physical kv head, group
        const int gr = min(GV, G - grp_i * GV);        // query heads (rows) of this group
        const int h0 = gp * G + grp_i * GV;            // its first query head
        const int ctx_raw = ctx_lens[s];
        const int ctx = ctx_raw < 0 ? 0 : (ctx_raw > cap ? cap : ctx_raw);
        const bool ctx_bad = ctx_raw < 0 || ctx_raw > cap;

        // Q operand (B of S^T = K Q^T): query row l16 (head h0 + l16 when l16 < gr).
        bf16x8 qf[KS];
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            u32x4 wq = {0u, 0u, 0u, 0u};
            if (l16 < gr) wq = ld16(q + ((size_t)s * Hq + h0 + l16) * D + QW * grp + 8 * ks);
            if (negate) wq = neg_bf16x8(wq);
            qf[ks] = __builtin_bit_cast(bf16x8, wq);
        }

        // Per-lane byte offsets inside a block: K row l16, dims QW*grp..;
        // V rows 4grp..4grp+3, dims DPL*l16...
        const uint32_t ul = threadIdx.x & 63u;
        const uint32_t koff = (ul & 15u) * (uint32_t)(D * 2) + (ul >> 4) * (uint32_t)(QW * 2);
        const uint32_t voff = (ul >> 4) * (uint32_t)(4 * D * 2) + (ul & 15u) * (uint32_t)(DPL * 2);
        const int32_t* trow = table + (size_t)s * max_blocks + b0;
        bool bad = false;
        int tab = 0;     // table entries of the current chunk (lane j: block cb + j)

        auto issue = [&](KVBuf<D>& R, int i, int cb, int cn) {
            int bytes = 0;
            size_t off = 0;
            if (i < cn) {
                const int e = __builtin_amdgcn_readlane(tab, i);
                const bool ok = e >= 0 && e < num_blocks;
                bad = bad || !ok;
                const int nv = min(kDecodeBlock, ctx - kDecodeBlock * (b0 + cb + i));
                bytes = ok ? nv * D * 2 : 0;
                off = ((size_t)(ok ? e : 0) * Hkv + gp) * (size_t)(kDecodeBlock * D);
            }
            const __amdgpu_buffer_rsrc_t rk = make_rsrc(kc + off, (uint32_t)bytes);
            const __amdgpu_buffer_rsrc_t rv = make_rsrc(vc + off, (uint32_t)bytes);
            // opaque copies keep the constant parts in the instructions'
            // offset fields instead of hoisted per-load address registers
            uint32_t ko = koff, vo = voff;
            asm volatile("" : "+v"(ko), "+v"(vo));
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) R.k[ks] = buf_ld16(rk, ko + (uint32_t)(ks * 16));
#pragma unroll
            for (int rr = 0; rr < 4; ++rr) R.v[rr] = buf_ld_vrow<D>(rv, vo + (uint32_t)(rr * D * 2));
        };

        // Running state (m, l, u) of the online softmax for this piece.
        float m_run = kNegInf, l_run = 0.f;
        f32x4 oacc[DPL];
#pragma unroll
        for (int j = 0; j < DPL; ++j) oacc[j] = f32x4{0.f, 0.f, 0.f, 0.f};
        const int key0 = 4 * grp;

        auto compute = [&](KVBuf<D>& R, int i, int cb) {
            f32x4 sc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < KS; ++ks)
                sc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, R.k[ks]), qf[ks], sc, 0, 0, 0);
            // lane: query row l16, keys key0 + rr of the block
            const int nv = min(kDecodeBlock, ctx - kDecodeBlock * (b0 + cb + i));
            float mx = kNegInf;
            bool ok[4];
#pragma unroll
            for (int rr = 0; rr < 4; ++rr) {
                ok[rr] = key0 < nv - rr;
                mx = fmaxf(mx, ok[rr] ? sc[rr] : kNegInf);
            }
            mx = fmaxf(mx, xor_shfl(mx, 16));
            mx = fmaxf(mx, xor_shfl(mx, 32));
            const float m_new = fmaxf(m_run, mx);
            const float alpha = (m_run == kNegInf) ? 0.f : fast_exp2((m_run - m_new) * c);
            m_run = m_new;
            const float mc = (m_run == kNegInf) ? 0.f : m_run * c;
            float ps = 0.f;
            s16x4 pb;
#pragma unroll
            for (int rr = 0; rr < 4; ++rr) {
                const float pv = ok[rr] ? fast_exp2(fmaf(sc[rr], c, -mc)) : 0.f;
                ps += pv;
                pb[rr] = __builtin_bit_cast(short, (__bf16)pv);
            }
            l_run = fmaf(l_run, alpha, ps);
#pragma unroll
            for (int j = 0; j < DPL; ++j) {
                const int wd = j >> 1;
                const uint32_t sel = (j & 1) ? 0x07060302u : 0x05040100u;
                u32x2 a2;
                a2.x = __builtin_amdgcn_perm(R.v[1][wd], R.v[0][wd], sel);
                a2.y = __builtin_amdgcn_perm(R.v[3][wd], R.v[2][wd], sel);
                oacc[j] *= alpha;
                oacc[j] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(s16x4, a2), pb,
                                                                    oacc[j], 0, 0, 0);
            }
        };

        // Chunks of up to 64 blocks (one table entry per lane).  Within a
        // chunk: NB blocks per trip, each trip issuing the loads LA blocks
        // ahead (past the chunk they are empty); then the last < NB blocks,
        // whose loads are in flight already.
        KVBuf<D> bufs[NB];
#pragma unroll 1
        for (int cb = 0; cb < nb; cb += 64) {
            const int cn = min(64, nb - cb);
            tab = (lane < cn) ? trow[cb + lane] : 0;
#pragma unroll
            for (int k = 0; k < LA; ++k) issue(bufs[k], k, cb, cn);
            int i = 0;
#pragma unroll 1
            for (; i + NB <= cn; i += NB) {
#pragma unroll
                for (int k = 0; k < NB; ++k) {
                    issue(bufs[(k + LA) % NB], i + k + LA, cb, cn);
                    __builtin_amdgcn_sched_barrier(0);
                    compute(bufs[k], i + k, cb);
                    __builtin_amdgcn_sched_barrier(0);
                }
            }
#pragma unroll
            for (int k = 0; k < LA; ++k)
                if (i + k < cn) compute(bufs[k], i + k, cb);
        }

        // ---- write the piece ----
        l_run += xor_shfl(l_run, 16);
        l_run += xor_shfl(l_run, 32);
        if (b0 == 0 && lane == 0) {
            recs[2 * p] = wt;                                  // first team of the pair
            recs[2 * p + 1] = wave_of_unit(pend - 1, U, W);    // last team of the pair
        }
        if (b0 == 0 && b1 == ns) {
            // the whole pair: final output
            const bool nan_out = bad || ctx_bad;
            const float inv = nan_out ? nanv : 1.f / l_run;
            if (l16 < gr) {
                uint16_t* orow = o + ((size_t)s * Hq + h0 + l16) * D + QW * grp;
#pragma unroll
                for (int rr = 0; rr < 4; ++rr) {
                    if constexpr (DPL == 8) {
                        u32x4 pk;
                        pk.x = pack_bf16x2(oacc[0][rr] * inv, oacc[1][rr] * inv);
                        pk.y = pack_bf16x2(oacc[2][rr] * inv, oacc[3][rr] * inv);
                        pk.z = pack_bf16x2(oacc[4][rr] * inv, oacc[5][rr] * inv);
                        pk.w = pack_bf16x2(oacc[6][rr] * inv, oacc[7][rr] * inv);
                        st16(orow + DPL * rr, pk);
                    } else {
                        u32x2 pk;
                        pk.x = pack_bf16x2(oacc[0][rr] * inv, oacc[1][rr] * inv);
                        pk.y = pack_bf16x2(oacc[2][rr] * inv, oacc[3][rr] * inv);
                        *reinterpret_cast<u32x2*>(orow + DPL * rr) = pk;
                    }
                }
                if (lse != nullptr && grp == 0)
                    lse[(size_t)s * Hq + h0 + l16] = nan_out ? nanv : (m_run * c + log2f(l_run)) * kLn2;
            }
        } else {
            // slot of (team, unit pair, member): teams visit the unit pairs
            // in increasing order, so wt + (s * HU + gu) is unique per piece
            float* slot = slots + ((size_t)(wt + s * HU + gu) * NL + jm) * sf;
            if (l16 < gr) {
                if (grp == 0) {
                    slot[l16] = m_run;
                    slot[GV + l16] = bad ? nanv : l_run;
                }
                float* ud = slot + mlp + (size_t)l16 * D + QW * grp;
#pragma unroll
                for (int rr = 0; rr < 4; ++rr)
#pragma unroll
                    for (int j4 = 0; j4 < DPL; j4 += 4)
                        *reinterpret_cast<f32x4*>(ud + DPL * rr + j4) =
                            f32x4{oacc[j4][rr], oacc[j4 + 1][rr], oacc[j4 + 2][rr], oacc[j4 + 3][rr]};
            }
        }

        // ---- next piece ----
        u = send;
        if (u >= u1) break;
        if (gu + 1 == HU) {
            Ps += ns;
            do {
                ++s;
                ns = nblocks_of(ctx_lens[s], cap);
            } while (ns == 0);
        }
    }
}

// Merge: one wave per (pair, 64 (row, 4-dim) elements).  Each lane walks
// the partial states that the teams wf..wl left for the pair, in team order
// (deterministic), sixteen at a time with all their loads issued together,
// and keeps a running merged state: when a part's m exceeds the running
// maximum the running l and u are rescaled first, so every part enters with
// the weight e^(m_k - M).  Pairs covered by one team were finished by it;
// empty sequences give o = 0 and lse = -inf (NaN for a length outside
// [0, max_blocks * 16]).
template <int D, int MODE>
__global__ void __launch_bounds__(64)
decode_merge_kernel(const int32_t* __restrict__ recs, const float* __restrict__ slots,
                    const int32_t* __restrict__ ctx_lens, uint16_t* __restrict__ o,
                    float* __restrict__ lse, int Hq, int Hkv, int max_blocks, float c) {
    constexpr int NQ = D / 4;     // 4-dim groups per row
    constexpr int BATCH = 16;
    const int p = blockIdx.x, lane = threadIdx.x;
    // pair p = (sequence, virtual kv head), as in the split kernel; its
    // pieces were left by teams wf..wl, member jm, in the slots of unit pair
    // pu = s * HU + gu
    const int G = Hq / Hkv, NG = MODE ? decode_groups(G) : 1, GV = MODE ? decode_group_rows(G) : G;
    const int HV = Hkv * NG, NL = MODE == 2 ? decode_team(G) : 1, HU = HV / NL;
    const int s = p / HV, g = p - s * HV;
    const int gp = g / NG, grp_i = g - gp * NG;
    const int gr = min(GV, G - grp_i * GV), h0 = gp * G + grp_i * GV;
    const int gu = g / NL, jm = g - gu * NL;
    const int e = blockIdx.y * 64 + lane;          // element: row e / NQ, dims 4*(e % NQ)..
    const int row = e / NQ, d4 = e - row * NQ;
    const bool act = row < gr;
    const int cap = max_blocks * kDecodeBlock;
    // the record is read before the length check so both loads are in flight together
    const int wf = recs[2 * p], wl = recs[2 * p + 1];
    const int ctx_raw = ctx_lens[s];
    const bool bad = ctx_raw < 0 || ctx_raw > cap;
    const float nanv = __builtin_nanf("");
    uint16_t* orow = o + ((size_t)s * Hq + h0 + row) * D + 4 * d4;
    float* lse_out = (lse != nullptr && act && d4 == 0) ? lse + (size_t)s * Hq + h0 + row : nullptr;
    if (nblocks_of(ctx_raw, cap) == 0) {
        if (act) {
            const uint32_t z = bad ? 0x7fc07fc0u : 0u;
            *reinterpret_cast<u32x2*>(orow) = u32x2{z, z};
        }
        if (lse_out) *lse_out = bad ? nanv : kNegInf;
        return;
    }
    if (wf == wl || !act) return;
    const int nk = wl - wf + 1;
    const size_t sf = decode_slot_floats(GV, D);
    const int mlp = decode_ml_pad(GV);
    const float* s0 = slots + ((size_t)(wf + s * HU + gu) * NL + jm) * sf;
    const size_t sstep = (size_t)NL * sf;     // the next team's slot of the pair

    float M = kNegInf, L = 0.f;
    f32x4 U = {0.f, 0.f, 0.f, 0.f};
    for (int k0 = 0; k0 < nk; k0 += BATCH) {
        float mk[BATCH], lk[BATCH];
        f32x4 uk[BATCH];
#pragma unroll
        for (int j = 0; j < BATCH; ++j) {
            const int k = min(k0 + j, nk - 1);
            const float* sl = s0 + (size_t)k * sstep;
            mk[j] = sl[row];
            lk[j] = sl[GV + row];
            uk[j] = *reinterpret_cast<const f32x4*>(sl + mlp + (size_t)row * D + 4 * d4);
        }
#pragma unroll
        for (int j = 0; j < BATCH; ++j) {
            if (k0 + j < nk && mk[j] > M) {
                const float r = (M == kNegInf) ? 0.f : fast_exp2((M - mk[j]) * c);
                L *= r;
                U *= r;
                M = mk[j];
            }
            const float f = (k0 + j >= nk || mk[j] == kNegInf) ? 0.f : fast_exp2((mk[j] - M) * c);
            L = fmaf(f, lk[j], L);
            U += f * uk[j];
        }
    }
    const float inv = bad ? nanv : (L > 0.f ? 1.f / L : (L == 0.f ? 0.f : nanv));
    u32x2 pk;
    pk.x = pack_bf16x2(U.x * inv, U.y * inv);
    pk.y = pack_bf16x2(U.z * inv, U.w * inv);
    *reinterpret_cast<u32x2*>(orow) = pk;
    if (lse_out) {
        float lv = (M == kNegInf) ? kNegInf : (M * c + log2f(L)) * kLn2;
        if (bad || L != L) lv = nanv;
        *lse_out = lv;
    }
}

template <int D, int MODE>
hipError_t launch_decode_t(const DecodeArgs& a, hipStream_t stream) {
    // ATTN_DECODE_WAVES (4..2048, a multiple of 4) sets the wave count, so
    // that tests can reach long pieces, many pieces per wave and wide merges
    // with small inputs.
    int waves = kDecodeWavesDefault;
    if (const char* env = getenv("ATTN_DECODE_WAVES")) {
        const int v = atoi(env);
        if (v >= 4 && v <= kDecodeWaves) waves = v / 4 * 4;
    }
    // virtual kv heads, waves per team, teams per workgroup
    const int G = a.Hq / a.Hkv, HV = a.Hkv * decode_groups(G), NL = MODE == 2 ? decode_team(G) : 1, tpw = 4 / NL;
    const long long units_max = (long long)a.S * (HV / NL) * a.max_blocks;
    if (units_max < (long long)(waves / 4) * tpw) waves = (int)((units_max + tpw - 1) / tpw * 4);
    int32_t* recs = reinterpret_cast<int32_t*>(a.workspace);
    float* slots = reinterpret_cast<float*>(reinterpret_cast<char*>(a.workspace) + decode_rec_bytes(a.S, HV));
    hipLaunchKernelGGL((decode_split_kernel<D, MODE>), dim3((unsigned)(waves / 4)), dim3(DS_THREADS), 0, stream,
                       static_cast<const uint16_t*>(a.q), static_cast<const uint16_t*>(a.k_cache),
                       static_cast<const uint16_t*>(a.v_cache), a.block_table, a.ctx_lens, recs, slots,
                       static_cast<uint16_t*>(a.o), a.lse, a.S, a.Hq, a.Hkv, a.max_blocks, a.num_blocks,
                       a.c, a.negate);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int elems = decode_group_rows(G) * (D / 4);
    const dim3 g2((unsigned)(a.S * HV), (unsigned)((elems + 63) / 64));
    hipLaunchKernelGGL((decode_merge_kernel<D, MODE>), g2, dim3(64), 0, stream, recs, slots, a.ctx_lens,
                       static_cast<uint16_t*>(a.o), a.lse, a.Hq, a.Hkv, a.max_blocks, a.c);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_paged_decode_bf16(const DecodeArgs& a, hipStream_t stream) {
    // one build per grouping (one group; groups without teams; teams), so
    // that each carries only its own index arithmetic
    const int G = a.Hq / a.Hkv;
    const int mode = decode_groups(G) == 1 ? 0 : (decode_team(G) > 1 ? 2 : 1);
    if (a.d == 128)
        return mode == 0 ? launch_decode_t<128, 0>(a, stream)
                         : (mode == 1 ? launch_decode_t<128, 1>(a, stream) : launch_decode_t<128, 2>(a, stream));
    return mode == 0 ? launch_decode_t<64, 0>(a, stream)
                     : (mode == 1 ? launch_decode_t<64, 1>(a, stream) : launch_decode_t<64, 2>(a, stream));
}

// The partial states of attn_paged_decode_noalloc: a device array owned by
// the library, one copy per GPU (each device's code object holds its own),
// alive until the process ends.  Host code never passes `scratch` itself to
// a kernel (in host code the name stands for a host-side shadow): each
// device's address is looked up once, with that device current, and kept.
// Nothing in it has to start at zero: every slot a merge reads was written
// by the same call's split kernel.
static __device__ __align__(256) unsigned char scratch[kDecodeScratchBytes];

namespace {
constexpr int kScratchDevices = 64;
std::atomic<void*> g_scratch_ptr[kScratchDevices];
}  // namespace

hipError_t launch_paged_decode_bf16_noalloc(DecodeArgs a, hipStream_t stream) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kScratchDevices) return hipErrorInvalidDevice;
    void* ptr = g_scratch_ptr[dev].load(std::memory_order_acquire);
    if (ptr == nullptr) {
        e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        if (ptr == nullptr) return hipErrorInvalidSymbol;
        g_scratch_ptr[dev].store(ptr, std::memory_order_release);
    }
    a.workspace = static_cast<float*>(ptr);
    return launch_paged_decode_bf16(a, stream);
}

}  // namespace attn

// Chunked prefill over a paged KV cache, bf16 in / bf16 out, fp32
// accumulation, for gfx950.
//
// The new query rows of several sequences arrive packed ([T, Hq, d]); the
// rows of sequence s are starts[s] .. starts[s+1]-1, and since their keys and
// values are already in the cache, its t-th new row sits at position
// ctx_lens[s] - n_s + t and attends to every cached position up to its own
// (causal, diagonal included).  Positions are translated through the block
// table into the pool of 16-token blocks ("Kernels de atención rápida y
// fusión de operadores", section "Atención tipo FlashAttention y atención
// paginada").  One 16-token block per wave per key tile keeps each load's
// physical block uniform across the wave, so both K and V go through one
// buffer resource per wave and tile, sized to the block's valid rows: slots
// past the sequence's length, and blocks whose table entry is outside the
// pool, read as zeros with no branch.
//
// Everything else is the dense kernel's tile recurrence (prefill_tile.h):
// 4 waves x 32 query rows per workgroup, 64-key tiles double-buffered in
// LDS, K and V loaded straight into LDS, MFMA 32x32x16 bf16
// on S^T = K Q^T and O^T += V^T P^T, lazy rescale of the running maximum.
// The work is cut into items: a run of up to cq consecutive query tiles of
// one sequence (a chunk) for one kv head, i.e. cq x G workgroups, one per
// (query tile, query head) of the chunk.  All workgroups of an item run on
// one XCD, side by side, so they read the chunk's keys and values from that
// XCD's L2 instead of each fetching them from HBM.  Sequence lengths vary
// widely, so the chunks run longest first: every workgroup ranks them by the
// keys their query tiles see, read from the device-resident lengths (up to
// 512 chunks; beyond that, later chunks first), and the ranked items are
// dealt to the 8 XCDs in a serpentine order, so each XCD gets a like share.
// The launch picks cq so that every XCD still gets at least 8 items and one
// item fits on an XCD at once.
//
// Device-resident values are checked before they form an address: a
// sequence with malformed row offsets (or more than max_new rows) is left
// unwritten; one whose length is below its row count or beyond the table
// gets NaN rows; a row that attends to a block with an out-of-range table
// entry gets NaN.

#include <algorithm>
#include <cstdlib>

#include "internal.h"
#include "prefill_tile.h"

namespace attn {
namespace {

// Up to this many chunks, every workgroup ranks them by cost to run the
// longest first (P^2 / 256 comparisons per thread).
constexpr int kRankPairs = 512;
// An item (cq x G workgroups) fits on one XCD: 32 CUs x 2 workgroups.
constexpr int kItemUnits = 64;
constexpr uint32_t kNaNBf16x2 = 0x7FC07FC0u;   // two quiet bf16 NaNs
constexpr uint32_t kNaN32 = 0x7FC00000u;       // quiet fp32 NaN

template <int D>
__global__ void __launch_bounds__(PF_THREADS) __attribute__((amdgpu_waves_per_eu(2, 2)))
prefill_paged_kernel(const uint16_t* __restrict__ q, const uint16_t* __restrict__ kc,
                     const uint16_t* __restrict__ vc, const int32_t* __restrict__ table,
                     const int32_t* __restrict__ ctx_lens, const int32_t* __restrict__ starts,
                     uint16_t* __restrict__ o, float* __restrict__ lse, int S, int T, int max_new,
                     int Hq, int Hkv, int max_blocks, int num_blocks, int n_qtiles, int cq,
                     float c, int negate) {
    using L = PfLayout<D>;
    constexpr int BS = kDecodeBlock;
    static_assert(PF_BN == PF_WAVES * BS, "one cache block per wave per key tile");
    __shared__ __attribute__((aligned(16))) uint16_t smem0[L::BUF];
    __shared__ __attribute__((aligned(16))) uint16_t smem1[L::BUF];
    __shared__ int bad_s[PF_WAVES];
    __shared__ long long rank_cost[kRankPairs];
    __shared__ int rank_pick;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int hi = lane >> 5, l32 = lane & 31;

    // Workgroup b runs on XCD b % 8.  The k-th item of XCD x is item slot
    // 8k + x (k even) or 8k + 7 - x (k odd); slot = rank * Hkv + kv head, rank
    // in the longest-first order of the chunks.  Within an item, later query
    // tiles first, the G query heads of the kv head side by side.
    const int G = Hq / Hkv;
    const int U = cq * G;                                     // workgroups per item
    const int n_ch = (n_qtiles + cq - 1) / cq;                // chunks per sequence
    const int P = n_ch * S;                                   // chunks
    const int xcd = blockIdx.x & (kXcds - 1), jx = blockIdx.x / kXcds;
    const int k = jx / U, e = jx - k * U;
    const int slot = k * kXcds + ((k & 1) ? kXcds - 1 - xcd : xcd);
    if (slot >= P * Hkv) return;
    const int rank = slot / Hkv, g = slot - rank * Hkv;
    const int h = g * G + e % G;
    int ch, s;
    if (P <= kRankPairs) {
        // Longest first: the chunk of rank `rank` in decreasing order of the
        // keys its query tiles see (ties by chunk index), from the lengths.
        for (int i = tid; i < P; i += PF_THREADS) {
            const int ci_ = i / S, si = i - ci_ * S;
            const int ai = starts[si], bi = starts[si + 1], li = ctx_lens[si];
            const int ni = bi - ai;
            const bool runs = !(ai < 0 || bi > T || ni < 0 || ni > max_new) && ci_ * cq * PF_BM < ni;
            const bool sane = li >= ni && li <= max_blocks * kDecodeBlock;
            long long cost = -1;
            if (runs) {
                cost = 0;
                const int t_end = min(ci_ * cq + cq, (ni + PF_BM - 1) / PF_BM);
                if (sane)
                    for (int t = ci_ * cq; t < t_end; ++t) cost += li - ni + min(t * PF_BM + PF_BM, ni);
            }
            rank_cost[i] = cost;
        }
        __syncthreads();
        for (int i = tid; i < P; i += PF_THREADS) {
            const long long ci = rank_cost[i];
            int r = 0;
            for (int j = 0; j < P; ++j) {
                const long long cj = rank_cost[j];
                r += (cj > ci || (cj == ci && j < i)) ? 1 : 0;
            }
            if (r == rank) rank_pick = i;
        }
        __syncthreads();
        ch = rank_pick / S;
        s = rank_pick - ch * S;
    } else {
        ch = n_ch - 1 - rank / S;                             // later chunks first
        s = rank - (rank / S) * S;
    }
    const int qt = ch * cq + cq - 1 - e / G;                  // later q tiles first

    const int a = starts[s], b = starts[s + 1], ctx = ctx_lens[s];
    const int n = b - a;
    if (a < 0 || b > T || n < 0 || n > max_new) return;     // not this call's rows
    const int q0 = qt * PF_BM;
    if (q0 >= n) return;
    const int row_end = min(q0 + PF_BM, n);
    const int wrow0 = q0 + wave * 32;
    const int myrow = wrow0 + l32;                            // row within the sequence
    const size_t orow = ((size_t)(a + myrow) * Hq + h);       // row index into o / lse

    if (ctx < n || ctx > max_blocks * BS) {                   // impossible length: NaN rows
        if (hi == 0 && myrow < row_end) {
            const u32x4 nan4 = {kNaNBf16x2, kNaNBf16x2, kNaNBf16x2, kNaNBf16x2};
#pragma unroll
            for (int c8 = 0; c8 < D / 8; ++c8) st16(o + orow * D + c8 * 8, nan4);
            if (lse != nullptr) reinterpret_cast<uint32_t*>(lse)[orow] = kNaN32;
        }
        return;
    }
    const int first = ctx - n;                                // position of row 0
    const bool wave_active = wrow0 < n;

    // Q rows myrow (zero past n), dims 16*ks + 8*hi .. +7.
    const uint32_t qstride = (uint32_t)Hq * D * 2;            // bytes between rows
    const __amdgpu_buffer_rsrc_t qrs =
        make_rsrc(q + ((size_t)a * Hq + h) * D, (uint32_t)(n - 1) * qstride + D * 2);
    bf16x8 qf[D / 16];
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks) {
        u32x4 w = buf_ld16(qrs, (uint32_t)myrow * qstride + (uint32_t)(ks * 16 + hi * 8) * 2);
        if (negate) w = neg_bf16x8(w);
        qf[ks] = __builtin_bit_cast(bf16x8, w);
    }

    // Keys 0 .. first + row_end - 1 are needed.
    const int n_kt = (first + row_end - 1) / PF_BN + 1;

    // This wave stages cache block kt*4 + wave of every tile: chunk p =
    // (wave * KINST + i) * 64 + lane of the K and of the V tile (row p / CPR,
    // a row of this block), straight to LDS with each tile's swizzle.
    uint32_t koff[L::KINST], voff[L::KINST];
#pragma unroll
    for (int i = 0; i < L::KINST; ++i) {
        const int p = (wave * L::KINST + i) * 64 + lane;
        const int r = p / L::CPR;
        koff[i] = (uint32_t)((r - wave * BS) * D + ((p % L::CPR) ^ kswz<L::CPR>(r)) * 8) * 2;
        voff[i] = (uint32_t)((r - wave * BS) * D + ((p % L::CPR) ^ vswz<L::CPR>(r)) * 8) * 2;
    }
    const size_t head_elems = (size_t)BS * D;                 // one (block, kv head) tile
    const int32_t* trow = table + (size_t)s * max_blocks;
    int bad = 0x7fffffff;                                     // lowest block with a bad entry

    auto issue_loads = [&](int kt, uint16_t* Ks) {
        const int blk = kt * PF_WAVES + wave;
        const int valid = min(max(ctx - blk * BS, 0), BS);    // rows of this block in the sequence
        int phys = 0;
        bool ok = valid > 0;
        if (ok) {
            phys = trow[blk];
            if (phys < 0 || phys >= num_blocks) {
                bad = min(bad, blk);
                phys = 0;
                ok = false;
            }
        }
        const size_t base = ((size_t)phys * Hkv + g) * head_elems;
        // (wave-uniform; readfirstlane keeps the resource in scalar registers)
        const uint32_t bytes = __builtin_amdgcn_readfirstlane(ok ? (uint32_t)valid * D * 2 : 0u);
        const __amdgpu_buffer_rsrc_t krs = make_rsrc(kc + base, bytes);
        const __amdgpu_buffer_rsrc_t vrs = make_rsrc(vc + base, bytes);
        uint16_t* Vs = Ks + L::KELEMS;
#pragma unroll
        for (int i = 0; i < L::KINST; ++i)
            buf_ld16_lds(krs, Ks + (wave * L::KINST + i) * 64 * 8, koff[i]);
#pragma unroll
        for (int i = 0; i < L::KINST; ++i)
            buf_ld16_lds(vrs, Vs + (wave * L::KINST + i) * 64 * 8, voff[i]);
    };

    f32x16 oacc[D / 32];
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[db][r] = 0.f;
    float m_run = kNegInf, l_run = 0.f;
    const int mypos = first + myrow;
    const int wpos0 = first + wrow0;

    issue_loads(0, smem0);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();

    // One key tile from `cur` while the next loads into `nxt` (separate LDS
    // arrays, loop unrolled by two, so the compiler sees they do not alias).
    auto step = [&](int kt, const uint16_t* cur, uint16_t* nxt) {
        const bool more = kt + 1 < n_kt;
        if (more) issue_loads(kt + 1, nxt);
        const int k0 = kt * PF_BN;
        if (wave_active && k0 <= wpos0 + 31) {
            const bool need_mask = k0 + PF_BN - 1 > wpos0;
            pf_tile_step<D, true>(cur, cur + L::KELEMS, qf, oacc, m_run, l_run, k0, ctx, mypos,
                                  need_mask, c, hi, l32);
        }
        if (more) __builtin_amdgcn_s_waitcnt(0);     // tile kt+1 in LDS
        __syncthreads();
    };
    for (int kt = 0; kt < n_kt; kt += 2) {
        step(kt, smem0, smem1);
        if (kt + 1 < n_kt) step(kt + 1, smem1, smem0);
    }

    // Lowest bad block seen by any wave of the workgroup.
    if (lane == 0) bad_s[wave] = bad;
    __syncthreads();
    int bad_all = bad_s[0];
#pragma unroll
    for (int w = 1; w < PF_WAVES; ++w) bad_all = min(bad_all, bad_s[w]);

    // Epilogue: o = u / l, lse = m + ln l (natural log); NaN for a row that
    // attends to a block with a bad table entry.
    const float l_tot = l_run + xor_shfl(l_run, 32);
    if (myrow < row_end) {
        // (NaN is written as a bit pattern: the arithmetic is compiled on
        // the assumption that it never meets a NaN)
        const bool poisoned = bad_all != 0x7fffffff && bad_all * BS <= mypos;
        const float inv = (l_tot > 0.f) ? 1.f / l_tot : 0.f;
        uint16_t* op = o + orow * D;
#pragma unroll
        for (int db = 0; db < D / 32; ++db)
#pragma unroll
            for (int rg = 0; rg < 4; ++rg) {
                const int dim0 = db * 32 + rg * 8 + hi * 4;
                u32x2 w = {pack_bf16x2(oacc[db][rg * 4 + 0] * inv, oacc[db][rg * 4 + 1] * inv),
                           pack_bf16x2(oacc[db][rg * 4 + 2] * inv, oacc[db][rg * 4 + 3] * inv)};
                if (poisoned) w = u32x2{kNaNBf16x2, kNaNBf16x2};
                *reinterpret_cast<u32x2*>(op + dim0) = w;
            }
        if (lse != nullptr && hi == 0) {
            const float lv = (m_run * c + log2f(l_tot)) * kLn2;
            reinterpret_cast<uint32_t*>(lse)[orow] = poisoned ? kNaN32 : __builtin_bit_cast(uint32_t, lv);
        }
    }
}

template <int D>
hipError_t launch_paged_prefill_t(const PagedPrefillArgs& a, hipStream_t stream) {
    const int n_qt = (a.max_new + PF_BM - 1) / PF_BM;
    const int G = a.Hq / a.Hkv;
    // Query tiles per item: as many as fit on one XCD (kItemUnits
    // workgroups), while the items still number at least 8 per XCD.
    // ATTN_PAGED_CQ=<n> (test hook) forces another cut, which must give the
    // same result bit for bit.
    int cq = std::max(1, std::min(n_qt, kItemUnits / G));
    while (cq > 1 && (long long)a.S * ((n_qt + cq - 1) / cq) * a.Hkv < 8LL * kXcds) --cq;
    if (const char* env = getenv("ATTN_PAGED_CQ")) {
        const int f = atoi(env);
        if (f >= 1 && f <= std::max(n_qt, 1)) cq = f;
    }
    auto grid_of = [&](int q) {
        const long long slots = (long long)((n_qt + q - 1) / q) * a.S * a.Hkv;
        return (slots + kXcds - 1) / kXcds * kXcds * q * G;
    };
    // (one tile per item always fits: the entry point bounds n_qt * S * Hq)
    if (grid_of(cq) >= (1LL << 31)) cq = 1;
    const long long ngrid = grid_of(cq);
    const dim3 grid((unsigned)ngrid), block(PF_THREADS);
    hipLaunchKernelGGL((prefill_paged_kernel<D>), grid, block, 0, stream,
                       static_cast<const uint16_t*>(a.q), static_cast<const uint16_t*>(a.k_cache),
                       static_cast<const uint16_t*>(a.v_cache), a.block_table, a.ctx_lens, a.starts,
                       static_cast<uint16_t*>(a.o), a.lse, a.S, a.T, a.max_new, a.Hq, a.Hkv,
                       a.max_blocks, a.num_blocks, n_qt, cq, a.c, a.negate);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_paged_prefill_bf16(const PagedPrefillArgs& a, hipStream_t stream) {
    return a.d == 128 ? launch_paged_prefill_t<128>(a, stream) : launch_paged_prefill_t<64>(a, stream);
}

}  // namespace attn

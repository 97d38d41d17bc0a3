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
//     before a tile skips its arithmetic for it.  In the pipelined kernel
//     the units that read one kv head stay on a subset of the XCDs
//     (causal_unit), which halves the K/V fetched past the L2s.
//   * Non-causal: the q tiles that read one kv head run as consecutive
//     workgroups of one XCD, so its K/V tiles come from HBM once and from
//     that XCD's L2 after.
//
// Two kernels share this layout: prefill_bf16_kernel runs each key tile's
// phases in order (tile step in prefill_tile.h); prefill_sp_kernel, used for
// causal d = 128, software-pipelines them inside each wave (see its comment).

#include <stdlib.h>

#include <type_traits>

#include "internal.h"
#include "prefill_tile.h"

namespace attn {
namespace {

// Waves per SIMD of prefill_bf16_kernel: 4 for d = 64 on 32-key tiles
// (state in 128 registers: one wave alone issues vector instructions at
// about half the SIMD's rate, so the softmax-heavy d = 64 loop gains from
// more resident waves), 2 elsewhere (256 registers).
template <int D, int BN>
constexpr int pf_waves_per_eu() {
    return (D == 64 && BN == 32) ? 4 : 2;
}

template <int D, bool CAUSAL, int BN>
__global__ void __launch_bounds__(PF_THREADS)
    __attribute__((amdgpu_waves_per_eu(pf_waves_per_eu<D, BN>(), pf_waves_per_eu<D, BN>())))
prefill_bf16_kernel(const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
                    const uint16_t* __restrict__ v, uint16_t* __restrict__ o,
                    float* __restrict__ lse, int Hq, int Hkv, int N, int BH, int n_qtiles,
                    float c, int negate, int xcd_runs) {
    using L = PfLayout<D, BN>;
    __shared__ __attribute__((aligned(16))) uint16_t smem0[L::BUF];
    __shared__ __attribute__((aligned(16))) uint16_t smem1[L::BUF];

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int hi = lane >> 5, l32 = lane & 31;

    // Work unit: (b, h, q tile); heaviest q tiles first when causal.
    const int wg = blockIdx.x;
    int qt, bh;
    if (!CAUSAL && xcd_runs) {
        // Workgroup w runs on XCD w % 8.  A run is the G * n_qtiles units
        // that read one kv head's K and V; run r goes to XCD r % 8, and the
        // j-th workgroup of XCD x takes unit j % (run length) of run
        // (j / run length) * 8 + x, so a run's units follow each other on
        // one XCD and the K/V tiles they share stay in its L2.  The grid is
        // padded to whole rounds of 8 runs; padding workgroups exit here.
        const int G = Hq / Hkv, R = G * n_qtiles;
        const int x = wg & 7, j = wg >> 3;
        const int r = (j / R) * 8 + x;
        if (r >= BH / G) return;
        const int i = j - (j / R) * R;
        qt = i / G;
        bh = r * G + (i - qt * G);
    } else {
        qt = CAUSAL ? (n_qtiles - 1 - wg / BH) : (wg / BH);
        bh = wg % BH;
    }
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
    const int n_kt = CAUSAL ? (row_end + BN - 1) / BN : (N + BN - 1) / BN;

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
        const uint32_t t0 = (uint32_t)kt * BN * D * 2;
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
        const int k0 = kt * BN;
        const bool compute = wave_active && (!CAUSAL || k0 <= wrow0 + 31);
        if (compute) {
            const bool need_mask = (k0 + BN > N) || (CAUSAL && k0 + BN - 1 > wrow0);
            pf_tile_step<D, CAUSAL, BN>(cur, cur + L::KELEMS, qf, oacc, m_run, l_run, k0, N, myrow,
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

// One step of the short-sequence kernel: a wave's 32 query rows against the
// NBLK 32-key blocks of keys GK0 .. GK0 + 32 NBLK - 1, staged from row 0 of
// Ks / Vs (d = 64), with the same online-softmax recurrence and MFMA layout
// as pf_tile_step but up to 64 keys per step and every LDS read a per-lane
// base plus an immediate.  Key `key` is allowed iff key < kend and (when
// CAUSAL) key <= mypos; need_mask must be true when some key of the step
// fails that for some row of the wave.  Only the first nvb 16-key blocks of
// V are staged (the rest lie past kend: weights 0, never read).
template <bool CAUSAL, int GK0, int NBLK>
__device__ __forceinline__ void sh_step(const uint16_t* Ks, const uint16_t* Vs, const int (&kofs)[4],
                                        const int (&vofs)[2], const bf16x8 (&qf)[4], f32x16 (&oacc)[2],
                                        float& m_run, float& l_run, int kend, int mypos, bool need_mask, int nvb,
                                        float c, int hi) {
    constexpr int D = 64;
    f32x16 sacc[NBLK];
#pragma unroll
    for (int kb = 0; kb < NBLK; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) sacc[kb][r] = 0.f;
    // S^T = K Q^T, block by block (K operands one MFMA ahead)
    bf16x8 ka[2];
    auto kread = [&](int i) {   // i = kb * 4 + ks
        return *reinterpret_cast<const bf16x8*>(Ks + kofs[i & 3] + (i >> 2) * 32 * D);
    };
    ka[0] = kread(0);
#pragma unroll
    for (int i = 0; i < NBLK * 4; ++i) {
        if (i + 1 < NBLK * 4) ka[(i + 1) & 1] = kread(i + 1);
        sacc[i >> 2] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka[i & 1], qf[i & 3], sacc[i >> 2], 0, 0, 0);
    }

    // row maximum (lane key of entry r in block kb: GK0 + 32 kb + 8 (r / 4) + 4 hi + r % 4)
    float mx = kNegInf;
    if (need_mask) {
        // allowed iff 32 kb + 8 (r / 4) + r % 4 <= lim; lim passes through an
        // empty asm so the compiler does not hoist the per-entry compares of
        // every step out of the row loop (they would fill the scalar
        // registers and spill)
        int lim = kend - 1 - (GK0 + 4 * hi);
        if (CAUSAL) lim = min(lim, mypos - (GK0 + 4 * hi));
        asm("" : "+v"(lim));
#pragma unroll
        for (int kb = 0; kb < NBLK; ++kb)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const bool ok = kb * 32 + 8 * (r >> 2) + (r & 3) <= lim;
                sacc[kb][r] = ok ? sacc[kb][r] : kNegInf;
                mx = fmaxf(mx, sacc[kb][r]);
            }
    } else {
#pragma unroll
        for (int kb = 0; kb < NBLK; ++kb)
#pragma unroll
            for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sacc[kb][r]);
    }
    mx = max_halves(mx);

    // lazy rescale, as in pf_tile_step
    const bool grow = (m_run == kNegInf) ? (mx != kNegInf) : ((mx - m_run) * c > kLazyLog2);
    if (__builtin_amdgcn_ballot_w64(grow) != 0) {
        const float m_new = grow ? mx : m_run;
        const float alpha = (m_run == kNegInf) ? 0.f : fast_exp2((m_run - m_new) * c);
        l_run *= alpha;
#pragma unroll
        for (int db = 0; db < 2; ++db)
#pragma unroll
            for (int r = 0; r < 16; ++r) oacc[db][r] *= alpha;
        m_run = m_new;
    }
    const float mc = (m_run == kNegInf) ? 0.f : m_run * c;

    // P = 2^(c s - c m) in bf16, row sum, and O^T += V^T P^T per 16 keys
    float lsum = 0.f;
    bf16x8 va[2][2];
    auto vread = [&](int c16, bf16x8* dst) {
#pragma unroll
        for (int db = 0; db < 2; ++db) {
            const uint16_t* base = Vs + vofs[db] + c16 * 16 * D;
            const bf16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)base);
            const bf16x4 hi4 = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(base + 8 * D));
            dst[db] = __builtin_shufflevector(lo, hi4, 0, 1, 2, 3, 4, 5, 6, 7);
        }
    };
    vread(0, va[0]);
#pragma unroll
    for (int c16 = 0; c16 < 2 * NBLK; ++c16) {
        const int kb = c16 >> 1, sh = (c16 & 1) * 8;
        bf16x8 pb;
        if (need_mask) {
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const float sv = sacc[kb][sh + i];
                const float p = (sv == kNegInf) ? 0.f : fast_exp2(fmaf(sv, c, -mc));
                lsum += p;
                pb[i] = (__bf16)p;
            }
        } else {
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const float p = fast_exp2(fmaf(sacc[kb][sh + i], c, -mc));
                lsum += p;
                pb[i] = (__bf16)p;
            }
        }
        if (c16 < nvb) {
            if (c16 + 1 < 2 * NBLK && c16 + 1 < nvb) vread(c16 + 1, va[(c16 + 1) & 1]);
#pragma unroll
            for (int db = 0; db < 2; ++db)
                oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va[c16 & 1][db], pb, oacc[db], 0, 0, 0);
        }
    }
    l_run += lsum;
}

// Short sequences at d = 64 (a ViT image: 196 tokens): one workgroup per
// (b, head) holds the head's whole K and V in LDS, and its 4 waves take the
// 32-row blocks of the head in turn (wave w: blocks w, w + 4, ...), each
// walking the staged keys in steps of 64 (sh_step).  At most SH_ROWS = 208
// keys: 52 KB of LDS, so three workgroups share a CU and a batch of 64
// images x 12 heads runs as a single round of workgroups.  The keys are
// staged in four parts (rows 0-63, 64-127, 128-191, 192-207), each in LDS
// arrays of its own, and a wave's first row block computes a step as soon as
// its part has landed (counted waits), so the loads of the later parts
// overlap the first steps.  Heads that share a kv head run back to back on
// one XCD (as in the non-causal tiled kernel), so the shared K/V come from
// its L2.
constexpr int SH_ROWS = 208;   // staged key rows: 3 parts of 64 and one of 16

template <bool CAUSAL, bool PIPE>
__global__ void __launch_bounds__(PF_THREADS) __attribute__((amdgpu_waves_per_eu(3, 3)))
prefill_short_kernel(const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
                     const uint16_t* __restrict__ v, uint16_t* __restrict__ o,
                     float* __restrict__ lse, int Hq, int Hkv, int N, int BH, float c, int negate) {
    constexpr int D = 64;
    constexpr int CPR = D / 8;
    constexpr int PR = 64;                    // rows of a full part
    // parts 0..2 (64 rows each) and part 3 (16 rows), each an array of its
    // own (K rows, then V rows), so every read names the array it reads and
    // the compiler does not wait for the loads still landing in the others
    __shared__ __attribute__((aligned(16))) uint16_t P0s[2 * PR * D], P1s[2 * PR * D], P2s[2 * PR * D];
    __shared__ __attribute__((aligned(16))) uint16_t P3s[2 * 16 * D];
    uint16_t *K0s = P0s, *V0s = P0s + PR * D, *K1s = P1s, *V1s = P1s + PR * D;
    uint16_t *K2s = P2s, *V2s = P2s + PR * D, *K3s = P3s, *V3s = P3s + 16 * D;

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int hi = lane >> 5, l32 = lane & 31;

    // Workgroup w runs on XCD w % 8; the G heads that read one kv head are
    // consecutive workgroups of one XCD.  Padding workgroups exit.
    const int G = Hq / Hkv;
    const int wg = blockIdx.x, x = wg & 7, j = wg >> 3;
    const int r = (j / G) * 8 + x;
    if (r >= BH / G) return;
    const int bh = r * G + (j - (j / G) * G);
    const int b = bh / Hq, h = bh - b * Hq;
    const int g = h / G;
    const uint32_t head_bytes = (uint32_t)N * D * 2;
    const __amdgpu_buffer_rsrc_t qrs = make_rsrc(q + (size_t)bh * N * D, head_bytes);
    const __amdgpu_buffer_rsrc_t krs = make_rsrc(k + ((size_t)b * Hkv + g) * N * D, head_bytes);
    const __amdgpu_buffer_rsrc_t vrs = make_rsrc(v + ((size_t)b * Hkv + g) * N * D, head_bytes);

    // q rows of a row block: raw loads, then the sign (negative scale) once
    // the loads are needed, so the first row block's loads stay in flight
    // while the K/V parts are issued
    auto load_q_raw = [&](int myrow, u32x4 (&qw)[4]) {
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) qw[ks] = buf_ld16(qrs, (uint32_t)(myrow * D + ks * 16 + hi * 8) * 2);
    };
    auto finish_q = [&](const u32x4 (&qw)[4], bf16x8 (&qf)[4]) {
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) qf[ks] = __builtin_bit_cast(bf16x8, negate ? neg_bf16x8(qw[ks]) : qw[ks]);
    };
    const int n_rb = (N + 31) / 32;
    bf16x8 qf[4];
    u32x4 qw[4];

    // Stage part p (rows 64p .. 64p + rows - 1 of K and V; rows past N read
    // as zero): 16-byte chunk i * 256 + tid of the part is its row
    // (i * 256 + tid) / 8, chunk ((i * 256 + tid) % 8) ^ swizzle(row).  A full
    // part is exactly 2 chunks of K and 2 of V per thread (no guard, so the
    // compiler counts them); a partial one guards whole waves.
    const int R = (N + 15) & ~15;             // staged rows
    auto stage_full = [&](int part, uint16_t* Kd, uint16_t* Vd) {
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const int pc = i * PF_THREADS + tid;
            const int row = pc / CPR;
            const int grow = part * PR + row;
            buf_ld16_lds(krs, Kd + (i * PF_THREADS + wave * 64) * 8,
                         (uint32_t)(grow * D + (((pc % CPR) ^ kswz<CPR>(row)) * 8)) * 2);
            buf_ld16_lds(vrs, Vd + (i * PF_THREADS + wave * 64) * 8,
                         (uint32_t)(grow * D + (((pc % CPR) ^ vswz<CPR>(row)) * 8)) * 2);
        }
    };
    auto stage_part = [&](int part, uint16_t* Kd, uint16_t* Vd, int rows) {
        const int chunks = rows * CPR;
        for (int p0 = 0; p0 < chunks; p0 += PF_THREADS) {
            if (p0 + wave * 64 < chunks) {
                const int pc = p0 + tid;
                const int row = pc / CPR;
                const int grow = part * PR + row;
                buf_ld16_lds(krs, Kd + (p0 + wave * 64) * 8,
                             (uint32_t)(grow * D + (((pc % CPR) ^ kswz<CPR>(row)) * 8)) * 2);
                buf_ld16_lds(vrs, Vd + (p0 + wave * 64) * 8,
                             (uint32_t)(grow * D + (((pc % CPR) ^ vswz<CPR>(row)) * 8)) * 2);
            }
        }
    };
    const int rows0 = min(PR, R), rows1 = min(PR, max(0, R - PR)), rows2 = min(PR, max(0, R - 2 * PR));
    const int rows3 = max(0, R - 3 * PR);
    // PIPE (193 <= N <= 208: parts 0-2 full, part 3 sixteen rows): the
    // 16-row part first, then parts 0, 1, 2, so that before step j < 3 the
    // loads this thread may still have in flight are the 4 of each full part
    // after j.  Otherwise every part is staged and waited for at once.
    // (The first row block's q loads go between the 16-row part and part 0:
    // the compiler counts the 12 part loads after them exactly, so its wait
    // for q leaves parts 0-2 in flight.)
    if (PIPE) {
        stage_full(0, K0s, V0s);
        // part 3 (16 rows, 128 chunks): waves 2 and 3 load the same chunks as
        // waves 0 and 1 into the same places (identical bytes), so every
        // thread issues exactly one K and one V load and nothing is guarded
        {
            const int pc = tid & 127;
            const int row = pc / CPR;
            const int grow = 3 * PR + row;
            buf_ld16_lds(krs, K3s + ((wave & 1) * 64) * 8,
                         (uint32_t)(grow * D + (((pc % CPR) ^ kswz<CPR>(row)) * 8)) * 2);
            buf_ld16_lds(vrs, V3s + ((wave & 1) * 64) * 8,
                         (uint32_t)(grow * D + (((pc % CPR) ^ vswz<CPR>(row)) * 8)) * 2);
        }
        load_q_raw(wave * 32 + l32, qw);
        stage_full(1, K1s, V1s);
        stage_full(2, K2s, V2s);
        __builtin_amdgcn_sched_barrier(0);
    } else {
        load_q_raw(wave * 32 + l32, qw);
        stage_part(0, K0s, V0s, rows0);
        stage_part(1, K1s, V1s, rows1);
        stage_part(2, K2s, V2s, rows2);
        stage_part(3, K3s, V3s, rows3);
        wait_vmcnt<0>();
        __syncthreads();
    }
    finish_q(qw, qf);
    auto part_ready = [&](auto jp_tag) {   // every thread's loads of part jp have landed
        constexpr int JP = decltype(jp_tag)::value;
        // issued: part 0 (4 loads per thread), part 3 (2), q (4), parts 1, 2.
        // A plain barrier: each thread has waited for its own loads of the
        // part, and the barrier orders that before every wave's reads (a
        // fenced barrier would drain every load still in flight).
        if constexpr (JP == 0) {
            wait_vmcnt<14>();
            __builtin_amdgcn_s_barrier();
        } else if constexpr (JP < 3) {
            wait_vmcnt<4 * (2 - JP)>();
            __builtin_amdgcn_s_barrier();
        }
    };

    // per-lane LDS read offsets (elements): K operand of k-step ks (row l32 of
    // a 32-key block; part 3 holds 16 rows, so its lanes 16..31 read row
    // l32 - 16 instead: those keys lie past N and are masked), and the two
    // V^T transpose reads per dims block; each one opaque, so every read stays
    // a base plus an immediate
    int kofs[4], kofs3[4], vofs[2];
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
        int off = l32 * D + (((ks * 2 + hi) ^ kswz<CPR>(l32)) * 8);
        asm("" : "+v"(off));
        kofs[ks] = off;
        const int r3 = l32 & 15;
        int off3 = r3 * D + (((ks * 2 + hi) ^ kswz<CPR>(r3)) * 8);
        asm("" : "+v"(off3));
        kofs3[ks] = off3;
    }
#pragma unroll
    for (int db = 0; db < 2; ++db) {
        int off = pf_vtr_offset<D>(lane, db);
        asm("" : "+v"(off));
        vofs[db] = off;
    }

    // One row block.  The first (row block `wave`, taken by every wave,
    // with or without rows) passes the part barriers, which are
    // workgroup-wide; its q rows were loaded before the parts.  It is a
    // separate instantiation, so the compiler's waits for a later block's q
    // rows do not tighten the part waits.
    auto row_block = [&](auto first_tag, int rb) {
        constexpr bool FIRST = decltype(first_tag)::value;
        const int wrow0 = rb * 32;
        const int myrow = wrow0 + l32;
        const bool active = rb < n_rb;
        if (!FIRST) {
            load_q_raw(myrow, qw);
            finish_q(qw, qf);
        }
        f32x16 oacc[2];
#pragma unroll
        for (int db = 0; db < 2; ++db)
#pragma unroll
            for (int i = 0; i < 16; ++i) oacc[db][i] = 0.f;
        float m_run = kNegInf, l_run = 0.f;

        // steps of 64 keys over parts 0..2, then the 16 keys of part 3
        const int key_end = CAUSAL ? min(N, wrow0 + 32) : N;
        auto step = [&](auto gk0_tag, auto nblk_tag, const uint16_t* Kp, const uint16_t* Vp, const int (&ko)[4],
                        int part_rows) {
            constexpr int GK0 = decltype(gk0_tag)::value, NB = decltype(nblk_tag)::value;
            if (PIPE && FIRST) part_ready(std::integral_constant<int, GK0 / PR>{});
            if (active && GK0 < key_end) {
                const bool need_mask = (GK0 + 32 * NB > N) || (CAUSAL && GK0 + 32 * NB - 1 > wrow0);
                sh_step<CAUSAL, GK0, NB>(Kp, Vp, ko, vofs, qf, oacc, m_run, l_run, N, myrow, need_mask,
                                         min(2 * NB, part_rows / 16), c, hi);
            }
        };
        using std::integral_constant;
        step(integral_constant<int, 0>{}, integral_constant<int, 2>{}, K0s, V0s, kofs, rows0);
        step(integral_constant<int, 64>{}, integral_constant<int, 2>{}, K1s, V1s, kofs, rows1);
        step(integral_constant<int, 128>{}, integral_constant<int, 2>{}, K2s, V2s, kofs, rows2);
        step(integral_constant<int, 192>{}, integral_constant<int, 1>{}, K3s, V3s, kofs3, rows3);

        // o = u / l, lse = m + ln l (natural log)
        const float l_tot = l_run + xor_shfl(l_run, 32);
        if (active && myrow < N) {
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
            if (lse != nullptr && hi == 0) lse[(size_t)bh * N + myrow] = (m_run * c + log2f(l_tot)) * kLn2;
        }
    };
    row_block(std::true_type{}, wave);
    for (int rb = wave + PF_WAVES; rb < n_rb; rb += PF_WAVES) row_block(std::false_type{}, rb);
}

// Causal work units (b, h, q tile), heaviest q tiles first, with the units
// that read one kv head's K and V kept on a subset of the XCDs (workgroup w
// runs on XCD w % 8), so that each XCD's L2 holds fewer kv heads.
//   mode 0: unit w of the heaviest-first order (no XCD placement);
//   mode 1 (kv heads a multiple of 8): XCD x takes kv heads x, x + 8, ...;
//           its j-th workgroup takes the j-th of their units, heaviest first;
//   mode 2 (8 a multiple of the kv heads): each kv head owns 8 / n_kv XCDs,
//           which deal its units (heaviest first) round-robin; workgroups past
//           the end of a kv head's units (grid padding) get none.
// Returns false for a padding workgroup.
__device__ __forceinline__ bool causal_unit(int wg, int BH, int G, int n_qtiles, int mode, int& qt, int& bh) {
    if (mode == 0) {
        qt = n_qtiles - 1 - wg / BH;
        bh = wg % BH;
        return true;
    }
    const int n_kv = BH / G;
    const int x = wg & 7, j = wg >> 3;
    if (mode == 1) {
        const int L = (n_kv / 8) * G;     // units of one q tile index on an XCD
        const int qi = j / L, rem = j - qi * L;
        if (qi >= n_qtiles) return false;
        qt = n_qtiles - 1 - qi;
        bh = (x + 8 * (rem / G)) * G + rem % G;
        return true;
    }
    const int S = 8 / n_kv;
    const int r = x / S;
    const int u = j * S + (x - r * S);
    if (u >= G * n_qtiles) return false;
    qt = n_qtiles - 1 - u / G;
    bh = r * G + u % G;
    return true;
}

// Software-pipelined variant: inside each wave, the vector work of key
// tile j runs between the matrix instructions of its neighbours, because a
// wave's own independent VALU instructions issue while its MFMAs execute
// (the matrix core and the vector unit then work at once), which two
// separate waves on a SIMD do not achieve.  Per tile j:
//   block A: S^T(j+1) = K(j+1) Q^T (16 MFMAs)  beside  P(j) = 2^(c s - c m)
//            against the running maximum, its row-sum parts and bf16 packing
//   then the quick lazy-rescale test of tile j (as in pf_tile_step): only
//            when a row-sum part exceeds 2^7 is tile j's maximum formed, the
//            running maximum moved if it grew past 2^8 in weight, and P(j)
//            formed again
//   block B: O^T += V^T(j) P^T(j) (16 MFMAs)    beside  the masking of tile
//            j+1 where needed
// The first maximum is taken in the prologue, from tile 0.  K and V have
// separate double buffers: block A reads K(j+1) and block B V(j), so both
// stay resident for one iteration while K(j+2) and V(j+1) load into the other
// halves.  The arithmetic per row is the same as in prefill_bf16_kernel (same
// products, same order, the same rescale decisions), only interleaved.
template <int D, bool CAUSAL>
__global__ void __launch_bounds__(PF_THREADS) __attribute__((amdgpu_waves_per_eu(2, 2)))
prefill_sp_kernel(const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
                  const uint16_t* __restrict__ v, uint16_t* __restrict__ o,
                  float* __restrict__ lse, int Hq, int Hkv, int N, int BH, int n_qtiles,
                  float c, int negate, int xcd_map) {
    constexpr int CPR = D / 8;
    constexpr int TILE = PF_BN * D;
    constexpr int LINST = PF_BN * CPR / PF_THREADS;
    constexpr int KS = D / 16;
    constexpr int NDB = D / 32;
    static_assert(LINST * PF_THREADS == PF_BN * CPR, "tile split");
    __shared__ __attribute__((aligned(16))) uint16_t kbuf0[TILE];
    __shared__ __attribute__((aligned(16))) uint16_t kbuf1[TILE];
    __shared__ __attribute__((aligned(16))) uint16_t vbuf0[TILE];
    __shared__ __attribute__((aligned(16))) uint16_t vbuf1[TILE];

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int hi = lane >> 5, l32 = lane & 31;

    int qt, bh;
    if (!causal_unit((int)blockIdx.x, BH, Hq / Hkv, n_qtiles, xcd_map, qt, bh)) return;
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

    bf16x8 qf[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
        u32x4 w = buf_ld16(qrs, (uint32_t)(myrow * D + ks * 16 + hi * 8) * 2);
        if (negate) w = neg_bf16x8(w);
        qf[ks] = __builtin_bit_cast(bf16x8, w);
    }

    const int row_end = min(q0 + PF_BM, N);
    const int n_kt = CAUSAL ? (row_end + PF_BN - 1) / PF_BN : (N + PF_BN - 1) / PF_BN;
    // this wave computes key tiles [0, my_kt)
    const int my_kt = !wave_active ? 0 : (CAUSAL ? min(n_kt, (wrow0 + 31) / PF_BN + 1) : n_kt);

    // Staging: unit p = (i * waves + wave) * 64 + lane holds the 16-byte
    // chunk (row p / CPR, chunk (p % CPR) ^ swizzle(row)).  Successive i are
    // 4096 bytes of rows apart and leave both swizzles unchanged, so one
    // offset per lane and tensor serves every i (the rest is scalar).
    uint32_t koff, voff;
    {
        const int p = wave * 64 + lane;
        const int r = p / CPR;
        koff = (uint32_t)(r * D + (((p % CPR) ^ kswz<CPR>(r)) * 8)) * 2;
        voff = (uint32_t)(r * D + (((p % CPR) ^ vswz<CPR>(r)) * 8)) * 2;
    }
    constexpr uint32_t kInstBytes = PF_WAVES * 64 * 16;
    auto load_k = [&](int kt, uint16_t* dst) {
#pragma unroll
        for (int i = 0; i < LINST; ++i)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(krs, (lds_void*)(dst + (i * PF_WAVES + wave) * 64 * 8), 16,
                                                     koff, (uint32_t)kt * TILE * 2 + i * kInstBytes, 0, 0);
    };
    auto load_v = [&](int kt, uint16_t* dst) {
#pragma unroll
        for (int i = 0; i < LINST; ++i)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(vrs, (lds_void*)(dst + (i * PF_WAVES + wave) * 64 * 8), 16,
                                                     voff, (uint32_t)kt * TILE * 2 + i * kInstBytes, 0, 0);
    };

    // Operand read offsets (one opaque offset each, so every LDS read's
    // address is a short chain from its array and the compiler can tell it
    // apart from the loads in flight into the other buffers).
    int kofs[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
        int off = l32 * D + (((ks * 2 + hi) ^ kswz<CPR>(l32)) * 8);
        asm("" : "+v"(off));
        kofs[ks] = off;
    }
    int vofs[NDB];
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
        int off = pf_vtr_offset<D>(lane, db);
        asm("" : "+v"(off));
        vofs[db] = off;
    }

    f32x16 oacc[NDB];
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[db][r] = 0.f;
    float m_run = kNegInf, l_run = 0.f;

    const PfPipe<D, CAUSAL> pp{qf, kofs, vofs, oacc, m_run, l_run, c, hi, N, myrow};
    auto tile_mask = [&](int j) {
        const int k0 = j * PF_BN;
        return (k0 + PF_BN > N) || (CAUSAL && k0 + PF_BN - 1 > wrow0);
    };

    f32x16 sa[2], sb[2];

    // Prologue: K(0), K(1), V(0) resident; scores of tile 0 and the first
    // running maximum.
    load_k(0, kbuf0);
    if (n_kt > 1) load_k(1, kbuf1);
    load_v(0, vbuf0);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (my_kt > 0) {
        pp.scores(kbuf0, sa);
        if (tile_mask(0)) pp.template mask<true>(sa, 0);
        pp.rescale(pp.rowmax_masked(sa));    // the first maximum (always a rescale)
    }
    __syncthreads();     // every wave's reads of K(0) precede the load into its buffer

    // Iteration j: K(j+1) in kn, V(j) in vc; loads of K(j+2) into kd and
    // V(j+1) into vd (their previous tiles were last read in iteration j-1).
    auto iter = [&](int j, const uint16_t* kn, const uint16_t* vc, uint16_t* kd, uint16_t* vd,
                    f32x16 (&scur)[2], f32x16 (&snxt)[2]) {
        if (j + 2 < n_kt) load_k(j + 2, kd);
        if (j + 1 < n_kt) load_v(j + 1, vd);
        // Tile j's weights were taken against the running maximum (row-sum
        // parts lsum); the full lazy-rescale test, from tile j's maximum, and
        // the weights again only when a part exceeds 2^7 or some row has no
        // maximum yet (as in pf_tile_step).
        auto settle = [&](bf16x8 (&pb)[4], float lsum) {
            if (__builtin_amdgcn_ballot_w64(m_run == kNegInf || !(lsum <= kLazyCheck)) != 0) {
                pp.rescale(pp.rowmax_masked(scur));
                lsum = pp.probs_part(scur, pb);
            }
            l_run += lsum;
        };
        if (j + 1 < my_kt) {
            const int k1 = (j + 1) * PF_BN;
            // One straight-line path per mask case of tile j+1, so that each
            // block is a single scheduling region.
            auto body = [&](auto mask_tag) {
                constexpr bool MASK = decltype(mask_tag)::value;
                bf16x8 pb[4];
                // block A
                pp.scores(kn, snxt);
                const float lsum = pp.probs_part(scur, pb);
                pf_interleave<2 * KS, 7, 6, 1>();
                __builtin_amdgcn_sched_barrier(0);
                settle(pb, lsum);
                __builtin_amdgcn_sched_barrier(0);
                // block B
                pp.pv(vc, pb);
                pp.template mask<MASK>(snxt, k1);
                pf_interleave<16, MASK ? 4 : 0, 12, 2>();
                __builtin_amdgcn_sched_barrier(0);
            };
            if (tile_mask(j + 1))
                body(std::true_type{});
            else
                body(std::false_type{});
        } else if (j < my_kt) {
            bf16x8 pb[4];
            settle(pb, pp.probs_part(scur, pb));
            pp.pv(vc, pb);
        }
        __builtin_amdgcn_s_waitcnt(0);     // K(j+2), V(j+1) in LDS
        __syncthreads();
    };
    for (int j = 0; j < n_kt; j += 2) {
        iter(j, kbuf1, vbuf0, kbuf0, vbuf1, sa, sb);
        if (j + 1 < n_kt) iter(j + 1, kbuf0, vbuf1, kbuf1, vbuf0, sb, sa);
    }

    // Epilogue: o = u / l, lse = m + ln l (natural log).
    const float l_tot = l_run + xor_shfl(l_run, 32);
    if (wave_active && myrow < N) {
        const float inv = (l_tot > 0.f) ? 1.f / l_tot : 0.f;
        uint16_t* orow = o + ((size_t)bh * N + myrow) * D;
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
            for (int rg = 0; rg < 4; ++rg) {
                const int dim0 = db * 32 + rg * 8 + hi * 4;
                const u32x2 w = {pack_bf16x2(oacc[db][rg * 4 + 0] * inv, oacc[db][rg * 4 + 1] * inv),
                                 pack_bf16x2(oacc[db][rg * 4 + 2] * inv, oacc[db][rg * 4 + 3] * inv)};
                *reinterpret_cast<u32x2*>(orow + dim0) = w;
            }
        if (lse != nullptr && hi == 0) lse[(size_t)bh * N + myrow] = (m_run * c + log2f(l_tot)) * kLn2;
    }
}

template <int D, bool CAUSAL>
hipError_t launch_bf16_t(const PrefillArgs& a, hipStream_t stream) {
    const int BH = a.B * a.Hq;
    const int n_qt = (a.N + PF_BM - 1) / PF_BM;
    const dim3 grid((unsigned)(BH * n_qt)), block(PF_THREADS);
    // The software-pipelined kernel for causal d = 128 (the long prefills);
    // the plain one elsewhere: at d = 64 on short sequences it is faster, and
    // the non-causal d = 128 build of the pipelined loop runs out of registers.
    // Scale 0 also takes the plain kernel: the pipelined one relies on
    // 2^(c * -inf - c m) being 0 for masked keys, which needs c > 0.
    // The plain kernel's key tiles: 64 keys at d = 128, 32 at d = 64 (four
    // waves per SIMD).  ATTN_PREFILL_BN=32 or 64 (test hook) forces the plain
    // kernel with that tile, another partition of the keys, which must give
    // the same result within the tolerances.
    const char* bn_env = getenv("ATTN_PREFILL_BN");
    const bool force32 = bn_env != nullptr && bn_env[0] == '3' && bn_env[1] == '2' && bn_env[2] == '\0';
    const bool force64 = bn_env != nullptr && bn_env[0] == '6' && bn_env[1] == '4' && bn_env[2] == '\0';
    const bool bn_forced = force32 || force64;
    const bool bn32 = force32 || (D == 64 && !force64);
    if constexpr (D == 128 && CAUSAL) {
        // ATTN_PREFILL_PLAIN=1 (test hook) keeps the plain kernel, so tests
        // can compare the two
        const char* plain = getenv("ATTN_PREFILL_PLAIN");
        if (a.c > 0.f && !bn_forced && !(plain != nullptr && plain[0] == '1')) {
            // XCD placement of the units by kv head (causal_unit); the grid of
            // mode 2 is padded to 8 equal XCD shares.  ATTN_PREFILL_XCD=0
            // (test hook) places them in plain heaviest-first order.
            const int G = a.Hq / a.Hkv, n_kv = BH / G;
            const char* xe = getenv("ATTN_PREFILL_XCD");
            int mode = 0;
            long long ngrid = (long long)BH * n_qt;
            if (!(xe != nullptr && xe[0] == '0')) {
                if (n_kv % 8 == 0) {
                    mode = 1;
                } else if (8 % n_kv == 0) {
                    const long long S = 8 / n_kv, per = ((long long)G * n_qt + S - 1) / S;
                    if (8 * per < (1LL << 31)) {
                        mode = 2;
                        ngrid = 8 * per;
                    }
                }
            }
            hipLaunchKernelGGL((prefill_sp_kernel<D, CAUSAL>), dim3((unsigned)ngrid), block, 0, stream,
                               static_cast<const uint16_t*>(a.q), static_cast<const uint16_t*>(a.k),
                               static_cast<const uint16_t*>(a.v), static_cast<uint16_t*>(a.o), a.lse,
                               a.Hq, a.Hkv, a.N, BH, n_qt, a.c, a.negate, mode);
            return hipGetLastError();
        }
    }
    // Short d = 64 sequences over enough heads to fill the machine: one
    // workgroup per head with the head's K and V staged whole.
    if constexpr (D == 64) {
        if (!bn_forced && a.N <= SH_ROWS && BH >= 256) {
            const long long padded = ((long long)BH / (a.Hq / a.Hkv) + 7) / 8 * 8 * (a.Hq / a.Hkv);
            if (a.N > 3 * 64 && a.N <= SH_ROWS)
                hipLaunchKernelGGL((prefill_short_kernel<CAUSAL, true>), dim3((unsigned)padded), block, 0, stream,
                                   static_cast<const uint16_t*>(a.q), static_cast<const uint16_t*>(a.k),
                                   static_cast<const uint16_t*>(a.v), static_cast<uint16_t*>(a.o), a.lse,
                                   a.Hq, a.Hkv, a.N, BH, a.c, a.negate);
            else
                hipLaunchKernelGGL((prefill_short_kernel<CAUSAL, false>), dim3((unsigned)padded), block, 0, stream,
                                   static_cast<const uint16_t*>(a.q), static_cast<const uint16_t*>(a.k),
                                   static_cast<const uint16_t*>(a.v), static_cast<uint16_t*>(a.o), a.lse,
                                   a.Hq, a.Hkv, a.N, BH, a.c, a.negate);
            return hipGetLastError();
        }
    }
    // Non-causal: XCD-local runs of the units that share a kv head (grid
    // padded to whole rounds of 8 runs), when the runs spread evenly over the
    // 8 XCDs (a multiple of 8 runs, or enough that one extra run per XCD
    // matters little) and the padded grid fits.
    const long long runs = (long long)BH / (a.Hq / a.Hkv);
    const long long padded = (runs + 7) / 8 * 8 * (a.Hq / a.Hkv) * n_qt;
    const int xcd_runs = (!CAUSAL && (runs % 8 == 0 || runs >= 128) && padded < (1LL << 31)) ? 1 : 0;
    const dim3 grid_p(xcd_runs ? (unsigned)padded : grid.x);
    if (bn32)
        hipLaunchKernelGGL((prefill_bf16_kernel<D, CAUSAL, 32>), grid_p, block, 0, stream,
                           static_cast<const uint16_t*>(a.q), static_cast<const uint16_t*>(a.k),
                           static_cast<const uint16_t*>(a.v), static_cast<uint16_t*>(a.o), a.lse,
                           a.Hq, a.Hkv, a.N, BH, n_qt, a.c, a.negate, xcd_runs);
    else
        hipLaunchKernelGGL((prefill_bf16_kernel<D, CAUSAL, PF_BN>), grid_p, block, 0, stream,
                           static_cast<const uint16_t*>(a.q), static_cast<const uint16_t*>(a.k),
                           static_cast<const uint16_t*>(a.v), static_cast<uint16_t*>(a.o), a.lse,
                           a.Hq, a.Hkv, a.N, BH, n_qt, a.c, a.negate, xcd_runs);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_prefill_bf16(const PrefillArgs& a, hipStream_t stream) {
    if (a.d == 128) return a.causal ? launch_bf16_t<128, true>(a, stream) : launch_bf16_t<128, false>(a, stream);
    return a.causal ? launch_bf16_t<64, true>(a, stream) : launch_bf16_t<64, false>(a, stream);
}

}  // namespace attn

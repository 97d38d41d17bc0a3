// The memory-bound fusions around attention in a transformer layer, for
// gfx950 ("Kernels de atención rápida y fusión de operadores", section
// "Fusión de operadores": a layer's residual additions, normalisation and
// activation would each be a kernel that writes its intermediate tensor to
// HBM and the next one reads back; fused, one pass reads the inputs once and
// writes the results once).
//
//   * add_rmsnorm: h = x + residual (the new residual stream, bf16) and
//     y = h / sqrt(mean(h^2) + eps) * w, one wave per row: the row's h stays
//     in registers between the sum of squares (a wave reduction) and the
//     scaling.  The norm reads h as stored (rounded to bf16), so the result
//     equals the unfused add-then-norm pair.
//   * swiglu: a = silu(g) * u between the gate/up projections and the down
//     projection, 8 elements per thread; gate and up may be one merged
//     [T, 2F] projection output or two tensors (row stride ld_in).
// Both are pure streams: fp32 arithmetic, 16-byte accesses, no LDS.

#include "common.h"
#include "internal.h"

namespace attn {
namespace {

constexpr int FU_THREADS = 256;

__device__ __forceinline__ float lo_f(uint32_t w) { return __builtin_bit_cast(float, w << 16); }
__device__ __forceinline__ float hi_f(uint32_t w) { return __builtin_bit_cast(float, w & 0xffff0000u); }

// CPL = 16-byte chunks per lane (the row has D / 8 <= 64 * CPL chunks).
template <int CPL>
__global__ void __launch_bounds__(FU_THREADS)
add_rmsnorm_kernel(const uint16_t* __restrict__ x, const uint16_t* r, const uint16_t* __restrict__ w,
                   uint16_t* __restrict__ y, uint16_t* h_out, int T, int D, float eps) {
    const int lane = threadIdx.x & 63;
    const long long row = (long long)blockIdx.x * (FU_THREADS / 64) + (threadIdx.x >> 6);
    if (row >= T) return;                           // whole wave
    const int nch = D / 8;
    const size_t base = (size_t)row * D;
    u32x4 hv[CPL];
    float ss = 0.f;
#pragma unroll
    for (int i = 0; i < CPL; ++i) {
        const int c = lane + 64 * i;
        if (c < nch) {
            const u32x4 a = ld16(x + base + c * 8);
            const u32x4 b = ld16(r + base + c * 8);
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const uint32_t p = pack_bf16x2(lo_f(a[j]) + lo_f(b[j]), hi_f(a[j]) + hi_f(b[j]));
                hv[i][j] = p;
                const float h0 = lo_f(p), h1 = hi_f(p);
                ss = fmaf(h0, h0, ss);
                ss = fmaf(h1, h1, ss);
            }
            st16(h_out + base + c * 8, hv[i]);
        }
    }
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) ss += __shfl_xor(ss, m, 64);
    const float inv = 1.0f / sqrtf(ss / (float)D + eps);
#pragma unroll
    for (int i = 0; i < CPL; ++i) {
        const int c = lane + 64 * i;
        if (c < nch) {
            const u32x4 wv = ld16(w + c * 8);
            u32x4 o;
#pragma unroll
            for (int j = 0; j < 4; ++j)
                o[j] = pack_bf16x2(lo_f(hv[i][j]) * inv * lo_f(wv[j]), hi_f(hv[i][j]) * inv * hi_f(wv[j]));
            st16(y + base + c * 8, o);
        }
    }
}

__device__ __forceinline__ float silu_mul(float g, float u) {
    return g / (1.0f + __expf(-g)) * u;
}

__global__ void __launch_bounds__(FU_THREADS)
swiglu_kernel(const uint16_t* __restrict__ g, const uint16_t* __restrict__ u, uint16_t* __restrict__ out,
              long long total, int f8, long long ld_in, long long ld_out) {
    const long long i = (long long)blockIdx.x * FU_THREADS + threadIdx.x;
    if (i >= total) return;
    const long long t = i / f8;
    const int c = (int)(i - t * f8);
    const u32x4 gv = ld16(g + t * ld_in + c * 8);
    const u32x4 uv = ld16(u + t * ld_in + c * 8);
    u32x4 o;
#pragma unroll
    for (int j = 0; j < 4; ++j)
        o[j] = pack_bf16x2(silu_mul(lo_f(gv[j]), lo_f(uv[j])), silu_mul(hi_f(gv[j]), hi_f(uv[j])));
    st16(out + t * ld_out + c * 8, o);
}

template <int CPL>
hipError_t launch_rms_t(const AddRmsNormArgs& a, hipStream_t stream) {
    const unsigned blocks = (unsigned)(((long long)a.T + 3) / 4);
    hipLaunchKernelGGL((add_rmsnorm_kernel<CPL>), dim3(blocks), dim3(FU_THREADS), 0, stream,
                       static_cast<const uint16_t*>(a.x), static_cast<const uint16_t*>(a.residual),
                       static_cast<const uint16_t*>(a.weight), static_cast<uint16_t*>(a.out),
                       static_cast<uint16_t*>(a.residual_out), a.T, a.D, a.eps);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_add_rmsnorm_bf16(const AddRmsNormArgs& a, hipStream_t stream) {
    const int nch = a.D / 8;
    if (nch <= 64) return launch_rms_t<1>(a, stream);
    if (nch <= 128) return launch_rms_t<2>(a, stream);
    if (nch <= 256) return launch_rms_t<4>(a, stream);
    if (nch <= 512) return launch_rms_t<8>(a, stream);
    return launch_rms_t<16>(a, stream);
}

hipError_t launch_swiglu_bf16(const SwigluArgs& a, hipStream_t stream) {
    const long long total = (long long)a.T * (a.F / 8);
    hipLaunchKernelGGL(swiglu_kernel, dim3((unsigned)((total + FU_THREADS - 1) / FU_THREADS)),
                       dim3(FU_THREADS), 0, stream, static_cast<const uint16_t*>(a.gate),
                       static_cast<const uint16_t*>(a.up), static_cast<uint16_t*>(a.out), total, a.F / 8,
                       (long long)a.ld_in, (long long)a.ld_out);
    return hipGetLastError();
}

}  // namespace attn

// Device-side helpers shared by the attention kernels (gfx950 / CDNA4 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace attn {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kNegInf = -__builtin_inff();

// 16-byte global load / store (global_load_dwordx4 / global_store_dwordx4).
__device__ __forceinline__ u32x4 ld16(const void* p) {
    return *reinterpret_cast<const u32x4*>(p);
}
__device__ __forceinline__ void st16(void* p, u32x4 v) {
    *reinterpret_cast<u32x4*>(p) = v;
}

// Flip the sign of the 8 bf16 lanes held in a 16-byte word (exact).
__device__ __forceinline__ u32x4 neg_bf16x8(u32x4 v) {
    const uint32_t s = 0x80008000u;
    return u32x4{v.x ^ s, v.y ^ s, v.z ^ s, v.w ^ s};
}

// Pack two fp32 into two bf16 (round to nearest even) in one 32-bit word,
// `lo` in the low half.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
    bf16x2 p = {(__bf16)lo, (__bf16)hi};
    return __builtin_bit_cast(uint32_t, p);
}

__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
    return __builtin_bit_cast(float, (uint32_t)b << 16);
}

// Raw buffer resource over `bytes` bytes at `base`: loads beyond the range
// return zero, so tile edges need no branches.  (Word 3 is the gfx9 raw
// buffer format used for 32-bit data.)
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}

__device__ __forceinline__ u32x4 buf_ld16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
}

typedef __attribute__((address_space(3))) void lds_void;

// 16 bytes per lane from the buffer straight into LDS: lane l's bytes land
// at lds_base + 16*l (lds_base must be wave-uniform).
__device__ __forceinline__ void buf_ld16_lds(__amdgpu_buffer_rsrc_t r, void* lds_base, uint32_t off) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void*)lds_base, 16, off, 0, 0, 0);
}

// 4 bytes per lane from the buffer straight into LDS: lane l's bytes land at
// lds_base + 4*l.
__device__ __forceinline__ void buf_ld4_lds(__amdgpu_buffer_rsrc_t r, void* lds_base, uint32_t off) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void*)lds_base, 4, off, 0, 0, 0);
}

// Wait until at most N vector memory operations of this wave are
// outstanding (loads complete in issue order); LDS and export counters are
// not waited on.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// Wave-wide exchange with lane ^ mask (ds_bpermute based).
__device__ __forceinline__ float xor_shfl(float x, int mask) {
    return __shfl_xor(x, mask, 64);
}

// max(x of this lane, x of lane l ^ 32) with v_permlane32_swap, a VALU
// exchange between the two 32-lane halves of the wave (no LDS traffic).  The
// instruction swaps the upper half of its first register with the lower half
// of its second: given x in both, the first ends up holding the lower half's
// values in both halves and the second the upper half's, so their maximum is
// the pairwise maximum in every lane.  Written as inline asm because the
// compiler's builtin for it returns the first register as both results (so a
// maximum of the two would silently be the lower half's value alone); the
// s_nop pairs cover the VALU hazards around the instruction, which the
// compiler cannot see inside the asm.  The instruction only moves register
// values between lanes.
__device__ __forceinline__ float max_halves(float x) {
    uint32_t a = __builtin_bit_cast(uint32_t, x), b = a;
    asm volatile("s_nop 1\n\tv_permlane32_swap_b32 %0, %1\n\ts_nop 1" : "+v"(a), "+v"(b));
    return fmaxf(__builtin_bit_cast(float, a), __builtin_bit_cast(float, b));
}

// Hardware base-2 exponential (v_exp_f32).
__device__ __forceinline__ float fast_exp2(float x) {
    return __builtin_amdgcn_exp2f(x);
}

}  // namespace attn

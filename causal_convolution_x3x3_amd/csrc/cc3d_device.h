// Device helpers shared by every gfx950 kernel file: bf16 conversions, the
// causal-window frame map, the fused act's transcendental forms and the raw
// buffer loads.  One definition of each, so the kernel families cannot drift
// apart.  Included by the .hip files only (the host runtime sees cc3d_kernels.h).
#pragma once

#include "cc3d_kernels.h"

namespace cc3d {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float bf2f(uint16_t h) { return __uint_as_float((uint32_t)h << 16); }

// float -> bfloat16, round to nearest, ties to even (NaN stays NaN): gfx950's
// v_cvt_pk_bf16_f32.
__device__ __forceinline__ uint16_t f2bf(float f) { return __builtin_bit_cast(uint16_t, (__bf16)f); }

// Two floats to a bf16 pair (low half = lo), round to nearest even: gfx950's
// v_cvt_pk_bf16_f32.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi)
{
    return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2){lo, hi}, bf16x2));
}

__device__ __forceinline__ bf16x8 as_bf16x8(uint4 v) { return __builtin_bit_cast(bf16x8, v); }

// 1/sqrt(mean of squares + eps) and SiLU(z) = z / (1 + e^-z) on the hardware's
// transcendental units (v_rsq_f32, v_exp_f32, v_rcp_f32; about 1 ulp of fp32
// each, far below the bf16 rounding of the stored result).
__device__ __forceinline__ float rms_scale(float mean_sq, float eps)
{
    return __builtin_amdgcn_rsqf(mean_sq + eps);
}
__device__ __forceinline__ float silu(float z)
{
    return z * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-1.4426950408889634f * z));
}

// 16-byte chunk swizzle inside a 64-byte LDS row (one pixel or one weight row of
// 32 channels): the 16 rows one fragment read touches spread over the banks.
__device__ __forceinline__ int swz(int row) { return (row >> 1) & 3; }

// Frame zi of the causal window Z = history (kt-1 frames) || V (ZWindow), as a
// byte address; nullptr for a zero history frame.  V[u] = X[(u + t_shift) / 2]
// when the conv doubles time, else X[u].  eb = bytes per element.
__device__ __forceinline__ const char* zframe_bytes(const ZWindow& z, int zi, int eb)
{
    const int hist = z.kt - 1;
    const int64_t fb = z.frame_elems * eb;
    if (zi < hist) {
        if (!z.first) return (const char*)z.cache + zi * fb;
        return z.zero_hist ? nullptr : (const char*)z.x;
    }
    const int u = zi - hist;
    const int src = (z.up_t == 2) ? ((u + z.t_shift) >> 1) : u;
    return (const char*)z.x + src * fb;
}
__device__ __forceinline__ const uint16_t* zframe(const ZWindow& z, int zi)
{
    return (const uint16_t*)zframe_bytes(z, zi, 2);
}

// Raw buffer descriptor (gfx9 family word 3) over `bytes` bytes at `base`; a
// load whose offset lies past the end returns zeros.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes)
{
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}

constexpr uint32_t OOB = 0x80000000u;  // an offset past every buffer used here

// 16 bytes per lane from buffer offset `off` straight into LDS: lane l writes
// the 16-byte slot lds_base + l (lds_base is the same for the whole wave).
__device__ __forceinline__ void load_to_lds(__amdgpu_buffer_rsrc_t r, uint32_t off, uint4* lds_base)
{
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)lds_base, 16, off, 0, 0, 0);
}

// 4 bytes per lane from buffer offset `off` into LDS at lds_base + 4 * lane.
__device__ __forceinline__ void load_to_lds4(__amdgpu_buffer_rsrc_t r, uint32_t off, char* lds_base)
{
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)lds_base, 4, off, 0, 0, 0);
}

// s_waitcnt vmcnt(N) (gfx9 encoding; expcnt and lgkmcnt left at their maxima)
template <int N>
__device__ __forceinline__ void wait_vmcnt()
{
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

}  // namespace cc3d

// txl_device.hpp -- device-side building blocks shared by the libtxl kernels.
//
// Matrix products run on the gfx950 matrix cores through one 32x32 output
// block shape, V_MFMA_F32_32X32X16_BF16 for bf16 storage and eight
// V_MFMA_F32_32X32X2_F32 for fp32 storage, so both dtypes share every tile
// layout. Lane l of a wave (64 lanes) owns
//   A operand: row l % 32, eight reduction slots k = 8*(l/32) + 0..7
//   B operand: column l % 32, the same eight slots
//   C/D:       column l % 32, rows 8*(i/4) + 4*(l/32) + i%4 for register i < 16.
// The reduction slots only need to agree between A and B, so a kernel may map
// its eight slots onto any eight reduction indices, as long as both operands
// use the same map.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace txl {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// Eight reduction slots of one operand for one 16-deep step.
template <typename T> struct Frag;
template <> struct Frag<bf16> { bf16x8 v; };
template <> struct Frag<float> { f32x4 lo, hi; };

__device__ __forceinline__ void mma16(f32x16 &acc, const Frag<bf16> &a, const Frag<bf16> &b) {
    acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a.v, b.v, acc, 0, 0, 0);
}
__device__ __forceinline__ void mma16(f32x16 &acc, const Frag<float> &a, const Frag<float> &b) {
    acc = __builtin_amdgcn_mfma_f32_32x32x2f32(a.lo[0], b.lo[0], acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_32x32x2f32(a.lo[1], b.lo[1], acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_32x32x2f32(a.lo[2], b.lo[2], acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_32x32x2f32(a.lo[3], b.lo[3], acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_32x32x2f32(a.hi[0], b.hi[0], acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_32x32x2f32(a.hi[1], b.hi[1], acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_32x32x2f32(a.hi[2], b.hi[2], acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_32x32x2f32(a.hi[3], b.hi[3], acc, 0, 0, 0);
}

// Eight consecutive elements (16-byte aligned for bf16, 32 for fp32) from LDS
// or global memory.
__device__ __forceinline__ void load8(Frag<bf16> &f, const bf16 *p) {
    f.v = *reinterpret_cast<const bf16x8 *>(p);
}
__device__ __forceinline__ void load8(Frag<float> &f, const float *p) {
    f.lo = *reinterpret_cast<const f32x4 *>(p);
    f.hi = *reinterpret_cast<const f32x4 *>(p + 4);
}
template <typename T> __device__ __forceinline__ void zero8(Frag<T> &f);
template <> __device__ __forceinline__ void zero8(Frag<bf16> &f) {
    f.v = bf16x8{0, 0, 0, 0, 0, 0, 0, 0};
}
template <> __device__ __forceinline__ void zero8(Frag<float> &f) {
    f.lo = f32x4{0.f, 0.f, 0.f, 0.f};
    f.hi = f.lo;
}

template <typename T> __device__ __forceinline__ T from_f32(float x);
template <> __device__ __forceinline__ float from_f32<float>(float x) { return x; }
template <> __device__ __forceinline__ bf16 from_f32<bf16>(float x) { return (bf16)x; }
__device__ __forceinline__ float to_f32(float x) { return x; }
__device__ __forceinline__ float to_f32(bf16 x) { return (float)x; }

__device__ __forceinline__ f32x16 zero16() {
    f32x16 z;
#pragma unroll
    for (int i = 0; i < 16; ++i) z[i] = 0.f;
    return z;
}

// Row of the 32x32 C block held in register i of lane l.
__device__ __forceinline__ int crow(int i, int lane) { return 8 * (i >> 2) + 4 * (lane >> 5) + (i & 3); }

// Exchange with the lane 32 positions away (the other half of the wave).
// Maximum and sum of x over the two lanes l and l ^ 32 (v_permlane32_swap: no LDS trip).
__device__ __forceinline__ float half_max(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float half_sum(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ __forceinline__ float swap_half(float x) {
    int l = threadIdx.x & 63;
    return __int_as_float(__builtin_amdgcn_ds_bpermute(((l ^ 32) << 2), __float_as_int(x)));
}

}  // namespace txl

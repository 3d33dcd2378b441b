// Device-side vector types and small helpers shared by the FP8 and BF16 kernels.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace attnfwd {

typedef int i32x2 __attribute__((ext_vector_type(2)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef short i16x8 __attribute__((ext_vector_type(8)));

#define ATTN_LDS __attribute__((address_space(3)))

constexpr float kLog2e = 1.4426950408889634f;

// Value of lane (l ^ 32) - the other half of the wave.  v_permlane32_swap
// exchanges the upper 32 lanes of its first operand with the lower 32 lanes of
// its second; with both operands equal, lanes < 32 find their partner's value
// in the second result and lanes >= 32 in the first.
__device__ __forceinline__ float other_half(float x) {
    int xi = __float_as_int(x);
    auto r = __builtin_amdgcn_permlane32_swap(xi, xi, false, false);
    return __int_as_float((threadIdx.x & 32) ? r[0] : r[1]);
}

__device__ __forceinline__ i32x4 load16(const void* p) {
    return *reinterpret_cast<const i32x4*>(p);
}

__device__ __forceinline__ i32x4 lds_load16(const ATTN_LDS uint8_t* p) {
    return *reinterpret_cast<const ATTN_LDS i32x4*>(p);
}

__device__ __forceinline__ void lds_store16(ATTN_LDS uint8_t* p, i32x4 v) {
    *reinterpret_cast<ATTN_LDS i32x4*>(p) = v;
}

// Transposing 64-bit LDS read (gfx950): within each group of 16 lanes, lanes 2t
// and 2t+1 address the two 8-byte halves of row t of an 8x16-byte tile and lane
// n receives column n (8 bytes, one per row).
__device__ __forceinline__ i32x2 lds_read_tr8(const ATTN_LDS uint8_t* p) {
    return __builtin_amdgcn_ds_read_tr8_b64_v2i32((ATTN_LDS i32x2*)p);
}

// Same for 16-bit elements: lanes 4t..4t+3 address row t (16 columns) of a 4x16
// tile and lane n receives column n (4 elements, one per row).
__device__ __forceinline__ i16x4 lds_read_tr16(const ATTN_LDS uint8_t* p) {
    return __builtin_amdgcn_ds_read_tr16_b64_v4i16((ATTN_LDS i16x4*)p);
}

__device__ __forceinline__ i16x8 i16x8_cat(i16x4 a, i16x4 b) {
    return i16x8{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
}

__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
    __bf16 x = (__bf16)a, y = (__bf16)b;
    return (uint32_t)__builtin_bit_cast(uint16_t, x) | ((uint32_t)__builtin_bit_cast(uint16_t, y) << 16);
}

}  // namespace attnfwd

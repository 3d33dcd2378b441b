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

// Value of lane (l ^ 32) - the other half of the wave.  v_permlane32_swap
// exchanges the upper 32 lanes of its first operand with the lower 32 lanes of
// its second; with both operands equal, lanes < 32 find their partner's value
// in the second result and lanes >= 32 in the first.
__device__ __forceinline__ float other_half(float x) {
    int xi = __float_as_int(x);
    auto r = __builtin_amdgcn_permlane32_swap(xi, xi, false, false);
    return __int_as_float((threadIdx.x & 32) ? r[0] : r[1]);
}

// max of x over the lane pair (l, l ^ 32).  v_permlane32_swap of x with itself
// leaves the lower half's 32 values in one result and the upper half's in the
// other, each in every lane, so one max of the two covers both lanes of a pair.
__device__ __forceinline__ float pair_max(float x) {
    const int xi = __float_as_int(x);
    const auto r = __builtin_amdgcn_permlane32_swap(xi, xi, false, false);
    return fmaxf(__int_as_float(r[0]), __int_as_float(r[1]));
}

__device__ __forceinline__ i32x4 load16(const void* p) {
    return *reinterpret_cast<const i32x4*>(p);
}

// Raw buffer resource over [base, base + bytes): 16-byte loads at byte offsets at
// or past `bytes` return zeros without touching memory.  Word 3 selects the
// 32-bit data format of untyped gfx9-family buffer accesses.
// The base and size must be wave-uniform; they are read from the first lane, so
// the descriptor lives in SGPRs (no per-lane waterfall around the loads).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_rsrc(const void* base, int bytes) {
    const unsigned long long a = (unsigned long long)base;
    const unsigned long long lo = (unsigned)__builtin_amdgcn_readfirstlane((int)a);
    const unsigned long long hi = (unsigned)__builtin_amdgcn_readfirstlane((int)(a >> 32));
    return __builtin_amdgcn_make_buffer_rsrc((void*)(lo | (hi << 32)), (short)0,
                                             __builtin_amdgcn_readfirstlane(bytes), 0x00020000);
}

// A wave-uniform pointer read from the first lane, so that it and the per-block addresses
// derived from it by uniform offsets are scalar values (no per-block readfirstlane).
__device__ __forceinline__ const uint8_t* uniform_ptr(const uint8_t* p) {
    const unsigned long long x = (unsigned long long)p;
    const unsigned long long lo = (unsigned)__builtin_amdgcn_readfirstlane((int)x);
    const unsigned long long hi = (unsigned)__builtin_amdgcn_readfirstlane((int)(x >> 32));
    return (const uint8_t*)(lo | (hi << 32));
}

// Query tile and (sequence, query head) index bh of workgroup L, in a grid of nt tiles
// (256 queries each) for each of BH query heads, ratio query heads per K/V head.
// Workgroups go to the 8 XCDs round-robin by index.  With more than 4 query heads per
// XCD, a tile-major order would run only a few tiles of each head together on an XCD,
// each streaming its own K/V prefix through that XCD's L2.  Instead XCD x then runs the
// query heads of the K/V heads g = x (mod 8) (so each K/V head is read through one
// L2), in bands of up to 32 tiles of one query head, the heads of one K/V head
// adjacent, heaviest band first: the workgroups running together on an XCD share one
// K/V prefix.  Otherwise (and when K/V heads do not divide over the XCDs) the order is
// tile-major, heaviest (longest causal prefix) tiles first.
__host__ __device__ __forceinline__ void tile_of(int L, int BH, int ratio, int nt, int& tile, int& bh) {
    if (BH > 32 && (BH / ratio) % 8 == 0) {
        constexpr int G = 32;                   // about one workgroup per CU of an XCD
        const int x = L & 7, idx = L >> 3, nh = BH >> 3;
        const int fb = nt / G;                  // full bands
        int k, t;
        if (idx < fb * G * nh) {
            const int band = idx / (G * nh), rem = idx - band * (G * nh);
            k = rem / G;
            t = band * G + (rem - k * G);
        } else {
            const int r = nt - fb * G, rem = idx - fb * G * nh;   // the last, partial band
            k = rem / r;
            t = fb * G + (rem - k * r);
        }
        tile = nt - 1 - t;
        bh = (x + 8 * (k / ratio)) * ratio + k % ratio;
    } else {
        tile = nt - 1 - L / BH;
        bh = L % BH;
    }
}

__device__ __forceinline__ i32x4 buffer_load16(__amdgpu_buffer_rsrc_t r, int offset) {
    return __builtin_amdgcn_raw_buffer_load_b128(r, offset, 0, 0);
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

// acc += A . B on the FP8 matrix cores (32x32x64, e4m3 operands) with per-lane E8M0
// scales: A's byte from scale_a, B's from scale_b.  The accumulator is tied to the
// destination registers (the builtin in VGPR form may give the result registers of
// its own and copy it back on every iteration, and, being free of side effects, is
// moved across the phase structure).  The compiler inserts no wait states around an
// instruction it cannot see: operands must not be written by a vector instruction just
// ahead of it (callers keep constants opaque so they are not rematerialised there; a
// test scans the built code for that hazard), and results are read only after
// vacc_settle.
__device__ __forceinline__ void mfma_f8_scaled_vacc(f32x16& acc, const i32x8& a, const i32x8& b, int scale_a,
                                                    int scale_b) {
    asm("v_mfma_scale_f32_32x32x64_f8f6f4 %0, %1, %2, %0, %3, %4 op_sel_hi:[0,0,0]"
        : "+v"(acc)
        : "v"(a), "v"(b), "v"(scale_a), "v"(scale_b));
}

// Before any other instruction touches accumulators written by mfma_f8_scaled_vacc:
// an XDL MFMA's result may be read or overwritten by a non-matrix instruction only a
// number of wait states after it that grows with its passes (the CDNA3/CDNA4 ISA
// guides' table of required independent instructions).  The compiler does not insert
// them for inline asm; for its own builtins on gfx950 it inserts 20 after the 16-pass
// FP8 32x32x64 and 12 after the 8-pass BF16 32x32x16, and 24 cover both.  Being
// volatile and tied to every accumulator, this also keeps all of those MFMAs in uniform
// control flow ahead of it.  (tests/test_mfma_hazards.py checks the built code.)
__device__ __forceinline__ void vacc_settle(f32x16 (&o)[4], f32x16& l) {
    asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" : "+v"(o[0]), "+v"(o[1]), "+v"(o[2]), "+v"(o[3]), "+v"(l));
}
__device__ __forceinline__ void vacc_settle(f32x16 (&o)[4]) {
    asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" : "+v"(o[0]), "+v"(o[1]), "+v"(o[2]), "+v"(o[3]));
}

// Workgroup barrier for LDS producer/consumer hand-off: waits for this wave's LDS
// operations only (outstanding global loads keep flowing across it), and fences
// the scheduler on both sides (ALU and matrix instructions that do not touch
// memory could otherwise be moved across s_barrier).
__device__ __forceinline__ void block_sync() {
    __builtin_amdgcn_sched_barrier(0);
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
}

// x / b for many x and one b (the epilogues' O / L): one reciprocal refined by a Newton step,
// then per value q = x y corrected by its residual x - b q (exact with an FMA), Markstein's
// final division step, which rounds like the division itself for the normal b of the
// epilogues (b within a few binades of 1).  b = infinity (a row without keys, x = 0) gives 0:
// y = 0, and the residual uses b = 0 (infinity times the zero quotient would be NaN).
struct Quotient {
    float b, y;
    __device__ __forceinline__ explicit Quotient(float b_) {
        const bool inf = b_ == INFINITY;
        const float r = __builtin_amdgcn_rcpf(b_);
        y = inf ? 0.0f : fmaf(fmaf(-b_, r, 1.0f), r, r);
        b = inf ? 0.0f : b_;
    }
    __device__ __forceinline__ float operator()(float x) const {
        const float q = x * y;
        return fmaf(fmaf(-b, q, x), y, q);
    }
};

__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
    __bf16 x = (__bf16)a, y = (__bf16)b;
    return (uint32_t)__builtin_bit_cast(uint16_t, x) | ((uint32_t)__builtin_bit_cast(uint16_t, y) << 16);
}

}  // namespace attnfwd

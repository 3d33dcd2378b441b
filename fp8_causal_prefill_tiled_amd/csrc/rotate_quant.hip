// Hadamard rotation and per-tensor FP8 (e4m3) quantisation of Q or K for gfx950.
//
// Method: "Zyphra ZYFA: FP8 FlashAttention for AMD MI355X, Up to 1.76x Faster"
// (MarkTechPost), section "How accurate is ZYFA's FP8 attention?": rotating Q and
// K by a Hadamard matrix before their FP8 quantisation cuts the input error to
// about half.  Every (token, head) vector is multiplied along the head dimension
// by the orthonormal Sylvester-Hadamard matrix H_n / sqrt(n), n = 128 (d = 128)
// or three blocks of n = 64 (d = 192); the rotated tensor is then quantised per
// tensor: scale = amax / 448, codes = e4m3 RNE(x / scale), saturating, scale 1
// for an all-zero tensor.  H is orthogonal, so the attention scores of rotated
// Q and K equal the originals: the rotated codes go straight into attn_fwd_fp8.
//
// Layout: rows are contiguous and d is a multiple of n, so the tensor is a
// sequence of n-element blocks.  LB = n/8 consecutive lanes hold one block, 8
// bf16 per lane (one 16-byte load); the fast Walsh-Hadamard transform runs its 3
// low butterfly stages inside the lane and log2(LB) stages across lanes (lane-xor
// moves within the block's aligned lane group, by DPP).  Four stream-ordered launches:
// zero the amax cell; rotate and reduce max|y| (per workgroup, then an atomic max
// on the float's bits, order-preserving for non-negative floats, skipped when
// the cell already holds more); rotate again and quantise with the final scale; turn
// the cell into the scale.  The work is HBM streaming: each of the two passes
// reads the bf16 tensor once, the second writes one byte per element.
#include "common.h"
#include "launch.h"

namespace attnfwd {
namespace {

constexpr float kE4M3Max = 448.0f;
constexpr int kThreads = 256;

// Value of lane i ^ M (M = 1, 2, 4, 8) by data-parallel-primitive moves, no LDS:
// quad permutations give xor 1, 2 and 3; the half-row mirror is xor 7 and the row
// mirror xor 15 within 16 lanes, so xor 4 = (xor 7 then xor 3) and xor 8 = (xor 15
// then xor 7).
template <int M>
__device__ __forceinline__ float xor_lane(float v) {
    constexpr int kQuadXor1 = 0xB1, kQuadXor2 = 0x4E, kQuadXor3 = 0x1B, kRowMirror = 0x140, kRowHalfMirror = 0x141;
    int x = __float_as_int(v);
    if constexpr (M == 1) {
        x = __builtin_amdgcn_update_dpp(0, x, kQuadXor1, 0xF, 0xF, false);
    } else if constexpr (M == 2) {
        x = __builtin_amdgcn_update_dpp(0, x, kQuadXor2, 0xF, 0xF, false);
    } else if constexpr (M == 4) {
        x = __builtin_amdgcn_update_dpp(0, x, kRowHalfMirror, 0xF, 0xF, false);
        x = __builtin_amdgcn_update_dpp(0, x, kQuadXor3, 0xF, 0xF, false);
    } else {
        static_assert(M == 8, "xor within 16 lanes");
        x = __builtin_amdgcn_update_dpp(0, x, kRowMirror, 0xF, 0xF, false);
        x = __builtin_amdgcn_update_dpp(0, x, kRowHalfMirror, 0xF, 0xF, false);
    }
    return __int_as_float(x);
}

// One cross-lane butterfly stage over the U blocks a lane holds: partner lane
// t ^ M (lower index a + b, upper a - b).
template <int M, int NU>
__device__ __forceinline__ void cross_stage(float (&x)[NU][8], int t) {
    const bool upper = (t & M) != 0;
#pragma unroll
    for (int u = 0; u < NU; ++u)
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const float p = xor_lane<M>(x[u][i]);
            x[u][i] = upper ? p - x[u][i] : x[u][i] + p;
        }
}

// Unnormalised transform of NU blocks at once (each stage runs over all of them
// before the next, so consecutive dependent lane moves are far apart), y_i =
// sum_j (-1)^popcount(i & j) x_j: bit b of the element index is one butterfly
// stage (lower index a + b, upper a - b).  Lane t of a block holds elements
// 8t .. 8t+7.
template <int LB, int NU>
__device__ __forceinline__ void fwht(float (&x)[NU][8], int t) {
#pragma unroll
    for (int h = 1; h < 8; h <<= 1)
#pragma unroll
        for (int u = 0; u < NU; ++u)
#pragma unroll
            for (int i = 0; i < 8; ++i)
                if (!(i & h)) {
                    const float a = x[u][i], b = x[u][i + h];
                    x[u][i] = a + b;
                    x[u][i + h] = a - b;
                }
    static_assert(LB == 8 || LB == 16, "blocks of 64 or 128 elements");
    cross_stage<1>(x, t);
    cross_stage<2>(x, t);
    cross_stage<4>(x, t);
    if constexpr (LB == 16) cross_stage<8>(x, t);
}

// The 8 bf16 of lane t of block blk as fp32 (zeros past the end; every lane then
// still takes part in the shuffles).
__device__ __forceinline__ void load_block(const __bf16* x, int64_t blk, int64_t nblocks, int nb, int t,
                                           float (&v)[8]) {
    i32x4 raw = {0, 0, 0, 0};
    if (blk < nblocks) raw = load16(x + blk * nb + 8 * t);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        v[2 * i] = __int_as_float(raw[i] << 16);
        v[2 * i + 1] = __int_as_float(raw[i] & (int)0xffff0000);
    }
}

template <int NB>
constexpr float inv_sqrt_nb() {
    return NB == 128 ? 0.088388347648318440550f : 0.125f;   // 1/sqrt(128), 1/sqrt(64)
}

__global__ void rq_init(unsigned* cell) { *cell = 0u; }

// Each wave takes U consecutive 1 KiB steps (BPW blocks each, contiguous in
// memory) and issues all U loads before using any, so every lane keeps U 16-byte
// loads in flight.
constexpr int U = 4;

// The max pass runs a fixed grid of grid-stride workgroups: each wave loops over
// groups of U steps, and each workgroup ends with one reduction and at most one
// atomic (these are device-scope operations on one address, served beyond the
// per-XCD L2s, so their number is kept small).
constexpr int kAmaxGrid = 2048;

template <int NB>
__global__ void __launch_bounds__(kThreads) rq_amax(const __bf16* __restrict__ x, int64_t nblocks, unsigned* cell) {
    constexpr int LB = NB / 8, BPW = 64 / LB;
    const int lane = threadIdx.x & 63, t = lane % LB;
    const int64_t wave = ((int64_t)blockIdx.x * kThreads + threadIdx.x) >> 6;
    const int64_t nwave = ((int64_t)gridDim.x * kThreads) >> 6;
    float m = 0.0f;
    for (int64_t w0 = wave * U; w0 * BPW < nblocks; w0 += nwave * U) {
        float v[U][8];
#pragma unroll
        for (int u = 0; u < U; ++u) load_block(x, (w0 + u) * BPW + lane / LB, nblocks, NB, t, v[u]);
        fwht<LB>(v, t);
#pragma unroll
        for (int u = 0; u < U; ++u)
#pragma unroll
            for (int i = 0; i < 8; ++i) m = fmaxf(m, fabsf(v[u][i]));
    }
    // max |y| of the normalised rotation: scaling by a positive constant commutes
    // with the maximum, rounding included
    m *= inv_sqrt_nb<NB>();
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) m = fmaxf(m, __shfl_xor(m, o, 64));
    __shared__ float wmax[kThreads / 64];
    if (lane == 0) wmax[threadIdx.x >> 6] = m;
    __syncthreads();
    if (threadIdx.x == 0) {
#pragma unroll
        for (int i = 1; i < kThreads / 64; ++i) m = fmaxf(m, wmax[i]);
        // the running maximum is usually larger already: read it and skip the atomic
        if (__float_as_uint(m) > __hip_atomic_load(cell, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT))
            atomicMax(cell, __float_as_uint(m));
    }
}

__device__ __forceinline__ float scale_of(float amax) { return amax > 0.0f ? amax / kE4M3Max : 1.0f; }

template <int NB>
__global__ void __launch_bounds__(kThreads) rq_quant(const __bf16* __restrict__ x, int64_t nblocks,
                                                     const unsigned* cell, uint8_t* __restrict__ out) {
    constexpr int LB = NB / 8, BPW = 64 / LB;
    const int lane = threadIdx.x & 63, t = lane % LB;
    const int64_t wave = ((int64_t)blockIdx.x * kThreads + threadIdx.x) >> 6;
    float v[U][8];
#pragma unroll
    for (int u = 0; u < U; ++u) load_block(x, (wave * U + u) * BPW + lane / LB, nblocks, NB, t, v[u]);
    // one multiply per element by 1/(sqrt(n) scale): within an ulp of dividing the
    // normalised value by the scale, so the rounding to e4m3 can differ only at ties
    const float f = inv_sqrt_nb<NB>() / scale_of(__uint_as_float(*cell));
    fwht<LB>(v, t);
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const int64_t blk = (wave * U + u) * BPW + lane / LB;
        float q[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) q[i] = fminf(fmaxf(v[u][i] * f, -kE4M3Max), kE4M3Max);
        int w0 = __builtin_amdgcn_cvt_pk_fp8_f32(q[0], q[1], 0, false);
        w0 = __builtin_amdgcn_cvt_pk_fp8_f32(q[2], q[3], w0, true);
        int w1 = __builtin_amdgcn_cvt_pk_fp8_f32(q[4], q[5], 0, false);
        w1 = __builtin_amdgcn_cvt_pk_fp8_f32(q[6], q[7], w1, true);
        if (blk < nblocks) *reinterpret_cast<int2*>(out + blk * NB + 8 * t) = make_int2(w0, w1);
    }
}

__global__ void rq_finish(unsigned* cell) {
    *reinterpret_cast<float*>(cell) = scale_of(__uint_as_float(*cell));
}

template <int NB>
hipError_t launch_t(const __bf16* x, uint8_t* x8, unsigned* cell, int64_t n_el, hipStream_t s) {
    const int64_t nblocks = n_el / NB;
    constexpr int BPW = 64 / (NB / 8);
    constexpr int64_t per_wg = (int64_t)BPW * U * (kThreads / 64);   // blocks per workgroup
    hipLaunchKernelGGL(rq_init, dim3(1), dim3(1), 0, s, cell);
    if (nblocks > 0) {
        const int64_t grid = (nblocks + per_wg - 1) / per_wg;
        if (grid > 0x7fffffffLL) return hipErrorInvalidConfiguration;
        const unsigned agrid = (unsigned)(grid < kAmaxGrid ? grid : kAmaxGrid);
        hipLaunchKernelGGL((rq_amax<NB>), dim3(agrid), dim3(kThreads), 0, s, x, nblocks, cell);
        hipLaunchKernelGGL((rq_quant<NB>), dim3((unsigned)grid), dim3(kThreads), 0, s, x, nblocks, cell, x8);
    }
    hipLaunchKernelGGL(rq_finish, dim3(1), dim3(1), 0, s, cell);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_rotate_quant(const void* x, void* x8, float* scale, int64_t n_el, int d, hipStream_t s) {
    auto* cell = reinterpret_cast<unsigned*>(scale);
    if (d % 128 == 0) return launch_t<128>(static_cast<const __bf16*>(x), static_cast<uint8_t*>(x8), cell, n_el, s);
    if (d % 64 == 0) return launch_t<64>(static_cast<const __bf16*>(x), static_cast<uint8_t*>(x8), cell, n_el, s);
    return hipErrorInvalidValue;
}

}  // namespace attnfwd

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
// low butterfly stages inside the lane and log2(LB) stages across lanes (xor
// shuffles within the block's aligned lane group).  Four stream-ordered launches:
// zero the amax cell; rotate and reduce max|y| (one atomic max per wave on the
// float's bits, order-preserving for non-negative floats); rotate again and
// quantise with the final scale; turn the cell into the scale.  The work is HBM
// streaming: each of the two passes reads the bf16 tensor once, the second
// writes one byte per element.
#include "common.h"
#include "launch.h"

namespace attnfwd {
namespace {

constexpr float kE4M3Max = 448.0f;
constexpr int kThreads = 256;

// Unnormalised transform of one block, y_i = sum_j (-1)^popcount(i & j) x_j: bit
// b of the element index is one butterfly stage (lower index a + b, upper a - b).
// Lane t of the block holds elements 8t .. 8t+7.
template <int LB>
__device__ __forceinline__ void fwht(float (&x)[8], int t) {
#pragma unroll
    for (int h = 1; h < 8; h <<= 1)
#pragma unroll
        for (int i = 0; i < 8; ++i)
            if (!(i & h)) {
                const float a = x[i], b = x[i + h];
                x[i] = a + b;
                x[i + h] = a - b;
            }
#pragma unroll
    for (int m = 1; m < LB; m <<= 1) {
        const bool upper = (t & m) != 0;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const float p = __shfl_xor(x[i], m, 64);
            x[i] = upper ? p - x[i] : x[i] + p;
        }
    }
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

template <int NB>
__global__ void __launch_bounds__(kThreads) rq_amax(const __bf16* __restrict__ x, int64_t nblocks, unsigned* cell) {
    constexpr int LB = NB / 8, BPW = 64 / LB;
    const int lane = threadIdx.x & 63, t = lane % LB;
    const int64_t wave = ((int64_t)blockIdx.x * kThreads + threadIdx.x) >> 6;
    const int64_t nwave = ((int64_t)gridDim.x * kThreads) >> 6;
    float m = 0.0f;
    for (int64_t b0 = wave * BPW; b0 < nblocks; b0 += nwave * BPW) {
        float v[8];
        load_block(x, b0 + lane / LB, nblocks, NB, t, v);
        fwht<LB>(v, t);
#pragma unroll
        for (int i = 0; i < 8; ++i) m = fmaxf(m, fabsf(v[i]));
    }
    // max |y| of the normalised rotation: scaling by a positive constant commutes
    // with the maximum, rounding included
    m *= inv_sqrt_nb<NB>();
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) m = fmaxf(m, __shfl_xor(m, o, 64));
    if (lane == 0) atomicMax(cell, __float_as_uint(m));
}

__device__ __forceinline__ float scale_of(float amax) { return amax > 0.0f ? amax / kE4M3Max : 1.0f; }

template <int NB>
__global__ void __launch_bounds__(kThreads) rq_quant(const __bf16* __restrict__ x, int64_t nblocks,
                                                     const unsigned* cell, uint8_t* __restrict__ out) {
    constexpr int LB = NB / 8, BPW = 64 / LB;
    const int lane = threadIdx.x & 63, t = lane % LB;
    const int64_t wave = ((int64_t)blockIdx.x * kThreads + threadIdx.x) >> 6;
    const int64_t nwave = ((int64_t)gridDim.x * kThreads) >> 6;
    const float scale = scale_of(__uint_as_float(*cell));
    for (int64_t b0 = wave * BPW; b0 < nblocks; b0 += nwave * BPW) {
        const int64_t blk = b0 + lane / LB;
        float v[8];
        load_block(x, blk, nblocks, NB, t, v);
        fwht<LB>(v, t);
        float q[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) q[i] = fminf(fmaxf(v[i] * inv_sqrt_nb<NB>() / scale, -kE4M3Max), kE4M3Max);
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
    hipLaunchKernelGGL(rq_init, dim3(1), dim3(1), 0, s, cell);
    if (nblocks > 0) {
        const int64_t want = (nblocks + BPW * (kThreads / 64) - 1) / (BPW * (kThreads / 64));
        const unsigned grid = (unsigned)(want < 4096 ? want : 4096);   // grid-stride beyond 4096 workgroups
        hipLaunchKernelGGL((rq_amax<NB>), dim3(grid), dim3(kThreads), 0, s, x, nblocks, cell);
        hipLaunchKernelGGL((rq_quant<NB>), dim3(grid), dim3(kThreads), 0, s, x, nblocks, cell, x8);
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

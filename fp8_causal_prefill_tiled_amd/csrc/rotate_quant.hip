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
// Rotation on the matrix cores.  Rows are contiguous and d is a multiple of n, so
// the tensor is a sequence of n-element blocks, n = 32 NA.  The Sylvester matrix
// factors as H_n = H_NA (x) H_32, so for a block split into NA chunks x_a of 32,
//     z_a = x_a H_32                   (matrix cores: exact bf16 inputs, fp32 sums)
//     y_b = sum_a H_NA[a][b] z_a       (an NA-point butterfly inside the lane, fp32)
// is y = x H_n.  A wave takes 32 consecutive blocks and computes the product
// transposed, Z_a^T = H_32 . X_a^T, with two v_mfma_f32_32x32x16_bf16 per chunk:
// the A operand is H_32 (constant +-1 in registers), the B operand the blocks, so
// each lane loads 16 contiguous bytes of one block per operand and ends holding,
// for block l%32, the rotated columns 8(r/4) + 4(l/32) + r%4 of every chunk: four
// consecutive columns per group of four accumulators, one 32-bit store of e4m3
// codes.  The vector work left is NA log2(NA) adds per 32 elements plus the
// maximum or the quantisation, so both passes stream at HBM rate.
//
// Four stream-ordered launches: zero the amax cell; rotate and reduce max|y| (per
// workgroup, then an atomic max on the float's bits, order-preserving for
// non-negative floats, skipped when the cell already holds more); rotate again
// and quantise with the final scale; turn the cell into the scale.  Each of the
// two passes reads the bf16 tensor once, the second writes one byte per element.
#include "common.h"
#include "launch.h"

namespace attnfwd {
namespace {

constexpr float kE4M3Max = 448.0f;
constexpr int kThreads = 256;
constexpr int U = 2;   // 32-block units per wave and loop step (loads in flight)

// Rows of the H_32 A operand held by this lane for K half kk: element i is
// H_32[l % 32][16 kk + 8 (l / 32) + i] = (-1)^popcount(row & col), as bf16.
__device__ __forceinline__ bf16x8 h32_operand(int lane, int kk) {
    const int row = lane & 31, col0 = 16 * kk + 8 * (lane >> 5);
    i16x8 bits;
#pragma unroll
    for (int i = 0; i < 8; ++i) bits[i] = (__builtin_popcount(row & (col0 + i)) & 1) ? (short)0xBF80 : (short)0x3F80;
    return __builtin_bit_cast(bf16x8, bits);
}

// Bytes of one bf16 block row in the LDS staging tile: padded by 16 so that the
// 16-byte operand reads of 32 rows fall on spread banks and stay aligned.
template <int NA>
constexpr int kInRow = 64 * NA + 16;

// Global -> registers -> LDS for U units of 32 blocks (each unit 64 NA bytes per
// block, contiguous): every load instruction reads 1 KiB of consecutive bytes.
// Blocks at or past nblocks read as zeros.
template <int NA>
__device__ __forceinline__ void stage_in(const __bf16* __restrict__ x, int64_t unit0, int64_t nblocks, int lane,
                                         ATTN_LDS uint8_t* tile) {
    constexpr int NB = 32 * NA, CPB = NB * 2 / 16;           // 16-byte chunks per block
    constexpr int IT = 32 * CPB / 64;                         // chunks per lane and unit
    i32x4 v[U][IT];
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
        for (int it = 0; it < IT; ++it) {
            const int k = it * 64 + lane, c = k / CPB;
            const int64_t blk = (unit0 + u) * 32 + c;
            v[u][it] = blk < nblocks ? load16(x + blk * NB + 8 * (k % CPB)) : i32x4{0, 0, 0, 0};
        }
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
        for (int it = 0; it < IT; ++it) {
            const int k = it * 64 + lane;
            lds_store16(tile + (u * 32 + k / CPB) * kInRow<NA> + 16 * (k % CPB), v[u][it]);
        }
}

// The NA-chunk rotation of one staged unit of 32 blocks, transposed: y[b][r] is
// column 32 b + 8 (r/4) + 4 (lane/32) + r%4 of block lane % 32 (unnormalised).
template <int NA>
__device__ __forceinline__ void rotate32(const ATTN_LDS uint8_t* unit_tile, int lane, const bf16x8 (&h)[2],
                                         f32x16 (&y)[NA]) {
    // B operand: lane l holds elements 32a + 16kk + 8(l/32) .. +7 of block l%32
    const ATTN_LDS uint8_t* p = unit_tile + (lane & 31) * kInRow<NA> + 16 * (lane >> 5);
    bf16x8 xb[NA][2];
#pragma unroll
    for (int a = 0; a < NA; ++a)
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) xb[a][kk] = __builtin_bit_cast(bf16x8, lds_load16(p + 64 * a + 32 * kk));
#pragma unroll
    for (int a = 0; a < NA; ++a) {
        y[a] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(h[0], xb[a][0], f32x16{0}, 0, 0, 0);
        y[a] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(h[1], xb[a][1], y[a], 0, 0, 0);
    }
    // y_b = sum_a H_NA[a][b] z_a: butterflies over the chunk index, inside the lane
#pragma unroll
    for (int st = 1; st < NA; st <<= 1)
#pragma unroll
        for (int a = 0; a < NA; ++a)
            if (!(a & st)) {
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const float u = y[a][r], v = y[a + st][r];
                    y[a][r] = u + v;
                    y[a + st][r] = u - v;
                }
            }
}

// Orders this wave's LDS writes before its reads of other lanes' data (and the
// reads before the next writes): LDS operations of one wave complete in order.
__device__ __forceinline__ void wave_lds_sync() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

template <int NB>
constexpr float inv_sqrt_nb() {
    return NB == 128 ? 0.088388347648318440550f : 0.125f;   // 1/sqrt(128), 1/sqrt(64)
}

__global__ void rq_init(unsigned* cell) { *cell = 0u; }

// Max over the workgroup of the per-thread maxima m of |y| (unnormalised), scaled to
// the normalised rotation (a positive constant commutes with the maximum, rounding
// included), folded into *cell by an atomic max on the float's bits (order-
// preserving for non-negative floats), skipped when the cell already holds more.
template <int NB>
__device__ __forceinline__ void commit_max(float m, int lane, unsigned* cell) {
    m *= inv_sqrt_nb<NB>();
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) m = fmaxf(m, __shfl_xor(m, o, 64));
    __shared__ float wmax[kThreads / 64];
    if (lane == 0) wmax[threadIdx.x >> 6] = m;
    __syncthreads();
    if (threadIdx.x == 0) {
#pragma unroll
        for (int i = 1; i < kThreads / 64; ++i) m = fmaxf(m, wmax[i]);
        if (__float_as_uint(m) > __hip_atomic_load(cell, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT))
            atomicMax(cell, __float_as_uint(m));
    }
}

// The max pass runs a fixed grid of grid-stride workgroups: each wave loops over
// steps of U units of 32 blocks, and each workgroup ends with one reduction and
// at most one atomic (device-scope operations on one address, served beyond the
// per-XCD L2s, so their number is kept small).
constexpr int kAmaxGrid = 2048;

template <int NB>
__global__ void __launch_bounds__(kThreads) rq_amax(const __bf16* __restrict__ x, int64_t nblocks, unsigned* cell) {
    constexpr int NA = NB / 32;
    __shared__ __attribute__((aligned(16))) uint8_t in_raw[kThreads / 64][U * 32 * kInRow<NA>];
    const int lane = threadIdx.x & 63;
    ATTN_LDS uint8_t* tile = (ATTN_LDS uint8_t*)in_raw[threadIdx.x >> 6];
    const int64_t wave = ((int64_t)blockIdx.x * kThreads + threadIdx.x) >> 6;
    const int64_t nwave = ((int64_t)gridDim.x * kThreads) >> 6;
    const bf16x8 h[2] = {h32_operand(lane, 0), h32_operand(lane, 1)};
    float m = 0.0f;
    for (int64_t u0 = wave * U; u0 * 32 < nblocks; u0 += nwave * U) {
        stage_in<NA>(x, u0, nblocks, lane, tile);
        wave_lds_sync();
#pragma unroll
        for (int u = 0; u < U; ++u) {
            f32x16 y[NA];
            rotate32<NA>(tile + u * 32 * kInRow<NA>, lane, h, y);
#pragma unroll
            for (int a = 0; a < NA; ++a)
#pragma unroll
                for (int r = 0; r < 16; ++r) m = fmaxf(m, fabsf(y[a][r]));
        }
        wave_lds_sync();
    }
    commit_max<NB>(m, lane, cell);
}

__device__ __forceinline__ float scale_of(float amax) { return amax > 0.0f ? amax / kE4M3Max : 1.0f; }

// PRESCALED: quantise with the caller's scale (*scale) instead of the amax cell of
// the max pass, and, when amax_out is given, fold this tensor's max |y| into it (one
// pass: the scale comes from an earlier step, the maximum is for the next one).
template <int NB, bool PRESCALED>
__global__ void __launch_bounds__(kThreads) rq_quant(const __bf16* __restrict__ x, int64_t nblocks,
                                                     const unsigned* cell, const float* scale, unsigned* amax_out,
                                                     uint8_t* __restrict__ out) {
    constexpr int NA = NB / 32;
    // The codes of a unit (32 blocks, contiguous in memory) go through LDS so that the
    // global stores are whole 16-byte chunks: rows of NB + 16 bytes keep the 16-byte
    // reads aligned and spread the 4-byte writes over the banks.
    constexpr int ROW = NB + 16;
    static_assert(32 * ROW <= U * 32 * kInRow<NA>, "the output staging reuses the input tile");
    __shared__ __attribute__((aligned(16))) uint8_t in_raw[kThreads / 64][U * 32 * kInRow<NA>];
    const int lane = threadIdx.x & 63;
    const int wv = threadIdx.x >> 6;
    ATTN_LDS uint8_t* tile = (ATTN_LDS uint8_t*)in_raw[wv];
    ATTN_LDS uint8_t* stage = tile;   // free once every unit's operands are in registers
    const int64_t wave = ((int64_t)blockIdx.x * kThreads + threadIdx.x) >> 6;
    const bf16x8 h[2] = {h32_operand(lane, 0), h32_operand(lane, 1)};
    stage_in<NA>(x, wave * U, nblocks, lane, tile);
    wave_lds_sync();
    f32x16 y[U][NA];
#pragma unroll
    for (int u = 0; u < U; ++u) rotate32<NA>(tile + u * 32 * kInRow<NA>, lane, h, y[u]);
    wave_lds_sync();
    // one multiply per element by 1/(sqrt(n) scale): within an ulp of dividing the
    // normalised value by the scale, so the rounding to e4m3 can differ only at ties
    const float f = inv_sqrt_nb<NB>() / (PRESCALED ? *scale : scale_of(__uint_as_float(*cell)));
    if constexpr (PRESCALED) {
        if (amax_out != nullptr) {   // uniform: the same pointer in every thread
            float m = 0.0f;
#pragma unroll
            for (int u = 0; u < U; ++u)
#pragma unroll
                for (int a = 0; a < NA; ++a)
#pragma unroll
                    for (int r = 0; r < 16; ++r) m = fmaxf(m, fabsf(y[u][a][r]));
            commit_max<NB>(m, lane, amax_out);
        }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
        // accumulators 4g..4g+3 of chunk a: columns 32a + 8g + 4(lane/32) + 0..3 of
        // block lane%32, one 32-bit word of codes
        ATTN_LDS uint8_t* row = stage + (lane & 31) * ROW + 4 * (lane >> 5);
#pragma unroll
        for (int a = 0; a < NA; ++a)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                float q[4];
#pragma unroll
                for (int t = 0; t < 4; ++t) q[t] = fminf(fmaxf(y[u][a][4 * g + t] * f, -kE4M3Max), kE4M3Max);
                int w = __builtin_amdgcn_cvt_pk_fp8_f32(q[0], q[1], 0, false);
                w = __builtin_amdgcn_cvt_pk_fp8_f32(q[2], q[3], w, true);
                *reinterpret_cast<ATTN_LDS int*>(row + 32 * a + 8 * g) = w;
            }
        wave_lds_sync();
        // 16-byte chunk k of the unit's 32 NB contiguous output bytes: block k / (NB/16)
        const int64_t blk0 = (wave * U + u) * 32;
#pragma unroll
        for (int it = 0; it < NB / 32; ++it) {
            const int k = it * 64 + lane;
            const int c = k / (NB / 16), col = 16 * (k % (NB / 16));
            const i32x4 v = lds_load16(stage + c * ROW + col);
            if (blk0 + c < nblocks) *reinterpret_cast<i32x4*>(out + (blk0 + c) * NB + col) = v;
        }
        wave_lds_sync();
    }
}

__global__ void rq_finish(unsigned* cell) {
    *reinterpret_cast<float*>(cell) = scale_of(__uint_as_float(*cell));
}

template <int NB>
hipError_t launch_t(const __bf16* x, uint8_t* x8, unsigned* cell, int64_t n_el, hipStream_t s) {
    const int64_t nblocks = n_el / NB;
    constexpr int64_t per_wg = (int64_t)32 * U * (kThreads / 64);   // blocks per workgroup
    hipLaunchKernelGGL(rq_init, dim3(1), dim3(1), 0, s, cell);
    if (nblocks > 0) {
        const int64_t grid = (nblocks + per_wg - 1) / per_wg;
        if (grid > 0x7fffffffLL) return hipErrorInvalidConfiguration;
        const unsigned agrid = (unsigned)(grid < kAmaxGrid ? grid : kAmaxGrid);
        hipLaunchKernelGGL((rq_amax<NB>), dim3(agrid), dim3(kThreads), 0, s, x, nblocks, cell);
        hipLaunchKernelGGL((rq_quant<NB, false>), dim3((unsigned)grid), dim3(kThreads), 0, s, x, nblocks, cell,
                           nullptr, nullptr, x8);
    }
    hipLaunchKernelGGL(rq_finish, dim3(1), dim3(1), 0, s, cell);
    return hipGetLastError();
}

template <int NB>
hipError_t launch_pre_t(const __bf16* x, uint8_t* x8, const float* scale, unsigned* amax, int64_t n_el,
                        hipStream_t s) {
    const int64_t nblocks = n_el / NB;
    constexpr int64_t per_wg = (int64_t)32 * U * (kThreads / 64);
    if (amax) hipLaunchKernelGGL(rq_init, dim3(1), dim3(1), 0, s, amax);
    if (nblocks > 0) {
        const int64_t grid = (nblocks + per_wg - 1) / per_wg;
        if (grid > 0x7fffffffLL) return hipErrorInvalidConfiguration;
        hipLaunchKernelGGL((rq_quant<NB, true>), dim3((unsigned)grid), dim3(kThreads), 0, s, x, nblocks, nullptr,
                           scale, amax, x8);
    }
    return hipGetLastError();
}

}  // namespace

hipError_t launch_rotate_quant_prescaled(const void* x, void* x8, const float* scale, float* amax, int64_t n_el,
                                         int d, hipStream_t s) {
    auto* cell = reinterpret_cast<unsigned*>(amax);
    if (d % 128 == 0)
        return launch_pre_t<128>(static_cast<const __bf16*>(x), static_cast<uint8_t*>(x8), scale, cell, n_el, s);
    if (d % 64 == 0)
        return launch_pre_t<64>(static_cast<const __bf16*>(x), static_cast<uint8_t*>(x8), scale, cell, n_el, s);
    return hipErrorInvalidValue;
}

hipError_t launch_rotate_quant(const void* x, void* x8, float* scale, int64_t n_el, int d, hipStream_t s) {
    auto* cell = reinterpret_cast<unsigned*>(scale);
    if (d % 128 == 0) return launch_t<128>(static_cast<const __bf16*>(x), static_cast<uint8_t*>(x8), cell, n_el, s);
    if (d % 64 == 0) return launch_t<64>(static_cast<const __bf16*>(x), static_cast<uint8_t*>(x8), cell, n_el, s);
    return hipErrorInvalidValue;
}

}  // namespace attnfwd

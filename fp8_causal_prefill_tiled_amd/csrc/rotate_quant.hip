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
constexpr int kWaves = kThreads / 64;

// Rows of the H_32 A operand held by this lane for K half kk: element i is
// H_32[l % 32][16 kk + 8 (l / 32) + i] = (-1)^popcount(row & col), as bf16.
__device__ __forceinline__ bf16x8 h32_operand(int lane, int kk) {
    const int row = lane & 31, col0 = 16 * kk + 8 * (lane >> 5);
    i16x8 bits;
#pragma unroll
    for (int i = 0; i < 8; ++i) bits[i] = (__builtin_popcount(row & (col0 + i)) & 1) ? (short)0xBF80 : (short)0x3F80;
    return __builtin_bit_cast(bf16x8, bits);
}

// A unit is 32 consecutive n-element blocks (32 rows of 2n bytes of bf16, contiguous in
// memory).  It moves from HBM to an LDS tile with direct loads (buffer_load ... lds), 1 KiB
// of consecutive bytes per instruction, and is read back as MFMA operands.  Rows are not
// padded: the 16-byte chunks of row r sit at chunk position (chunk ^ swz(r)), which puts
// the operand reads of 16 consecutive rows (one logical chunk each) on 16 distinct groups
// of banks.
template <int NB>
struct RqTile {
    static constexpr int NA = NB / 32;             // 32-element chunks per block
    static constexpr int ROWB = 2 * NB;            // bytes per block row
    static constexpr int UNIT = 32 * ROWB;         // bytes per unit
    static constexpr int NDMA = UNIT / 1024;       // direct loads per unit
    static constexpr int OROW = NB + 16;           // output staging row (codes), padded
    static_assert(32 * OROW <= UNIT, "the output staging reuses the unit's tile");
    __device__ static int swz(int row) { return NB == 128 ? (row & 15) : ((row >> 1) & 7); }
};

// Direct HBM -> LDS load of 16 bytes per lane (lane i writes LDS bytes [l + 16 i, +16)
// from buffer offset v).  Inline asm, so the compiler does not wait for it before every
// LDS access; the waits are explicit (s_waitcnt vmcnt).  M0 is saved and restored; the
// s_nop covers the wait states a buffer instruction needs after its descriptor SGPRs were
// written by v_readfirstlane.
__device__ __forceinline__ void dma16(i32x4 r, int v, unsigned l) {
    int t;
    asm volatile(
        "s_mov_b32 %0, m0\n\t"
        "s_mov_b32 m0, %2\n\t"
        "s_nop 4\n\t"
        "buffer_load_dwordx4 %1, %3, 0 offen lds\n\t"
        "s_mov_b32 m0, %0"
        : "=&s"(t)
        : "v"(v), "s"(l), "s"(r)
        : "memory");
}

// Buffer resource words over [base, base + bytes): loads at or past `bytes` return zeros.
__device__ __forceinline__ i32x4 rsrc_words(const void* base, int bytes) {
    const unsigned long long a = (unsigned long long)base;
    return i32x4{__builtin_amdgcn_readfirstlane((int)a), __builtin_amdgcn_readfirstlane((int)(a >> 32)) & 0xffff,
                 __builtin_amdgcn_readfirstlane(bytes), 0x00020000};
}

// Issue the direct loads of unit `unit` into the LDS tile at `lds` (blocks at or past
// nblocks read as zeros).  Lane i of load m fills physical row (1024 m + 16 i) / ROWB,
// chunk position (16 i / 16) % (ROWB / 16), with the logical chunk that position holds.
template <int NB>
__device__ __forceinline__ void load_unit(const __bf16* x, int64_t unit, int64_t nblocks, int lane, unsigned lds) {
    using T = RqTile<NB>;
    const int64_t b0 = unit * 32;
    const int64_t left = nblocks - b0;
    const int rows = left <= 0 ? 0 : left >= 32 ? 32 : (int)left;
    const i32x4 r = rsrc_words(x + (b0 < nblocks ? b0 : 0) * NB, rows * T::ROWB);
#pragma unroll
    for (int m = 0; m < T::NDMA; ++m) {
        const int byte = 1024 * m + 16 * lane;
        const int row = byte / T::ROWB, pos = (byte % T::ROWB) / 16;
        dma16(r, row * T::ROWB + 16 * (pos ^ T::swz(row)), lds + 1024 * m);
    }
}

// The rotation of one unit of 32 blocks from its LDS tile, transposed: y[b][r] is column
// 32 b + 8 (r/4) + 4 (lane/32) + r%4 of block lane % 32 (unnormalised).
template <int NB>
__device__ __forceinline__ void rotate_unit(const ATTN_LDS uint8_t* tile, int lane, const bf16x8 (&h)[2],
                                            f32x16 (&y)[RqTile<NB>::NA]) {
    using T = RqTile<NB>;
    constexpr int NA = T::NA;
    // B operand: lane l holds elements 32a + 16kk + 8(l/32) .. +7 of block l%32
    const int row = lane & 31;
    const ATTN_LDS uint8_t* p = tile + row * T::ROWB;
    bf16x8 xb[NA][2];
#pragma unroll
    for (int a = 0; a < NA; ++a)
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
            const int chunk = 4 * a + 2 * kk + (lane >> 5);
            xb[a][kk] = __builtin_bit_cast(bf16x8, lds_load16(p + 16 * (chunk ^ T::swz(row))));
        }
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
    __shared__ float wmax[kWaves];
    if (lane == 0) wmax[threadIdx.x >> 6] = m;
    __syncthreads();
    if (threadIdx.x == 0) {
#pragma unroll
        for (int i = 1; i < kWaves; ++i) m = fmaxf(m, wmax[i]);
        if (__float_as_uint(m) > __hip_atomic_load(cell, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT))
            atomicMax(cell, __float_as_uint(m));
    }
}

__device__ __forceinline__ float scale_of(float amax) { return amax > 0.0f ? amax / kE4M3Max : 1.0f; }

// One streaming kernel for both passes.  A fixed grid of workgroups; every wave walks the
// units wave, wave + W, ... (W waves in the grid) with two LDS tiles: the direct loads of
// its next unit are in flight while it rotates the current one.
//   MODE 0: max |rotated| into *cell (the first pass).
//   MODE 1: quantise with the scale the first pass left in *cell.
//   MODE 2: quantise with *scale (one pass), and fold max |rotated| into *amax_out when
//           that pointer is not null.
// Quantisation: one multiply per element by 1/(sqrt(n) scale), within an ulp of dividing
// the normalised value by the scale, so the rounding to e4m3 can differ only at ties;
// saturate at +-448, RNE convert.  The codes of a unit go through the LDS tile (rows of
// n + 16 bytes) so that the global stores are whole 16-byte chunks.
// Workgroups resident per CU: LDS-bound (two 8 KiB tiles per wave at n = 128, 4 KiB at
// n = 64); the grid is one full wave of them over the 256 CUs.
template <int NB>
constexpr int kStreamGrid = 256 * (NB == 128 ? 2 : 4);

template <int NB, int MODE>
__global__ void __launch_bounds__(kThreads) rq_stream(const __bf16* __restrict__ x, int64_t nblocks,
                                                      unsigned* cell, const float* scale, unsigned* amax_out,
                                                      uint8_t* __restrict__ out) {
    using T = RqTile<NB>;
    constexpr int NA = T::NA;
    __shared__ __attribute__((aligned(16))) uint8_t tiles_raw[kWaves][2][T::UNIT];
    const int lane = threadIdx.x & 63;
    const int wv = threadIdx.x >> 6;
    ATTN_LDS uint8_t* tiles = (ATTN_LDS uint8_t*)tiles_raw[wv];
    const unsigned lds0 = __builtin_amdgcn_readfirstlane((unsigned)(uintptr_t)tiles);
    const int64_t wave = ((int64_t)blockIdx.x * kThreads + threadIdx.x) >> 6;
    const int64_t nwave = ((int64_t)gridDim.x * kThreads) >> 6;
    const int64_t nunits = (nblocks + 31) / 32;
    const bf16x8 h[2] = {h32_operand(lane, 0), h32_operand(lane, 1)};
    const bool want_max = MODE == 0 || (MODE == 2 && amax_out != nullptr);   // uniform
    float f = 0.0f;
    if (MODE == 1) f = inv_sqrt_nb<NB>() / scale_of(__uint_as_float(*cell));
    if (MODE == 2) f = inv_sqrt_nb<NB>() / *scale;
    float m = 0.0f;
    int buf = 0;
    if (wave < nunits) load_unit<NB>(x, wave, nblocks, lane, lds0);
    for (int64_t u = wave; u < nunits; u += nwave, buf ^= 1) {
        // next unit's loads (zeros past the end), then wait for all but those
        load_unit<NB>(x, u + nwave, nblocks, lane, lds0 + (buf ^ 1) * T::UNIT);
        asm volatile("s_waitcnt vmcnt(%0)" ::"n"(T::NDMA) : "memory");
        ATTN_LDS uint8_t* tile = tiles + buf * T::UNIT;
        f32x16 y[NA];
        rotate_unit<NB>(tile, lane, h, y);
        if (want_max) {
#pragma unroll
            for (int a = 0; a < NA; ++a)
#pragma unroll
                for (int r = 0; r < 16; ++r) m = fmaxf(m, fabsf(y[a][r]));
        }
        if constexpr (MODE != 0) {
            wave_lds_sync();   // every operand read of the tile is done: it becomes the output staging
            // accumulators 4g..4g+3 of chunk a: columns 32a + 8g + 4(lane/32) + 0..3 of
            // block lane%32, one 32-bit word of codes
            ATTN_LDS uint8_t* orow = tile + (lane & 31) * T::OROW + 4 * (lane >> 5);
#pragma unroll
            for (int a = 0; a < NA; ++a)
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    float q[4];
#pragma unroll
                    for (int t = 0; t < 4; ++t) q[t] = fminf(fmaxf(y[a][4 * g + t] * f, -kE4M3Max), kE4M3Max);
                    int wd = __builtin_amdgcn_cvt_pk_fp8_f32(q[0], q[1], 0, false);
                    wd = __builtin_amdgcn_cvt_pk_fp8_f32(q[2], q[3], wd, true);
                    *reinterpret_cast<ATTN_LDS int*>(orow + 32 * a + 8 * g) = wd;
                }
            wave_lds_sync();
            // 16-byte chunk k of the unit's 32 NB contiguous output bytes: block k / (NB/16)
            const int64_t blk0 = u * 32;
#pragma unroll
            for (int it = 0; it < NB / 32; ++it) {
                const int k = it * 64 + lane;
                const int c = k / (NB / 16), col = 16 * (k % (NB / 16));
                const i32x4 v = lds_load16(tile + c * T::OROW + col);
                if (blk0 + c < nblocks) *reinterpret_cast<i32x4*>(out + (blk0 + c) * NB + col) = v;
            }
        }
        // the tile's reads are complete before the loads of the unit after next overwrite it
        wave_lds_sync();
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    }
    // the last (empty) prefetch must land before the workgroup's LDS is released
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    if (want_max) commit_max<NB>(m, lane, MODE == 0 ? cell : amax_out);
}

__global__ void rq_finish(unsigned* cell) {
    *reinterpret_cast<float*>(cell) = scale_of(__uint_as_float(*cell));
}

template <int NB>
unsigned stream_grid(int64_t nblocks) {
    const int64_t nunits = (nblocks + 31) / 32;
    const int64_t wgs = (nunits + kWaves - 1) / kWaves;
    return (unsigned)(wgs < kStreamGrid<NB> ? wgs : kStreamGrid<NB>);
}

template <int NB>
hipError_t launch_t(const __bf16* x, uint8_t* x8, unsigned* cell, int64_t n_el, hipStream_t s) {
    const int64_t nblocks = n_el / NB;
    hipLaunchKernelGGL(rq_init, dim3(1), dim3(1), 0, s, cell);
    if (nblocks > 0) {
        const unsigned grid = stream_grid<NB>(nblocks);
        hipLaunchKernelGGL((rq_stream<NB, 0>), dim3(grid), dim3(kThreads), 0, s, x, nblocks, cell, nullptr, nullptr,
                           nullptr);
        hipLaunchKernelGGL((rq_stream<NB, 1>), dim3(grid), dim3(kThreads), 0, s, x, nblocks, cell, nullptr, nullptr,
                           x8);
    }
    hipLaunchKernelGGL(rq_finish, dim3(1), dim3(1), 0, s, cell);
    return hipGetLastError();
}

template <int NB>
hipError_t launch_pre_t(const __bf16* x, uint8_t* x8, const float* scale, unsigned* amax, int64_t n_el,
                        hipStream_t s) {
    const int64_t nblocks = n_el / NB;
    if (amax) hipLaunchKernelGGL(rq_init, dim3(1), dim3(1), 0, s, amax);
    if (nblocks > 0)
        hipLaunchKernelGGL((rq_stream<NB, 2>), dim3(stream_grid<NB>(nblocks)), dim3(kThreads), 0, s, x, nblocks,
                           nullptr, scale, amax, x8);
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

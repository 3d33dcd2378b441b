// Shared device code of the two FP8 attention kernels: tile geometry, kernel
// parameters, the work-item map, scales, the Q load and the output epilogue.  The
// method and the mapping on CDNA4 are described in attn_fwd_fp8.hip.
#pragma once
#include <type_traits>

#include "common.h"
#include "launch.h"

namespace attnfwd {
namespace {

constexpr int KB = 64;               // keys per block = the probability scaling block
constexpr float kRefSlack = 16.0f;   // move the reference only if a block exceeds it by more

template <int DQK>
struct Fp8Tile {
    static constexpr int NKK = DQK / 64;          // 32x32x64 steps over d_qk
    static constexpr int K_STRIDE = DQK + 16;     // padded LDS row of K, bytes
    static constexpr int K_BYTES = KB * K_STRIDE;
    static constexpr int V_BYTES = KB * 128;      // key-major V staging tile, chunk-swizzled
    static constexpr int VT_STRIDE = KB + 16;     // padded LDS row of V^T (one d, 64 keys), bytes
    static constexpr int VT_BYTES = 128 * VT_STRIDE;
    // LDS: 2 slots each of K, V^T and the key-major V staging tile; block j uses slot j%2
    static constexpr int OFF_VT = 2 * K_BYTES;
    static constexpr int OFF_VS = OFF_VT + 2 * VT_BYTES;
    static constexpr int LDS_BYTES = OFF_VS + 2 * V_BYTES;
    static constexpr int K_CHUNKS = KB * DQK / 16;
    static constexpr int V_CHUNKS = KB * 128 / 16;
};

template <int DQK>
struct PairTile {
    static constexpr int NKK = DQK / 64;          // 32x32x64 steps over d_qk
    // K block in LDS: region A holds d in [0, 128) as 128-byte rows, region B (d_qk = 192)
    // d in [128, 192) as 64-byte rows; 16-byte chunks XOR-swizzled by row (kswz_a, kswz_b)
    // so that the operand reads are free of bank conflicts.  Unpadded, so that one wave's
    // direct-to-LDS load fills 1 KB of consecutive rows.
    static constexpr int KA_BYTES = KB * 128;
    static constexpr int K_BYTES = KB * DQK;
    static constexpr int V_BYTES = KB * 128;      // key-major V staging tile, chunk-swizzled
    static constexpr int VT_STRIDE = KB + 16;     // padded LDS row of V^T (one d, 64 keys), bytes
    static constexpr int VT_BYTES = 128 * VT_STRIDE;
    // An iteration covers NB = 2 64-key blocks.  LDS: NSLOT = 2*NB slots each of K, V^T
    // and the key-major V staging tile; block jb uses slot jb % NSLOT.
    static constexpr int NB = 2;
    static constexpr int NSLOT = 2 * NB;
    static constexpr int OFF_VT = NSLOT * K_BYTES;
    static constexpr int OFF_VS = OFF_VT + NSLOT * VT_BYTES;
    static constexpr int LDS_BYTES = OFF_VS + NSLOT * V_BYTES;

};

struct Fp8Params {
    const uint8_t* q;
    const uint8_t* k;
    const uint8_t* v;
    __bf16* o;
    float* lse;     // (B, Hq, S) natural-log normaliser per query row, or null
    float c;        // q_scale * k_scale * sm * log2(e)
    float a8;       // 8 * c, the Lean-P slope
    float v_scale;
    int B, Hq, Hkv, S;
    int n_tiles;    // query tiles per head
    const int* cu;    // variable-length batches: B + 1 query row offsets (device), else null
    int total;        // variable-length batches: rows of the packed Q and O
    const int* cu_k;  // variable-length batches: B + 1 key row offsets (device)
    int total_k;      // variable-length batches: rows of the packed K and V
    const float* dq;  // per-tensor scales in device memory (one float each), or null:
    const float* dk;  //   then c, a8 and v_scale above are used as given
    const float* dv;
    float sm;         // softmax scale (for scales read from device memory)
};

// 16-byte chunk swizzle of a V row in LDS.  The transposing read of one 16-lane
// group touches keys {b..b+3, b+8..b+11} (b = 0 mod 4); this maps them to 8
// distinct chunk positions, so the group's 128 bytes hit distinct banks.
__device__ __forceinline__ int v_swz(int row) { return (row & 3) | (((row >> 3) & 1) << 2); }
// Workgroup barrier after this wave's direct-to-LDS loads and LDS operations have
// completed: the loads' data is then visible to every wave after the barrier.
__device__ __forceinline__ void vmem_lds_sync() {
    __builtin_amdgcn_sched_barrier(0);
    asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
}
// 16-byte chunk swizzles of the K regions: 16 lanes reading the same logical chunk of 16
// consecutive rows hit 16 distinct 16-byte bank groups.
__device__ __forceinline__ int kswz_a(int row) { return (row >> 1) & 7; }   // 128-byte rows
__device__ __forceinline__ int kswz_b(int row) { return (row >> 2) & 3; }   // 64-byte rows

// Work of one workgroup: a 256-query tile of one (sequence, head).  Workgroup L
// takes tile n_tiles-1-L/(B*Hq) (the longest causal prefixes first, for load
// balance) of head L % (B*Hq) (consecutive workgroups take consecutive heads, so
// each XCD keeps the same heads' K/V in its L2).  Sequence b has S query rows from
// packed row tok0 and Sk key rows from packed row tok0k; causal query i sees keys
// j <= i + qoff (qoff = Sk - S, the mask aligned at the bottom right).  Equal-length
// batches are (B, S, H, d) with Sk = S and qoff = 0; a variable-length batch packs
// its sequences along the rows, a.S being the longest query run.  The offsets are
// clamped into the tensors, so any contents of cu and cu_k keep every access inside
// them.
struct Work {
    int b, h, g;            // sequence, query head, key/value head
    int S, Sk, qoff;
    int64_t tok0, tok0k;
    int q0;                 // first query of the tile
    int nblk;               // 64-key blocks the workgroup walks
    int jdiag;              // first block that needs a mask: the diagonal one (causal) or the ragged last one
};

template <bool CAUSAL, bool VARLEN>
__device__ __forceinline__ bool work_of(const Fp8Params& a, Work& u) {
    constexpr int BM = 256;
    const int BH = a.B * a.Hq;
    const int L = blockIdx.x;
    int tile, bh;
    tile_of(L, BH, a.Hq / a.Hkv, a.n_tiles, tile, bh);
    u.b = bh / a.Hq;
    u.h = bh - u.b * a.Hq;
    u.g = u.h / (a.Hq / a.Hkv);
    u.S = a.S;
    u.Sk = u.S;
    u.qoff = 0;
    u.tok0 = (int64_t)u.b * u.S;
    u.tok0k = u.tok0;
    if constexpr (VARLEN) {
        const int t0 = min(max(a.cu[u.b], 0), a.total);
        const int t1 = min(max(a.cu[u.b + 1], t0), a.total);
        const int u0 = min(max(a.cu_k[u.b], 0), a.total_k);
        const int u1 = min(max(a.cu_k[u.b + 1], u0), a.total_k);
        u.S = min(t1 - t0, a.S);
        u.Sk = u1 - u0;
        u.qoff = u.Sk - u.S;
        u.tok0 = t0;
        u.tok0k = u0;
        if (tile * BM >= u.S) return false;   // whole workgroup: past the end of this sequence
    }
    u.q0 = tile * BM;
    const int kend = !CAUSAL ? u.Sk : VARLEN ? max(min(u.Sk, u.q0 + BM + u.qoff), 0) : min(u.S, u.q0 + BM);
    u.nblk = (kend + KB - 1) / KB;
    u.jdiag = !CAUSAL ? (u.Sk - 1) / KB : VARLEN ? max(u.q0 + u.qoff, 0) / KB : u.q0 / KB;
    return true;
}

// The scales: by value, or read from device memory where an earlier kernel on the
// stream (the rotation's quantisation) wrote them; the same double-precision
// formula as the host's, so both give the same bits.
struct Scales {
    float c, a8, v;
};
template <bool DSCALE>
__device__ __forceinline__ Scales scales_of(const Fp8Params& a) {
    Scales s{a.c, a.a8, a.v_scale};
    if constexpr (DSCALE) {
        const double cd = (double)*a.dq * (double)*a.dk * (double)a.sm * 1.4426950408889634;
        s.c = (float)cd;
        s.a8 = (float)(8.0 * cd);
        s.v = *a.dv;
    }
    return s;
}

// Q^T operands: lane (query c, half hh) holds d in [64kk + 32hh, +32) for each step kk.
template <int DQK, int NKK>
__device__ __forceinline__ void load_q(const Fp8Params& a, const Work& u, int qabs, int hh, i32x8 (&qr)[NKK]) {
    const bool ok = qabs < u.S;
    const uint8_t* qp = a.q + (u.tok0 + (ok ? qabs : 0)) * ((int64_t)a.Hq * DQK) + (int64_t)u.h * DQK + 32 * hh;
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) {
        i32x4 lo = ok ? load16(qp + 64 * kk) : i32x4{0, 0, 0, 0};
        i32x4 hi = ok ? load16(qp + 64 * kk + 16) : i32x4{0, 0, 0, 0};
        qr[kk] = i32x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    }
}

// Epilogue: out = bf16(v_scale * (O / L)), lane holds query c,
// d = 32dt + 8(r/4) + 4hh + r%4.  L = sum_j 2^(t_j - ref) over the rounded
// probabilities, so the row's natural-log normaliser is ln2 * (log2 L + ref).
template <bool LSE, bool VARLEN>
__device__ __forceinline__ void store_out(const Fp8Params& a, const Work& u, int qabs, int hh, const f32x16 (&o)[4],
                                          const f32x16& lsum, float ref, float sc_v) {
    const float l0 = lsum[0];
    // a query of a variable-length sequence that sees no key (more queries than keys)
    // has L = 0 and O = 0: divide by infinity instead, so its output is 0
    const float l0d = (VARLEN && !(l0 > 0.0f)) ? INFINITY : l0;
    if (LSE && hh == 0 && qabs < u.S)
        a.lse[(VARLEN ? (int64_t)u.h * a.total + u.tok0 : ((int64_t)u.b * a.Hq + u.h) * u.S) + qabs] =
            (log2f(l0) + ref) * 0.6931471805599453f;
    const Quotient quot(l0d);   // O / L, one reciprocal for the lane's 64 values
    if (qabs < u.S) {
        __bf16* op = a.o + ((u.tok0 + qabs) * a.Hq + u.h) * 128;
#pragma unroll
        for (int dt = 0; dt < 4; ++dt) {
#pragma unroll
            for (int r4 = 0; r4 < 4; ++r4) {
                float x0 = quot(o[dt][4 * r4 + 0]) * sc_v;
                float x1 = quot(o[dt][4 * r4 + 1]) * sc_v;
                float x2 = quot(o[dt][4 * r4 + 2]) * sc_v;
                float x3 = quot(o[dt][4 * r4 + 3]) * sc_v;
                uint2 pk = make_uint2(pack_bf16x2(x0, x1), pack_bf16x2(x2, x3));
                *reinterpret_cast<uint2*>(op + 32 * dt + 8 * r4 + 4 * hh) = pk;
            }
        }
    }
}

constexpr int kFp8Rows = 256;   // query rows per workgroup (8 waves of 32)

// Kernel parameters of a validated problem.  c is the log2-domain score scale.
inline Fp8Params fp8_params(const Problem& p) {
    Fp8Params a;
    a.q = static_cast<const uint8_t*>(p.q);
    a.k = static_cast<const uint8_t*>(p.k);
    a.v = static_cast<const uint8_t*>(p.v);
    a.o = static_cast<__bf16*>(p.o);
    a.lse = p.lse;
    const double c = (double)p.q_scale * p.k_scale * p.sm * 1.4426950408889634;
    a.c = (float)c;
    a.a8 = (float)(8.0 * c);
    a.v_scale = p.v_scale;
    a.B = p.B;
    a.Hq = p.Hq;
    a.Hkv = p.Hkv;
    a.S = p.S;
    a.cu = p.cu;
    a.total = p.total;
    a.cu_k = p.cu_k;
    a.total_k = p.total_k;
    a.dq = p.dq;
    a.dk = p.dk;
    a.dv = p.dv;
    a.sm = p.sm;
    a.n_tiles = (p.S + kFp8Rows - 1) / kFp8Rows;
    return a;
}

}  // namespace
}  // namespace attnfwd

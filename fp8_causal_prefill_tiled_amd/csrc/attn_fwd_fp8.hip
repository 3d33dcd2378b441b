// FP8 (OCP e4m3fn) causal prefill attention for gfx950.
//
// Method: "Zyphra ZYFA: FP8 FlashAttention for AMD MI355X, Up to 1.76x Faster"
// (MarkTechPost), sections "Lean P: one multiply-add instead of an exponential"
// and "Per-block scaling and a rounded row sum"; "Breaking the FP8 Attention
// Bottleneck on AMD MI355X" (kg.zhiyong.dev), section "ZYFA's Technical
// Solutions".  Per query row and 64-key block:
//   s   = <Q8_i, K8_j> on the FP8 matrix cores (fp32 accumulate)
//   t   = s * c,  c = q_scale * k_scale * sm * log2(e)        (log2-domain score)
//   M   = ceil(max_j t)                                         (block exponent)
//   p~  = e4m3(2^(t - M + 8))   exact path: v_exp_f32 + RNE convert
//       = byte rint(8c*s + 120 - 8M) clamped to [0,255]        Lean P: FMA + convert
//   O  += 2^(M-8-R) * p~ . V8   scaled MFMA, the power of two is the E8M0 B scale
//   L  += 2^(M-8-R) * sum p~    one more scaled MFMA against an all-ones operand
//   out = bf16(v_scale * (O / L))
// R is a per-row power-of-two reference that only moves (with an exact
// rescale of O and L) when a block exponent exceeds it by more than 16.
//
// Mapping on CDNA4.  Each wave owns 32 query rows of one head and computes the
// score tile transposed, S^T = K . Q^T (v_mfma_f32_32x32x64_f8f6f4, A = K rows
// from LDS, B = the wave's Q in registers), so lane l holds query l%32 and 32 of
// the block's 64 keys: the row max is 32 in-lane maxima plus one
// v_permlane32_swap, and the packed FP8 probabilities are already the B operand
// of O^T = V^T . P^T.
//
// Two kernels share that mapping and the two-wave ping-pong schedule:
// fp8_causal_fwd takes one 64-key block per phase and stages K and V through
// registers (the exponential path); fp8_causal_fwd_pair takes two blocks per
// phase (128 keys, the block size of the pages' ping-pong) and stages K and V
// with direct HBM-to-LDS loads, which keep the staging out of the registers that
// the second block's scores need (Lean P).
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
    static constexpr int OFF_ONES = OFF_VS + NSLOT * V_BYTES;   // 32 bytes of e4m3 1.0
    static constexpr int LDS_BYTES = OFF_ONES + 32;

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
    const int tile = a.n_tiles - 1 - L / BH;
    const int bh = L % BH;
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
    if (qabs < u.S) {
        __bf16* op = a.o + ((u.tok0 + qabs) * a.Hq + u.h) * 128;
#pragma unroll
        for (int dt = 0; dt < 4; ++dt) {
#pragma unroll
            for (int r4 = 0; r4 < 4; ++r4) {
                float x0 = (o[dt][4 * r4 + 0] / l0d) * sc_v;
                float x1 = (o[dt][4 * r4 + 1] / l0d) * sc_v;
                float x2 = (o[dt][4 * r4 + 2] / l0d) * sc_v;
                float x3 = (o[dt][4 * r4 + 3] / l0d) * sc_v;
                uint2 pk = make_uint2(pack_bf16x2(x0, x1), pack_bf16x2(x2, x3));
                *reinterpret_cast<uint2*>(op + 32 * dt + 8 * r4 + 4 * hh) = pk;
            }
        }
    }
}

// Two-wave ping-pong ("Two-wave ping-pong schedule", Zyphra ZYFA page,
// MarkTechPost).  A workgroup of 8 waves covers 256 query rows of one head;
// waves w and w+4 share a SIMD and form the two groups G0 (waves 0-3) and G1
// (waves 4-7).  In iteration j the two groups run their phases in opposite
// order:
//     G0:  MFMA(j), then VALU(j+1)
//     G1:  VALU(j), then MFMA(j)
// MFMA(j): S^T(j+1) = K(j+1).Q^T, O^T += V^T(j).P(j)^T, L += 1.P(j)^T, and in the
// shadow of the P.V MFMAs the mask, row max and block exponent of block j+1.
// VALU(j): P(j) bytes and the reference update.  One workgroup barrier ends the
// iteration; starting from it, on every SIMD one wave feeds the matrix core while
// its partner runs the probability code, and the order is restored at every
// barrier.  A single wave issues roughly one vector instruction per 5-6 cycles,
// so one wave alone cannot both keep a 64-cycle MFMA pipeline busy and issue the
// ~100 vector instructions each 9-MFMA phase needs; two waves can.
// The MFMA wave also does the block staging between its MFMAs, while the matrix
// pipe is busy:
//     G0 (MFMA(j)):  K block j+2 registers -> LDS, buffer loads of K block j+3;
//                    V^T(j+1) with the exponential path
//     G1 (MFMA(j)):  V block j+2 registers -> LDS staging, buffer loads of V block j+3;
//                    V^T(j+1) with Lean P
// K, V^T and V staging tiles each have 2 LDS slots (block j in slot j%2); the
// buffer loads run one iteration ahead of their LDS stores, and every LDS
// producer/consumer pair is separated by the end-of-iteration barrier.  V^T row
// d holds the block's 64 keys in the byte order of the probability operand, so
// both matrix operands are plain 16-byte LDS reads; it is built once per
// workgroup with the transposing ds_read_b64_tr_b8, far slower per byte than
// ds_read_b128 on gfx950.  Buffer loads use a range ending at row S, so rows
// past S read as zeros.
template <int DQK, int PMODE, bool CAUSAL, bool LSE, bool VARLEN, bool DSCALE>
__global__ void __launch_bounds__(512) fp8_causal_fwd(Fp8Params a) {
    using T = Fp8Tile<DQK>;
    constexpr int NT = 256;                       // threads per group
    constexpr int BM = 256;                       // query rows per workgroup
    constexpr int KPT = T::K_CHUNKS / NT;         // K chunks staged per G0 thread
    constexpr int VPT = T::V_CHUNKS / NT;         // V chunks staged per G1 thread
    constexpr int SPT = KPT > VPT ? KPT : VPT;
    constexpr int TPT = (128 * 4) / NT;           // V^T chunks built per G0 thread
    constexpr int KCH_ROW = DQK / 16;
    static_assert(T::K_CHUNKS % NT == 0 && T::V_CHUNKS % NT == 0, "staging split");

    __shared__ __attribute__((aligned(16))) uint8_t smem_raw[T::LDS_BYTES];
    ATTN_LDS uint8_t* smem = (ATTN_LDS uint8_t*)smem_raw;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave index, uniform
    const int grp = w >> 2;                                   // 0: G0, 1: G1
    const int tg = tid & (NT - 1);                            // thread index in its group
    Work u;
    if (!work_of<CAUSAL, VARLEN>(a, u)) return;
    const int S = u.S, Sk = u.Sk, qoff = u.qoff, q0 = u.q0, nblk = u.nblk, jdiag = u.jdiag;
    const int c = lane & 31;
    const int hh = lane >> 5;
    const int qabs = q0 + 32 * w + c;             // query of this lane
    const Scales scl = scales_of<DSCALE>(a);
    const float sc_c = scl.c, sc_a8 = scl.a8;
    const int k_row = a.Hkv * DQK;                // bytes between consecutive keys
    const int v_row = a.Hkv * 128;
    const uint8_t* kbase = a.k + u.tok0k * k_row + (int64_t)u.g * DQK;
    const uint8_t* vbase = a.v + u.tok0k * v_row + (int64_t)u.g * 128;
    i32x8 qr[T::NKK];
    load_q<DQK>(a, u, qabs, hh, qr);

    // ---- staging.  G0 moves K blocks, G1 V blocks: HBM -> registers (gload, one
    // iteration ahead) -> LDS (lstore).  Per-lane byte offsets of the staged chunks
    // inside a block (global) and inside an LDS slot.
    i32x4 st[SPT];
    int go[SPT], so[SPT];
#pragma unroll
    for (int i = 0; i < SPT; ++i) {
        const int idx = tg + i * NT;
        if (grp == 0) {
            const int row = idx / KCH_ROW, cc = idx % KCH_ROW;
            go[i] = row * k_row + 16 * cc;
            so[i] = row * T::K_STRIDE + 16 * cc;
        } else {
            const int row = (idx >> 3) & (KB - 1), cc = idx & 7;
            go[i] = row * v_row + 16 * cc;
            so[i] = T::OFF_VS + row * 128 + 16 * (cc ^ v_swz(row));
        }
    }
    // Every block index is loaded (blocks past the last one read zeros through an
    // empty range), so the staging steps need no guards.
    auto gload = [&](int j) {
        // rows of block j inside the tensor, clamped to [0, KB]; uniform, so kept on the
        // scalar unit (a fused vector med3 would cost three vector instructions per block)
        const int rows = min(__builtin_amdgcn_readfirstlane(max(Sk - j * KB, 0)), KB);
        if (grp == 0) {
            const auto r = buffer_rsrc(kbase + (int64_t)j * KB * k_row, rows * k_row);
#pragma unroll
            for (int i = 0; i < KPT; ++i) st[i] = buffer_load16(r, go[i]);
        } else {
            const auto r = buffer_rsrc(vbase + (int64_t)j * KB * v_row, rows * v_row);
#pragma unroll
            for (int i = 0; i < VPT; ++i) st[i] = buffer_load16(r, go[i]);
        }
    };
    auto lstore = [&](int j) {   // G0: K slot j%2, G1: staging slot j%2
        if (grp == 0) {
            ATTN_LDS uint8_t* base = smem + (j & 1) * T::K_BYTES;
#pragma unroll
            for (int i = 0; i < KPT; ++i) lds_store16(base + so[i], st[i]);
        } else {
            ATTN_LDS uint8_t* base = smem + (j & 1) * T::V_BYTES;
#pragma unroll
            for (int i = 0; i < VPT; ++i) lds_store16(base + so[i], st[i]);
        }
    };

    // ---- V^T construction: V^T row d holds the 64 keys at positions
    // p = 32h + t in the probability-byte order key(h, t) = 32(t/16) + 8((t%16)/4)
    // + 4h + t%4.  16-lane group Gi (of 32) builds the chunk d in [16(Gi%8), +16),
    // p in [16(Gi/8), +16) from two transposing reads of 8 keys (rows) x 16 d
    // (columns) of the key-major staging tile.
    int tr_off[TPT][2];
    int tr_dst[TPT];
#pragma unroll
    for (int u = 0; u < TPT; ++u) {
        const int Gi = 4 * (w & 3) + (lane >> 4) + 16 * u, n = lane & 15, t = n >> 1;
        const int dbase = 16 * (Gi & 7), p0 = 16 * (Gi >> 3);
#pragma unroll
        for (int x = 0; x < 2; ++x) {
            const int pos = p0 + 8 * x + t;
            const int hk = pos >> 5, tk = pos & 31;
            const int key = 32 * (tk >> 4) + 8 * ((tk & 15) >> 2) + 4 * hk + (tk & 3);
            tr_off[u][x] = T::OFF_VS + key * 128 + 16 * ((dbase >> 4) ^ v_swz(key)) + 8 * (n & 1);
        }
        tr_dst[u] = T::OFF_VT + (dbase + n) * T::VT_STRIDE + p0;
    }
    // Split in two so the transposing reads can be issued early and their latency
    // hidden behind other work before the stores.
    i32x2 tlo[TPT], thi[TPT];
    auto transpose_read = [&](int j) {   // staging slot j%2 -> registers
        const ATTN_LDS uint8_t* src = smem + (j & 1) * T::V_BYTES;
#pragma unroll
        for (int u = 0; u < TPT; ++u) {
            tlo[u] = lds_read_tr8(src + tr_off[u][0]);
            thi[u] = lds_read_tr8(src + tr_off[u][1]);
        }
    };
    auto transpose_write = [&](int j) {   // registers -> V^T slot j%2
        ATTN_LDS uint8_t* dst = smem + (j & 1) * T::VT_BYTES;
#pragma unroll
        for (int u = 0; u < TPT; ++u)
            lds_store16(dst + tr_dst[u], i32x4{tlo[u][0], tlo[u][1], thi[u][0], thi[u][1]});
    };
    auto transpose_v = [&](int j) {
        transpose_read(j);
        transpose_write(j);
    };

    f32x16 o[4];
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) o[dt] = f32x16{0};
    f32x16 lsum = f32x16{0};
    float ref = -INFINITY;
    // e4m3 1.0 in every byte: the A operand of the row-sum MFMA.  Kept live in
    // registers (the empty asm hides the constant, so it is not rebuilt per block).
    i32x8 ones;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        int one4 = 0x38383838;
        asm volatile("" : "+v"(one4));
        ones[i] = one4;
    }
    // The A-side E8M0 scale of the P.V MFMAs (127 = 2^0), set once here under a
    // full EXEC mask: matrix instructions read every lane's scale byte whatever
    // EXEC is, so the constant must never be materialised inside divergent code.
    int sa = 127;
    asm volatile("" : "+v"(sa));

    auto read32 = [&](const ATTN_LDS uint8_t* p) {
        i32x4 lo = lds_load16(p), hi = lds_load16(p + 16);
        return i32x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    };

    // ---- MFMA phase of block j: S^T(j+1) from K slot (j+1)%2 (when block j+1
    // exists) and P(j).V^T(j) from V^T slot j%2.  Lane (row c, half hh) reads its
    // operands 32 bytes at 32hh of K row c (+32 for keys [32,64)) and V^T row 32dt + c.
    f32x16 s0, s1;              // S^T of the next block: keys [0,32) and [32,64)
    i32x8 pv_bytes;             // P(j), the B operand of the P.V MFMAs
    int sb = 127;               // its E8M0 scale byte
    // ---- probabilities of block j in two parts.  prep: mask (diagonal blocks),
    // block exponent M, the bias of the byte formula and the reference update
    // decision; it runs on the MFMA wave right after the score MFMAs, in the shadow
    // of the P.V MFMAs.  finish: P bytes, the rare exact rescale of O and L when the
    // power-of-two reference moves (by more than kRefSlack), E8M0 scale byte; it is
    // the vector phase.
    float bias_n = 0.0f, nref_n = 0.0f;
    bool need_n = false;
    int sb_n = 127;
    auto prep_mask = [&](int j) {
        if (j >= jdiag) {
            // key kb0 + off(r) + 4hh is visible iff off(r) <= qlim - kb0 - 4hh, qlim the
            // last key the query sees
            const int qlim = CAUSAL ? min(qabs + qoff, Sk - 1) : Sk - 1;
            const int lim = qlim - j * KB - 4 * hh;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int off = 8 * (r >> 2) + (r & 3);
                s0[r] = off <= lim ? s0[r] : -INFINITY;
                s1[r] = off + 32 <= lim ? s1[r] : -INFINITY;
            }
        }
    };
    float mx_n = -INFINITY;
    auto prep_max = [&](int r0, int r1) {
        if (r0 == 0) mx_n = -INFINITY;
#pragma unroll
        for (int r = r0; r < r1; ++r) mx_n = fmaxf(fmaxf(mx_n, s0[r]), s1[r]);
    };
    auto prep_exponent = [&]() {
        const float mx = pair_max(mx_n);
        const float M = fmaxf(ceilf(mx * sc_c), -1.0e30f);  // floor: rows with no visible key here
        bias_n = PMODE == 0 ? 8.0f - M : 120.0f - 8.0f * M;
        need_n = M > ref + kRefSlack;
        nref_n = need_n ? M : ref;
        // E8M0 byte of 2^(M-8-nref), exponent clamped to [-127, 127]: all terms are
        // integers in float, so one median and one conversion give it exactly
        sb_n = (int)__builtin_amdgcn_fmed3f(M - nref_n + 119.0f, 0.0f, 254.0f);
    };
    auto prep = [&](int j) {
        prep_mask(j);
        prep_max(0, 16);
        prep_exponent();
    };
    auto finish = [&]() {
        int pw[8];
        if (PMODE == 0) {
#pragma unroll
            for (int q4 = 0; q4 < 8; ++q4) {
                const f32x16& x = q4 < 4 ? s0 : s1;
                const int e = 4 * (q4 & 3);
                const float p0 = __builtin_amdgcn_exp2f(fmaf(x[e + 0], sc_c, bias_n));
                const float p1 = __builtin_amdgcn_exp2f(fmaf(x[e + 1], sc_c, bias_n));
                const float p2 = __builtin_amdgcn_exp2f(fmaf(x[e + 2], sc_c, bias_n));
                const float p3 = __builtin_amdgcn_exp2f(fmaf(x[e + 3], sc_c, bias_n));
                const int wd = __builtin_amdgcn_cvt_pk_fp8_f32(p0, p1, 0, false);
                pw[q4] = __builtin_amdgcn_cvt_pk_fp8_f32(p2, p3, wd, true);
            }
        } else {
#pragma unroll
            for (int q4 = 0; q4 < 8; ++q4) {
                const f32x16& x = q4 < 4 ? s0 : s1;
                const int e = 4 * (q4 & 3);
                unsigned wd = 0;
                wd = __builtin_amdgcn_cvt_pk_u8_f32(fmaf(x[e + 0], sc_a8, bias_n), 0, wd);
                wd = __builtin_amdgcn_cvt_pk_u8_f32(fmaf(x[e + 1], sc_a8, bias_n), 1, wd);
                wd = __builtin_amdgcn_cvt_pk_u8_f32(fmaf(x[e + 2], sc_a8, bias_n), 2, wd);
                wd = __builtin_amdgcn_cvt_pk_u8_f32(fmaf(x[e + 3], sc_a8, bias_n), 3, wd);
                pw[q4] = (int)wd;
            }
        }
        pv_bytes = i32x8{pw[0], pw[1], pw[2], pw[3], pw[4], pw[5], pw[6], pw[7]};
        if (__ballot(need_n)) {
            vacc_settle(o, lsum);
            const float f = __builtin_amdgcn_exp2f(ref - nref_n);   // exactly 1 for rows that do not move
#pragma unroll
            for (int dt = 0; dt < 4; ++dt)
#pragma unroll
                for (int r = 0; r < 16; ++r) o[dt][r] *= f;
#pragma unroll
            for (int r = 0; r < 16; ++r) lsum[r] *= f;
            vacc_settle(o, lsum);   // the rescaled values are back before the next MFMA reads them
        }
        ref = nref_n;
        sb = sb_n;
    };

    constexpr int NS = 2 * T::NKK;      // score MFMAs per block
    // Issue order: operand i (i < NS: K operand, key half i%2, d step i/2; else V^T
    // rows 32(i-NS)) is read two MFMAs ahead of its use.
    // extra(i) runs after MFMA i: the staging work of the MFMA wave, issued while the
    // matrix pipe is busy.
    auto mfma_phase = [&](int j, auto&& extra) {
        __builtin_amdgcn_s_setprio(1);   // matrix issue wins arbitration against the partner wave
        const ATTN_LDS uint8_t* kp = smem + ((j + 1) & 1) * T::K_BYTES + c * T::K_STRIDE + 32 * hh;
        const ATTN_LDS uint8_t* vp = smem + T::OFF_VT + (j & 1) * T::VT_BYTES + c * T::VT_STRIDE + 32 * hh;
        auto operand = [&](int i) {
            return i < NS ? read32(kp + (i & 1) * 32 * T::K_STRIDE + 64 * (i >> 1))
                          : read32(vp + 32 * (i - NS) * T::VT_STRIDE);
        };
        // S^T(j+1) is computed even for the last block (from the stale K slot, in
        // bounds, result unused): one branch-free sequence keeps the accumulators in
        // fixed registers.
        i32x8 opb[3];
        opb[0] = operand(0);
        opb[1] = operand(1);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int i = 0; i < NS + 4; ++i) {
            if (i + 2 < NS + 4) opb[(i + 2) % 3] = operand(i + 2);
            if (i < NS) {
                f32x16& sd = (i & 1) ? s1 : s0;
                sd = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(opb[i % 3], qr[i >> 1], i < 2 ? f32x16{0} : sd,
                                                                      0, 0, 0, 0, 0, 0);
            } else {
                mfma_f8_scaled_vacc(o[i - NS], opb[i % 3], pv_bytes, sa, sb);
            }
            // prep of block j+1 once its score MFMAs have completed
            if (i == NS + 1) prep_mask(j + 1);
            if (i == NS + 2) prep_max(0, 8);
            if (i == NS + 3) prep_max(8, 16);
            extra(i);
            __builtin_amdgcn_sched_barrier(0);
        }
        mfma_f8_scaled_vacc(lsum, ones, pv_bytes, sa, sb);
        prep_exponent();
        __builtin_amdgcn_s_setprio(0);
    };

    // ---- prologue: K(0), K(1) and V(0), V(1) staged, blocks 2 and 3 in flight,
    // V^T(0) built, S^T(0) for every wave, P(0) for G0.
    // Issue order keeps the rule lstore relies on: when block jb is stored, the
    // loads of block jb+1 (if it exists) are the only ones issued after its own.
    gload(0);
    lstore(0);
    gload(1);
    lstore(1);
    gload(2);
    block_sync();
    if (grp == 0) transpose_v(0);
    {
        const ATTN_LDS uint8_t* kp = smem + c * T::K_STRIDE + 32 * hh;
        s0 = f32x16{0};
        s1 = f32x16{0};
#pragma unroll
        for (int kk = 0; kk < T::NKK; ++kk) {
            s0 = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(read32(kp + 64 * kk), qr[kk], s0, 0, 0, 0, 0, 0, 0);
            s1 = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(read32(kp + 32 * T::K_STRIDE + 64 * kk), qr[kk], s1,
                                                                  0, 0, 0, 0, 0, 0);
        }
    }
    block_sync();

    // ---- main loop.  Each group runs a loop of its own (one code path per loop
    // keeps the accumulators in fixed registers); both execute one barrier per
    // iteration.  Nothing is guarded: staging past the last block moves zeros into
    // free slots, a vector phase past it sees only masked keys (P = 0, no reference
    // move), and an MFMA phase past it adds 0 * 0.
    // V^T is built inside an MFMA phase, between MFMAs: by G1 with Lean P (G1's
    // iteration is otherwise the shorter one), by G0 with the exponential path.
    constexpr bool kTransposeOnG0 = PMODE == 0;
    prep(0);
    if (grp == 0) {
        finish();
        for (int j = 0; j < nblk; ++j) {
            mfma_phase(j, [&](int i) {                    // MFMA(j)
                if (kTransposeOnG0 && i == 0) transpose_read(j + 1);
                if (i == 1) lstore(j + 2);
                if (i == 2) gload(j + 3);
                if (kTransposeOnG0 && i == 4) transpose_write(j + 1);
            });
            finish();                                     // VALU(j+1)
            block_sync();
        }
    } else {
        for (int j = 0; j < nblk; ++j) {
            finish();                                     // VALU(j)
            mfma_phase(j, [&](int i) {                    // MFMA(j)
                if (!kTransposeOnG0 && i == 0) transpose_read(j + 1);
                if (i == 1) lstore(j + 2);
                if (i == 2) gload(j + 3);
                if (!kTransposeOnG0 && i == 4) transpose_write(j + 1);
            });
            block_sync();
        }
    }
    // The matrix instructions ignore EXEC: settling the accumulators here also keeps
    // all matrix work (and any operand copies it needs) out of the divergent stores.
    vacc_settle(o, lsum);

    store_out<LSE, VARLEN>(a, u, qabs, hh, o, lsum, ref, scl.v);
}

// Ping-pong over block pairs: the same two groups and phase order as
// fp8_causal_fwd, with 128 keys (blocks 2p, 2p+1, each with its own exponent
// and E8M0 scale) per phase, so that the per-phase costs (operand latency at the
// start of a phase, barrier, reference decision) are paid once per 128 keys.
//     G0:  MFMA(p), then VALU(p+1)        G1:  VALU(p), then MFMA(p)
// MFMA(p): O^T += V^T.P^T and L += 1.P^T for pair p (scaled MFMAs), then S^T of
// pair p+1 (its scores feed the next vector phase); VALU(p): mask, exponents,
// reference decision and probability bytes of pair p.  K and V move from HBM to
// LDS with direct-to-LDS buffer loads issued at the start of each wave's vector
// phase (no staging registers); each wave waits for its own loads before the
// end-of-iteration barrier.  Each group builds the V^T tile of one block of the
// next pair between its MFMAs.
template <int DQK, int PMODE, bool CAUSAL, bool LSE, bool VARLEN, bool DSCALE>
__global__ void __launch_bounds__(512) fp8_causal_fwd_pair(Fp8Params a) {
    using T = PairTile<DQK>;
    constexpr int NT = 256;                       // threads per group
    constexpr int BM = 256;                       // query rows per workgroup
    constexpr int NB = T::NB;                     // 64-key blocks per iteration
    constexpr int NSLOT = T::NSLOT;
    constexpr int TPT = (128 * 4) / NT;           // V^T chunks of one block built per thread

    __shared__ __attribute__((aligned(16))) uint8_t smem_raw[T::LDS_BYTES];
    ATTN_LDS uint8_t* smem = (ATTN_LDS uint8_t*)smem_raw;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave index, uniform
    const int grp = w >> 2;                                   // 0: G0, 1: G1
    const int tg = tid & (NT - 1);                            // thread index in its group
    Work u;
    if (!work_of<CAUSAL, VARLEN>(a, u)) return;
    const int S = u.S, Sk = u.Sk, qoff = u.qoff, q0 = u.q0, nblk = u.nblk, jdiag = u.jdiag;
    const int c = lane & 31;
    const int hh = lane >> 5;
    const int qabs = q0 + 32 * w + c;             // query of this lane
    const Scales scl = scales_of<DSCALE>(a);
    const float sc_c = scl.c, sc_a8 = scl.a8;
    const int k_row = a.Hkv * DQK;                // bytes between consecutive keys
    const int v_row = a.Hkv * 128;
    const uint8_t* kbase = a.k + u.tok0k * k_row + (int64_t)u.g * DQK;
    const uint8_t* vbase = a.v + u.tok0k * v_row + (int64_t)u.g * 128;
    i32x8 qr[T::NKK];
    load_q<DQK>(a, u, qabs, hh, qr);

    // ---- staging: direct loads from HBM into LDS (no registers), G0 moves K blocks,
    // G1 V blocks.  One wave instruction fills 1 KB of consecutive LDS bytes, lane i the
    // 16 bytes at 16i: for a region of 128-byte rows that is row 8m + i/8, physical chunk
    // i%8, whose logical chunk (the global one) undoes the swizzle.  Per block, each wave
    // of a group issues 2 such loads (K region A, or the V staging tile) and, for
    // d_qk = 192, one more for K region B (64-byte rows: row 16m + i/4, chunk i%4).
    // Rows past the end of the keys read as zeros through the buffer range.
    const int wq = w & 3;                         // wave within its group
    int goff[2];
#pragma unroll
    for (int m2 = 0; m2 < 2; ++m2) {
        const int m = 2 * wq + m2;
        const int row = 8 * m + (lane >> 3), pos = lane & 7;
        goff[m2] = grp == 0 ? row * k_row + 16 * (pos ^ kswz_a(row)) : row * v_row + 16 * (pos ^ v_swz(row));
    }
    int goff_b = 0;
    if (DQK == 192) {
        const int row = 16 * wq + (lane >> 2), pos = lane & 3;
        goff_b = row * k_row + 128 + 16 * (pos ^ kswz_b(row));
    }
    auto dload = [&](int p) {   // blocks NB*p .. NB*p+NB-1 into their slots
#pragma unroll
        for (int bl = 0; bl < NB; ++bl) {
            const int jb = NB * p + bl;
            const int slot = jb & (NSLOT - 1);
            // rows of block jb inside the tensor, clamped to [0, KB]; uniform, on the scalar unit
            const int rows = min(__builtin_amdgcn_readfirstlane(max(Sk - jb * KB, 0)), KB);
            if (grp == 0) {
                const auto r = buffer_rsrc(kbase + (int64_t)jb * KB * k_row, rows * k_row);
                ATTN_LDS uint8_t* dst = smem + slot * T::K_BYTES;
#pragma unroll
                for (int m2 = 0; m2 < 2; ++m2)
                    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (ATTN_LDS void*)(dst + 1024 * (2 * wq + m2)), 16,
                                                             goff[m2], 0, 0, 0);
                if (DQK == 192)
                    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (ATTN_LDS void*)(dst + T::KA_BYTES + 1024 * wq), 16,
                                                             goff_b, 0, 0, 0);
            } else {
                const auto r = buffer_rsrc(vbase + (int64_t)jb * KB * v_row, rows * v_row);
                ATTN_LDS uint8_t* dst = smem + T::OFF_VS + slot * T::V_BYTES;
#pragma unroll
                for (int m2 = 0; m2 < 2; ++m2)
                    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (ATTN_LDS void*)(dst + 1024 * (2 * wq + m2)), 16,
                                                             goff[m2], 0, 0, 0);
            }
        }
    };

    // ---- V^T construction: V^T row d holds the 64 keys at positions
    // p = 32h + t in the probability-byte order key(h, t) = 32(t/16) + 8((t%16)/4)
    // + 4h + t%4.  16-lane group Gi (of 32) builds the chunk d in [16(Gi%8), +16),
    // p in [16(Gi/8), +16) from two transposing reads of 8 keys (rows) x 16 d
    // (columns) of the key-major staging tile.  Each group builds one block of a pair.
    int tr_off[TPT][2];
    int tr_dst[TPT];
#pragma unroll
    for (int u = 0; u < TPT; ++u) {
        const int Gi = 4 * (w & 3) + (lane >> 4) + 16 * u, n = lane & 15, t = n >> 1;
        const int dbase = 16 * (Gi & 7), p0 = 16 * (Gi >> 3);
#pragma unroll
        for (int x = 0; x < 2; ++x) {
            const int pos = p0 + 8 * x + t;
            const int hk = pos >> 5, tk = pos & 31;
            const int key = 32 * (tk >> 4) + 8 * ((tk & 15) >> 2) + 4 * hk + (tk & 3);
            tr_off[u][x] = T::OFF_VS + key * 128 + 16 * ((dbase >> 4) ^ v_swz(key)) + 8 * (n & 1);
        }
        tr_dst[u] = T::OFF_VT + (dbase + n) * T::VT_STRIDE + p0;
    }
    i32x2 tlo[TPT], thi[TPT];
    auto transpose_read = [&](int jb) {   // staging slot of block jb -> registers
        const ATTN_LDS uint8_t* src = smem + (jb & (NSLOT - 1)) * T::V_BYTES;
#pragma unroll
        for (int u = 0; u < TPT; ++u) {
            tlo[u] = lds_read_tr8(src + tr_off[u][0]);
            thi[u] = lds_read_tr8(src + tr_off[u][1]);
        }
    };
    auto transpose_write = [&](int jb) {   // registers -> V^T slot of block jb
        ATTN_LDS uint8_t* dst = smem + (jb & (NSLOT - 1)) * T::VT_BYTES;
#pragma unroll
        for (int u = 0; u < TPT; ++u)
            lds_store16(dst + tr_dst[u], i32x4{tlo[u][0], tlo[u][1], thi[u][0], thi[u][1]});
    };

    f32x16 o[4];
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) o[dt] = f32x16{0};
    f32x16 lsum = f32x16{0};
    float ref = -INFINITY;
    // e4m3 1.0 in every byte, the A operand of the row-sum MFMAs: 32 bytes of LDS that
    // every lane reads (a broadcast read) at the start of each MFMA phase.
    if (tid < 2) lds_store16(smem + T::OFF_ONES + 16 * tid, i32x4{0x38383838, 0x38383838, 0x38383838, 0x38383838});
    // The A-side E8M0 scale of the P.V MFMAs (127 = 2^0), set once here under a
    // full EXEC mask: matrix instructions read every lane's scale byte whatever
    // EXEC is, so the constant must never be materialised inside divergent code.
    int sa = 127;
    asm volatile("" : "+v"(sa));

    auto read32 = [&](const ATTN_LDS uint8_t* p) {
        i32x4 lo = lds_load16(p), hi = lds_load16(p + 16);
        return i32x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    };
    // K operand of block slot `slot`, key half kh, d step kk: lane (c, hh) takes row
    // 32kh + c, d in [64kk + 32hh, +32), i.e. two logical chunks of its region.
    auto kread = [&](int slot, int kh, int kk) {
        const int row = 32 * kh + c;
        const ATTN_LDS uint8_t* base = smem + slot * T::K_BYTES;
        int a0, a1;
        if (kk < 2) {
            const int j = 4 * kk + 2 * hh, sw = kswz_a(row);
            a0 = row * 128 + 16 * (j ^ sw);
            a1 = row * 128 + 16 * ((j + 1) ^ sw);
        } else {
            const int j = 2 * hh, sw = kswz_b(row);
            a0 = T::KA_BYTES + row * 64 + 16 * (j ^ sw);
            a1 = T::KA_BYTES + row * 64 + 16 * ((j + 1) ^ sw);
        }
        i32x4 lo = lds_load16(base + a0), hi = lds_load16(base + a1);
        return i32x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    };

    f32x16 sc[NB][2];           // S^T of the next block pair: block bl, keys [0,32) / [32,64)
    i32x8 pv[NB];               // P of the current pair, the B operands of the P.V MFMAs
    int sb[NB];                 // their E8M0 scale bytes
#pragma unroll
    for (int bl = 0; bl < NB; ++bl) sb[bl] = 127;

    // ---- the vector phase of block pair p: masks (pairs from the diagonal one on), block
    // exponents M (row max over each block), the reference decision for the pair,
    // probability bytes, the rare exact rescale of O and L when the power-of-two
    // reference moves (by more than kRefSlack), E8M0 scale bytes.  The two blocks'
    // dependency chains (the row maxima, the byte packing of each word) are interleaved:
    // a wave issues a dependent vector instruction more slowly than an independent one.
    auto valu_phase = [&](int p) {
        // masks: only pairs that reach the diagonal (or the ragged last block); the
        // formula leaves a block that lies wholly inside the visible range unchanged
        if (NB * p + NB - 1 >= jdiag) {
            const int qlim = CAUSAL ? min(qabs + qoff, Sk - 1) : Sk - 1;
#pragma unroll
            for (int bl = 0; bl < NB; ++bl) {
                const int lim = qlim - (NB * p + bl) * KB - 4 * hh;
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int off = 8 * (r >> 2) + (r & 3);
                    sc[bl][0][r] = off <= lim ? sc[bl][0][r] : -INFINITY;
                    sc[bl][1][r] = off + 32 <= lim ? sc[bl][1][r] : -INFINITY;
                }
            }
        }
        // row maxima of the blocks: independent chains, interleaved
        float mx[NB], M[NB];
#pragma unroll
        for (int bl = 0; bl < NB; ++bl) mx[bl] = fmaxf(sc[bl][0][0], sc[bl][1][0]);
#pragma unroll
        for (int r = 1; r < 16; ++r)
#pragma unroll
            for (int bl = 0; bl < NB; ++bl) mx[bl] = fmaxf(fmaxf(mx[bl], sc[bl][0][r]), sc[bl][1][r]);
#pragma unroll
        for (int bl = 0; bl < NB; ++bl) {
            mx[bl] = pair_max(mx[bl]);
            M[bl] = fmaxf(ceilf(mx[bl] * sc_c), -1.0e30f);  // floor: rows with no visible key here
        }
        float Mmax = M[0];
#pragma unroll
        for (int bl = 1; bl < NB; ++bl) Mmax = fmaxf(Mmax, M[bl]);
        const bool need = Mmax > ref + kRefSlack;
        const float nref = need ? Mmax : ref;
        float bias[NB];
#pragma unroll
        for (int bl = 0; bl < NB; ++bl) {
            bias[bl] = PMODE == 0 ? 8.0f - M[bl] : 120.0f - 8.0f * M[bl];
            // E8M0 byte of 2^(M-8-nref), exponent clamped to [-127, 127]: all terms are
            // integers in float, so one median and one conversion give it exactly
            sb[bl] = (int)__builtin_amdgcn_fmed3f(M[bl] - nref + 119.0f, 0.0f, 254.0f);
        }
        // probability bytes: byte e of all 16 words, then byte e + 1, ... (each word packs its
        // four bytes in sequence; stepping through the words keeps those chains apart)
        int pw[NB][8];
        if (PMODE == 0) {
#pragma unroll
            for (int q4 = 0; q4 < 8; ++q4)
#pragma unroll
                for (int bl = 0; bl < NB; ++bl) {
                    const f32x16& x = q4 < 4 ? sc[bl][0] : sc[bl][1];
                    const int e = 4 * (q4 & 3);
                    const float p0 = __builtin_amdgcn_exp2f(fmaf(x[e + 0], sc_c, bias[bl]));
                    const float p1 = __builtin_amdgcn_exp2f(fmaf(x[e + 1], sc_c, bias[bl]));
                    const float p2 = __builtin_amdgcn_exp2f(fmaf(x[e + 2], sc_c, bias[bl]));
                    const float p3 = __builtin_amdgcn_exp2f(fmaf(x[e + 3], sc_c, bias[bl]));
                    const int wd = __builtin_amdgcn_cvt_pk_fp8_f32(p0, p1, 0, false);
                    pw[bl][q4] = __builtin_amdgcn_cvt_pk_fp8_f32(p2, p3, wd, true);
                }
        } else {
#pragma unroll
            for (int g = 0; g < 8; g += 2) {   // two words of each block at a time
#pragma unroll
                for (int e = 0; e < 4; ++e)
#pragma unroll
                    for (int q4 = g; q4 < g + 2; ++q4)
#pragma unroll
                        for (int bl = 0; bl < NB; ++bl) {
                            const f32x16& x = q4 < 4 ? sc[bl][0] : sc[bl][1];
                            const float y = fmaf(x[4 * (q4 & 3) + e], sc_a8, bias[bl]);
                            pw[bl][q4] = (int)__builtin_amdgcn_cvt_pk_u8_f32(y, e, e == 0 ? 0u : (unsigned)pw[bl][q4]);
                        }
                __builtin_amdgcn_sched_barrier(0);
            }
        }
#pragma unroll
        for (int bl = 0; bl < NB; ++bl)
            pv[bl] = i32x8{pw[bl][0], pw[bl][1], pw[bl][2], pw[bl][3], pw[bl][4], pw[bl][5], pw[bl][6], pw[bl][7]};
        if (__ballot(need)) {
            vacc_settle(o, lsum);
            const float f = __builtin_amdgcn_exp2f(ref - nref);   // exactly 1 for rows that do not move
#pragma unroll
            for (int dt = 0; dt < 4; ++dt)
#pragma unroll
                for (int r = 0; r < 16; ++r) o[dt][r] *= f;
#pragma unroll
            for (int r = 0; r < 16; ++r) lsum[r] *= f;
            vacc_settle(o, lsum);   // the rescaled values are back before the next MFMA reads them
        }
        ref = nref;
    };

    constexpr int NS = 2 * T::NKK;      // score MFMAs per block
    constexpr int NPV = NB * 4;         // P.V MFMAs per pair
    constexpr int NMF = NPV + NB * NS;  // P.V, then score MFMAs of the next pair
    // ---- MFMA phase of pair p: O^T += V^T(pair p).P^T, L += 1.P^T (one scaled MFMA
    // per block) from the V^T slots, then S^T(pair p+1) from the K slots (computed
    // even past the last pair, from stale slots, in bounds, result unused).  The P.V
    // MFMAs come first so that the P registers are free before the score
    // accumulators are written.  Operand i (i < NPV: V^T rows 32(i%4) of block i/4;
    // else K operand: block (i-NPV)/NS, key half, d step) is read two MFMAs ahead of
    // its use; extra(i) runs after MFMA i: the staging work of the MFMA wave, issued
    // while the matrix pipe is busy.
    auto mfma_phase = [&](int p, auto&& extra) {
        __builtin_amdgcn_s_setprio(1);   // matrix issue wins arbitration against the partner wave
        auto operand = [&](int i) {
            if (i < NPV) {
                const int jb = NB * p + i / 4;
                return read32(smem + T::OFF_VT + (jb & (NSLOT - 1)) * T::VT_BYTES + c * T::VT_STRIDE + 32 * hh +
                              32 * (i % 4) * T::VT_STRIDE);
            }
            const int k = i - NPV, jb = NB * (p + 1) + k / NS, ks = k % NS;
            return kread(jb & (NSLOT - 1), ks & 1, ks >> 1);
        };
        const i32x8 ones = read32(smem + T::OFF_ONES);
        constexpr int PD = 2;            // operands read this many MFMAs ahead
        i32x8 opb[PD + 1];
#pragma unroll
        for (int i = 0; i < PD; ++i) opb[i] = operand(i);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int i = 0; i < NMF; ++i) {
            if (i + PD < NMF) opb[(i + PD) % (PD + 1)] = operand(i + PD);
            if (i < NPV) {
                const int bl = i / 4;
                mfma_f8_scaled_vacc(o[i % 4], opb[i % (PD + 1)], pv[bl], sa, sb[bl]);
                if (i % 4 == 3) mfma_f8_scaled_vacc(lsum, ones, pv[bl], sa, sb[bl]);
            } else {
                const int k = i - NPV, bl = k / NS, ks = k % NS;
                f32x16& sd = sc[bl][ks & 1];
                sd = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(opb[i % (PD + 1)], qr[ks >> 1],
                                                                      ks < 2 ? f32x16{0} : sd, 0, 0, 0, 0, 0, 0);
            }
            extra(i);
            __builtin_amdgcn_sched_barrier(0);
        }
        __builtin_amdgcn_s_setprio(0);
    };

    // ---- prologue: pairs 0 and 1 of K and V in LDS, V^T of pair 0 built (one block per
    // group), S^T of pair 0 for every wave.
    dload(0);
    dload(1);
    vmem_lds_sync();
    transpose_read(grp);
    transpose_write(grp);
#pragma unroll
    for (int bl = 0; bl < NB; ++bl) {
        f32x16 s0 = f32x16{0}, s1 = f32x16{0};
#pragma unroll
        for (int kk = 0; kk < T::NKK; ++kk) {
            s0 = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(kread(bl, 0, kk), qr[kk], s0, 0, 0, 0, 0, 0, 0);
            s1 = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(kread(bl, 1, kk), qr[kk], s1, 0, 0, 0, 0, 0, 0);
        }
        sc[bl][0] = s0;
        sc[bl][1] = s1;
    }
    block_sync();

    // ---- main loop over block pairs.  Each group runs a loop of its own (one code
    // path per loop keeps the accumulators in fixed registers); both execute one
    // barrier per iteration.  Nothing is guarded: staging past the last block moves
    // zeros into free slots, a vector phase past it sees only masked keys (P = 0, no
    // reference move), and an MFMA phase past it adds 0 * 0.
    // Iteration p: MFMA(p) reads V^T of pair p and K of pair p+1 (loaded in iteration
    // p-1), loads pair p+2 directly into LDS (into the slots of pair p, which nobody
    // reads in iteration p), and builds V^T of pair p+1 (one block per group) from the
    // staging slots loaded in iteration p-1.  Each wave waits for its own direct loads
    // before the end-of-iteration barrier.  LDS slots: block jb in slot jb % NSLOT,
    // NSLOT = 2*NB.
    const int npair = (nblk + NB - 1) / NB;
    if (grp == 0) {
        valu_phase(0);
        for (int p = 0; p < npair; ++p) {
            mfma_phase(p, [&](int i) {                    // MFMA(p)
                if (i == 0) transpose_read(NB * (p + 1));
                if (i == 4) transpose_write(NB * (p + 1));
            });
            dload(p + 2);
            valu_phase(p + 1);                            // VALU(p+1)
            vmem_lds_sync();
        }
    } else {
        for (int p = 0; p < npair; ++p) {
            dload(p + 2);
            valu_phase(p);                                // VALU(p)
            mfma_phase(p, [&](int i) {                    // MFMA(p)
                if (i == 0) transpose_read(NB * (p + 1) + 1);
                if (i == 4) transpose_write(NB * (p + 1) + 1);
            });
            vmem_lds_sync();
        }
    }
    // The matrix instructions ignore EXEC: settling the accumulators here also keeps
    // all matrix work (and any operand copies it needs) out of the divergent stores.
    vacc_settle(o, lsum);

    store_out<LSE, VARLEN>(a, u, qabs, hh, o, lsum, ref, scl.v);
}

template <int DQK, int PMODE, bool CAUSAL, bool LSE, bool VARLEN, bool DSCALE>
hipError_t launch_t(const Problem& p) {
    constexpr int NW = 8;
    constexpr int BM = 256;
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
    a.n_tiles = (p.S + BM - 1) / BM;
    const long long nblocks = (long long)a.n_tiles * p.B * p.Hq;
    if (nblocks <= 0 || nblocks > 0x7fffffffLL) return hipErrorInvalidConfiguration;
    // Lean P runs two blocks per phase; the exponential path one (its longer vector
    // phase fits the single-block schedule better: measured 12% faster there).
    if constexpr (PMODE == 1)
        hipLaunchKernelGGL((fp8_causal_fwd_pair<DQK, PMODE, CAUSAL, LSE, VARLEN, DSCALE>), dim3((unsigned)nblocks),
                           dim3(NW * 64), 0, p.stream, a);
    else
        hipLaunchKernelGGL((fp8_causal_fwd<DQK, PMODE, CAUSAL, LSE, VARLEN, DSCALE>), dim3((unsigned)nblocks),
                           dim3(NW * 64), 0, p.stream, a);
    return hipGetLastError();
}

// The log-sum-exp store is a template switch: the kernels without it keep exactly the
// code (and code layout) they have when no caller asks for it.
template <bool CAUSAL, bool LSE, bool VARLEN, bool DSCALE>
hipError_t launch_c(const Problem& p) {
    if (p.d_qk == 128)
        return p.p_mode == 0 ? launch_t<128, 0, CAUSAL, LSE, VARLEN, DSCALE>(p)
                             : launch_t<128, 1, CAUSAL, LSE, VARLEN, DSCALE>(p);
    if (p.d_qk == 192)
        return p.p_mode == 0 ? launch_t<192, 0, CAUSAL, LSE, VARLEN, DSCALE>(p)
                             : launch_t<192, 1, CAUSAL, LSE, VARLEN, DSCALE>(p);
    return hipErrorInvalidValue;
}

// Scales in device memory are a template switch too (equal-length calls only), so
// the kernels that take them by value keep their code.
template <bool VARLEN, bool DSCALE>
hipError_t launch_v(const Problem& p) {
    if (p.lse) return p.causal ? launch_c<true, true, VARLEN, DSCALE>(p) : launch_c<false, true, VARLEN, DSCALE>(p);
    return p.causal ? launch_c<true, false, VARLEN, DSCALE>(p) : launch_c<false, false, VARLEN, DSCALE>(p);
}

}  // namespace

hipError_t launch_fp8(const Problem& p) {
    if (p.cu) return p.dq ? hipErrorInvalidValue : launch_v<true, false>(p);
    return p.dq ? launch_v<false, true>(p) : launch_v<false, false>(p);
}

}  // namespace attnfwd

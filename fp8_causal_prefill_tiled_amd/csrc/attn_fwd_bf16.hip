// BF16 causal prefill attention for gfx950.
//
// The pages say only that the BF16 kernels are plain HIP and gain 1.01-1.02x
// over the vendor library ("Zyphra ZYFA: FP8 FlashAttention for AMD MI355X, Up to
// 1.76x Faster", sections "What is ZYFA?" and TL;DR); the arithmetic here is the
// standard FlashAttention-2 online softmax:
//   s = <Q_i, K_j> (bf16 matrix cores, fp32 accumulate), t = s * sm * log2(e)
//   p = 2^(t - R)          fp32 v_exp_f32, R a per-row power-of-two reference
//   O += bf16(p) . V,  l += p (fp32, unrounded)
//   out = bf16(O / l)
// R only moves (with an exact rescale of O and l by a power of two) when a
// block's integer maximum exceeds it by more than 8, so p <= 2^8 always.
//
// Mapping mirrors the FP8 kernel: S^T = K . Q^T with v_mfma_f32_32x32x16_bf16 so
// lane l owns query l%32; P^T packs straight into the B operand of
// O^T = V^T . P^T.  V^T is built once per workgroup from the key-major V tile
// with the transposing ds_read_b64_tr_b16 (far slower per byte than
// ds_read_b128), its rows holding the keys in the order of the P operand, so the
// P.V operands are plain 16-byte LDS reads.
//
// Schedule: the two-wave ping-pong of the FP8 kernel ("Two-wave ping-pong
// schedule", Zyphra ZYFA page, MarkTechPost).  Waves w and w+4 share a SIMD and
// form the groups G0 (waves 0-3) and G1 (waves 4-7); in iteration j
//     G0:  MFMA(j), then VALU(j+1)
//     G1:  VALU(j), then MFMA(j)
// MFMA(j): S^T(j+1) (2 d_qk/16 MFMAs), O^T += V^T(j).P(j)^T (16 MFMAs), in the
// shadow of the P.V MFMAs the mask, row maximum and reference decision of block
// j+1, and between the MFMAs this wave's share (1/8) of V^T(j+1).  VALU(j): p, the row-sum part and the bf16 P operand of block j, and the
// rare rescale.  One workgroup barrier ends the iteration.  Per wave and block the
// matrix work (1024 cycles at d_qk = 128) exceeds the probability code, so on
// every SIMD the partner wave's probability code runs under this wave's MFMAs.
// G0 stages K blocks, G1 V blocks (2 LDS slots each, block j in slot j%2) between
// their MFMAs; buffer loads run one iteration ahead of the LDS stores, over a
// range ending at row S, so rows past S read as zeros.
#include "common.h"
#include "launch.h"

namespace attnfwd {
namespace {

constexpr int KB = 64;
constexpr float kRefSlack = 8.0f;

template <int DQK>
struct Bf16Tile {
    static constexpr int NKS = DQK / 16;              // 32x32x16 steps over d_qk
    static constexpr int K_STRIDE = DQK * 2 + 16;     // padded LDS row of K, bytes
    static constexpr int K_BYTES = KB * K_STRIDE;
    static constexpr int V_BYTES = KB * 256;          // d_v = 128 bf16 per key, chunk-swizzled
    static constexpr int VT_STRIDE = KB * 2 + 16;     // padded LDS row of V^T (one d, 64 keys), bytes
    static constexpr int VT_BYTES = 128 * VT_STRIDE;
    // LDS: 2 slots each of K, the key-major V staging tile and V^T; block j in slot j%2
    static constexpr int OFF_V = 2 * K_BYTES;
    static constexpr int OFF_VT = OFF_V + 2 * V_BYTES;
    static constexpr int LDS_BYTES = OFF_VT + 2 * VT_BYTES;
    static constexpr int K_CHUNKS = KB * DQK * 2 / 16;
    static constexpr int V_CHUNKS = KB * 256 / 16;
};

struct Bf16Params {
    const __bf16* q;
    const __bf16* k;
    const __bf16* v;
    __bf16* o;
    float* lse;   // (B, Hq, S) natural-log normaliser per query row, or null
    float c;      // sm * log2(e)
    int B, Hq, Hkv, S;
    int n_tiles;
    const int* cu;    // variable-length batches: B + 1 query row offsets (device), else null
    int total;        // variable-length batches: rows of the packed Q and O
    const int* cu_k;  // variable-length batches: B + 1 key row offsets (device)
    int total_k;      // variable-length batches: rows of the packed K and V
};

// 16-byte chunk swizzle of a V row (16 chunks of 8 bf16).  A transposing read of
// one 16-lane group covers 4 consecutive keys x 32 bytes (a chunk pair); XOR-ing
// the pair index with key%4 puts the 4 rows on 4 distinct 32-byte bank groups.
__device__ __forceinline__ int v_swz16(int row) { return (row & 3) << 1; }

// acc += A . B on the BF16 matrix cores (32x32x16), the accumulator tied to the
// destination registers (the builtin may give the result registers of its own
// and copy it back every iteration).  Results are read only after vacc_settle; the
// leading s_nop gives a vector write of an operand register just before it the wait
// states the compiler does not insert around inline asm.
__device__ __forceinline__ void mfma_bf16_vacc(f32x16& acc, const bf16x8& a, const bf16x8& b) {
    asm("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(acc) : "v"(a), "v"(b));
}

template <int DQK, bool CAUSAL, bool LSE, bool VARLEN>
__global__ void __launch_bounds__(512) bf16_causal_fwd(Bf16Params a) {
    using T = Bf16Tile<DQK>;
    constexpr int NT = 256;                       // threads per group
    constexpr int BM = 256;                       // query rows per workgroup
    constexpr int KPT = T::K_CHUNKS / NT;         // K chunks staged per G0 thread
    constexpr int VPT = T::V_CHUNKS / NT;         // V chunks staged per G1 thread
    static_assert(T::K_CHUNKS % NT == 0 && T::V_CHUNKS % NT == 0, "staging split");

    __shared__ __attribute__((aligned(16))) uint8_t smem_raw[T::LDS_BYTES];
    ATTN_LDS uint8_t* smem = (ATTN_LDS uint8_t*)smem_raw;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave index, uniform
    const int grp = w >> 2;                                   // 0: G0, 1: G1
    const int tg = tid & (NT - 1);                            // thread index in its group
    const int BH = a.B * a.Hq;
    const int L = blockIdx.x;
    int tile, bh;
    tile_of(L, BH, a.Hq / a.Hkv, a.n_tiles, tile, bh);
    const int b = bh / a.Hq;
    const int h = bh - b * a.Hq;
    const int g = h / (a.Hq / a.Hkv);
    // Sequence b: S query rows from packed row tok0, Sk key rows from packed row
    // tok0k; causal query i sees keys j <= i + qoff (qoff = Sk - S, the mask aligned
    // at the bottom right).  Equal-length batches are (B, S, H, d) with Sk = S and
    // qoff = 0; a variable-length batch packs its sequences along the rows, a.S
    // being the longest query run.  The offsets are clamped into the tensors, so
    // any contents of cu and cu_k keep every access inside them.
    int S = a.S;
    int Sk = S;
    int qoff = 0;
    int64_t tok0 = (int64_t)b * S;
    int64_t tok0k = tok0;
    if constexpr (VARLEN) {
        const int t0 = min(max(a.cu[b], 0), a.total);
        const int t1 = min(max(a.cu[b + 1], t0), a.total);
        const int u0 = min(max(a.cu_k[b], 0), a.total_k);
        const int u1 = min(max(a.cu_k[b + 1], u0), a.total_k);
        S = min(t1 - t0, a.S);
        Sk = u1 - u0;
        qoff = Sk - S;
        tok0 = t0;
        tok0k = u0;
        if (tile * BM >= S) return;   // whole workgroup: past the end of this sequence
    }
    const int q0 = tile * BM;
    const int kend = !CAUSAL ? Sk : VARLEN ? max(min(Sk, q0 + BM + qoff), 0) : min(S, q0 + BM);
    const int nblk = (kend + KB - 1) / KB;        // key blocks the workgroup walks
    // first block that needs a mask: the diagonal one (causal) or the ragged last one
    const int jdiag = !CAUSAL ? (Sk - 1) / KB : VARLEN ? max(q0 + qoff, 0) / KB : q0 / KB;

    const int c = lane & 31;
    const int hh = lane >> 5;
    const int qabs = q0 + 32 * w + c;             // query of this lane

    const int64_t q_row = (int64_t)a.Hq * DQK;    // elements between consecutive queries
    const int k_row = a.Hkv * DQK * 2;            // bytes between consecutive keys
    const int v_row = a.Hkv * 128 * 2;
    const uint8_t* kbase = reinterpret_cast<const uint8_t*>(a.k) + (tok0k * a.Hkv + g) * DQK * 2;
    const uint8_t* vbase = reinterpret_cast<const uint8_t*>(a.v) + (tok0k * a.Hkv + g) * 128 * 2;

    // Q^T operand: lane (query c, half hh) holds d in [16ks + 8hh, +8) for each step ks.
    bf16x8 qreg[T::NKS];
    {
        const bool ok = qabs < S;
        const uint8_t* qp = reinterpret_cast<const uint8_t*>(
            a.q + (tok0 + (ok ? qabs : 0)) * q_row + (int64_t)h * DQK + 8 * hh);
#pragma unroll
        for (int ks = 0; ks < T::NKS; ++ks) {
            i32x4 x = ok ? load16(qp + 32 * ks) : i32x4{0, 0, 0, 0};
            qreg[ks] = __builtin_bit_cast(bf16x8, x);
        }
    }

    // ---- staging.  G0 moves K blocks, G1 V blocks: HBM -> registers (gload, one
    // iteration ahead) -> LDS (lstore).  TPR consecutive threads cover TPR
    // consecutive 16-byte chunks of a row (16 for V and d_qk = 128 K rows, 8 for
    // d_qk = 192), so each 16-lane LDS store pass writes one or two rows: distinct
    // bank groups (K rows are padded by 16 bytes, V chunks XOR-swizzled within the
    // row).  Load i covers row pass i / CG (NT / TPR rows apart) and chunk group
    // i % CG (TPR chunks apart); the row pass is added to the vector offset, which
    // alone is range-checked.
    constexpr int K_TPR = (DQK / 8) % 16 == 0 ? 16 : 8;   // K threads per row
    constexpr int K_CG = DQK / 8 / K_TPR;                  // chunk groups per K row
    static_assert(K_CG * (KB / (NT / K_TPR)) == KPT && (NT / 16) * 4 == KB && VPT == 4, "staging split");
    // Staging registers: one array when both groups stage as many chunks, one per group
    // when the counts differ.  The compiler merges the groups' loops when their shapes
    // allow it: one shared array with two counts becomes one loop of run-time length, and
    // two arrays with one count one loop over a selected array, both indexed in scratch.
    i32x4 stk[KPT], stv_own[KPT == VPT ? 1 : VPT];
    auto stv = [&](int i) -> i32x4& {
        if constexpr (KPT == VPT) return stk[i];
        else return stv_own[i];
    };
    int g_base, s_base, g_step;
    {
        const int tpr = grp == 0 ? K_TPR : 16;
        const int row = tg / tpr, cc = tg % tpr;
        if (grp == 0) {
            g_base = row * k_row + 16 * cc;
            s_base = row * T::K_STRIDE + 16 * cc;
            g_step = (NT / K_TPR) * k_row;
        } else {
            g_base = row * v_row + 16 * cc;
            s_base = T::OFF_V + row * 256 + 16 * (cc ^ v_swz16(row));   // row%4 is the same in every pass
            g_step = 16 * v_row;
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
            for (int i = 0; i < KPT; ++i)
                stk[i] = buffer_load16(r, g_base + (i / K_CG) * g_step + 16 * K_TPR * (i % K_CG));
        } else {
            const auto r = buffer_rsrc(vbase + (int64_t)j * KB * v_row, rows * v_row);
#pragma unroll
            for (int i = 0; i < VPT; ++i) stv(i) = buffer_load16(r, g_base + i * g_step);
        }
    };
    auto lstore = [&](int j) {   // G0: K slot j%2, G1: V slot j%2
        if (grp == 0) {
            ATTN_LDS uint8_t* base = smem + s_base + (j & 1) * T::K_BYTES;
#pragma unroll
            for (int i = 0; i < KPT; ++i)
                lds_store16(base + (i / K_CG) * (NT / K_TPR) * T::K_STRIDE + 16 * K_TPR * (i % K_CG), stk[i]);
        } else {
            ATTN_LDS uint8_t* base = smem + s_base + (j & 1) * T::V_BYTES;
#pragma unroll
            for (int i = 0; i < VPT; ++i) lds_store16(base + i * 16 * 256, stv(i));
        }
    };

    // ---- V^T construction.  The P.V A operand for d tile dt and K-step ks (keys
    // 16ks + [0,16)) gives lane (row c, half hh) d = 32dt + c and the keys 16ks +
    // {4hh..4hh+3, 8+4hh..8+4hh+3} (the P operand's order).  It is read from the
    // key-major V tile by two transposing reads per lane: 16-lane group G reads rows
    // key = 16ks + 8e4 + 4hh + (i/4), columns d = 32dt + 16(G&1) + 4(i%4) .. +3 (8
    // bytes per lane), and stored as bytes [32ks + 16hh, +16) of V^T row d.  Chunk
    // (4dt + vcol_chunk) ^ swz = 4(dt ^ (swz/4)) + (vcol_chunk ^ swz%4), so the byte
    // offset of d tile dt is voff[dt%2] + 128(dt/2).  Each wave builds 2 of the 16
    // (dt, ks) operands: 8 grp + 2(w%4) + u.
    int voff[2];
    {
        const int G = lane >> 4, il = lane & 15;
        const int vrow0 = 4 * hh + (il >> 2);
        const int vcol_chunk = 2 * (G & 1) + ((il & 3) >> 1);
#pragma unroll
        for (int dt = 0; dt < 2; ++dt)
            voff[dt] = T::OFF_V + vrow0 * 256 + 16 * ((4 * dt + vcol_chunk) ^ v_swz16(vrow0)) + 8 * (il & 1);
    }
    const int tcb = 8 * grp + 2 * (w & 3);        // first (dt, ks) operand this wave builds
    i16x4 tlo[2], thi[2];
    auto transpose_read = [&](int j) {   // V staging slot j%2 -> registers
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            const int cb = tcb + u, dt = cb & 3, ks = cb >> 2;
            const int va = (j & 1) * T::V_BYTES + (dt & 1 ? voff[1] : voff[0]) + 128 * (dt >> 1) + 4096 * ks;
            tlo[u] = lds_read_tr16(smem + va);
            thi[u] = lds_read_tr16(smem + va + 2048);
        }
    };
    auto transpose_write = [&](int j) {   // registers -> V^T slot j%2
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            const int cb = tcb + u, dt = cb & 3, ks = cb >> 2;
            lds_store16(smem + T::OFF_VT + (j & 1) * T::VT_BYTES + (32 * dt + c) * T::VT_STRIDE + 32 * ks + 16 * hh,
                        __builtin_bit_cast(i32x4, i16x8_cat(tlo[u], thi[u])));
        }
    };

    f32x16 o[4];
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) o[dt] = f32x16{0};
    float lpart = 0.0f;   // this lane's half of the row sum (its 32 of the 64 keys per block)
    float ref = -INFINITY;

    f32x16 s0, s1;        // S^T of the next block: keys [0,32) and [32,64)
    bf16x8 pb[4];         // P(j)^T, the B operand of K-step ks (keys 16ks + [0,16))
    // ---- probabilities in two parts.  prep (MFMA wave, in the shadow of the P.V
    // MFMAs): mask on diagonal blocks, row maximum, reference decision.  finish
    // (vector phase): p, its row-sum part and bf16 operand, the rare rescale.
    float nref_n = 0.0f;
    bool need_n = false;
    float mx_n = -INFINITY;
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
    auto prep_max = [&](int r0, int r1) {
        if (r0 == 0) mx_n = -INFINITY;
#pragma unroll
        for (int r = r0; r < r1; ++r) mx_n = fmaxf(fmaxf(mx_n, s0[r]), s1[r]);
    };
    auto prep_ref = [&]() {
        const float mx = pair_max(mx_n);
        const float M = fmaxf(ceilf(mx * a.c), -1.0e30f);   // floor: rows with no visible key here
        need_n = M > ref + kRefSlack;
        nref_n = need_n ? M : ref;
    };
    auto prep = [&](int j) {
        prep_mask(j);
        prep_max(0, 16);
        prep_ref();
    };
    auto finish = [&]() {
        const float nb = -nref_n;
        float bl = 0.0f;
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
            float p[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const float sv = (ks < 2) ? s0[8 * (ks & 1) + e] : s1[8 * (ks & 1) + e];
                p[e] = __builtin_amdgcn_exp2f(fmaf(sv, a.c, nb));
                bl += p[e];
            }
            pb[ks] = bf16x8{(__bf16)p[0], (__bf16)p[1], (__bf16)p[2], (__bf16)p[3],
                            (__bf16)p[4], (__bf16)p[5], (__bf16)p[6], (__bf16)p[7]};
        }
        // P complete here, in the vector phase: without this the compiler sinks the
        // probability code next to its use, into the MFMA phase
        asm volatile("" : "+v"(pb[0]), "+v"(pb[1]), "+v"(pb[2]), "+v"(pb[3]), "+v"(bl));
        if (__ballot(need_n)) {
            vacc_settle(o);
            const float f = __builtin_amdgcn_exp2f(ref - nref_n);   // exactly 1 for rows that do not move
#pragma unroll
            for (int dt = 0; dt < 4; ++dt)
#pragma unroll
                for (int r = 0; r < 16; ++r) o[dt][r] *= f;
            lpart *= f;
            vacc_settle(o);   // the rescaled values are back before the next MFMA reads them
        }
        lpart += bl;
        ref = nref_n;
    };

    constexpr int NS = 2 * T::NKS;      // score MFMAs per block
    constexpr int NM = NS + 16;         // MFMAs per phase
    constexpr int AHEAD = 3;            // operands are read this many MFMAs ahead of use
    // MFMA phase of block j.  Slot i < NS: score MFMA (key half i%2, d step i/2) of
    // S^T(j+1) from K slot (j+1)%2; slot NS + m: P.V MFMA for K-step m/4 and d tile
    // m%4 (consecutive MFMAs on different accumulators) from V^T slot j%2.  extra(i)
    // runs after MFMA i: the staging and V^T work of the MFMA wave.
    auto mfma_phase = [&](int j, auto&& extra) {
        __builtin_amdgcn_s_setprio(1);   // matrix issue wins arbitration against the partner wave
        const ATTN_LDS uint8_t* kp = smem + ((j + 1) & 1) * T::K_BYTES + c * T::K_STRIDE + 16 * hh;
        const ATTN_LDS uint8_t* vp = smem + T::OFF_VT + (j & 1) * T::VT_BYTES + c * T::VT_STRIDE + 16 * hh;
        auto operand = [&](int i) {
            if (i < NS) return __builtin_bit_cast(bf16x8, lds_load16(kp + (i & 1) * 32 * T::K_STRIDE + 32 * (i >> 1)));
            const int m = i - NS, ks = m >> 2, dt = m & 3;
            return __builtin_bit_cast(bf16x8, lds_load16(vp + 32 * dt * T::VT_STRIDE + 32 * ks));
        };
        // S^T(j+1) is computed even for the last block (from the stale K slot, in
        // bounds, result unused): one branch-free sequence keeps the accumulators in
        // fixed registers.
        bf16x8 opb[AHEAD + 1];
#pragma unroll
        for (int i = 0; i < AHEAD; ++i) opb[i] = operand(i);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int i = 0; i < NM; ++i) {
            if (i + AHEAD < NM) opb[(i + AHEAD) % (AHEAD + 1)] = operand(i + AHEAD);
            const bf16x8& op = opb[i % (AHEAD + 1)];
            if (i < NS) {
                f32x16& sd = (i & 1) ? s1 : s0;
                sd = __builtin_amdgcn_mfma_f32_32x32x16_bf16(op, qreg[i >> 1], i < 2 ? f32x16{0} : sd, 0, 0, 0);
            } else {
                const int m = i - NS;
                mfma_bf16_vacc(o[m & 3], op, pb[m >> 2]);
            }
            // prep of block j+1 once its score MFMAs have completed
            if (i == NS + 2) prep_mask(j + 1);
            if (i == NS + 4) prep_max(0, 4);
            if (i == NS + 5) prep_max(4, 8);
            if (i == NS + 6) prep_max(8, 12);
            if (i == NS + 7) prep_max(12, 16);
            if (i == NS + 8) prep_ref();
            extra(i);
            __builtin_amdgcn_sched_barrier(0);
        }
        __builtin_amdgcn_s_setprio(0);
    };

    // ---- prologue: K(0), K(1) and V(0), V(1) staged, block 2 in flight, V^T(0)
    // built, S^T(0) for every wave.
    gload(0);
    lstore(0);
    gload(1);
    lstore(1);
    gload(2);
    block_sync();
    transpose_read(0);
    transpose_write(0);
    {
        const ATTN_LDS uint8_t* kp = smem + c * T::K_STRIDE + 16 * hh;
        s0 = f32x16{0};
        s1 = f32x16{0};
#pragma unroll
        for (int ks = 0; ks < T::NKS; ++ks) {
            s0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, lds_load16(kp + 32 * ks)),
                                                         qreg[ks], s0, 0, 0, 0);
            s1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                __builtin_bit_cast(bf16x8, lds_load16(kp + 32 * T::K_STRIDE + 32 * ks)), qreg[ks], s1, 0, 0, 0);
        }
    }
    block_sync();   // V^T(0) complete; K slot 0 is restaged in the first iteration

    // ---- main loop: one loop per group (one code path keeps the accumulators in
    // fixed registers), one barrier per iteration.  Nothing is guarded: staging
    // past the last block moves zeros into free slots, a vector phase past it sees
    // only masked keys (p = 0, no reference move), and an MFMA phase past it adds
    // 0 * 0.
    prep(0);
    if constexpr (DQK == 128) {
        // unrolled by two blocks: every LDS slot index (j % 2) is a constant in each copy, so the
        // operand and staging addresses fold into instruction offsets (+1.2% on the Qwen shape;
        // at d_qk = 192 the unrolled loop spills, so it keeps the plain loop below)
        auto iter0 = [&] [[gnu::always_inline]] (int j) {
            mfma_phase(j, [&](int i) {                    // MFMA(j)
                if (i == 0) transpose_read(j + 1);
                if (i == 1) lstore(j + 2);
                if (i == 3) gload(j + 3);
                if (i == 4) transpose_write(j + 1);
            });
            finish();                                     // VALU(j+1)
            block_sync();
        };
        auto iter1 = [&] [[gnu::always_inline]] (int j) {
            finish();                                     // VALU(j)
            mfma_phase(j, [&](int i) {                    // MFMA(j)
                if (i == 0) transpose_read(j + 1);
                if (i == 1) lstore(j + 2);
                if (i == 3) gload(j + 3);
                if (i == 4) transpose_write(j + 1);
            });
            block_sync();
        };
        if (grp == 0) {
            finish();
            for (int jj = 0; 2 * jj < nblk; ++jj) {
                iter0(2 * jj);
                if (2 * jj + 1 < nblk) iter0(2 * jj + 1);
            }
        } else {
            for (int jj = 0; 2 * jj < nblk; ++jj) {
                iter1(2 * jj);
                if (2 * jj + 1 < nblk) iter1(2 * jj + 1);
            }
        }
    } else {
        if (grp == 0) {
            finish();
            for (int j = 0; j < nblk; ++j) {
                mfma_phase(j, [&](int i) {                    // MFMA(j)
                    if (i == 0) transpose_read(j + 1);
                    if (i == 1) lstore(j + 2);
                    if (i == 3) gload(j + 3);
                    if (i == 4) transpose_write(j + 1);
                });
                finish();                                     // VALU(j+1)
                block_sync();
            }
        } else {
            for (int j = 0; j < nblk; ++j) {
                finish();                                     // VALU(j)
                mfma_phase(j, [&](int i) {                    // MFMA(j)
                    if (i == 0) transpose_read(j + 1);
                    if (i == 1) lstore(j + 2);
                    if (i == 3) gload(j + 3);
                    if (i == 4) transpose_write(j + 1);
                });
                block_sync();
            }
        }
    }
    // The matrix instructions ignore EXEC: settling the accumulators here also keeps
    // all matrix work (and any operand copies it needs) out of the divergent stores.
    vacc_settle(o);

    // ---- epilogue: out = bf16(O / l), lane holds query c, d = 32dt + 8(r/4) + 4hh + r%4.
    // l = sum_j 2^(t_j - ref), so the row's natural-log normaliser is ln2 * (log2 l + ref).
    const float lsum = lpart + other_half(lpart);
    // a query of a variable-length sequence that sees no key (more queries than keys)
    // has l = 0 and O = 0: divide by infinity instead, so its output is 0
    const float lsumd = (VARLEN && !(lsum > 0.0f)) ? INFINITY : lsum;
    if (LSE && hh == 0 && qabs < S)
        a.lse[(VARLEN ? (int64_t)h * a.total + tok0 : ((int64_t)b * a.Hq + h) * S) + qabs] = (log2f(lsum) + ref) * 0.6931471805599453f;
    const Quotient quot(lsumd);   // O / l, one reciprocal for the lane's 64 values
    if (qabs < S) {
        __bf16* op = a.o + ((tok0 + qabs) * a.Hq + h) * 128;
#pragma unroll
        for (int dt = 0; dt < 4; ++dt) {
#pragma unroll
            for (int r4 = 0; r4 < 4; ++r4) {
                float x0 = quot(o[dt][4 * r4 + 0]);
                float x1 = quot(o[dt][4 * r4 + 1]);
                float x2 = quot(o[dt][4 * r4 + 2]);
                float x3 = quot(o[dt][4 * r4 + 3]);
                uint2 pk = make_uint2(pack_bf16x2(x0, x1), pack_bf16x2(x2, x3));
                *reinterpret_cast<uint2*>(op + 32 * dt + 8 * r4 + 4 * hh) = pk;
            }
        }
    }
}

template <int DQK, bool CAUSAL, bool LSE, bool VARLEN>
hipError_t launch_t(const Problem& p) {
    constexpr int BM = 256;
    Bf16Params a;
    a.q = static_cast<const __bf16*>(p.q);
    a.k = static_cast<const __bf16*>(p.k);
    a.v = static_cast<const __bf16*>(p.v);
    a.o = static_cast<__bf16*>(p.o);
    a.lse = p.lse;
    a.c = (float)((double)p.sm * 1.4426950408889634);
    a.B = p.B;
    a.Hq = p.Hq;
    a.Hkv = p.Hkv;
    a.S = p.S;
    a.cu = p.cu;
    a.total = p.total;
    a.cu_k = p.cu_k;
    a.total_k = p.total_k;
    a.n_tiles = (p.S + BM - 1) / BM;
    const long long nblocks = (long long)a.n_tiles * p.B * p.Hq;
    if (nblocks <= 0 || nblocks > 0x7fffffffLL) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL((bf16_causal_fwd<DQK, CAUSAL, LSE, VARLEN>), dim3((unsigned)nblocks), dim3(512), 0, p.stream, a);
    return hipGetLastError();
}

// The log-sum-exp store is a template switch: the kernels without it keep exactly the
// code they have when no caller asks for it.
template <bool CAUSAL, bool LSE, bool VARLEN>
hipError_t launch_c(const Problem& p) {
    if (p.d_qk == 128) return launch_t<128, CAUSAL, LSE, VARLEN>(p);
    if (p.d_qk == 192) return launch_t<192, CAUSAL, LSE, VARLEN>(p);
    return hipErrorInvalidValue;
}

template <bool VARLEN>
hipError_t launch_v(const Problem& p) {
    if (p.lse) return p.causal ? launch_c<true, true, VARLEN>(p) : launch_c<false, true, VARLEN>(p);
    return p.causal ? launch_c<true, false, VARLEN>(p) : launch_c<false, false, VARLEN>(p);
}

}  // namespace

hipError_t launch_bf16(const Problem& p) { return p.cu ? launch_v<true>(p) : launch_v<false>(p); }

}  // namespace attnfwd

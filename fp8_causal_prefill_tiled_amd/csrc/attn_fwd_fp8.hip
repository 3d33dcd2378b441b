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
// fp8_causal_fwd (this file) takes one 64-key block per phase and stages K and V
// through registers (the exponential path); fp8_causal_fwd_pair
// (attn_fwd_fp8_pair.hip) takes two blocks per phase (128 keys, the block size of
// the pages' ping-pong) and stages K and V with direct HBM-to-LDS loads, which keep
// the staging out of the registers that the second block's scores need (Lean P).
// They are separate translation units because they are compiled with different
// code-generation options; the device code they share is in fp8_common.h.
#include "fp8_common.h"

// This file is compiled once per head dimension, FP8_EXP_DQK = 128 or 192, each
// build with its own code-generation options, and each defines its own entry
// point launch_fp8_exp_d<FP8_EXP_DQK>.
#if !defined(FP8_EXP_DQK) || (FP8_EXP_DQK != 128 && FP8_EXP_DQK != 192)
#error "compile attn_fwd_fp8.hip with -DFP8_EXP_DQK=128 or -DFP8_EXP_DQK=192"
#endif

namespace attnfwd {
namespace {

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
    // Staging registers: one array when both groups stage as many chunks, one per group
    // when the counts differ.  The compiler merges the groups' loops when their shapes
    // allow it: one shared array with two counts becomes one loop of run-time length, and
    // two arrays with one count one loop over a selected array, both indexed in scratch.
    i32x4 stk[KPT], stv_own[KPT == VPT ? 1 : VPT];
    auto stv = [&](int i) -> i32x4& {
        if constexpr (KPT == VPT) return stk[i];
        else return stv_own[i];
    };
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
            for (int i = 0; i < KPT; ++i) stk[i] = buffer_load16(r, go[i]);
        } else {
            const auto r = buffer_rsrc(vbase + (int64_t)j * KB * v_row, rows * v_row);
#pragma unroll
            for (int i = 0; i < VPT; ++i) stv(i) = buffer_load16(r, go[i]);
        }
    };
    auto lstore = [&](int j) {   // G0: K slot j%2, G1: staging slot j%2
        if (grp == 0) {
            ATTN_LDS uint8_t* base = smem + (j & 1) * T::K_BYTES;
#pragma unroll
            for (int i = 0; i < KPT; ++i) lds_store16(base + so[i], stk[i]);
        } else {
            ATTN_LDS uint8_t* base = smem + (j & 1) * T::V_BYTES;
#pragma unroll
            for (int i = 0; i < VPT; ++i) lds_store16(base + so[i], stv(i));
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
    if constexpr (DQK == 192) {
        // unrolled by two blocks: every LDS slot index (j % 2) is a constant in each copy, so the
        // operand and staging addresses fold into instruction offsets (+0.9% on the MLA shape; at
        // d_qk = 128 the unrolled loop measured 5% slower, so that kernel keeps the plain loop)
        auto iter0 = [&] [[gnu::always_inline]] (int j) {
            mfma_phase(j, [&](int i) {                    // MFMA(j)
                if (kTransposeOnG0 && i == 0) transpose_read(j + 1);
                if (i == 1) lstore(j + 2);
                if (i == 2) gload(j + 3);
                if (kTransposeOnG0 && i == 4) transpose_write(j + 1);
            });
            finish();                                     // VALU(j+1)
            block_sync();
        };
        auto iter1 = [&] [[gnu::always_inline]] (int j) {
            finish();                                     // VALU(j)
            mfma_phase(j, [&](int i) {                    // MFMA(j)
                if (!kTransposeOnG0 && i == 0) transpose_read(j + 1);
                if (i == 1) lstore(j + 2);
                if (i == 2) gload(j + 3);
                if (!kTransposeOnG0 && i == 4) transpose_write(j + 1);
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
    }
    // The matrix instructions ignore EXEC: settling the accumulators here also keeps
    // all matrix work (and any operand copies it needs) out of the divergent stores.
    vacc_settle(o, lsum);

    store_out<LSE, VARLEN>(a, u, qabs, hh, o, lsum, ref, scl.v);
}

template <int DQK, bool CAUSAL, bool LSE, bool VARLEN, bool DSCALE>
hipError_t launch_t(const Problem& p) {
    const Fp8Params a = fp8_params(p);
    const long long nblocks = (long long)a.n_tiles * p.B * p.Hq;
    if (nblocks <= 0 || nblocks > 0x7fffffffLL) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL((fp8_causal_fwd<DQK, 0, CAUSAL, LSE, VARLEN, DSCALE>), dim3((unsigned)nblocks), dim3(512), 0,
                       p.stream, a);
    return hipGetLastError();
}

// The log-sum-exp store is a template switch: the kernels without it keep exactly the
// code (and code layout) they have when no caller asks for it.
template <bool CAUSAL, bool LSE, bool VARLEN, bool DSCALE>
hipError_t launch_c(const Problem& p) {
    if (p.d_qk == FP8_EXP_DQK) return launch_t<FP8_EXP_DQK, CAUSAL, LSE, VARLEN, DSCALE>(p);
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

#define FP8_EXP_CAT2(a, b) a##b
#define FP8_EXP_CAT(a, b) FP8_EXP_CAT2(a, b)
hipError_t FP8_EXP_CAT(launch_fp8_exp_d, FP8_EXP_DQK)(const Problem& p) {
    if (p.cu) return p.dq ? hipErrorInvalidValue : launch_v<true, false>(p);
    return p.dq ? launch_v<false, true>(p) : launch_v<false, false>(p);
}

}  // namespace attnfwd

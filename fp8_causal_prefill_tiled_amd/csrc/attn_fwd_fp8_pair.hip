// FP8 causal prefill attention for gfx950, Lean P probabilities: the two-block
// ping-pong kernel fp8_causal_fwd_pair.  The method, the mapping on CDNA4 and the
// one-block kernel of the exponential path are in attn_fwd_fp8.hip; the device
// code both kernels share is in fp8_common.h.
#include "fp8_common.h"

namespace attnfwd {
namespace {

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
    constexpr int NB = T::NB;                     // 64-key blocks per iteration
    constexpr int NSLOT = T::NSLOT;
    constexpr int TPT = (128 * 4) / NT;           // V^T chunks of one block built per thread

    __shared__ __attribute__((aligned(16))) uint8_t smem_raw[T::LDS_BYTES];
    ATTN_LDS uint8_t* smem = (ATTN_LDS uint8_t*)smem_raw;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave index, uniform
    const int grp = w >> 2;                                   // 0: G0, 1: G1
    Work u;
    if (!work_of<CAUSAL, VARLEN>(a, u)) return;
    const int S = u.S, Sk = u.Sk, qoff = u.qoff, q0 = u.q0, nblk = u.nblk, jdiag = u.jdiag;
    const int c = lane & 31;
    const int hh = lane >> 5;
    const int qabs = q0 + 32 * w + c;             // query of this lane
    const Scales scl = scales_of<DSCALE>(a);
    const float sc_a8 = scl.a8;
    // Lean P codes as f32 subnormals.  The score MFMAs scale S by 2^-ksh (E8M0 operand
    // scales, exact), so that m0 = a8 * 2^(ksh-149) is a normal float; then one fused
    // fma(S', m0, (120 - 8M) * 2^-149) rounds a8 S + 120 - 8M to the subnormal grid, whose
    // ulp is one code: the result's bit pattern is the integer code, and the output clamp to
    // [0, 1] sends negative codes (and masked -inf scores) to 0.  This replaces the
    // float-to-byte conversion of every probability with a quarter as many byte permutes.
    const int ea8 = (int)((__float_as_uint(sc_a8) >> 23) & 0xff) - 127;   // a8 = 8c > 0, normal
    const int ksh = PMODE == 1 ? min(max(24 - ea8, 0), 254) : 0;
    const float sc_c = ldexpf(scl.c, ksh);        // c in units of S' (c * S = sc_c * S')
    const float sc_m0 = ldexpf(sc_a8, ksh - 149);
    // E8M0 scale bytes of the score MFMAs, set once under a full EXEC mask like sa below:
    // byte 0 (K operand) 2^-max(ksh-127, 0), byte 1 (Q operand) 2^-min(ksh, 127)
    int sks = (127 - max(ksh - 127, 0)) | ((127 - min(ksh, 127)) << 8);
    asm volatile("" : "+v"(sks));
    const int k_row = a.Hkv * DQK;                // bytes between consecutive keys
    const int v_row = a.Hkv * 128;
    // wave-uniform bases, so that the per-block staging addresses are scalar arithmetic
    const uint8_t* kbase = uniform_ptr(a.k + u.tok0k * k_row + (int64_t)u.g * DQK);
    const uint8_t* vbase = uniform_ptr(a.v + u.tok0k * v_row + (int64_t)u.g * 128);
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
    // The A-side E8M0 scale of the P.V MFMAs (127 = 2^0), set once here under a
    // full EXEC mask: matrix instructions read every lane's scale byte whatever
    // EXEC is, so the constant must never be materialised inside divergent code.
    int sa = 127;
    asm volatile("" : "+v"(sa));
    // e4m3 1.0 in every byte, the A operand of the row-sum MFMAs, kept in registers across the
    // loop (read from LDS it cost two reads and a wait per phase).  Opaque to the compiler, so
    // it is never rematerialised by vector moves just ahead of an (inline asm) matrix
    // instruction that reads it, a hazard the compiler does not see.
    i32x8 ones = i32x8{0x38383838, 0x38383838, 0x38383838, 0x38383838,
                       0x38383838, 0x38383838, 0x38383838, 0x38383838};
    asm volatile("" : "+v"(ones));

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

    // S^T += K.Q^T over one d step; on the Lean P path scaled by 2^-ksh (scale bytes in sks)
    auto score_mfma = [&](const i32x8& kop, const i32x8& qop, const f32x16& acc) {
        if (PMODE == 1) return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(kop, qop, acc, 0, 0, 0, sks, 1, sks);
        return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(kop, qop, acc, 0, 0, 0, 0, 0, 0);
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
    auto valu_phase = [&] [[gnu::always_inline]] (int p) {
        // masks: only pairs that reach the diagonal (or the ragged last block); the
        // formula leaves a block that lies wholly inside the visible range unchanged
        if (NB * p + NB - 1 >= jdiag) {
            const int qlim = CAUSAL ? min(qabs + qoff, Sk - 1) : Sk - 1;
            // the same bound for the wave's first and last query (qlim grows with the
            // query): a block every lane sees whole, or none of, needs no per-key test
            const int qw = __builtin_amdgcn_readfirstlane(q0 + 32 * w);
            const int qlo = CAUSAL ? min(qw + qoff, Sk - 1) : Sk - 1;
            const int qhi = CAUSAL ? min(qw + 31 + qoff, Sk - 1) : Sk - 1;
#pragma unroll
            for (int bl = 0; bl < NB; ++bl) {
                const int kb0 = (NB * p + bl) * KB;
                if (qlo - kb0 - 4 >= 32 + 27) continue;   // every key visible to every lane
                if (qhi - kb0 < 0) {                       // no key visible to any lane
#pragma unroll
                    for (int r = 0; r < 16; ++r) sc[bl][0][r] = sc[bl][1][r] = -INFINITY;
                    continue;
                }
                const int lim = qlim - kb0 - 4 * hh;
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
        // Block exponents.  Lane l holds the maximum of 32 of a block's keys for query l%32;
        // the other 32 are in lane l^32.  One v_permlane32_swap of the two blocks' maxima
        // puts both halves of block 0 into lanes 0-31 and both halves of block 1 into
        // lanes 32-63, so one max and one exponent computation serve both blocks, and a
        // second swap hands each lane the exponents of both.
        static_assert(NB == 2, "the exponent exchange pairs the two blocks of a pair");
        {
            const auto r = __builtin_amdgcn_permlane32_swap(__float_as_int(mx[0]), __float_as_int(mx[1]), false, false);
            const float t = fmaxf(__int_as_float(r[0]), __int_as_float(r[1]));
            // floor: rows with no visible key in the block
            const int e = __float_as_int(fmaxf(ceilf(t * sc_c), -1.0e30f));
            const auto m = __builtin_amdgcn_permlane32_swap(e, e, false, false);
            M[0] = __int_as_float(m[0]);
            M[1] = __int_as_float(m[1]);
        }
        const float Mmax = fmaxf(M[0], M[1]);
        const bool need = Mmax > ref + kRefSlack;
        const float nref = need ? Mmax : ref;
        // E8M0 byte of 2^(M-8-nref), exponent clamped to [-127, 127]: all terms are integers
        // in float (or the -1e30 floor), so the sums are exact and one median and one
        // conversion give it
        const float sbase = 119.0f - nref;
        float bias[NB];
#pragma unroll
        for (int bl = 0; bl < NB; ++bl) {
            // Lean P: (120 - 8M) * 2^-149, exact (an integer times the subnormal ulp)
            bias[bl] = PMODE == 0 ? 8.0f - M[bl] : fmaf(M[bl], -0x1p-146f, 120.0f * 0x1p-149f);
            sb[bl] = (int)__builtin_amdgcn_fmed3f(M[bl] + sbase, 0.0f, 254.0f);
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
            // every clamped multiply-add first, in place over the scores (all independent; the
            // clamp folds into the FMA), then the codes into words: bytes (c0, c1) and (c2, c3)
            // of each word into the low halves of two words, then those into one, three byte
            // permutes per word (written as shifts and ors they are re-associated into four)
#pragma unroll
            for (int h = 0; h < 2; ++h)
#pragma unroll
                for (int r = 0; r < 16; ++r)
#pragma unroll
                    for (int bl = 0; bl < NB; ++bl)
                        sc[bl][h][r] = __builtin_amdgcn_fmed3f(fmaf(sc[bl][h][r], sc_m0, bias[bl]), 0.0f, 1.0f);
            __builtin_amdgcn_sched_barrier(0);
            auto code = [&](int bl, int q4, int e) {   // code of word q4, byte e, as an integer
                return __float_as_uint((q4 < 4 ? sc[bl][0] : sc[bl][1])[4 * (q4 & 3) + e]);
            };
            unsigned lo2[NB][8], hi2[NB][8];
#pragma unroll
            for (int q4 = 0; q4 < 8; ++q4)
#pragma unroll
                for (int bl = 0; bl < NB; ++bl) lo2[bl][q4] = __builtin_amdgcn_perm(code(bl, q4, 1), code(bl, q4, 0), 0x0c0c0400u);
#pragma unroll
            for (int q4 = 0; q4 < 8; ++q4)
#pragma unroll
                for (int bl = 0; bl < NB; ++bl) hi2[bl][q4] = __builtin_amdgcn_perm(code(bl, q4, 3), code(bl, q4, 2), 0x0c0c0400u);
#pragma unroll
            for (int q4 = 0; q4 < 8; ++q4)
#pragma unroll
                for (int bl = 0; bl < NB; ++bl) pw[bl][q4] = (int)__builtin_amdgcn_perm(hi2[bl][q4], lo2[bl][q4], 0x05040100u);
            __builtin_amdgcn_sched_barrier(0);
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
    auto mfma_phase = [&] [[gnu::always_inline]] (int p, auto&& extra) {
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
                sd = score_mfma(opb[i % (PD + 1)], qr[ks >> 1], ks < 2 ? f32x16{0} : sd);
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
            s0 = score_mfma(kread(bl, 0, kk), qr[kk], s0);
            s1 = score_mfma(kread(bl, 1, kk), qr[kk], s1);
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
    // The loop is unrolled by two pairs (NSLOT / NB): within each copy every slot index is a
    // constant, so LDS operand and staging addresses fold into instruction offsets (the
    // phases are forced inline: called five times, the vector phase would otherwise become
    // a function call).
    static_assert(NSLOT == 2 * NB, "two pairs per unrolled iteration cycle through the slots");
    if (grp == 0) {
        auto iter = [&] [[gnu::always_inline]] (int p) {
            mfma_phase(p, [&](int i) {                    // MFMA(p)
                if (i == 0) transpose_read(NB * (p + 1));
                if (i == 4) transpose_write(NB * (p + 1));
            });
            dload(p + 2);
            valu_phase(p + 1);                            // VALU(p+1)
            vmem_lds_sync();
        };
        valu_phase(0);
        for (int pp = 0; 2 * pp < npair; ++pp) {
            iter(2 * pp);
            if (2 * pp + 1 < npair) iter(2 * pp + 1);
        }
    } else {
        auto iter = [&] [[gnu::always_inline]] (int p) {
            dload(p + 2);
            valu_phase(p);                                // VALU(p)
            mfma_phase(p, [&](int i) {                    // MFMA(p)
                if (i == 0) transpose_read(NB * (p + 1) + 1);
                if (i == 4) transpose_write(NB * (p + 1) + 1);
            });
            vmem_lds_sync();
        };
        for (int pp = 0; 2 * pp < npair; ++pp) {
            iter(2 * pp);
            if (2 * pp + 1 < npair) iter(2 * pp + 1);
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
    hipLaunchKernelGGL((fp8_causal_fwd_pair<DQK, 1, CAUSAL, LSE, VARLEN, DSCALE>), dim3((unsigned)nblocks), dim3(512), 0,
                       p.stream, a);
    return hipGetLastError();
}

// The log-sum-exp store is a template switch: the kernels without it keep exactly the
// code (and code layout) they have when no caller asks for it.
template <bool CAUSAL, bool LSE, bool VARLEN, bool DSCALE>
hipError_t launch_c(const Problem& p) {
    if (p.d_qk == 128) return launch_t<128, CAUSAL, LSE, VARLEN, DSCALE>(p);
    if (p.d_qk == 192) return launch_t<192, CAUSAL, LSE, VARLEN, DSCALE>(p);
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

hipError_t launch_fp8_lean(const Problem& p) {
    if (p.cu) return p.dq ? hipErrorInvalidValue : launch_v<true, false>(p);
    return p.dq ? launch_v<false, true>(p) : launch_v<false, false>(p);
}

}  // namespace attnfwd

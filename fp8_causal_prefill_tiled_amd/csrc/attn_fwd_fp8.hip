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
// Mapping on CDNA4.  A workgroup is NW waves; each wave owns 32 consecutive
// query rows of one head and walks the causal key blocks.  The score tile is
// computed transposed, S^T = K . Q^T (v_mfma_f32_32x32x64_f8f6f4, A = K rows
// from LDS, B = the wave's Q held in registers), so lane l holds query l%32 and
// 32 of the block's 64 keys: the row max is 32 in-lane maxima plus one
// v_permlane32_swap, and the packed FP8 probabilities are already the B operand
// of O^T = V^T . P^T.  V^T comes straight from LDS with the transposing
// ds_read_b64_tr_b8.  K and V blocks are staged HBM -> registers -> LDS with
// 16-byte coalesced loads, double-buffered, one barrier per block.
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
    // LDS: 3 slots each of K, V^T and the key-major V staging tile; block j uses slot j%3
    static constexpr int OFF_VT = 3 * K_BYTES;
    static constexpr int OFF_VS = OFF_VT + 3 * VT_BYTES;
    static constexpr int LDS_BYTES = OFF_VS + 3 * V_BYTES;
    static constexpr int K_CHUNKS = KB * DQK / 16;
    static constexpr int V_CHUNKS = KB * 128 / 16;
};

struct Fp8Params {
    const uint8_t* q;
    const uint8_t* k;
    const uint8_t* v;
    __bf16* o;
    float c;        // q_scale * k_scale * sm * log2(e)
    float a8;       // 8 * c, the Lean-P slope
    float v_scale;
    int B, Hq, Hkv, S;
    int n_tiles;    // query tiles per head
};

// 16-byte chunk swizzle of a V row in LDS.  The transposing read of one 16-lane
// group touches keys {b..b+3, b+8..b+11} (b = 0 mod 4); this maps them to 8
// distinct chunk positions, so the group's 128 bytes hit distinct banks.
__device__ __forceinline__ int v_swz(int row) { return (row & 3) | (((row >> 3) & 1) << 2); }

// One wave per SIMD, two query halves in ping-pong.
//
// A workgroup of 4 waves (one per SIMD, 512 registers each) covers 256 query
// rows of one head; wave w owns rows [64w, 64w + 64) of the tile as two 32-row
// halves A and B.  Each iteration j is two phases whose matrix and vector work
// are independent of each other:
//     phase 1:  MFMA  S^T of half B, block j  and  P.V of half B, block j-1
//               VALU  probabilities of half A, block j
//     phase 2:  MFMA  S^T of half A, block j+1  and  P.V of half A, block j
//               VALU  probabilities of half B, block j
// This is the pages' two-wave ping-pong ("Two-wave ping-pong schedule", Zyphra
// ZYFA page, MarkTechPost) moved inside one wave: the two halves take the roles
// of the two waves.  In the fully visible loop every phase is issued as fixed
// slots (the LDS reads of the operand two MFMAs ahead, one MFMA, about ten vector
// instructions), the number a 64-cycle 32x32x64 MFMA hides on gfx950 when one
// wave runs per SIMD.  Only two score tiles are live at any time.
//
// LDS.  K tiles (row-major, padded rows), V^T tiles and key-major V staging tiles
// each live in 3 slots, block j in slot j%3; the fully visible loop is unrolled
// three times so every LDS address is a per-lane base plus a constant.  V^T row
// d holds the block's 64 keys in the byte order of the probability operand, so
// both matrix operands are plain 16-byte LDS reads; it is built once per
// workgroup with the transposing ds_read_b64_tr_b8, which is far slower per byte
// than ds_read_b128 on gfx950.  Iteration j builds V^T(j+1), stores K(j+2) and
// V(j+2) from registers and issues the buffer loads of block j+3 (rows past S
// read as zeros); one barrier ends the iteration.
template <int DQK, int PMODE>
__global__ void __launch_bounds__(256, 1) fp8_causal_fwd(Fp8Params a) {
    using T = Fp8Tile<DQK>;
    constexpr int NW = 4;
    constexpr int NT = NW * 64;
    constexpr int BM = NW * 64;
    constexpr int KPT = (T::K_CHUNKS + NT - 1) / NT;
    constexpr int VPT = (T::V_CHUNKS + NT - 1) / NT;
    constexpr int TPT = (128 * 4) / NT;          // V^T chunks built per thread
    constexpr int KCH_ROW = DQK / 16;

    __shared__ __attribute__((aligned(16))) uint8_t smem_raw[T::LDS_BYTES];
    ATTN_LDS uint8_t* smem = (ATTN_LDS uint8_t*)smem_raw;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave index, uniform
    const int BH = a.B * a.Hq;
    const int L = blockIdx.x;
    const int tile = a.n_tiles - 1 - L / BH;      // heaviest (longest causal prefix) tiles first
    const int bh = L % BH;                        // consecutive blocks: consecutive heads (XCD spread)
    const int b = bh / a.Hq;
    const int h = bh - b * a.Hq;
    const int g = h / (a.Hq / a.Hkv);
    const int S = a.S;
    const int q0 = tile * BM;
    const int qw0 = q0 + 64 * w;
    const int kend = min(S, q0 + BM);
    const int nblk = (kend + KB - 1) / KB;        // key blocks the workgroup walks

    const int c = lane & 31;
    const int hh = lane >> 5;
    const int qA = qw0 + c;                       // query of this lane in half A
    const int qB = qw0 + 32 + c;                  // and in half B

    const int64_t q_row = (int64_t)a.Hq * DQK;
    const int k_row = a.Hkv * DQK;                // bytes between consecutive keys
    const int v_row = a.Hkv * 128;
    const uint8_t* kbase = a.k + (int64_t)b * S * k_row + (int64_t)g * DQK;
    const uint8_t* vbase = a.v + (int64_t)b * S * v_row + (int64_t)g * 128;

    // Q^T operands: lane (query c, half hh) holds d in [64kk + 32hh, +32) for each step kk.
    i32x8 qa[T::NKK], qb[T::NKK];
    auto load_q = [&](int qabs, i32x8 (&qr)[T::NKK]) {
        const bool ok = qabs < S;
        const uint8_t* qp = a.q + ((int64_t)b * S + (ok ? qabs : 0)) * q_row + (int64_t)h * DQK + 32 * hh;
#pragma unroll
        for (int kk = 0; kk < T::NKK; ++kk) {
            i32x4 lo = ok ? load16(qp + 64 * kk) : i32x4{0, 0, 0, 0};
            i32x4 hi = ok ? load16(qp + 64 * kk + 16) : i32x4{0, 0, 0, 0};
            qr[kk] = i32x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
        }
    };
    load_q(qA, qa);
    load_q(qB, qb);

    // ---- staging: HBM -> registers (gload, one buffer resource per block whose range
    // ends at row S, so rows past S read as zeros), registers -> LDS slot (lstore).
    i32x4 kst[KPT];
    i32x4 vst[VPT];
    int kgo[KPT], vgo[VPT];     // per-lane byte offsets of the staged chunks inside a block
    int kso[KPT], vso[VPT];     // and their LDS offsets inside a slot
#pragma unroll
    for (int i = 0; i < KPT; ++i) {
        const int idx = min(tid + i * NT, T::K_CHUNKS - 1);
        const int row = idx / KCH_ROW, cc = idx % KCH_ROW;
        kgo[i] = row * k_row + 16 * cc;
        kso[i] = row * T::K_STRIDE + 16 * cc;
    }
#pragma unroll
    for (int i = 0; i < VPT; ++i) {
        const int idx = tid + i * NT;
        const int row = idx >> 3, cc = idx & 7;
        vgo[i] = row * v_row + 16 * cc;
        vso[i] = row * 128 + 16 * (cc ^ v_swz(row));
    }
    auto gload = [&](int j) {
        const int rows = min(S - j * KB, KB);
        const auto kr = buffer_rsrc(kbase + (int64_t)j * KB * k_row, rows * k_row);
        const auto vr = buffer_rsrc(vbase + (int64_t)j * KB * v_row, rows * v_row);
#pragma unroll
        for (int i = 0; i < KPT; ++i)
            if (T::K_CHUNKS % NT == 0 || tid + i * NT < T::K_CHUNKS) kst[i] = buffer_load16(kr, kgo[i]);
#pragma unroll
        for (int i = 0; i < VPT; ++i) vst[i] = buffer_load16(vr, vgo[i]);
    };
    auto lstore = [&](int slot) {   // K -> K slot, V -> staging slot
        ATTN_LDS uint8_t* Ks = smem + slot * T::K_BYTES;
        ATTN_LDS uint8_t* Vs = smem + T::OFF_VS + slot * T::V_BYTES;
#pragma unroll
        for (int i = 0; i < KPT; ++i)
            if (T::K_CHUNKS % NT == 0 || tid + i * NT < T::K_CHUNKS) lds_store16(Ks + kso[i], kst[i]);
#pragma unroll
        for (int i = 0; i < VPT; ++i) lds_store16(Vs + vso[i], vst[i]);
    };

    // ---- V^T construction: V^T row d holds the 64 keys at positions p = 32h + t in the
    // probability-byte order key(h, t) = 32(t/16) + 8((t%16)/4) + 4h + t%4.  16-lane group
    // G (of 32) builds the chunk d in [16(G%8), +16), p in [16(G/8), +16) from two
    // transposing reads of 8 keys (rows) x 16 d (columns) of the key-major staging tile.
    int tr_off[TPT][2];
    int tr_dst[TPT];
#pragma unroll
    for (int u = 0; u < TPT; ++u) {
        const int G = 4 * w + (lane >> 4) + 16 * u, n = lane & 15, t = n >> 1;
        const int dbase = 16 * (G & 7), p0 = 16 * (G >> 3);
#pragma unroll
        for (int x = 0; x < 2; ++x) {
            const int pos = p0 + 8 * x + t;
            const int hk = pos >> 5, tk = pos & 31;
            const int key = 32 * (tk >> 4) + 8 * ((tk & 15) >> 2) + 4 * hk + (tk & 3);
            tr_off[u][x] = key * 128 + 16 * ((dbase >> 4) ^ v_swz(key)) + 8 * (n & 1);
        }
        tr_dst[u] = (dbase + n) * T::VT_STRIDE + p0;
    }
    i32x2 tlo[TPT], thi[TPT];
    auto transpose_read = [&](int slot) {   // staging slot -> registers
        const ATTN_LDS uint8_t* Vs = smem + T::OFF_VS + slot * T::V_BYTES;
#pragma unroll
        for (int u = 0; u < TPT; ++u) {
            tlo[u] = lds_read_tr8(Vs + tr_off[u][0]);
            thi[u] = lds_read_tr8(Vs + tr_off[u][1]);
        }
    };
    auto transpose_write = [&](int slot) {   // registers -> V^T slot
#pragma unroll
        for (int u = 0; u < TPT; ++u)
            lds_store16(smem + T::OFF_VT + slot * T::VT_BYTES + tr_dst[u],
                        i32x4{tlo[u][0], tlo[u][1], thi[u][0], thi[u][1]});
    };

    f32x16 oa[4], ob[4];
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) {
        oa[dt] = f32x16{0};
        ob[dt] = f32x16{0};
    }
    f32x16 la = f32x16{0}, lb = f32x16{0};
    float refa = -INFINITY, refb = -INFINITY;
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
    // Matrix operands, read from LDS once per block and kept in registers for both
    // halves.  op[i], i < NS, is a K operand of the score MFMAs (key half i%2, d step
    // i/2); op[NS + dt] is the V^T operand of d rows [32dt, +32).  Lane (row c, half
    // hh) reads 32 bytes at 32hh.  Phase 2 of iteration j reads K(j+1) and V^T(j);
    // phase 1 of iteration j+1 reuses both (S^T of half B, block j+1 and P.V of half
    // B, block j), so it issues no operand reads at all.
    constexpr int NS = 2 * T::NKK;      // score MFMAs per phase
    constexpr int NM = NS + 5;          // all MFMAs per phase
    i32x8 op[NS + 4];
    auto read_operand = [&](int kslot, int vslot, int i) {
        if (i < NS)
            op[i] = read32(smem + kslot * T::K_BYTES + c * T::K_STRIDE + 32 * hh + (i & 1) * 32 * T::K_STRIDE +
                           64 * (i >> 1));
        else if (i < NS + 4)
            op[i] = read32(smem + T::OFF_VT + vslot * T::VT_BYTES + (32 * (i - NS) + c) * T::VT_STRIDE + 32 * hh);
    };
    auto read_k = [&](int kslot) {
#pragma unroll
        for (int i = 0; i < NS; ++i) read_operand(kslot, 0, i);
    };
    auto read_v = [&](int vslot) {
#pragma unroll
        for (int i = NS; i < NS + 4; ++i) read_operand(0, vslot, i);
    };
    // S^T = K . Q^T for one half from the kept K operands: keys [0,32) in s0, [32,64) in s1.
    auto qk = [&](const i32x8 (&qr)[T::NKK], f32x16& s0, f32x16& s1) {
        s0 = f32x16{0};
        s1 = f32x16{0};
#pragma unroll
        for (int kk = 0; kk < T::NKK; ++kk) {
            s0 = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(op[2 * kk], qr[kk], s0, 0, 0, 0, 0, 0, 0);
            s1 = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(op[2 * kk + 1], qr[kk], s1, 0, 0, 0, 0, 0, 0);
        }
    };
    // O^T += V^T . P^T and L += 1 . P^T for one half from the kept V^T operands, both
    // scaled by the E8M0 byte sb.
    auto pv = [&](const i32x8& pvv, int sb, f32x16 (&o)[4], f32x16& l) {
#pragma unroll
        for (int dt = 0; dt < 4; ++dt) mfma_f8_scaled_acc(o[dt], op[NS + dt], pvv, sa, sb);
        mfma_f8_scaled_acc(l, ones, pvv, sa, sb);
    };

    // ---- probabilities of block j for one half: mask (diagonal blocks), block
    // exponent M, e4m3 bytes.  Independent of the running reference.  Written as
    // stages so the fully visible loop can spread them over the MFMAs of a phase.
    auto prob_mask = [&](int j, int qabs, f32x16& s0, f32x16& s1) {
        // key kb0 + off(r) + 4hh is visible iff off(r) <= min(qabs, S-1) - kb0 - 4hh
        const int lim = min(qabs, S - 1) - j * KB - 4 * hh;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int off = 8 * (r >> 2) + (r & 3);
            s0[r] = off <= lim ? s0[r] : -INFINITY;
            s1[r] = off + 32 <= lim ? s1[r] : -INFINITY;
        }
    };
    auto prob_max = [&](const f32x16& s0, const f32x16& s1, int r0, int r1, float& mx) {
#pragma unroll
        for (int r = r0; r < r1; ++r) mx = fmaxf(fmaxf(mx, s0[r]), s1[r]);
    };
    // block exponent M and the per-row bias of the probability formula
    auto prob_exponent = [&](float mx, float& M, float& bias) {
        mx = fmaxf(mx, other_half(mx));
        M = fmaxf(ceilf(mx * a.c), -1.0e30f);  // floor: rows with no visible key here
        bias = PMODE == 0 ? 8.0f - M : 120.0f - 8.0f * M;
    };
    // bytes of the 4 scores x[4q4 .. 4q4+3]: one packed dword of the P operand
    auto prob_bytes = [&](const f32x16& x, int q4, float bias) -> int {
        if (PMODE == 0) {
            const float p0 = __builtin_amdgcn_exp2f(fmaf(x[4 * q4 + 0], a.c, bias));
            const float p1 = __builtin_amdgcn_exp2f(fmaf(x[4 * q4 + 1], a.c, bias));
            const float p2 = __builtin_amdgcn_exp2f(fmaf(x[4 * q4 + 2], a.c, bias));
            const float p3 = __builtin_amdgcn_exp2f(fmaf(x[4 * q4 + 3], a.c, bias));
            const int wd = __builtin_amdgcn_cvt_pk_fp8_f32(p0, p1, 0, false);
            return __builtin_amdgcn_cvt_pk_fp8_f32(p2, p3, wd, true);
        } else {
            unsigned wd = 0;
            wd = __builtin_amdgcn_cvt_pk_u8_f32(fmaf(x[4 * q4 + 0], a.a8, bias), 0, wd);
            wd = __builtin_amdgcn_cvt_pk_u8_f32(fmaf(x[4 * q4 + 1], a.a8, bias), 1, wd);
            wd = __builtin_amdgcn_cvt_pk_u8_f32(fmaf(x[4 * q4 + 2], a.a8, bias), 2, wd);
            wd = __builtin_amdgcn_cvt_pk_u8_f32(fmaf(x[4 * q4 + 3], a.a8, bias), 3, wd);
            return (int)wd;
        }
    };
    auto probs = [&](int j, int qabs, f32x16& s0, f32x16& s1, float& M, i32x8& pvv) {
        prob_mask(j, qabs, s0, s1);
        float mx = -INFINITY, bias;
        prob_max(s0, s1, 0, 16, mx);
        prob_exponent(mx, M, bias);
        pvv = i32x8{prob_bytes(s0, 0, bias), prob_bytes(s0, 1, bias), prob_bytes(s0, 2, bias),
                    prob_bytes(s0, 3, bias), prob_bytes(s1, 0, bias), prob_bytes(s1, 1, bias),
                    prob_bytes(s1, 2, bias), prob_bytes(s1, 3, bias)};
    };
    // Lazy power-of-two reference of one half: it moves (an exact rescale of that
    // half's O and L) only when the block exponent exceeds it by more than
    // kRefSlack; then the E8M0 scale of the block.
    auto commit = [&](float M, float& ref, f32x16 (&o)[4], f32x16& l, int& sb) {
        const bool need = M > ref + kRefSlack;
        if (__ballot(need)) {
            acc_settle(o, l);
            const float nr = need ? M : ref;
            const float f = need ? __builtin_amdgcn_exp2f(ref - nr) : 1.0f;
#pragma unroll
            for (int dt = 0; dt < 4; ++dt)
#pragma unroll
                for (int r = 0; r < 16; ++r) o[dt][r] *= f;
#pragma unroll
            for (int r = 0; r < 16; ++r) l[r] *= f;
            acc_settle(o, l);   // the rescaled values are back before the next MFMA reads them
            ref = nr;
        }
        sb = (int)fminf(fmaxf(M - 8.0f - ref, -127.0f), 127.0f) + 127;
    };

    // ---- pipeline.  Entering iteration j: S^T(A, j) in sa0/sa1; P(B, j-1) in pb with
    // scale sbb; op holds K(j) and V^T(j-1); LDS holds K(j+1) and V^T(j), staging slot
    // (j+1)%3 holds V(j+1); registers hold block j+2.
    f32x16 sa0, sa1, sb0, sb1;
    i32x8 pa, pb = i32x8{0, 0, 0, 0, 0, 0, 0, 0};
    int sba = 127, sbb = 127;
    gload(0);
    lstore(0);
    if (nblk > 1) {
        gload(1);
        lstore(1);
    }
    if (nblk > 2) gload(2);
    __syncthreads();
    transpose_read(0);
    transpose_write(0);
    read_k(0);
    qk(qa, sa0, sa1);
    __syncthreads();

    // General body (block 0, diagonal blocks, pipeline tail, unroll remainder):
    // masked, every staging step guarded, slots computed at run time.  Score MFMAs
    // come first in each phase: the tile they produce is read by the vector code
    // of the next phase.
    auto iteration = [&](int j) {
        float Ma, Mb;
        const int s0 = j % 3, s1 = (j + 1) % 3, s2 = (j + 2) % 3;
        // phase 1: operands K(j), V^T(j-1) already in op
        qk(qb, sb0, sb1);
        if (j >= 1) pv(pb, sbb, ob, lb);
        probs(j, qA, sa0, sa1, Ma, pa);
        if (j + 1 < nblk) {
            transpose_read(s1);
            transpose_write(s1);
        }
        if (j + 2 < nblk) lstore(s2);
        if (j + 3 < nblk) gload(j + 3);
        commit(Ma, refa, oa, la, sba);
        // phase 2: read K(j+1), V^T(j)
        if (j + 1 < nblk) {
            read_k(s1);
            qk(qa, sa0, sa1);
        }
        read_v(s0);
        pv(pa, sba, oa, la);
        probs(j, qB, sb0, sb1, Mb, pb);
        commit(Mb, refb, ob, lb, sbb);
        block_sync();
    };

    // One phase of the fully visible loop as an explicit instruction order: slot i
    // issues (with `reads`) the LDS reads of the operand two MFMAs ahead, MFMA i, a
    // share of the probability stages of the other half and any staging work, and
    // ends in a scheduling fence.  MFMAs 0 .. NS-1 compute S^T into (so0, so1) from
    // the K operands; MFMAs NS .. NS+4 accumulate P.V and the row sum from pin with
    // scale sbin; the vector work turns (si0, si1) into the bytes and exponent of
    // the next P.
    constexpr int NSTAGE = 11;          // 2 max, exponent, 8 byte groups
    auto fast_phase = [&](bool reads, int ks, int vs, const i32x8 (&qr)[T::NKK], f32x16& so0, f32x16& so1,
                          const i32x8& pin, int sbin, f32x16 (&o)[4], f32x16& l, f32x16& si0, f32x16& si1,
                          float& M, i32x8& pout, auto&& extra) {
        float mx = -INFINITY, bias = 0.0f;
        int pw[8];
        if (reads) {
            read_operand(ks, vs, 0);
            read_operand(ks, vs, 1);
        }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int i = 0; i < NM; ++i) {
            if (reads) read_operand(ks, vs, i + 2);
            if (i < NS) {
                f32x16& sd = (i & 1) ? so1 : so0;
                sd = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(op[i], qr[i >> 1], i < 2 ? f32x16{0} : sd,
                                                                      0, 0, 0, 0, 0, 0);
            } else if (i < NS + 4) {
                mfma_f8_scaled_acc(o[i - NS], op[i], pin, sa, sbin);
            } else {
                mfma_f8_scaled_acc(l, ones, pin, sa, sbin);
            }
            // the MFMA issues first; the slot's vector work then runs in its shadow
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int st = (i * NSTAGE) / NM; st < ((i + 1) * NSTAGE) / NM; ++st) {
                if (st == 0) prob_max(si0, si1, 0, 8, mx);
                else if (st == 1) prob_max(si0, si1, 8, 16, mx);
                else if (st == 2) prob_exponent(mx, M, bias);
                else {
                    pw[st - 3] = prob_bytes((st - 3) < 4 ? si0 : si1, (st - 3) & 3, bias);
                    asm volatile("" : "+v"(pw[st - 3]));   // computed here, not sunk to its use
                }
            }
            extra(i);
            __builtin_amdgcn_sched_barrier(0);
        }
        pout = i32x8{pw[0], pw[1], pw[2], pw[3], pw[4], pw[5], pw[6], pw[7]};
    };
    // Fully visible block j (slot r = j%3, a compile-time constant) with every
    // neighbour in range.  Phase 1 issues no operand reads, so the LDS staging work
    // (V^T build, K and V stores) goes there.
    auto fast_iteration = [&](int j, auto rc) {
        constexpr int r = decltype(rc)::value;
        constexpr int s0 = r, s1 = (r + 1) % 3, s2 = (r + 2) % 3;
        float Ma, Mb;
        fast_phase(false, 0, 0, qb, sb0, sb1, pb, sbb, ob, lb, sa0, sa1, Ma, pa, [&](int i) {
            if (i == 0) transpose_read(s1);
            if (i == 3) transpose_write(s1);
            if (i == 4) lstore(s2);
            if (i == 5) gload(j + 3);
        });
        commit(Ma, refa, oa, la, sba);
        fast_phase(true, s1, s0, qa, sa0, sa1, pa, sba, oa, la, sb0, sb1, Mb, pb, [&](int) {});
        commit(Mb, refb, ob, lb, sbb);
        block_sync();
    };

    // Blocks [1, jfast) are fully visible to every wave of the workgroup and have all
    // neighbours in range.
    int jfast = max(1, min(nblk - 3, q0 / KB));
    asm volatile("" : "+s"(jfast));   // opaque bound: keep the fast loop a loop of its own
    iteration(0);
    int j = 1;
    for (; j + 2 < jfast; j += 3) {
        fast_iteration(j, std::integral_constant<int, 1>{});
        fast_iteration(j + 1, std::integral_constant<int, 2>{});
        fast_iteration(j + 2, std::integral_constant<int, 0>{});
    }
    for (; j < nblk; ++j) iteration(j);
    pv(pb, sbb, ob, lb);   // op holds V^T(nblk-1)
    // The matrix instructions ignore EXEC: settling the accumulators here also keeps
    // all matrix work (and any operand copies it needs) out of the divergent stores.
    acc_settle(oa, la);
    acc_settle(ob, lb);

    // ---- epilogue: out = bf16(v_scale * (O / L)), lane holds query c of a half,
    // d = 32dt + 8(r/4) + 4hh + r%4
    auto store = [&](int qabs, const f32x16 (&o)[4], const f32x16& l) {
        if (qabs < S) {
            const float lsum = l[0];
            __bf16* op = a.o + (((int64_t)b * S + qabs) * a.Hq + h) * 128;
#pragma unroll
            for (int dt = 0; dt < 4; ++dt) {
#pragma unroll
                for (int r4 = 0; r4 < 4; ++r4) {
                    float x0 = (o[dt][4 * r4 + 0] / lsum) * a.v_scale;
                    float x1 = (o[dt][4 * r4 + 1] / lsum) * a.v_scale;
                    float x2 = (o[dt][4 * r4 + 2] / lsum) * a.v_scale;
                    float x3 = (o[dt][4 * r4 + 3] / lsum) * a.v_scale;
                    uint2 pk = make_uint2(pack_bf16x2(x0, x1), pack_bf16x2(x2, x3));
                    *reinterpret_cast<uint2*>(op + 32 * dt + 8 * r4 + 4 * hh) = pk;
                }
            }
        }
    };
    store(qA, oa, la);
    store(qB, ob, lb);
}

template <int DQK, int PMODE>
hipError_t launch_t(const Problem& p) {
    constexpr int NW = 4;
    constexpr int BM = NW * 64;
    Fp8Params a;
    a.q = static_cast<const uint8_t*>(p.q);
    a.k = static_cast<const uint8_t*>(p.k);
    a.v = static_cast<const uint8_t*>(p.v);
    a.o = static_cast<__bf16*>(p.o);
    const double c = (double)p.q_scale * p.k_scale * p.sm * 1.4426950408889634;
    a.c = (float)c;
    a.a8 = (float)(8.0 * c);
    a.v_scale = p.v_scale;
    a.B = p.B;
    a.Hq = p.Hq;
    a.Hkv = p.Hkv;
    a.S = p.S;
    a.n_tiles = (p.S + BM - 1) / BM;
    const long long nblocks = (long long)a.n_tiles * p.B * p.Hq;
    if (nblocks <= 0 || nblocks > 0x7fffffffLL) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL((fp8_causal_fwd<DQK, PMODE>), dim3((unsigned)nblocks), dim3(NW * 64), 0, p.stream, a);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_fp8(const Problem& p) {
    if (p.d_qk == 128) return p.p_mode == 0 ? launch_t<128, 0>(p) : launch_t<128, 1>(p);
    if (p.d_qk == 192) return p.p_mode == 0 ? launch_t<192, 0>(p) : launch_t<192, 1>(p);
    return hipErrorInvalidValue;
}

}  // namespace attnfwd

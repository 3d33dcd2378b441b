// BF16 causal prefill attention for gfx950.
//
// The pages say only that the BF16 kernels are plain HIP and gain 1.01-1.02x
// over the vendor library ("Zyphra ZYFA: FP8 FlashAttention for AMD MI355X, Up to
// 1.76x Faster", sections "What is ZYFA?" and TL;DR); the internals here are the
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
// O^T = V^T . P^T; V^T is read with the transposing ds_read_b64_tr_b16.
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
    static constexpr int STAGE = K_BYTES + V_BYTES;
    static constexpr int K_CHUNKS = KB * DQK * 2 / 16;
    static constexpr int V_CHUNKS = KB * 256 / 16;
};

struct Bf16Params {
    const __bf16* q;
    const __bf16* k;
    const __bf16* v;
    __bf16* o;
    float c;   // sm * log2(e)
    int B, Hq, Hkv, S;
    int n_tiles;
};

// 16-byte chunk swizzle of a V row (16 chunks of 8 bf16).  A transposing read of
// one 16-lane group covers 4 consecutive keys x 32 bytes (a chunk pair); XOR-ing
// the pair index with key%4 puts the 4 rows on 4 distinct 32-byte bank groups.
__device__ __forceinline__ int v_swz16(int row) { return (row & 3) << 1; }

template <int DQK, int NW>
__global__ void __launch_bounds__(NW * 64) bf16_causal_fwd(Bf16Params a) {
    using T = Bf16Tile<DQK>;
    constexpr int NT = NW * 64;
    constexpr int BM = NW * 32;
    constexpr int KPT = (T::K_CHUNKS + NT - 1) / NT;
    constexpr int VPT = (T::V_CHUNKS + NT - 1) / NT;
    constexpr int KCH_ROW = DQK / 8;

    __shared__ __attribute__((aligned(16))) uint8_t smem_raw[2 * T::STAGE];
    ATTN_LDS uint8_t* smem = (ATTN_LDS uint8_t*)smem_raw;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int w = tid >> 6;
    const int BH = a.B * a.Hq;
    const int L = blockIdx.x;
    const int tile = a.n_tiles - 1 - L / BH;
    const int bh = L % BH;
    const int b = bh / a.Hq;
    const int h = bh - b * a.Hq;
    const int g = h / (a.Hq / a.Hkv);
    const int S = a.S;
    const int q0 = tile * BM;
    const int qw0 = q0 + 32 * w;
    const int kend = min(S, q0 + BM);
    const int nblk = (kend + KB - 1) / KB;
    const int wnblk = qw0 < S ? (min(qw0 + 31, S - 1) / KB + 1) : 0;

    const int c = lane & 31;
    const int hh = lane >> 5;
    const int qabs = qw0 + c;

    const int64_t q_row = (int64_t)a.Hq * DQK;
    const int64_t k_row = (int64_t)a.Hkv * DQK;
    const int64_t v_row = (int64_t)a.Hkv * 128;
    const uint8_t* kbase = reinterpret_cast<const uint8_t*>(a.k + (int64_t)b * S * k_row + (int64_t)g * DQK);
    const uint8_t* vbase = reinterpret_cast<const uint8_t*>(a.v + (int64_t)b * S * v_row + (int64_t)g * 128);

    // Q^T operand: lane (query c, half hh) holds d in [16ks + 8hh, +8) for each step ks.
    bf16x8 qreg[T::NKS];
    {
        const bool ok = qabs < S;
        const uint8_t* qp = reinterpret_cast<const uint8_t*>(
            a.q + ((int64_t)b * S + (ok ? qabs : 0)) * q_row + (int64_t)h * DQK + 8 * hh);
#pragma unroll
        for (int ks = 0; ks < T::NKS; ++ks) {
            i32x4 x = ok ? load16(qp + 32 * ks) : i32x4{0, 0, 0, 0};
            qreg[ks] = __builtin_bit_cast(bf16x8, x);
        }
    }

    i32x4 kst[KPT];
    i32x4 vst[VPT];
    // Stage loads of key block j; only a block that crosses S is predicated.
    auto gload = [&](int j) {
        const bool full = (j + 1) * KB <= S;
#pragma unroll
        for (int i = 0; i < KPT; ++i) {
            const int idx = tid + i * NT;
            if (T::K_CHUNKS % NT == 0 || idx < T::K_CHUNKS) {
                const int row = idx / KCH_ROW, cc = idx % KCH_ROW;
                const int key = j * KB + row;
                const uint8_t* src = kbase + (int64_t)key * k_row * 2 + 16 * cc;
                if (full) kst[i] = load16(src);
                else kst[i] = key < S ? load16(src) : i32x4{0, 0, 0, 0};
            }
        }
#pragma unroll
        for (int i = 0; i < VPT; ++i) {
            const int idx = tid + i * NT;
            if (T::V_CHUNKS % NT == 0 || idx < T::V_CHUNKS) {
                const int row = idx >> 4, cc = idx & 15;
                const int key = j * KB + row;
                const uint8_t* src = vbase + (int64_t)key * v_row * 2 + 16 * cc;
                if (full) vst[i] = load16(src);
                else vst[i] = key < S ? load16(src) : i32x4{0, 0, 0, 0};
            }
        }
    };
    auto lstore = [&](int st) {
        ATTN_LDS uint8_t* Ks = smem + st * T::STAGE;
        ATTN_LDS uint8_t* Vs = Ks + T::K_BYTES;
#pragma unroll
        for (int i = 0; i < KPT; ++i) {
            const int idx = tid + i * NT;
            if (T::K_CHUNKS % NT == 0 || idx < T::K_CHUNKS) {
                const int row = idx / KCH_ROW, cc = idx % KCH_ROW;
                lds_store16(Ks + row * T::K_STRIDE + 16 * cc, kst[i]);
            }
        }
#pragma unroll
        for (int i = 0; i < VPT; ++i) {
            const int idx = tid + i * NT;
            if (T::V_CHUNKS % NT == 0 || idx < T::V_CHUNKS) {
                const int row = idx >> 4, cc = idx & 15;
                lds_store16(Vs + row * 256 + 16 * (cc ^ v_swz16(row)), vst[i]);
            }
        }
    };

    // Transposing V reads: for K-step ks (keys 16ks + [0,16)) and half e4 of the
    // operand, group G reads rows key = 16ks + 8*e4 + 4hh + (i/4), columns
    // d = 32dt + 16(G&1) + 4(i%4) .. +3 (8 bytes per lane).
    const int G = lane >> 4, il = lane & 15;
    const int vrow0 = 4 * hh + (il >> 2);          // + 16ks + 8e4
    const int vcol_chunk = 2 * (G & 1) + ((il & 3) >> 1);   // + 4dt  (chunk of 8 bf16)
    const int vcol_byte = 8 * (il & 1);

    f32x16 o[4];
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) o[dt] = f32x16{0};
    float lpart = 0.0f;   // this lane's half of the row sum
    float ref = -INFINITY;

    gload(0);
    lstore(0);
    __syncthreads();

    for (int j = 0; j < nblk; ++j) {
        const int st = j & 1;
        if (j + 1 < nblk) gload(j + 1);
        if (j < wnblk) {
            const ATTN_LDS uint8_t* Ks = smem + st * T::STAGE;
            const ATTN_LDS uint8_t* Vs = Ks + T::K_BYTES;

            f32x16 s0 = f32x16{0}, s1 = f32x16{0};
#pragma unroll
            for (int ks = 0; ks < T::NKS; ++ks) {
                const ATTN_LDS uint8_t* kp = Ks + c * T::K_STRIDE + 32 * ks + 16 * hh;
                bf16x8 a0 = __builtin_bit_cast(bf16x8, lds_load16(kp));
                bf16x8 a1 = __builtin_bit_cast(bf16x8, lds_load16(kp + 32 * T::K_STRIDE));
                s0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a0, qreg[ks], s0, 0, 0, 0);
                s1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a1, qreg[ks], s1, 0, 0, 0);
            }

            // causal / tail mask: key kb0 + off(r) + 4hh is visible iff off(r) <= min(qabs, S-1) - kb0 - 4hh
            const int kb0 = j * KB;
            if (kb0 + KB - 1 > qw0) {
                const int lim = min(qabs, S - 1) - kb0 - 4 * hh;
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int off = 8 * (r >> 2) + (r & 3);
                    s0[r] = off <= lim ? s0[r] : -INFINITY;
                    s1[r] = off + 32 <= lim ? s1[r] : -INFINITY;
                }
            }

            float mx = -INFINITY;
#pragma unroll
            for (int r = 0; r < 16; ++r) mx = fmaxf(fmaxf(mx, s0[r]), s1[r]);
            mx = fmaxf(mx, other_half(mx));
            const float M = fmaxf(ceilf(mx * a.c), -1.0e30f);
            const bool need = M > ref + kRefSlack;
            if (__ballot(need)) {
                const float nref = need ? M : ref;
                const float f = need ? __builtin_amdgcn_exp2f(ref - nref) : 1.0f;
#pragma unroll
                for (int dt = 0; dt < 4; ++dt)
#pragma unroll
                    for (int r = 0; r < 16; ++r) o[dt][r] *= f;
                lpart *= f;
                ref = nref;
            }
            const float nb = -ref;

            // p = 2^(t - R), summed unrounded, packed to bf16 as the B operand of each K-step:
            // K-step ks covers keys 16ks + [0,16): registers 8(ks%2)..+7 of tile ks/2.
            bf16x8 pb[4];
#pragma unroll
            for (int ks = 0; ks < 4; ++ks) {
                float p[8];
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const float sv = (ks < 2) ? s0[8 * (ks & 1) + e] : s1[8 * (ks & 1) + e];
                    p[e] = __builtin_amdgcn_exp2f(fmaf(sv, a.c, nb));
                    lpart += p[e];
                }
                pb[ks] = bf16x8{(__bf16)p[0], (__bf16)p[1], (__bf16)p[2], (__bf16)p[3],
                                (__bf16)p[4], (__bf16)p[5], (__bf16)p[6], (__bf16)p[7]};
            }

#pragma unroll
            for (int dt = 0; dt < 4; ++dt) {
#pragma unroll
                for (int ks = 0; ks < 4; ++ks) {
                    i16x4 lo, hi;
                    {
                        const int key = 16 * ks + vrow0;
                        lo = lds_read_tr16(Vs + key * 256 + 16 * ((4 * dt + vcol_chunk) ^ v_swz16(key)) + vcol_byte);
                    }
                    {
                        const int key = 16 * ks + 8 + vrow0;
                        hi = lds_read_tr16(Vs + key * 256 + 16 * ((4 * dt + vcol_chunk) ^ v_swz16(key)) + vcol_byte);
                    }
                    bf16x8 va = __builtin_bit_cast(bf16x8, i16x8_cat(lo, hi));
                    o[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, pb[ks], o[dt], 0, 0, 0);
                }
            }
        }
        if (j + 1 < nblk) lstore(st ^ 1);
        __syncthreads();
    }

    const float lsum = lpart + other_half(lpart);
    if (qabs < S && wnblk > 0) {
        __bf16* op = a.o + (((int64_t)b * S + qabs) * a.Hq + h) * 128;
#pragma unroll
        for (int dt = 0; dt < 4; ++dt) {
#pragma unroll
            for (int r4 = 0; r4 < 4; ++r4) {
                float x0 = o[dt][4 * r4 + 0] / lsum;
                float x1 = o[dt][4 * r4 + 1] / lsum;
                float x2 = o[dt][4 * r4 + 2] / lsum;
                float x3 = o[dt][4 * r4 + 3] / lsum;
                uint2 pk = make_uint2(pack_bf16x2(x0, x1), pack_bf16x2(x2, x3));
                *reinterpret_cast<uint2*>(op + 32 * dt + 8 * r4 + 4 * hh) = pk;
            }
        }
    }
}

template <int DQK, int NW>
hipError_t launch_t(const Problem& p) {
    constexpr int BM = NW * 32;
    Bf16Params a;
    a.q = static_cast<const __bf16*>(p.q);
    a.k = static_cast<const __bf16*>(p.k);
    a.v = static_cast<const __bf16*>(p.v);
    a.o = static_cast<__bf16*>(p.o);
    a.c = (float)((double)p.sm * 1.4426950408889634);
    a.B = p.B;
    a.Hq = p.Hq;
    a.Hkv = p.Hkv;
    a.S = p.S;
    a.n_tiles = (p.S + BM - 1) / BM;
    const long long nblocks = (long long)a.n_tiles * p.B * p.Hq;
    if (nblocks <= 0 || nblocks > 0x7fffffffLL) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL((bf16_causal_fwd<DQK, NW>), dim3((unsigned)nblocks), dim3(NW * 64), 0, p.stream, a);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_bf16(const Problem& p) {
    constexpr int NW = 8;
    if (p.d_qk == 128) return launch_t<128, NW>(p);
    if (p.d_qk == 192) return launch_t<192, NW>(p);
    return hipErrorInvalidValue;
}

}  // namespace attnfwd

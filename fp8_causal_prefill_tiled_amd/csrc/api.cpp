// C-ABI layer of libattnfwd.so: argument validation, defaults, dispatch and
// error reporting.  Every check runs on the host before any HIP call.
#include "../../include/attn_fwd.h"
#include "launch.h"

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdint>
#include <cstdio>

namespace {

thread_local char g_err[512] = {0};

int fail(int status, const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof(g_err), fmt, ap);
    va_end(ap);
    return status;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

bool overlaps(const void* a, size_t na, const void* b, size_t nb) {
    uintptr_t a0 = reinterpret_cast<uintptr_t>(a), b0 = reinterpret_cast<uintptr_t>(b);
    return a0 < b0 + nb && b0 < a0 + na;
}

int finish(hipError_t e, const char* who);

// Shared checks; elem_qkv = bytes per Q/K/V element, rows / rows_k = rows of Q,O /
// K,V (B*S, or the packed totals of a variable-length batch).  Returns ATTN_OK, an
// error, or -1 for "empty problem, nothing to do".
int check_common(const void* q, const void* k, const void* v, void* o, const float* lse,
                 float softmax_scale, int B, int Hq, int Hkv, int S, int64_t rows, int64_t rows_k, int d_qk,
                 int d_v, int causal, size_t elem_qkv, const char* who) {
    if (B < 0 || S < 0) return fail(ATTN_E_INVALID_ARG, "%s: B=%d and S=%d must be >= 0", who, B, S);
    if (rows < 0 || rows_k < 0)
        return fail(ATTN_E_INVALID_ARG, "%s: total rows %lld / %lld must be >= 0", who, (long long)rows, (long long)rows_k);
    if (Hq <= 0 || Hkv <= 0) return fail(ATTN_E_INVALID_ARG, "%s: Hq=%d and Hkv=%d must be >= 1", who, Hq, Hkv);
    if (Hq % Hkv != 0) return fail(ATTN_E_INVALID_ARG, "%s: Hq=%d is not a multiple of Hkv=%d", who, Hq, Hkv);
    if (d_qk <= 0 || d_v <= 0) return fail(ATTN_E_INVALID_ARG, "%s: head dims d_qk=%d d_v=%d must be > 0", who, d_qk, d_v);
    if (!(std::isfinite(softmax_scale))) return fail(ATTN_E_INVALID_ARG, "%s: softmax_scale is not finite", who);
    if (causal != 0 && causal != 1) return fail(ATTN_E_INVALID_ARG, "%s: causal=%d must be 0 or 1", who, causal);
    if (d_qk != 128 && d_qk != 192) return fail(ATTN_E_UNSUPPORTED, "%s: d_qk=%d unsupported (128 or 192)", who, d_qk);
    if (d_v != 128) return fail(ATTN_E_UNSUPPORTED, "%s: d_v=%d unsupported (128)", who, d_v);
    // Every element offset is formed in 64-bit arithmetic by the kernels; the row
    // index and the head count must fit comfortably in 32-bit integers.
    const int64_t most = std::max<int64_t>(rows, rows_k);
    if (most > (int64_t)1 << 30) return fail(ATTN_E_UNSUPPORTED, "%s: %lld rows too many", who, (long long)most);
    // The kernels address one 64-key block of K or V (64 rows of H*d elements) and the
    // per-row strides inside it with 32-bit offsets and buffer ranges.
    const int64_t block_bytes = (int64_t)64 * std::max(Hq, Hkv) * std::max(d_qk, d_v) * (int64_t)elem_qkv;
    if (block_bytes >= ((int64_t)1 << 31))
        return fail(ATTN_E_UNSUPPORTED, "%s: Hq=%d / Hkv=%d heads too many (a 64-row block exceeds 2 GiB)", who, Hq,
                    Hkv);
    // one workgroup per (256-query tile, sequence, head)
    const int64_t grid = ((int64_t)S + 255) / 256 * B * Hq;
    if (grid > 0x7fffffffLL) return fail(ATTN_E_UNSUPPORTED, "%s: %lld workgroups too many", who, (long long)grid);
    if (B == 0 || S == 0 || rows == 0) return -1;
    if (!q || !k || !v || !o) return fail(ATTN_E_INVALID_ARG, "%s: null tensor pointer", who);
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o))
        return fail(ATTN_E_INVALID_ARG, "%s: tensor pointers must be 16-byte aligned", who);
    const size_t nq = (size_t)rows * Hq * d_qk * elem_qkv;
    const size_t nk = (size_t)rows_k * Hkv * d_qk * elem_qkv;
    const size_t nv = (size_t)rows_k * Hkv * d_v * elem_qkv;
    const size_t no = (size_t)rows * Hq * d_v * 2;
    if (overlaps(o, no, q, nq) || overlaps(o, no, k, nk) || overlaps(o, no, v, nv))
        return fail(ATTN_E_INVALID_ARG, "%s: output overlaps an input", who);
    if (lse) {
        if ((reinterpret_cast<uintptr_t>(lse) & 3u) != 0)
            return fail(ATTN_E_INVALID_ARG, "%s: lse pointer must be 4-byte aligned", who);
        const size_t nl = (size_t)rows * Hq * sizeof(float);
        if (overlaps(lse, nl, q, nq) || overlaps(lse, nl, k, nk) || overlaps(lse, nl, v, nv) || overlaps(lse, nl, o, no))
            return fail(ATTN_E_INVALID_ARG, "%s: lse overlaps another tensor", who);
    }
    return ATTN_OK;
}

// Checks of a variable-length batch's offsets pointer (its contents live on the
// device and are clamped by the kernels, so any values stay in bounds).
int check_cu(const int* cu, int n_seqs, const char* who) {
    if (n_seqs > 0 && !cu) return fail(ATTN_E_INVALID_ARG, "%s: null cu_seqlens", who);
    if (cu && (reinterpret_cast<uintptr_t>(cu) & 3u) != 0)
        return fail(ATTN_E_INVALID_ARG, "%s: cu_seqlens must be 4-byte aligned", who);
    return ATTN_OK;
}

int run_fp8(const void* q, const void* k, const void* v, void* o, float* lse, bool varlen, const int* cu, int total,
            const int* cu_k, int total_k, const float* dq, const float* dk, const float* dv,
            float q_scale, float k_scale, float v_scale, float softmax_scale, int B, int Hq, int Hkv, int S,
            int d_qk, int d_v, int causal, int p_mode, hipStream_t stream, const char* who) {
    const int64_t rows = varlen ? (int64_t)total : (int64_t)B * S;
    const int64_t rows_k = varlen ? (int64_t)total_k : rows;
    int st = check_common(q, k, v, o, lse, softmax_scale, B, Hq, Hkv, S, rows, rows_k, d_qk, d_v, causal, 1, who);
    if (st == -1) { g_err[0] = 0; return ATTN_OK; }
    if (st != ATTN_OK) return st;
    const bool dscale = dq != nullptr;
    if (dscale) {
        if (!dk || !dv) return fail(ATTN_E_INVALID_ARG, "%s: null scale pointer", who);
        const float* sp[3] = {dq, dk, dv};
        for (const float* x : sp)
            if ((reinterpret_cast<uintptr_t>(x) & 3u) != 0)
                return fail(ATTN_E_INVALID_ARG, "%s: scale pointers must be 4-byte aligned", who);
    } else if (!(std::isfinite(q_scale) && q_scale > 0.f) || !(std::isfinite(k_scale) && k_scale > 0.f) ||
               !(std::isfinite(v_scale) && v_scale > 0.f)) {
        return fail(ATTN_E_INVALID_ARG, "%s: q/k/v scales must be finite and > 0", who);
    }
    if (p_mode != ATTN_P_EXACT && p_mode != ATTN_P_LEAN)
        return fail(ATTN_E_INVALID_ARG, "%s: p_mode=%d must be 0 (exact) or 1 (lean)", who, p_mode);
    attnfwd::Problem p{q, k, v, o, q_scale, k_scale, v_scale,
                       softmax_scale > 0.f ? softmax_scale : 1.0f / std::sqrt((float)d_qk),
                       B, Hq, Hkv, S, d_qk, d_v, p_mode, stream, lse, causal, cu, (int)rows, cu_k, (int)rows_k,
                       dq, dk, dv};
    const double c = (double)q_scale * k_scale * p.sm * 1.4426950408889634;
    if (!dscale && !(c < 1e30 && c > 1e-30))
        return fail(ATTN_E_INVALID_ARG, "%s: q_scale*k_scale*softmax_scale out of range", who);
    return finish(attnfwd::launch_fp8(p), who);
}

int run_bf16(const void* q, const void* k, const void* v, void* o, float* lse, bool varlen, const int* cu, int total,
             const int* cu_k, int total_k,
             float softmax_scale, int B, int Hq, int Hkv, int S, int d_qk, int d_v, int causal,
             hipStream_t stream, const char* who) {
    const int64_t rows = varlen ? (int64_t)total : (int64_t)B * S;
    const int64_t rows_k = varlen ? (int64_t)total_k : rows;
    int st = check_common(q, k, v, o, lse, softmax_scale, B, Hq, Hkv, S, rows, rows_k, d_qk, d_v, causal, 2, who);
    if (st == -1) { g_err[0] = 0; return ATTN_OK; }
    if (st != ATTN_OK) return st;
    attnfwd::Problem p{q, k, v, o, 1.f, 1.f, 1.f,
                       softmax_scale > 0.f ? softmax_scale : 1.0f / std::sqrt((float)d_qk),
                       B, Hq, Hkv, S, d_qk, d_v, 0, stream, lse, causal, cu, (int)rows, cu_k, (int)rows_k};
    return finish(attnfwd::launch_bf16(p), who);
}

int finish(hipError_t e, const char* who) {
    if (e != hipSuccess) return fail(ATTN_E_HIP, "%s: HIP error %d (%s)", who, (int)e, hipGetErrorString(e));
    g_err[0] = 0;
    return ATTN_OK;
}

}  // namespace

extern "C" {

int attn_fwd_fp8_lse(const void* q, const void* k, const void* v, void* o, float* lse,
                     float q_scale, float k_scale, float v_scale, float softmax_scale,
                     int B, int Hq, int Hkv, int S, int d_qk, int d_v,
                     int causal, int p_mode, hipStream_t stream) {
    return run_fp8(q, k, v, o, lse, false, nullptr, 0, nullptr, 0, nullptr, nullptr, nullptr, q_scale, k_scale, v_scale, softmax_scale, B, Hq, Hkv, S, d_qk, d_v,
                   causal, p_mode, stream, lse ? "attn_fwd_fp8_lse" : "attn_fwd_fp8");
}

int attn_fwd_fp8(const void* q, const void* k, const void* v, void* o,
                 float q_scale, float k_scale, float v_scale, float softmax_scale,
                 int B, int Hq, int Hkv, int S, int d_qk, int d_v,
                 int causal, int p_mode, hipStream_t stream) {
    return attn_fwd_fp8_lse(q, k, v, o, nullptr, q_scale, k_scale, v_scale, softmax_scale,
                            B, Hq, Hkv, S, d_qk, d_v, causal, p_mode, stream);
}

int attn_fwd_fp8_varlen(const void* q, const void* k, const void* v, void* o, float* lse,
                        const int* cu_seqlens_q, const int* cu_seqlens_k, int n_seqs, int max_seqlen_q,
                        int total_q, int total_k, float q_scale, float k_scale, float v_scale,
                        float softmax_scale, int Hq, int Hkv, int d_qk, int d_v, int causal, int p_mode,
                        hipStream_t stream) {
    const char* who = "attn_fwd_fp8_varlen";
    if (int st = check_cu(cu_seqlens_q, n_seqs, who)) return st;
    if (int st = check_cu(cu_seqlens_k, 0, who)) return st;
    const int* cu_k = cu_seqlens_k ? cu_seqlens_k : cu_seqlens_q;
    return run_fp8(q, k, v, o, lse, true, cu_seqlens_q, total_q, cu_k, cu_seqlens_k ? total_k : total_q,
                   nullptr, nullptr, nullptr, q_scale, k_scale,
                   v_scale, softmax_scale, n_seqs, Hq, Hkv, max_seqlen_q, d_qk, d_v, causal, p_mode, stream, who);
}

int attn_fwd_fp8_dscale(const void* q, const void* k, const void* v, void* o, float* lse,
                        const float* q_scale, const float* k_scale, const float* v_scale, float softmax_scale,
                        int B, int Hq, int Hkv, int S, int d_qk, int d_v, int causal, int p_mode,
                        hipStream_t stream) {
    const char* who = "attn_fwd_fp8_dscale";
    if (!q_scale || !k_scale || !v_scale) return fail(ATTN_E_INVALID_ARG, "%s: null scale pointer", who);
    return run_fp8(q, k, v, o, lse, false, nullptr, 0, nullptr, 0, q_scale, k_scale, v_scale, 1.f, 1.f, 1.f,
                   softmax_scale, B, Hq, Hkv, S, d_qk, d_v, causal, p_mode, stream, who);
}

int attn_fwd_bf16_lse(const void* q, const void* k, const void* v, void* o, float* lse, float softmax_scale,
                      int B, int Hq, int Hkv, int S, int d_qk, int d_v, int causal, hipStream_t stream) {
    return run_bf16(q, k, v, o, lse, false, nullptr, 0, nullptr, 0, softmax_scale, B, Hq, Hkv, S, d_qk, d_v, causal, stream,
                    lse ? "attn_fwd_bf16_lse" : "attn_fwd_bf16");
}

int attn_fwd_bf16(const void* q, const void* k, const void* v, void* o, float softmax_scale,
                  int B, int Hq, int Hkv, int S, int d_qk, int d_v, int causal, hipStream_t stream) {
    return attn_fwd_bf16_lse(q, k, v, o, nullptr, softmax_scale, B, Hq, Hkv, S, d_qk, d_v, causal, stream);
}

int attn_fwd_bf16_varlen(const void* q, const void* k, const void* v, void* o, float* lse,
                         const int* cu_seqlens_q, const int* cu_seqlens_k, int n_seqs, int max_seqlen_q,
                         int total_q, int total_k, float softmax_scale, int Hq, int Hkv, int d_qk, int d_v,
                         int causal, hipStream_t stream) {
    const char* who = "attn_fwd_bf16_varlen";
    if (int st = check_cu(cu_seqlens_q, n_seqs, who)) return st;
    if (int st = check_cu(cu_seqlens_k, 0, who)) return st;
    const int* cu_k = cu_seqlens_k ? cu_seqlens_k : cu_seqlens_q;
    return run_bf16(q, k, v, o, lse, true, cu_seqlens_q, total_q, cu_k, cu_seqlens_k ? total_k : total_q,
                    softmax_scale, n_seqs, Hq, Hkv, max_seqlen_q, d_qk, d_v, causal, stream, who);
}

int attn_rotate_quant_bf16(const void* x, void* x8, float* scale, int B, int S, int H, int d,
                           hipStream_t stream) {
    const char* who = "attn_rotate_quant_bf16";
    if (B < 0 || S < 0 || H <= 0) return fail(ATTN_E_INVALID_ARG, "%s: B=%d S=%d H=%d out of range", who, B, S, H);
    if (d != 128 && d != 192) return fail(ATTN_E_UNSUPPORTED, "%s: d=%d unsupported (128 or 192)", who, d);
    if (!scale) return fail(ATTN_E_INVALID_ARG, "%s: null scale pointer", who);
    const int64_t n_el = (int64_t)B * S * H * d;
    if (n_el * 2 > ((int64_t)1 << 31)) return fail(ATTN_E_UNSUPPORTED, "%s: tensor of %lld elements too large", who, (long long)n_el);
    if (n_el > 0) {
        if (!x || !x8) return fail(ATTN_E_INVALID_ARG, "%s: null tensor pointer", who);
        if (!aligned16(x) || !aligned16(x8)) return fail(ATTN_E_INVALID_ARG, "%s: tensor pointers must be 16-byte aligned", who);
        if (overlaps(x8, (size_t)n_el, x, (size_t)n_el * 2) || overlaps(scale, 4, x, (size_t)n_el * 2) ||
            overlaps(scale, 4, x8, (size_t)n_el))
            return fail(ATTN_E_INVALID_ARG, "%s: output overlaps an input", who);
    }
    return finish(attnfwd::launch_rotate_quant(x, x8, scale, n_el, d, stream), who);
}

int attn_rotate_quant_bf16_prescaled(const void* x, void* x8, const float* scale, float* amax, int B, int S, int H,
                                     int d, hipStream_t stream) {
    const char* who = "attn_rotate_quant_bf16_prescaled";
    if (B < 0 || S < 0 || H <= 0) return fail(ATTN_E_INVALID_ARG, "%s: B=%d S=%d H=%d out of range", who, B, S, H);
    if (d != 128 && d != 192) return fail(ATTN_E_UNSUPPORTED, "%s: d=%d unsupported (128 or 192)", who, d);
    if (!scale) return fail(ATTN_E_INVALID_ARG, "%s: null scale pointer", who);
    if ((reinterpret_cast<uintptr_t>(scale) & 3u) != 0 || (reinterpret_cast<uintptr_t>(amax) & 3u) != 0)
        return fail(ATTN_E_INVALID_ARG, "%s: scale and amax pointers must be 4-byte aligned", who);
    const int64_t n_el = (int64_t)B * S * H * d;
    if (n_el * 2 > ((int64_t)1 << 31)) return fail(ATTN_E_UNSUPPORTED, "%s: tensor of %lld elements too large", who, (long long)n_el);
    if (n_el > 0) {
        if (!x || !x8) return fail(ATTN_E_INVALID_ARG, "%s: null tensor pointer", who);
        if (!aligned16(x) || !aligned16(x8)) return fail(ATTN_E_INVALID_ARG, "%s: tensor pointers must be 16-byte aligned", who);
        if (overlaps(x8, (size_t)n_el, x, (size_t)n_el * 2) ||
            (amax && (overlaps(amax, 4, x, (size_t)n_el * 2) || overlaps(amax, 4, x8, (size_t)n_el) ||
                      overlaps(amax, 4, scale, 4))))
            return fail(ATTN_E_INVALID_ARG, "%s: output overlaps an input", who);
    }
    if (n_el == 0 && !amax) { g_err[0] = 0; return ATTN_OK; }   // nothing to write: no HIP call
    return finish(attnfwd::launch_rotate_quant_prescaled(x, x8, scale, amax, n_el, d, stream), who);
}

const char* attn_last_error(void) { return g_err; }

int attn_abi_version(void) { return 105; }

}  // extern "C"

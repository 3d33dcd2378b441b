/*
 * attn_fwd.h - C ABI of libattnfwd.so: forward prefill attention (causal or
 * not, equal-length or variable-length batches) on AMD Instinct MI355X (CDNA4,
 * gfx950), and the Hadamard rotation + FP8 quantisation of its Q and K.
 *
 * Operation (every attention entry point): for every batch b, query head h and
 * query position i < S,
 *
 *     O[b,i,h,:] = sum_{j in K(i)} softmax_j( sm * <Q[b,i,h,:], K[b,j,g,:]> ) * V[b,j,g,:]
 *
 * with g = h / (Hq / Hkv) (grouped-query attention by consecutive groups), sm
 * the softmax scale and K(i) the keys query i sees: j <= i when causal == 1,
 * every j < S when causal == 0.  The causal case is the equal-length forward
 * prefill the pages scope the kernels to ("Breaking the FP8 Attention Bottleneck on AMD
 * MI355X: How Zyphra ZYFA Unleashes Performance", section "Application
 * Boundaries and Engineering Decisions"; "Zyphra ZYFA: FP8 FlashAttention for
 * AMD MI355X, Up to 1.76x Faster", TL;DR and comparison table row "Scope"),
 * computed FlashAttention-style as an online softmax over 64-key blocks.
 *
 * Layout: every tensor is contiguous (B, S, H, d) - the flash_attn_func
 * convention ("drop-in flash_attn_func interface", TL;DR of the second page).
 * Q: (B,S,Hq,d_qk), K: (B,S,Hkv,d_qk), V: (B,S,Hkv,d_v), O: (B,S,Hq,d_v) bf16.
 *
 * Ownership and execution: all pointers are device pointers owned by the
 * caller; the library keeps no state, allocates nothing and is reentrant.
 * The call enqueues its kernels on `stream` (0 = the default stream) and
 * returns without synchronising; O is valid once the stream has completed.
 * O must not overlap Q, K or V.
 *
 * The non-causal case (causal == 0) is the same loop over every key block, with
 * only the ragged last block masked.
 *
 * Supported shapes: d_qk in {128, 192}, d_v == 128, Hq % Hkv == 0, S >= 1
 * (any S; the ragged last tile is masked), causal in {0, 1}, tensor pointers
 * 16-byte aligned, and 64 * max(Hq, Hkv) * max(d_qk, d_v) * (bytes per Q/K/V
 * element) below 2^31 (the kernels address a 64-key block with 32-bit
 * offsets; larger head counts are ATTN_E_UNSUPPORTED).  B == 0 or S == 0 is an
 * empty problem: ATTN_OK, nothing launched.
 *
 * Errors: every argument check happens on the host before any HIP call and
 * returns ATTN_E_INVALID_ARG (a malformed argument) or ATTN_E_UNSUPPORTED (a
 * well-formed request outside the supported set); a launch failure returns
 * ATTN_E_HIP.  The library never aborts and never writes errno.
 * attn_last_error() describes the last non-OK status of the calling thread.
 */
#ifndef ATTN_FWD_H
#define ATTN_FWD_H

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    ATTN_OK = 0,
    ATTN_E_INVALID_ARG = 1,
    ATTN_E_UNSUPPORTED = 2,
    ATTN_E_HIP = 3
} attn_status;

/* Probability path of the FP8 kernel. */
typedef enum {
    /* p = e4m3_RNE(2^(t - M + 8)) from a true exponential on the vector unit
     * (the "exact P" of "Zyphra ZYFA: FP8 FlashAttention...", section
     * "Two-wave ping-pong schedule"). */
    ATTN_P_EXACT = 0,
    /* Lean P: the e4m3 code of 2^x is about 8x + 56, so the probability's FP8
     * byte is one multiply-add and one round-to-integer ("Zyphra ZYFA: FP8
     * FlashAttention...", section "Lean P: one multiply-add instead of an
     * exponential"). */
    ATTN_P_LEAN = 1
} attn_p_mode;

/*
 * FP8 causal prefill attention.
 *
 * q, k, v: OCP e4m3fn bytes; the dequantised value is scale * decode(byte)
 *          with q_scale, k_scale, v_scale > 0 and finite (per-tensor scales).
 * o:       bfloat16 output (round to nearest even).
 * softmax_scale: sm; a value <= 0 selects 1/sqrt(d_qk).
 * p_mode:  attn_p_mode.
 *
 * Method ("Zyphra ZYFA: FP8 FlashAttention for AMD MI355X, Up to 1.76x
 * Faster", section "Per-block scaling and a rounded row sum"): per query row
 * and 64-key block the probabilities are taken relative to 2^(M-8), M the
 * ceiling of the block's largest log2-domain score, rounded to e4m3, and
 * multiplied into V by the block-scaled FP8 matrix instruction whose E8M0
 * operand scale restores the power of two; the row is normalised by the sum
 * of the rounded probabilities (one extra matrix instruction per block).
 */
int attn_fwd_fp8(const void* q, const void* k, const void* v, void* o,
                 float q_scale, float k_scale, float v_scale, float softmax_scale,
                 int B, int Hq, int Hkv, int S, int d_qk, int d_v,
                 int causal, int p_mode, hipStream_t stream);

/*
 * attn_fwd_fp8 that also writes the log-sum-exp of every query row.
 *
 * lse: device pointer to B*Hq*S floats, layout (B, Hq, S) contiguous, 4-byte
 *      aligned, owned by the caller, not overlapping q, k, v or o; NULL makes
 *      the call identical to attn_fwd_fp8.  lse[b,h,i] = ln sum_{j in K(i)}
 *      exp(sm * <q_i, k_j>) on the dequantised inputs, taken from the very
 *      normaliser the kernel divides by: the sum of the rounded e4m3
 *      probabilities times their block powers of two.  It therefore carries the
 *      probability rounding: |lse - exact| <= ln(1 + 2^-4) per row on the exact
 *      path (each e4m3 rounding moves a term by at most 2^-4 of itself), and
 *      within the Lean-P code law's ratio range (the linear-mantissa chord
 *      overstates 2^x by at most 6.2%, plus half a code step) on Lean P.
 *      (B, Hq, S) is the layout FlashAttention-style libraries return it in;
 *      with O it is what exact merging of partial attention over key subsets
 *      needs (two partial results combine as a softmax over their lse values).
 * Other arguments, behaviour and errors as attn_fwd_fp8; a misaligned or
 * overlapping lse is ATTN_E_INVALID_ARG.
 */
int attn_fwd_fp8_lse(const void* q, const void* k, const void* v, void* o, float* lse,
                     float q_scale, float k_scale, float v_scale, float softmax_scale,
                     int B, int Hq, int Hkv, int S, int d_qk, int d_v,
                     int causal, int p_mode, hipStream_t stream);

/*
 * attn_fwd_fp8_lse with the per-tensor scales read from device memory, so that a
 * call can follow attn_rotate_quant_bf16 (which writes Q's and K's scales to
 * device memory) on the same stream with no host synchronisation in between.
 *
 * q_scale, k_scale, v_scale: device pointers to one float each, 4-byte aligned,
 *      read by the kernel when it runs (values as for attn_fwd_fp8: finite and
 *      > 0; they cannot be checked on the host - other values give undefined
 *      outputs, e.g. NaN from a zero scale times a masked score, never an
 *      out-of-bounds access).  The kernel forms
 *      q_scale * k_scale * softmax_scale * log2(e) in double precision as the
 *      host does for attn_fwd_fp8, so both entry points give the same bits.
 * lse: NULL or as for attn_fwd_fp8_lse.  Other arguments, behaviour and errors
 *      as attn_fwd_fp8_lse; a null or misaligned scale pointer is
 *      ATTN_E_INVALID_ARG.
 */
int attn_fwd_fp8_dscale(const void* q, const void* k, const void* v, void* o, float* lse,
                        const float* q_scale, const float* k_scale, const float* v_scale, float softmax_scale,
                        int B, int Hq, int Hkv, int S, int d_qk, int d_v, int causal, int p_mode,
                        hipStream_t stream);

/*
 * BF16 causal prefill attention (the BF16 kernel of "Zyphra ZYFA: FP8
 * FlashAttention...", section "What is ZYFA?").
 *
 * q, k, v: bfloat16; o: bfloat16.  softmax_scale <= 0 selects 1/sqrt(d_qk).
 * Probabilities are fp32 exponentials relative to a running per-row power-of-
 * two reference, rounded to bf16 for the P.V product; the row sum adds the
 * unrounded fp32 probabilities (standard FlashAttention-2 normalisation; the
 * pages do not describe the BF16 internals).
 */
int attn_fwd_bf16(const void* q, const void* k, const void* v, void* o,
                  float softmax_scale,
                  int B, int Hq, int Hkv, int S, int d_qk, int d_v,
                  int causal, hipStream_t stream);

/*
 * attn_fwd_bf16 that also writes the log-sum-exp of every query row: lse as
 * for attn_fwd_fp8_lse (B*Hq*S floats, (B, Hq, S), NULL = none), here from the
 * fp32 sum of the unrounded probabilities, so it matches the exact value on
 * the bf16 inputs to fp32 accuracy.
 */
int attn_fwd_bf16_lse(const void* q, const void* k, const void* v, void* o, float* lse,
                      float softmax_scale,
                      int B, int Hq, int Hkv, int S, int d_qk, int d_v,
                      int causal, hipStream_t stream);

/*
 * Hadamard rotation and per-tensor FP8 quantisation of a Q or K tensor ("Zyphra
 * ZYFA: FP8 FlashAttention for AMD MI355X, Up to 1.76x Faster", section "How
 * accurate is ZYFA's FP8 attention?": rotating Q and K by a Hadamard matrix
 * before quantisation cuts the input error to about half).
 *
 * x:     bfloat16 (B, S, H, d), contiguous, 16-byte aligned; d = 128 or 192.
 * x8:    output e4m3fn bytes (B, S, H, d), 16-byte aligned, not overlapping x.
 * scale: output, device pointer to one float: amax / 448 of the rotated tensor
 *        (1 if it is all zero); dequantised rotated value = scale * decode(byte).
 *
 * Each (token, head) vector is multiplied along d by the orthonormal
 * Sylvester-Hadamard matrix H_n / sqrt(n): n = 128 for d = 128, three blocks of
 * n = 64 for d = 192.  The codes are e4m3 RNE(rotated / scale), saturating at
 * +-448.  H is orthogonal, so rotating both Q and K leaves the attention scores
 * unchanged: pass the rotated codes and their scales to attn_fwd_fp8 (V is not
 * rotated).  Enqueues four small kernels on stream; allocates nothing; the
 * caller owns x, x8 and scale.  Errors as for attn_fwd_fp8: ATTN_E_INVALID_ARG
 * for null or misaligned pointers, negative sizes or overlapping buffers,
 * ATTN_E_UNSUPPORTED for d other than 128 or 192 or a tensor above 2^31 bytes.
 */
int attn_rotate_quant_bf16(const void* x, void* x8, float* scale, int B, int S, int H, int d,
                           hipStream_t stream);

/*
 * Variable-length batches: n_seqs sequences packed along the rows (the
 * flash_attn_varlen_func convention), each attending only to itself.  The
 * pages list variable batch sizing among what their kernels do not yet cover
 * ("Breaking the FP8 Attention Bottleneck on AMD MI355X", section
 * "Application Boundaries and Engineering Decisions"); this is the same kernel
 * with per-sequence row offsets.  A sequence may have fewer queries than keys
 * (a chunk of queries after a cached key prefix) or more: with Sq queries and
 * Sk keys the causal mask is aligned at the bottom right, query i seeing keys
 * j <= i + Sk - Sq (FlashAttention's convention; equal lengths give the usual
 * mask).  A query that sees no key gets O = 0 and lse = -inf.
 *
 * q: (total_q, Hq, d_qk), o: (total_q, Hq, d_v) bf16, k: (total_k, Hkv, d_qk),
 *    v: (total_k, Hkv, d_v); contiguous, 16-byte aligned.
 * cu_seqlens_q: device pointer to n_seqs + 1 int32 row offsets, 4-byte aligned:
 *    sequence i's queries are rows cu_seqlens_q[i] .. cu_seqlens_q[i+1]-1 of q/o.
 * cu_seqlens_k: the same for k/v, or NULL: keys at the query offsets
 *    (total_k is then ignored and taken equal to total_q).
 * Expected: offsets start at 0, never decrease, end at most at the totals,
 *    every query run at most max_seqlen_q.  The contents are not read on the host
 *    (no synchronisation); the kernels clamp every offset into its tensor and
 *    every query run to max_seqlen_q, so any contents keep all accesses in
 *    bounds.  Rows outside every sequence are left unwritten.
 * lse: NULL, or Hq * total_q floats, layout (Hq, total_q).
 * The grid covers ceil(max_seqlen_q / 256) query tiles per (sequence, head);
 * tiles past a sequence's end exit at once.  Other arguments, behaviour and
 * errors as attn_fwd_fp8_lse / attn_fwd_bf16_lse; n_seqs == 0,
 * max_seqlen_q == 0 or total_q == 0 is an empty problem (ATTN_OK, nothing
 * launched).
 */
int attn_fwd_fp8_varlen(const void* q, const void* k, const void* v, void* o, float* lse,
                        const int* cu_seqlens_q, const int* cu_seqlens_k, int n_seqs, int max_seqlen_q,
                        int total_q, int total_k, float q_scale, float k_scale, float v_scale,
                        float softmax_scale, int Hq, int Hkv, int d_qk, int d_v, int causal, int p_mode,
                        hipStream_t stream);
int attn_fwd_bf16_varlen(const void* q, const void* k, const void* v, void* o, float* lse,
                         const int* cu_seqlens_q, const int* cu_seqlens_k, int n_seqs, int max_seqlen_q,
                         int total_q, int total_k, float softmax_scale, int Hq, int Hkv, int d_qk, int d_v,
                         int causal, hipStream_t stream);

/*
 * One-pass form of attn_rotate_quant_bf16 for a scale known in advance (for
 * example from the previous step or a calibration run; per-tensor "delayed"
 * scaling): the same rotation, codes e4m3 RNE(rotated / *scale) saturating at
 * +-448, and, when amax is not NULL, *amax = max |rotated| of this tensor (the
 * next call's scale is amax / 448).  One streaming pass instead of two.
 *
 * scale: device pointer to one float (> 0 and finite; not checkable on the host),
 *        read by the kernel.  amax: device pointer to one float, or NULL.  Both
 *        4-byte aligned, amax not overlapping x, x8 or scale.  Other arguments,
 *        behaviour and errors as attn_rotate_quant_bf16.  Enqueues one kernel (two
 *        with amax); allocates nothing.
 */
int attn_rotate_quant_bf16_prescaled(const void* x, void* x8, const float* scale, float* amax, int B, int S, int H,
                                     int d, hipStream_t stream);

/* Message for the calling thread's last non-OK status ("" if none).  The
 * returned storage is thread-local and valid until that thread's next call. */
const char* attn_last_error(void);

/* ABI version of this header (major * 100 + minor). */
int attn_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* ATTN_FWD_H */

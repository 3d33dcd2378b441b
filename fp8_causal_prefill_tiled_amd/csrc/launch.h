// Internal interface between the C-ABI layer (api.cpp) and the kernel launchers.
#pragma once
#include <hip/hip_runtime_api.h>
#include <stdint.h>

namespace attnfwd {

// A validated problem.  Shapes follow include/attn_fwd.h; sm is the final
// softmax scale (already defaulted to 1/sqrt(d_qk)).
struct Problem {
    const void* q;
    const void* k;
    const void* v;
    void* o;
    float q_scale, k_scale, v_scale, sm;
    int B, Hq, Hkv, S, d_qk, d_v;
    int p_mode;
    hipStream_t stream;
    float* lse;   // (B, Hq, S) fp32 per-row log-sum-exp output, or null
    int causal;   // 1: key j visible to query i iff j <= i; 0: every key visible
    // Variable-length batch: B sequences packed along the rows, sequence b's queries at
    // rows cu[b]..cu[b+1]-1 of Q and O and its keys at rows cu_k[b]..cu_k[b+1]-1 of K
    // and V (device pointers, B + 1 entries each); S = the longest query run, total and
    // total_k = rows of the packed Q/O and K/V.  cu == nullptr: equal-length
    // (B, S, H, d) tensors.
    const int* cu;
    int total;
    const int* cu_k;
    int total_k;
    // FP8 only: per-tensor scales in device memory (one float each), or null (use the
    // values above)
    const float* dq;
    const float* dk;
    const float* dv;
};

// FP8 attention by probability mode and head dimension, each in a translation unit
// of its own: Lean P (p_mode 1) in attn_fwd_fp8_pair.hip, the exponential path in
// the two builds of attn_fwd_fp8.hip.
hipError_t launch_fp8_lean(const Problem& p);
hipError_t launch_fp8_exp_d128(const Problem& p);
hipError_t launch_fp8_exp_d192(const Problem& p);
inline hipError_t launch_fp8(const Problem& p) {
    if (p.p_mode == 1) return launch_fp8_lean(p);
    return p.d_qk == 192 ? launch_fp8_exp_d192(p) : launch_fp8_exp_d128(p);
}
hipError_t launch_bf16(const Problem& p);
// Hadamard rotation + per-tensor e4m3 quantisation of n_el bf16 values (rows of
// d elements); scale points to one device float.
hipError_t launch_rotate_quant(const void* x, void* x8, float* scale, int64_t n_el, int d, hipStream_t s);
// The same with the caller's scale (one pass); amax (nullable) receives max |rotated|.
hipError_t launch_rotate_quant_prescaled(const void* x, void* x8, const float* scale, float* amax, int64_t n_el,
                                         int d, hipStream_t s);

}  // namespace attnfwd

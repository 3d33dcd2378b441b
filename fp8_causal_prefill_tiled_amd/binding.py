"""ctypes binding of libattnfwd.so (argument marshalling only).

Every step of the attention runs in the library's HIP kernels; this module only
turns torch tensors into (pointer, shape) arguments, passes torch's current HIP
stream, and raises ``AttnError`` on a non-OK status.  It fails loudly when the
library has not been built - there is no fallback implementation.
"""
import ctypes
import math
import os
import subprocess

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_PKG, "libattnfwd.so")

ATTN_OK, ATTN_E_INVALID_ARG, ATTN_E_UNSUPPORTED, ATTN_E_HIP = 0, 1, 2, 3
P_EXACT, P_LEAN = 0, 1
_P_MODES = {"exact": P_EXACT, "lean": P_LEAN, P_EXACT: P_EXACT, P_LEAN: P_LEAN}

_EXPORTS = ("attn_fwd_fp8", "attn_fwd_fp8_lse", "attn_fwd_fp8_varlen", "attn_fwd_fp8_dscale", "attn_fwd_bf16", "attn_fwd_bf16_lse",
            "attn_fwd_bf16_varlen", "attn_rotate_quant_bf16", "attn_rotate_quant_bf16_prescaled", "attn_last_error",
            "attn_abi_version")


class AttnError(RuntimeError):
    def __init__(self, status, message):
        super().__init__(f"status {status}: {message}")
        self.status = status


_lib = None


def library_path():
    return _LIB_PATH


def load_library():
    """Load libattnfwd.so once; raise if it is missing."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        raise ImportError(f"{_LIB_PATH} is not built; run `python -m fp8_causal_prefill_tiled_amd.build`")
    lib = ctypes.CDLL(_LIB_PATH)
    vp, f, i = ctypes.c_void_p, ctypes.c_float, ctypes.c_int
    lib.attn_fwd_fp8.argtypes = [vp, vp, vp, vp, f, f, f, f, i, i, i, i, i, i, i, i, vp]
    lib.attn_fwd_fp8.restype = i
    lib.attn_fwd_fp8_lse.argtypes = [vp, vp, vp, vp, vp, f, f, f, f, i, i, i, i, i, i, i, i, vp]
    lib.attn_fwd_fp8_lse.restype = i
    lib.attn_fwd_fp8_dscale.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, f, i, i, i, i, i, i, i, i, vp]
    lib.attn_fwd_fp8_dscale.restype = i
    lib.attn_fwd_bf16.argtypes = [vp, vp, vp, vp, f, i, i, i, i, i, i, i, vp]
    lib.attn_fwd_bf16.restype = i
    lib.attn_fwd_bf16_lse.argtypes = [vp, vp, vp, vp, vp, f, i, i, i, i, i, i, i, vp]
    lib.attn_fwd_bf16_lse.restype = i
    lib.attn_fwd_fp8_varlen.argtypes = [vp, vp, vp, vp, vp, vp, vp, i, i, i, i, f, f, f, f, i, i, i, i, i, i, vp]
    lib.attn_fwd_fp8_varlen.restype = i
    lib.attn_fwd_bf16_varlen.argtypes = [vp, vp, vp, vp, vp, vp, vp, i, i, i, i, f, i, i, i, i, i, vp]
    lib.attn_fwd_bf16_varlen.restype = i
    lib.attn_rotate_quant_bf16.argtypes = [vp, vp, vp, i, i, i, i, vp]
    lib.attn_rotate_quant_bf16.restype = i
    lib.attn_rotate_quant_bf16_prescaled.argtypes = [vp, vp, vp, vp, i, i, i, i, vp]
    lib.attn_rotate_quant_bf16_prescaled.restype = i
    lib.attn_last_error.argtypes = []
    lib.attn_last_error.restype = ctypes.c_char_p
    lib.attn_abi_version.argtypes = []
    lib.attn_abi_version.restype = i
    _lib = lib
    return lib


def attn_last_error():
    return load_library().attn_last_error().decode()


def exported_symbols():
    """Dynamic symbols exported by the built library (via `nm -D`)."""
    out = subprocess.run(["nm", "-D", "--defined-only", _LIB_PATH], capture_output=True, text=True, check=True)
    return {ln.split()[-1] for ln in out.stdout.splitlines() if ln.strip()}


def _check(status):
    if status != ATTN_OK:
        raise AttnError(status, attn_last_error())


def _stream_ptr(stream, device):
    if stream is None:
        stream = torch.cuda.current_stream(device)
    return stream.cuda_stream


def _bshd(x, name):
    if x.dim() != 4:
        raise ValueError(f"{name} must be (B, S, H, d), got shape {tuple(x.shape)}")
    if not x.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if not x.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    return x.shape


def attn_fwd_fp8_raw(q, k, v, o, q_scale, k_scale, v_scale, softmax_scale, B, Hq, Hkv, S, d_qk, d_v,
                     causal, p_mode, stream=0):
    """Direct C call with integer pointers; returns the status code (no exception)."""
    return load_library().attn_fwd_fp8(q, k, v, o, q_scale, k_scale, v_scale, softmax_scale,
                                       B, Hq, Hkv, S, d_qk, d_v, causal, p_mode, stream)


def attn_fwd_fp8_lse_raw(q, k, v, o, lse, q_scale, k_scale, v_scale, softmax_scale, B, Hq, Hkv, S, d_qk, d_v,
                         causal, p_mode, stream=0):
    return load_library().attn_fwd_fp8_lse(q, k, v, o, lse, q_scale, k_scale, v_scale, softmax_scale,
                                           B, Hq, Hkv, S, d_qk, d_v, causal, p_mode, stream)


def attn_fwd_fp8_dscale_raw(q, k, v, o, lse, q_scale, k_scale, v_scale, softmax_scale, B, Hq, Hkv, S, d_qk, d_v,
                            causal, p_mode, stream=0):
    """Direct C call with the three scales as device pointers."""
    return load_library().attn_fwd_fp8_dscale(q, k, v, o, lse, q_scale, k_scale, v_scale, softmax_scale,
                                              B, Hq, Hkv, S, d_qk, d_v, causal, p_mode, stream)


def attn_fwd_bf16_raw(q, k, v, o, softmax_scale, B, Hq, Hkv, S, d_qk, d_v, causal, stream=0):
    return load_library().attn_fwd_bf16(q, k, v, o, softmax_scale, B, Hq, Hkv, S, d_qk, d_v, causal, stream)


def attn_fwd_bf16_lse_raw(q, k, v, o, lse, softmax_scale, B, Hq, Hkv, S, d_qk, d_v, causal, stream=0):
    return load_library().attn_fwd_bf16_lse(q, k, v, o, lse, softmax_scale, B, Hq, Hkv, S, d_qk, d_v, causal,
                                            stream)


def attn_fwd_fp8_varlen_raw(q, k, v, o, lse, cu_seqlens_q, cu_seqlens_k, n_seqs, max_seqlen_q, total_q, total_k,
                            q_scale, k_scale, v_scale, softmax_scale, Hq, Hkv, d_qk, d_v, causal, p_mode, stream=0):
    return load_library().attn_fwd_fp8_varlen(q, k, v, o, lse, cu_seqlens_q, cu_seqlens_k, n_seqs, max_seqlen_q,
                                              total_q, total_k, q_scale, k_scale, v_scale, softmax_scale, Hq, Hkv,
                                              d_qk, d_v, causal, p_mode, stream)


def attn_fwd_bf16_varlen_raw(q, k, v, o, lse, cu_seqlens_q, cu_seqlens_k, n_seqs, max_seqlen_q, total_q, total_k,
                             softmax_scale, Hq, Hkv, d_qk, d_v, causal, stream=0):
    return load_library().attn_fwd_bf16_varlen(q, k, v, o, lse, cu_seqlens_q, cu_seqlens_k, n_seqs, max_seqlen_q,
                                               total_q, total_k, softmax_scale, Hq, Hkv, d_qk, d_v, causal, stream)


def attn_rotate_quant_bf16_raw(x, x8, scale, B, S, H, d, stream=0):
    return load_library().attn_rotate_quant_bf16(x, x8, scale, B, S, H, d, stream)


def rotate_quant_bf16(x, out=None, scale=None, stream=None):
    """Hadamard-rotate a bf16 (B,S,H,d) Q or K tensor along d and quantise it per tensor
    to e4m3.  Returns (codes: uint8 (B,S,H,d), scale: one-element float32 device tensor)."""
    B, S, H, d = _bshd(x, "x")
    if x.dtype != torch.bfloat16:
        raise TypeError(f"x must be bfloat16, got {x.dtype}")
    if out is None:
        out = torch.empty(x.shape, dtype=torch.uint8, device=x.device)
    elif out.shape != x.shape or out.dtype != torch.uint8 or not out.is_contiguous():
        raise ValueError("out must be a contiguous uint8 tensor of x's shape")
    if scale is None:
        scale = torch.empty(1, dtype=torch.float32, device=x.device)
    _check(load_library().attn_rotate_quant_bf16(x.data_ptr(), out.data_ptr(), scale.data_ptr(), B, S, H, d,
                                                 _stream_ptr(stream, x.device)))
    return out, scale


def attn_rotate_quant_bf16_prescaled_raw(x, x8, scale, amax, B, S, H, d, stream=0):
    return load_library().attn_rotate_quant_bf16_prescaled(x, x8, scale, amax, B, S, H, d, stream)


def rotate_quant_bf16_prescaled(x, scale, out=None, with_amax=True, stream=None):
    """One-pass Hadamard rotation + e4m3 quantisation of a bf16 (B,S,H,d) Q or K tensor with a
    scale known in advance (one-element float32 GPU tensor).  Returns (codes, amax) where amax
    is a one-element float32 GPU tensor holding max |rotated| (None if not with_amax)."""
    B, S, H, d = _bshd(x, "x")
    if x.dtype != torch.bfloat16:
        raise TypeError(f"x must be bfloat16, got {x.dtype}")
    if not (isinstance(scale, torch.Tensor) and scale.is_cuda and scale.dtype == torch.float32
            and scale.numel() == 1):
        raise ValueError("scale must be a one-element float32 GPU tensor")
    if out is None:
        out = torch.empty(x.shape, dtype=torch.uint8, device=x.device)
    elif out.shape != x.shape or out.dtype != torch.uint8 or not out.is_contiguous():
        raise ValueError("out must be a contiguous uint8 tensor of x's shape")
    amax = torch.empty(1, dtype=torch.float32, device=x.device) if with_amax else None
    _check(load_library().attn_rotate_quant_bf16_prescaled(x.data_ptr(), out.data_ptr(), scale.data_ptr(),
                                                           0 if amax is None else amax.data_ptr(), B, S, H, d,
                                                           _stream_ptr(stream, x.device)))
    return out, amax


def _lse_out(return_lse, B, Hq, S, device):
    if not return_lse:
        return None
    return torch.empty((B, Hq, S), dtype=torch.float32, device=device)


def attn_fwd_fp8(q8, k8, v8, q_scale, k_scale, v_scale, softmax_scale=None, causal=True,
                 p_mode="exact", out=None, stream=None, return_lse=False):
    """FP8 attention (causal by default); q8/k8/v8 are e4m3fn bytes (uint8 or float8_e4m3fn), (B,S,H,d).

    Returns the bf16 output (B, S, Hq, d_v), enqueued on ``stream`` (default:
    torch's current stream of the inputs' device); with ``return_lse`` returns
    (out, lse), lse the fp32 (B, Hq, S) natural-log normaliser of every row.
    The scales are floats, or one-element float32 GPU tensors (all three), which
    the kernel reads when it runs - e.g. the scales rotate_quant_bf16 wrote on the
    same stream, with no host synchronisation.
    """
    for t, n in ((q8, "q8"), (k8, "k8"), (v8, "v8")):
        if t.dtype not in (torch.uint8, torch.float8_e4m3fn):
            raise TypeError(f"{n} must hold e4m3fn bytes (uint8 or float8_e4m3fn), got {t.dtype}")
    B, S, Hq, dqk = _bshd(q8, "q8")
    Bk, Sk, Hkv, dk = _bshd(k8, "k8")
    Bv, Sv, Hv, dv = _bshd(v8, "v8")
    if (Bk, Sk, dk) != (B, S, dqk) or (Bv, Sv, Hv) != (B, S, Hkv):
        raise ValueError(f"shape mismatch q{tuple(q8.shape)} k{tuple(k8.shape)} v{tuple(v8.shape)}")
    if out is None:
        out = torch.empty((B, S, Hq, dv), dtype=torch.bfloat16, device=q8.device)
    elif out.dtype != torch.bfloat16 or tuple(out.shape) != (B, S, Hq, dv) or not out.is_contiguous():
        raise ValueError("out must be a contiguous bf16 tensor of shape (B, S, Hq, d_v)")
    sm = 0.0 if softmax_scale is None else float(softmax_scale)
    lse = _lse_out(return_lse, B, Hq, S, q8.device)
    dev_scales = [isinstance(x, torch.Tensor) for x in (q_scale, k_scale, v_scale)]
    if any(dev_scales):
        if not all(dev_scales):
            raise TypeError("q_scale, k_scale and v_scale must be all floats or all device tensors")
        for x in (q_scale, k_scale, v_scale):
            if not x.is_cuda or x.dtype != torch.float32 or x.numel() != 1 or not x.is_contiguous():
                raise ValueError("device scales must be one-element contiguous float32 GPU tensors")
        st = attn_fwd_fp8_dscale_raw(q8.data_ptr(), k8.data_ptr(), v8.data_ptr(), out.data_ptr(),
                                     0 if lse is None else lse.data_ptr(), q_scale.data_ptr(), k_scale.data_ptr(),
                                     v_scale.data_ptr(), sm, B, Hq, Hkv, S, dqk, dv, int(bool(causal)),
                                     _P_MODES[p_mode], _stream_ptr(stream, q8.device))
        _check(st)
        return (out, lse) if return_lse else out
    st = attn_fwd_fp8_lse_raw(q8.data_ptr(), k8.data_ptr(), v8.data_ptr(), out.data_ptr(),
                              0 if lse is None else lse.data_ptr(),
                              float(q_scale), float(k_scale), float(v_scale), sm,
                              B, Hq, Hkv, S, dqk, dv, int(bool(causal)), _P_MODES[p_mode],
                              _stream_ptr(stream, q8.device))
    _check(st)
    return (out, lse) if return_lse else out


def attn_fwd_bf16(q, k, v, softmax_scale=None, causal=True, out=None, stream=None, return_lse=False):
    """BF16 attention (causal by default) on bf16 (B,S,H,d) tensors; returns bf16 (B,S,Hq,d_v),
    or (out, lse) with ``return_lse`` (lse fp32 (B, Hq, S))."""
    for t, n in ((q, "q"), (k, "k"), (v, "v")):
        if t.dtype != torch.bfloat16:
            raise TypeError(f"{n} must be bfloat16, got {t.dtype}")
    B, S, Hq, dqk = _bshd(q, "q")
    Bk, Sk, Hkv, dk = _bshd(k, "k")
    Bv, Sv, Hv, dv = _bshd(v, "v")
    if (Bk, Sk, dk) != (B, S, dqk) or (Bv, Sv, Hv) != (B, S, Hkv):
        raise ValueError(f"shape mismatch q{tuple(q.shape)} k{tuple(k.shape)} v{tuple(v.shape)}")
    if out is None:
        out = torch.empty((B, S, Hq, dv), dtype=torch.bfloat16, device=q.device)
    elif out.dtype != torch.bfloat16 or tuple(out.shape) != (B, S, Hq, dv) or not out.is_contiguous():
        raise ValueError("out must be a contiguous bf16 tensor of shape (B, S, Hq, d_v)")
    sm = 0.0 if softmax_scale is None else float(softmax_scale)
    lse = _lse_out(return_lse, B, Hq, S, q.device)
    st = attn_fwd_bf16_lse_raw(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
                               0 if lse is None else lse.data_ptr(), sm,
                               B, Hq, Hkv, S, dqk, dv, int(bool(causal)), _stream_ptr(stream, q.device))
    _check(st)
    return (out, lse) if return_lse else out


def causal_flops(B, Hq, S, d_qk, d_v):
    """2*B*Hq*S^2*(d_qk+d_v)/2 - the causal FLOP count throughput is quoted in."""
    return 2.0 * B * Hq * S * S * (d_qk + d_v) / 2.0


def default_softmax_scale(d_qk):
    return 1.0 / math.sqrt(d_qk)


def _thd(x, name):
    if x.dim() != 3:
        raise ValueError(f"{name} must be (total_tokens, H, d), got shape {tuple(x.shape)}")
    if not x.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if not x.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    return x.shape


def _check_cu(cu, name):
    if cu.dtype != torch.int32 or cu.dim() != 1 or not cu.is_cuda or not cu.is_contiguous() or cu.numel() < 1:
        raise ValueError(f"{name} must be a contiguous 1-D int32 GPU tensor of n_seqs + 1 offsets")


def _varlen_common(q, k, v, cu_seqlens, out, return_lse, cu_seqlens_k=None):
    T, Hq, dqk = _thd(q, "q")
    Tk, Hkv, dk = _thd(k, "k")
    Tv, Hv, dv = _thd(v, "v")
    if dk != dqk or (Tv, Hv) != (Tk, Hkv) or (cu_seqlens_k is None and Tk != T):
        raise ValueError(f"shape mismatch q{tuple(q.shape)} k{tuple(k.shape)} v{tuple(v.shape)}")
    _check_cu(cu_seqlens, "cu_seqlens")
    if cu_seqlens_k is not None:
        _check_cu(cu_seqlens_k, "cu_seqlens_k")
        if cu_seqlens_k.numel() != cu_seqlens.numel():
            raise ValueError("cu_seqlens and cu_seqlens_k must hold the same number of offsets")
    if out is None:
        out = torch.empty((T, Hq, dv), dtype=torch.bfloat16, device=q.device)
    elif out.dtype != torch.bfloat16 or tuple(out.shape) != (T, Hq, dv) or not out.is_contiguous():
        raise ValueError("out must be a contiguous bf16 tensor of shape (total_tokens, Hq, d_v)")
    lse = torch.empty((Hq, T), dtype=torch.float32, device=q.device) if return_lse else None
    return T, Tk, Hq, Hkv, dqk, dv, out, lse


def attn_fwd_fp8_varlen(q8, k8, v8, cu_seqlens, max_seqlen, q_scale, k_scale, v_scale, softmax_scale=None,
                        causal=True, p_mode="exact", out=None, stream=None, return_lse=False, cu_seqlens_k=None):
    """FP8 attention over a variable-length batch packed along the rows: q8 (total_q, Hq, d_qk),
    k8/v8 (total_k, Hkv, d), sequence i's queries at rows cu_seqlens[i]..cu_seqlens[i+1]-1 (int32
    GPU tensor) and its keys at the same rows of k8/v8, or at cu_seqlens_k's rows when given
    (bottom-right aligned causal mask when the lengths differ); max_seqlen is the longest query
    run (host int).  Returns bf16 (total_q, Hq, d_v), or (out, lse) with lse fp32 (Hq, total_q)."""
    for t, n in ((q8, "q8"), (k8, "k8"), (v8, "v8")):
        if t.dtype not in (torch.uint8, torch.float8_e4m3fn):
            raise TypeError(f"{n} must hold e4m3fn bytes (uint8 or float8_e4m3fn), got {t.dtype}")
    T, Tk, Hq, Hkv, dqk, dv, out, lse = _varlen_common(q8, k8, v8, cu_seqlens, out, return_lse, cu_seqlens_k)
    sm = 0.0 if softmax_scale is None else float(softmax_scale)
    _check(attn_fwd_fp8_varlen_raw(q8.data_ptr(), k8.data_ptr(), v8.data_ptr(), out.data_ptr(),
                                   0 if lse is None else lse.data_ptr(), cu_seqlens.data_ptr(),
                                   0 if cu_seqlens_k is None else cu_seqlens_k.data_ptr(),
                                   cu_seqlens.numel() - 1, int(max_seqlen), T, Tk, float(q_scale), float(k_scale),
                                   float(v_scale), sm, Hq, Hkv, dqk, dv, int(bool(causal)), _P_MODES[p_mode],
                                   _stream_ptr(stream, q8.device)))
    return (out, lse) if return_lse else out


def attn_fwd_bf16_varlen(q, k, v, cu_seqlens, max_seqlen, softmax_scale=None, causal=True, out=None, stream=None,
                         return_lse=False, cu_seqlens_k=None):
    """BF16 attention over a variable-length batch (layout as attn_fwd_fp8_varlen)."""
    for t, n in ((q, "q"), (k, "k"), (v, "v")):
        if t.dtype != torch.bfloat16:
            raise TypeError(f"{n} must be bfloat16, got {t.dtype}")
    T, Tk, Hq, Hkv, dqk, dv, out, lse = _varlen_common(q, k, v, cu_seqlens, out, return_lse, cu_seqlens_k)
    sm = 0.0 if softmax_scale is None else float(softmax_scale)
    _check(attn_fwd_bf16_varlen_raw(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
                                    0 if lse is None else lse.data_ptr(), cu_seqlens.data_ptr(),
                                    0 if cu_seqlens_k is None else cu_seqlens_k.data_ptr(),
                                    cu_seqlens.numel() - 1, int(max_seqlen), T, Tk, sm, Hq, Hkv, dqk, dv,
                                    int(bool(causal)), _stream_ptr(stream, q.device)))
    return (out, lse) if return_lse else out

"""``flash_attn_func``-style entry point and torch.library custom operators.

The pages describe the kernels as a drop-in replacement for ``flash_attn_func``
("Zyphra ZYFA: FP8 FlashAttention for AMD MI355X, Up to 1.76x Faster", TL;DR).
This module gives that calling convention (and ``flash_attn_varlen_func``'s)
over the C ABI, and registers the attention calls as torch custom operators
(``fp8_prefill::attn_fwd_fp8``, ``fp8_prefill::attn_fwd_bf16`` and their
``_varlen`` forms) with shape-only fake implementations, so that
``torch.compile`` traces them as single opaque nodes instead of breaking the graph.

Every call still runs in the library's HIP kernels through ``binding``; this
module holds no attention arithmetic and no fallback.
"""
import torch

from . import binding

_OPS = "fp8_prefill"
_FP8_DTYPES = (torch.float8_e4m3fn, torch.uint8)


@torch.library.custom_op(f"{_OPS}::attn_fwd_fp8", mutates_args=(), device_types="cuda")
def _attn_fwd_fp8_op(q8: torch.Tensor, k8: torch.Tensor, v8: torch.Tensor, q_scale: float, k_scale: float,
                     v_scale: float, softmax_scale: float, causal: bool, p_mode: int, with_lse: bool
                     ) -> tuple[torch.Tensor, torch.Tensor]:
    sm = softmax_scale if softmax_scale > 0 else None
    if not with_lse:
        out = binding.attn_fwd_fp8(q8, k8, v8, q_scale, k_scale, v_scale, softmax_scale=sm, causal=causal,
                                   p_mode=p_mode)
        return out, q8.new_empty((0,), dtype=torch.float32)
    return binding.attn_fwd_fp8(q8, k8, v8, q_scale, k_scale, v_scale, softmax_scale=sm, causal=causal,
                                p_mode=p_mode, return_lse=True)


def _fake_outputs(q, v, with_lse):
    B, S, Hq, _ = q.shape
    lse_shape = (B, Hq, S) if with_lse else (0,)
    return (q.new_empty((B, S, Hq, v.shape[3]), dtype=torch.bfloat16),
            q.new_empty(lse_shape, dtype=torch.float32))


@_attn_fwd_fp8_op.register_fake
def _(q8, k8, v8, q_scale, k_scale, v_scale, softmax_scale, causal, p_mode, with_lse):
    return _fake_outputs(q8, v8, with_lse)


@torch.library.custom_op(f"{_OPS}::attn_fwd_fp8_dscale", mutates_args=(), device_types="cuda")
def _attn_fwd_fp8_dscale_op(q8: torch.Tensor, k8: torch.Tensor, v8: torch.Tensor, q_scale: torch.Tensor,
                            k_scale: torch.Tensor, v_scale: torch.Tensor, softmax_scale: float, causal: bool,
                            p_mode: int, with_lse: bool) -> tuple[torch.Tensor, torch.Tensor]:
    sm = softmax_scale if softmax_scale > 0 else None
    if not with_lse:
        out = binding.attn_fwd_fp8(q8, k8, v8, q_scale, k_scale, v_scale, softmax_scale=sm, causal=causal,
                                   p_mode=p_mode)
        return out, q8.new_empty((0,), dtype=torch.float32)
    return binding.attn_fwd_fp8(q8, k8, v8, q_scale, k_scale, v_scale, softmax_scale=sm, causal=causal,
                                p_mode=p_mode, return_lse=True)


@_attn_fwd_fp8_dscale_op.register_fake
def _(q8, k8, v8, q_scale, k_scale, v_scale, softmax_scale, causal, p_mode, with_lse):
    return _fake_outputs(q8, v8, with_lse)


@torch.library.custom_op(f"{_OPS}::attn_fwd_bf16", mutates_args=(), device_types="cuda")
def _attn_fwd_bf16_op(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, softmax_scale: float, causal: bool,
                      with_lse: bool) -> tuple[torch.Tensor, torch.Tensor]:
    sm = softmax_scale if softmax_scale > 0 else None
    if not with_lse:
        return binding.attn_fwd_bf16(q, k, v, softmax_scale=sm, causal=causal), q.new_empty((0,), dtype=torch.float32)
    return binding.attn_fwd_bf16(q, k, v, softmax_scale=sm, causal=causal, return_lse=True)


@_attn_fwd_bf16_op.register_fake
def _(q, k, v, softmax_scale, causal, with_lse):
    return _fake_outputs(q, v, with_lse)


@torch.library.custom_op(f"{_OPS}::attn_fwd_fp8_varlen", mutates_args=(), device_types="cuda")
def _attn_fwd_fp8_varlen_op(q8: torch.Tensor, k8: torch.Tensor, v8: torch.Tensor, cu_seqlens_q: torch.Tensor,
                            cu_seqlens_k: torch.Tensor, max_seqlen_q: int, q_scale: float, k_scale: float,
                            v_scale: float, softmax_scale: float, causal: bool, p_mode: int, with_lse: bool
                            ) -> tuple[torch.Tensor, torch.Tensor]:
    res = binding.attn_fwd_fp8_varlen(q8, k8, v8, cu_seqlens_q, max_seqlen_q, q_scale, k_scale, v_scale,
                                      softmax_scale=softmax_scale if softmax_scale > 0 else None, causal=causal,
                                      p_mode=p_mode, return_lse=with_lse, cu_seqlens_k=cu_seqlens_k)
    return res if with_lse else (res, q8.new_empty((0,), dtype=torch.float32))


def _fake_varlen_outputs(q, v, with_lse):
    T, Hq, _ = q.shape
    return (q.new_empty((T, Hq, v.shape[2]), dtype=torch.bfloat16),
            q.new_empty((Hq, T) if with_lse else (0,), dtype=torch.float32))


@_attn_fwd_fp8_varlen_op.register_fake
def _(q8, k8, v8, cu_seqlens_q, cu_seqlens_k, max_seqlen_q, q_scale, k_scale, v_scale, softmax_scale, causal,
      p_mode, with_lse):
    return _fake_varlen_outputs(q8, v8, with_lse)


@torch.library.custom_op(f"{_OPS}::attn_fwd_bf16_varlen", mutates_args=(), device_types="cuda")
def _attn_fwd_bf16_varlen_op(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, cu_seqlens_q: torch.Tensor,
                             cu_seqlens_k: torch.Tensor, max_seqlen_q: int, softmax_scale: float, causal: bool,
                             with_lse: bool) -> tuple[torch.Tensor, torch.Tensor]:
    res = binding.attn_fwd_bf16_varlen(q, k, v, cu_seqlens_q, max_seqlen_q,
                                       softmax_scale=softmax_scale if softmax_scale > 0 else None, causal=causal,
                                       return_lse=with_lse, cu_seqlens_k=cu_seqlens_k)
    return res if with_lse else (res, q.new_empty((0,), dtype=torch.float32))


@_attn_fwd_bf16_varlen_op.register_fake
def _(q, k, v, cu_seqlens_q, cu_seqlens_k, max_seqlen_q, softmax_scale, causal, with_lse):
    return _fake_varlen_outputs(q, v, with_lse)


def _scale(x, name):
    if x is None:
        raise ValueError(f"FP8 inputs need {name} (the per-tensor dequantisation scale)")
    if isinstance(x, torch.Tensor):
        if x.numel() != 1:
            raise ValueError(f"{name} must be a single per-tensor scale, got {x.numel()} elements")
        x = float(x.item())
    return float(x)


def flash_attn_func(q, k, v, dropout_p=0.0, softmax_scale=None, causal=False, window_size=(-1, -1),
                    softcap=0.0, alibi_slopes=None, deterministic=False, return_attn_probs=False, *,
                    q_descale=None, k_descale=None, v_descale=None, p_mode="lean"):
    """Forward attention in the ``flash_attn_func`` calling convention.

    q: (B, S, Hq, d_qk), k: (B, S, Hkv, d_qk), v: (B, S, Hkv, d_v), contiguous, on
    the GPU, equal query and key lengths.  bfloat16 inputs run the BF16 kernel;
    float8_e4m3fn (or uint8 e4m3 bytes) inputs run the FP8 kernel and need the
    per-tensor scales ``q_descale``/``k_descale``/``v_descale`` (float or
    one-element tensor: dequantised value = descale * code; GPU tensors for all
    three are read by the kernel itself, with no host synchronisation), with
    ``p_mode`` "lean" or "exact".  Returns the bf16 output (B, S, Hq, d_v); with
    ``return_attn_probs`` returns (out, lse, None), lse fp32 (B, Hq, S), as
    flash_attn_func does (its third value, the dropout mask, is always None).
    Scales given as CPU tensors are read with ``.item()``.

    Options outside the kernels' scope raise NotImplementedError: dropout,
    sliding windows, softcapping and ALiBi.  ``deterministic`` is accepted and
    always holds (fixed reduction order, no atomics).
    """
    if dropout_p != 0.0:
        raise NotImplementedError("dropout is not supported (forward inference kernels)")
    if tuple(window_size) != (-1, -1):
        raise NotImplementedError("sliding-window attention is not supported")
    if softcap != 0.0:
        raise NotImplementedError("softcapping is not supported")
    if alibi_slopes is not None:
        raise NotImplementedError("ALiBi is not supported")
    sm = 0.0 if softmax_scale is None else float(softmax_scale)
    if q.dtype in _FP8_DTYPES:
        if k.dtype not in _FP8_DTYPES or v.dtype not in _FP8_DTYPES:
            raise TypeError("q, k and v must all be FP8 e4m3 (or all bfloat16)")
        q8, k8, v8 = (t.view(torch.uint8) if t.dtype != torch.uint8 else t for t in (q, k, v))
        scales = (q_descale, k_descale, v_descale)
        if all(isinstance(x, torch.Tensor) and x.is_cuda for x in scales):
            # scales in device memory: read by the kernel, no host synchronisation
            out, lse = _attn_fwd_fp8_dscale_op(q8, k8, v8, *(x.reshape(1).float() for x in scales), sm, bool(causal),
                                               int(binding._P_MODES[p_mode]), bool(return_attn_probs))
        else:
            out, lse = _attn_fwd_fp8_op(q8, k8, v8, _scale(q_descale, "q_descale"), _scale(k_descale, "k_descale"),
                                        _scale(v_descale, "v_descale"), sm, bool(causal),
                                        int(binding._P_MODES[p_mode]), bool(return_attn_probs))
    elif q.dtype == torch.bfloat16:
        if k.dtype != torch.bfloat16 or v.dtype != torch.bfloat16:
            raise TypeError("q, k and v must all be bfloat16 (or all FP8 e4m3)")
        out, lse = _attn_fwd_bf16_op(q, k, v, sm, bool(causal), bool(return_attn_probs))
    else:
        raise TypeError(f"unsupported input dtype {q.dtype}: bfloat16 or float8_e4m3fn")
    if return_attn_probs:
        return out, lse, None
    return out


def flash_attn_varlen_func(q, k, v, cu_seqlens_q, cu_seqlens_k, max_seqlen_q, max_seqlen_k=None, dropout_p=0.0,
                           softmax_scale=None, causal=False, window_size=(-1, -1), softcap=0.0, alibi_slopes=None,
                           deterministic=False, return_attn_probs=False, *, q_descale=None, k_descale=None,
                           v_descale=None, p_mode="lean"):
    """Variable-length forward attention in the ``flash_attn_varlen_func`` calling convention.

    q: (total_q, Hq, d_qk), k/v: (total_k, Hkv, d), sequences packed along the rows at the int32
    GPU offsets ``cu_seqlens_q`` / ``cu_seqlens_k``; a sequence with fewer (or more) queries than
    keys uses the bottom-right aligned causal mask.  ``max_seqlen_q`` is the longest query run
    (``max_seqlen_k`` is accepted for the signature and not needed).  bfloat16 or e4m3 inputs as
    for flash_attn_func.  Returns O (total_q, Hq, d_v), or (O, lse (Hq, total_q), None).
    """
    if dropout_p != 0.0 or tuple(window_size) != (-1, -1) or softcap != 0.0 or alibi_slopes is not None:
        raise NotImplementedError("dropout, sliding windows, softcapping and ALiBi are not supported")
    sm = 0.0 if softmax_scale is None else float(softmax_scale)
    if q.dtype in _FP8_DTYPES:
        if k.dtype not in _FP8_DTYPES or v.dtype not in _FP8_DTYPES:
            raise TypeError("q, k and v must all be FP8 e4m3 (or all bfloat16)")
        q8, k8, v8 = (t.view(torch.uint8) if t.dtype != torch.uint8 else t for t in (q, k, v))
        out, lse = _attn_fwd_fp8_varlen_op(q8, k8, v8, cu_seqlens_q, cu_seqlens_k, int(max_seqlen_q),
                                           _scale(q_descale, "q_descale"), _scale(k_descale, "k_descale"),
                                           _scale(v_descale, "v_descale"), sm, bool(causal),
                                           int(binding._P_MODES[p_mode]), bool(return_attn_probs))
    elif q.dtype == torch.bfloat16:
        if k.dtype != torch.bfloat16 or v.dtype != torch.bfloat16:
            raise TypeError("q, k and v must all be bfloat16 (or all FP8 e4m3)")
        out, lse = _attn_fwd_bf16_varlen_op(q, k, v, cu_seqlens_q, cu_seqlens_k, int(max_seqlen_q), sm, bool(causal),
                                            bool(return_attn_probs))
    else:
        raise TypeError(f"unsupported input dtype {q.dtype}: bfloat16 or float8_e4m3fn")
    if return_attn_probs:
        return out, lse, None
    return out

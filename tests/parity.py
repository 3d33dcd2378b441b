"""Helpers shared by the GPU parity tests: run the HIP path through the C-ABI
binding and evaluate the CPU oracle on the same seeded inputs.

Tolerances (derived from the arithmetic; the FP8 path cannot be closer to fp64
than the method itself):

* GPU vs the step-by-step emulation of the method: relative RMS <= 5e-3.  The
  emulation rounds P exactly as the kernel does, so what remains is the bf16
  output rounding (relative RMS 1.1e-3 to 2.3e-3 depending on where values sit
  in their binade) plus the rare e4m3 rounding decisions of P that fp32 scores
  (MFMA accumulation, fp32 FMA and exp2) flip relative to the fp64 oracle; a
  flip moves one probability by an e4m3 step (12.5%), which weighs most when
  the attention is concentrated on a few keys (outlier channels: up to 3.4e-3
  measured).
* GPU vs fp64 attention on the dequantised inputs: <= max(2e-2, 1.1 * e + 2e-3)
  where e is the emulation's own error vs fp64 - rounding P to e4m3 alone leaves
  1-3% relative RMS on Gaussian values, so the bar is the method's own error
  plus the output rounding.
* BF16 path vs fp64: <= 4e-3.
"""
import numpy as np
import torch

from fp8_causal_prefill_tiled_amd import binding
from fp8_causal_prefill_tiled_amd import workloads as W
from oracle.attention64 import attention_fp64, dequantize, lse_fp64, rel_rms
from oracle.emulate import emulate_fp8
from oracle.e4m3 import bf16_rne, decode_e4m3

TOL_EMU = 5e-3
TOL_BF16 = 4e-3


def tol_fp64(emu_err):
    return max(2e-2, 1.1 * emu_err + 2e-3)


def run_fp8(d, mode, dev="cuda:0", causal=True, return_lse=False):
    q8, k8, v8 = (d[n].to(dev) for n in ("q8", "k8", "v8"))
    out = binding.attn_fwd_fp8(q8, k8, v8, d["q_scale"], d["k_scale"], d["v_scale"], p_mode=mode,
                               causal=causal, return_lse=return_lse)
    torch.cuda.synchronize()
    return out


def run_bf16(d, dev="cuda:0", causal=True, return_lse=False):
    q, k, v = (d[n].to(dev) for n in ("q", "k", "v"))
    out = binding.attn_fwd_bf16(q, k, v, causal=causal, return_lse=return_lse)
    torch.cuda.synchronize()
    return out


def oracle_fp8(d, mode, heads=None, rows=None, causal=True, with_lse=False):
    """(emulation, fp64) for the given query heads and rows; arrays (B, rows, heads, d_v).

    With ``with_lse`` also (emulated, fp64) natural-log normalisers, arrays (B, heads, rows)."""
    q8, k8, v8 = d["q8"].numpy(), d["k8"].numpy(), d["v8"].numpy()
    Hq, Hkv = q8.shape[2], k8.shape[2]
    heads = list(range(Hq)) if heads is None else list(heads)
    emus, refs, lemus, lrefs = [], [], [], []
    for h in heads:
        g = h // (Hq // Hkv)
        qs, ks, vs = q8[:, :, h:h + 1], k8[:, :, g:g + 1], v8[:, :, g:g + 1]
        e = emulate_fp8(qs, ks, vs, d["q_scale"], d["k_scale"], d["v_scale"], p_mode=mode, rows=rows,
                        causal=causal, return_lse=with_lse)
        if with_lse:
            e, log2L = e
            lemus.append(np.log(2.0) * log2L.transpose(0, 2, 1))
            lrefs.append(lse_fp64(dequantize(qs, d["q_scale"]), dequantize(ks, d["k_scale"]), rows=rows,
                                  causal=causal))
        emus.append(e)
        refs.append(attention_fp64(dequantize(qs, d["q_scale"]), dequantize(ks, d["k_scale"]),
                                   dequantize(vs, d["v_scale"]), rows=rows, causal=causal))
    res = (np.concatenate(emus, axis=2), np.concatenate(refs, axis=2))
    if with_lse:
        res += (np.concatenate(lemus, axis=1), np.concatenate(lrefs, axis=1))
    return res


def oracle_bf16(d, heads=None, rows=None, causal=True, with_lse=False):
    q, k, v = (d[n].float().numpy() for n in ("q", "k", "v"))
    Hq, Hkv = q.shape[2], k.shape[2]
    heads = list(range(Hq)) if heads is None else list(heads)
    refs, lrefs = [], []
    for h in heads:
        g = h // (Hq // Hkv)
        refs.append(attention_fp64(q[:, :, h:h + 1], k[:, :, g:g + 1], v[:, :, g:g + 1], rows=rows,
                                   causal=causal))
        if with_lse:
            lrefs.append(lse_fp64(q[:, :, h:h + 1], k[:, :, g:g + 1], rows=rows, causal=causal))
    if with_lse:
        return np.concatenate(refs, axis=2), np.concatenate(lrefs, axis=1)
    return np.concatenate(refs, axis=2)


def gpu_select(out, heads=None, rows=None):
    o = out.float().cpu().numpy().astype(np.float64)
    if rows is not None:
        o = o[:, np.asarray(rows)]
    if heads is not None:
        o = o[:, :, list(heads)]
    return o


def row0_expected_fp8(d):
    """Row 0 sees one key: O_0 = bf16(fp32(decode(V8[0]) * v_scale)), bit-exact."""
    v0 = decode_e4m3(d["v8"][:, 0].numpy()).astype(np.float32)   # (B, Hkv, d_v), exact in fp32
    return bf16_rne(v0 * np.float32(d["v_scale"]))


def check_fp8(got, emu, ref, label=""):
    e_emu = rel_rms(got, emu)
    e_ref = rel_rms(got, ref)
    e_meth = rel_rms(emu, ref)
    print(f"[parity] {label}: vs emulation {e_emu:.2e}  vs fp64 {e_ref:.4f}  (emulation vs fp64 {e_meth:.4f})")
    assert np.all(np.isfinite(got)), label
    assert e_emu <= TOL_EMU, (label, e_emu)
    assert e_ref <= tol_fp64(e_meth), (label, e_ref, e_meth)
    return e_emu, e_ref, e_meth


__all__ = ["W", "rel_rms", "np", "torch", "binding"]

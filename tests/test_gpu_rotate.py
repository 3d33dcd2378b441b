"""GPU parity of the Hadamard rotation + per-tensor FP8 quantisation of Q and K
(attn_rotate_quant_bf16, through the C ABI) against oracle/rotate.py, and its
end-to-end effect on the FP8 attention ([MTP] section "How accurate is ZYFA's FP8
attention?": the rotation cuts the input error to about half)."""
import numpy as np
import pytest
import torch

from parity import W, binding, rel_rms
from oracle.attention64 import attention_fp64
from oracle.e4m3 import E4M3_MAX, decode_e4m3, encode_e4m3_rne
from oracle.rotate import block_size, rotate

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def bf16_input(shape, seed, outlier_channels=0, gain=8.0):
    g = torch.Generator().manual_seed(seed)
    x = torch.randn(shape, generator=g, dtype=torch.float32)
    if outlier_channels:
        ch = torch.randperm(shape[-1], generator=g)[:outlier_channels]
        x[..., ch] *= gain
    return x.to(torch.bfloat16)


def run(x):
    codes, scale = binding.rotate_quant_bf16(x.to(DEV))
    torch.cuda.synchronize()
    return codes.cpu().numpy(), float(scale.item())


def check_codes(x_bf16, codes, scale, rows=None):
    """Codes equal the oracle's, except where the fp64 rotated value lies within the
    fp32 rounding error of the GPU's butterflies and division of a rounding boundary:
    there either neighbouring code is correct.  `rows` restricts the comparison to a
    sample of (flattened) vectors; the scale is checked separately."""
    d = x_bf16.shape[-1]
    x = x_bf16.float().numpy().astype(np.float64).reshape(-1, d)
    c = codes.reshape(-1, d)
    if rows is not None:
        x, c = x[rows], c[rows]
    y = rotate(x)
    n = block_size(d)
    blk_l1 = np.repeat(np.abs(x).reshape(-1, d // n, n).sum(-1), n, axis=-1) / np.sqrt(n)
    q = y / scale
    tol = (np.log2(n) + 3) * 2.0 ** -24 * blk_l1 / scale + 3 * 2.0 ** -24 * np.abs(q)
    got = decode_e4m3(c)
    lo = decode_e4m3(encode_e4m3_rne(np.clip(q - tol, -E4M3_MAX, E4M3_MAX)))
    hi = decode_e4m3(encode_e4m3_rne(np.clip(q + tol, -E4M3_MAX, E4M3_MAX)))
    exact = decode_e4m3(encode_e4m3_rne(q))
    assert np.all((got >= lo) & (got <= hi)), "a code outside the rounding-tolerance interval"
    assert np.mean(got == exact) > 0.999
    return np.mean(got == exact)


def reference_scale(x_bf16):
    amax = float(np.max(np.abs(rotate(x_bf16.float().numpy().astype(np.float64)))))
    return float(np.float32(amax / E4M3_MAX)) if amax > 0 else 1.0


@pytest.mark.parametrize("shape,seed,outliers", [
    ((1, 64, 2, 128), 1, 0), ((2, 129, 3, 128), 2, 0), ((1, 65, 2, 192), 3, 0),
    ((1, 1, 1, 128), 4, 0), ((3, 7, 5, 192), 5, 0), ((1, 300, 4, 128), 6, 4), ((2, 33, 2, 192), 7, 4),
])
def test_rotate_quant_matches_oracle(shape, seed, outliers):
    x = bf16_input(shape, seed, outliers)
    codes, scale = run(x)
    ref = reference_scale(x)
    assert abs(scale - ref) <= 4e-7 * ref
    frac = check_codes(x, codes, scale)
    print(f"[parity] rotate_quant {shape}: scale {scale:.6g} (oracle {ref:.6g}), exact codes {frac:.5f}")


def test_all_zero_and_empty_tensors():
    codes, scale = run(torch.zeros((1, 5, 2, 128), dtype=torch.bfloat16))
    assert scale == 1.0 and np.all(decode_e4m3(codes) == 0)
    codes, scale = run(torch.zeros((1, 0, 2, 192), dtype=torch.bfloat16))
    assert scale == 1.0 and codes.size == 0


def test_extreme_values_saturate_at_448():
    x = bf16_input((1, 16, 2, 128), 9)
    x[0, 3, 1, 5] = 3.0e4                       # one huge element: it alone sets amax
    codes, scale = run(x)
    assert abs(scale - reference_scale(x)) <= 4e-7 * scale
    check_codes(x, codes, scale)
    assert np.max(np.abs(decode_e4m3(codes))) == 448.0


def test_full_size_q_sampled_rows():
    # Q of the 32K-token Gaussian workload (B=1, S=32768, Hq=32, d=128) as bf16, the
    # shape the benchmark times; the scale covers the whole tensor, codes compared on
    # 4096 sampled vectors.
    w = W.WORKLOADS["gauss32k"]
    q = W.draw_fp32(w)[0].to(torch.bfloat16)
    codes, scale = run(q)
    x = q.float().numpy().reshape(-1, w.d_qk)
    amax = 0.0
    for i in range(0, x.shape[0], 1 << 18):
        amax = max(amax, float(np.max(np.abs(rotate(x[i:i + (1 << 18)].astype(np.float64))))))
    ref = float(np.float32(amax / E4M3_MAX))
    assert abs(scale - ref) <= 4e-7 * ref
    rows = np.random.default_rng(3).choice(x.shape[0], 4096, replace=False)
    check_codes(q, codes, scale, rows=rows)


def test_deterministic_over_repeated_launches():
    x = bf16_input((1, 512, 8, 192), 12).to(DEV)
    first_codes, first_scale = binding.rotate_quant_bf16(x)
    first_codes, first_scale = first_codes.clone(), first_scale.clone()
    out = torch.empty_like(first_codes)
    sc = torch.empty_like(first_scale)
    bad = 0
    for _ in range(100):
        binding.rotate_quant_bf16(x, out=out, scale=sc)
        bad += int(not (torch.equal(out, first_codes) and torch.equal(sc, first_scale)))
    torch.cuda.synchronize()
    assert bad == 0


@pytest.mark.parametrize("mode", ["exact", "lean"])
def test_rotation_cuts_end_to_end_error_with_outlier_channels(mode):
    # Mistral-shaped inputs (4 outlier channels x8, shared by a KV head and its query
    # heads), bf16 activations; reference: fp64 attention of those bf16 values.
    w = W.WORKLOADS["mistral"].with_(S=512, Hq=8, Hkv=2)
    q, k, v = (t.to(torch.bfloat16) for t in W.draw_fp32(w))
    ref = attention_fp64(*(t.float().numpy().astype(np.float64) for t in (q, k, v)))
    v8, vs = W.quantize_e4m3(v.float())
    vd = v8.to(DEV)

    def attend(q8, qs, k8, ks):
        out = binding.attn_fwd_fp8(q8.to(DEV), k8.to(DEV), vd, qs, ks, vs, p_mode=mode)
        torch.cuda.synchronize()
        return out.float().cpu().numpy()

    q8, qs = W.quantize_e4m3(q.float())
    k8, ks = W.quantize_e4m3(k.float())
    e_plain = rel_rms(attend(q8, qs, k8, ks), ref)
    rq, rqs = binding.rotate_quant_bf16(q.to(DEV))
    rk, rks = binding.rotate_quant_bf16(k.to(DEV))
    e_rot = rel_rms(attend(rq, float(rqs.item()), rk, float(rks.item())), ref)
    print(f"[parity] rotation end to end ({mode}): rel-RMS {e_plain:.4f} -> {e_rot:.4f}")
    assert e_rot < 0.5 * e_plain


@pytest.mark.parametrize("mode", ["lean", "exact"])
@pytest.mark.parametrize("dqk", [128, 192])
def test_rotation_then_attention_with_device_scales(mode, dqk):
    # rotate Q and K, then attend with the scales the rotation wrote, all on one stream with no
    # host synchronisation; byte-identical to the call taking the same scales by value
    w = W.Workload("chain", 1, 4, 2, 777, dqk, 128)
    d = W.make_bf16(w, seed=23)
    dev = "cuda:0"
    q, k = d["q"].to(dev), d["k"].to(dev)
    v8, vs = W.quantize_e4m3(d["v"].float())
    v8 = v8.to(dev)
    q8, qs = binding.rotate_quant_bf16(q)
    k8, ks = binding.rotate_quant_bf16(k)
    vs_dev = torch.tensor([vs], dtype=torch.float32, device=dev)
    out_dev, lse_dev = binding.attn_fwd_fp8(q8, k8, v8, qs, ks, vs_dev, p_mode=mode, return_lse=True)
    torch.cuda.synchronize()
    out_val, lse_val = binding.attn_fwd_fp8(q8, k8, v8, float(qs.item()), float(ks.item()), vs, p_mode=mode,
                                            return_lse=True)
    torch.cuda.synchronize()
    assert torch.equal(out_dev.view(torch.int16), out_val.view(torch.int16))
    assert torch.equal(lse_dev, lse_val)


@pytest.mark.parametrize("dqk", [128, 192])
def test_prescaled_one_pass_matches_two_pass(dqk):
    # with the two-pass scale, the one-pass form writes the same codes, and its amax / 448 is that
    # scale (the same maximum of the same rotated values)
    w = W.Workload("pre", 2, 3, 3, 301, dqk, 128)
    x = W.make_bf16(w, seed=41)["q"].to("cuda:0")
    codes, scale = binding.rotate_quant_bf16(x)
    codes2, amax = binding.rotate_quant_bf16_prescaled(x, scale)
    torch.cuda.synchronize()
    assert torch.equal(codes, codes2)
    assert np.float32(amax.item()) / np.float32(E4M3_MAX) == np.float32(scale.item())
    # a different scale gives the oracle's codes for that scale (up to fp32 ties)
    s2 = torch.tensor([scale.item() * 1.37], dtype=torch.float32, device="cuda:0")
    codes3, _ = binding.rotate_quant_bf16_prescaled(x, s2, with_amax=False)
    torch.cuda.synchronize()
    r = rotate(x.float().cpu().numpy().astype(np.float64))
    exp = encode_e4m3_rne(np.clip(r / np.float64(np.float32(s2.item())), -E4M3_MAX, E4M3_MAX))
    assert np.mean(codes3.cpu().numpy() == exp) > 0.999

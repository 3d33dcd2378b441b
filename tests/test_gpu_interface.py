"""GPU checks of the flash_attn_func-style wrapper and the torch custom operators: the
same bytes as the direct binding calls (every call runs the HIP kernels), the same
bytes under torch.compile (the operators trace as opaque nodes, no graph break), and
torch.library.opcheck's registration checks."""
import pytest
import torch

from fp8_causal_prefill_tiled_amd import binding
from fp8_causal_prefill_tiled_amd import workloads as W
from fp8_causal_prefill_tiled_amd.interface import (flash_attn_func, _attn_fwd_bf16_op, _attn_fwd_fp8_dscale_op,
                                                    _attn_fwd_fp8_op)

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _fp8(S=300, Hq=4, Hkv=2, dqk=128, seed=8):
    d = W.make_fp8(W.Workload("iface", 1, Hq, Hkv, S, dqk, 128), seed=seed)
    q8, k8, v8 = (d[n].to(DEV) for n in ("q8", "k8", "v8"))
    return d, q8, k8, v8


@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("mode", ["lean", "exact"])
def test_fp8_wrapper_matches_binding(mode, causal):
    d, q8, k8, v8 = _fp8()
    ref, ref_lse = binding.attn_fwd_fp8(q8, k8, v8, d["q_scale"], d["k_scale"], d["v_scale"], p_mode=mode,
                                        causal=causal, return_lse=True)
    qf, kf, vf = (t.view(torch.float8_e4m3fn) for t in (q8, k8, v8))
    scales = dict(q_descale=d["q_scale"], k_descale=torch.tensor([d["k_scale"]], device=DEV),
                  v_descale=d["v_scale"])
    out, lse, none = flash_attn_func(qf, kf, vf, causal=causal, return_attn_probs=True, p_mode=mode, **scales)
    out2 = flash_attn_func(qf, kf, vf, causal=causal, p_mode=mode, **scales)
    torch.cuda.synchronize()
    assert none is None
    assert torch.equal(out.view(torch.int16), ref.view(torch.int16))
    assert torch.equal(out2.view(torch.int16), ref.view(torch.int16))
    assert torch.equal(lse, ref_lse)


@pytest.mark.parametrize("causal", [True, False])
def test_bf16_wrapper_matches_binding(causal):
    d = W.make_bf16(W.Workload("iface", 2, 4, 2, 257, 192, 128), seed=9)
    q, k, v = (d[n].to(DEV) for n in ("q", "k", "v"))
    ref, ref_lse = binding.attn_fwd_bf16(q, k, v, causal=causal, return_lse=True, softmax_scale=0.07)
    out, lse, _ = flash_attn_func(q, k, v, causal=causal, softmax_scale=0.07, return_attn_probs=True)
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), ref.view(torch.int16)) and torch.equal(lse, ref_lse)


def test_torch_compile_full_graph_same_bytes():
    d, q8, k8, v8 = _fp8(S=200)
    qb, kb, vb = (W.make_bf16(W.Workload("iface", 1, 4, 2, 200, 128, 128), seed=3)[n].to(DEV) for n in "qkv")
    qs, ks, vs = d["q_scale"], d["k_scale"], d["v_scale"]

    def f(q8, k8, v8, qb, kb, vb):
        a = flash_attn_func(q8, k8, v8, causal=True, q_descale=qs, k_descale=ks, v_descale=vs)
        b, lse, _ = flash_attn_func(qb, kb, vb, causal=True, return_attn_probs=True)
        return a.float() + b.float(), lse

    qf, kf, vf = (t.view(torch.float8_e4m3fn) for t in (q8, k8, v8))
    eager = f(qf, kf, vf, qb, kb, vb)
    compiled = torch.compile(f, backend="aot_eager", fullgraph=True)(qf, kf, vf, qb, kb, vb)
    torch.cuda.synchronize()
    assert torch.equal(eager[0], compiled[0]) and torch.equal(eager[1], compiled[1])


def test_opcheck():
    d, q8, k8, v8 = _fp8(S=130)
    torch.library.opcheck(_attn_fwd_fp8_op, (q8, k8, v8, d["q_scale"], d["k_scale"], d["v_scale"], 0.0, True, 1,
                                             True))
    b = W.make_bf16(W.Workload("iface", 1, 4, 2, 130, 128, 128), seed=4)
    q, k, v = (b[n].to(DEV) for n in ("q", "k", "v"))
    torch.library.opcheck(_attn_fwd_bf16_op, (q, k, v, 0.0, False, True))


def test_varlen_wrapper_matches_binding():
    from fp8_causal_prefill_tiled_amd.interface import flash_attn_varlen_func
    g = torch.Generator().manual_seed(5)
    q = torch.randn((150, 4, 128), generator=g).to(torch.bfloat16).to(DEV)
    k = torch.randn((400, 2, 128), generator=g).to(torch.bfloat16).to(DEV)
    v = torch.randn((400, 2, 128), generator=g).to(torch.bfloat16).to(DEV)
    cq = torch.tensor([0, 50, 150], dtype=torch.int32, device=DEV)
    ck = torch.tensor([0, 300, 400], dtype=torch.int32, device=DEV)
    ref, ref_lse = binding.attn_fwd_bf16_varlen(q, k, v, cq, 100, causal=True, return_lse=True, cu_seqlens_k=ck)
    out, lse, _ = flash_attn_varlen_func(q, k, v, cq, ck, 100, 300, causal=True, return_attn_probs=True)
    q8, qs = W.quantize_e4m3(q.float().cpu())
    k8, ks = W.quantize_e4m3(k.float().cpu())
    v8, vs = W.quantize_e4m3(v.float().cpu())
    q8, k8, v8 = q8.to(DEV), k8.to(DEV), v8.to(DEV)
    ref8 = binding.attn_fwd_fp8_varlen(q8, k8, v8, cq, 100, qs, ks, vs, p_mode="lean", cu_seqlens_k=ck)
    out8 = flash_attn_varlen_func(q8.view(torch.float8_e4m3fn), k8.view(torch.float8_e4m3fn),
                                  v8.view(torch.float8_e4m3fn), cq, ck, 100, causal=True,
                                  q_descale=qs, k_descale=ks, v_descale=vs)
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), ref.view(torch.int16)) and torch.equal(lse, ref_lse)
    assert torch.equal(out8.view(torch.int16), ref8.view(torch.int16))


def test_varlen_opcheck_and_compile():
    from fp8_causal_prefill_tiled_amd.interface import (flash_attn_varlen_func, _attn_fwd_bf16_varlen_op,
                                                         _attn_fwd_fp8_varlen_op)
    g = torch.Generator().manual_seed(6)
    q = torch.randn((96, 4, 128), generator=g).to(torch.bfloat16).to(DEV)
    k = torch.randn((160, 2, 128), generator=g).to(torch.bfloat16).to(DEV)
    cq = torch.tensor([0, 40, 96], dtype=torch.int32, device=DEV)
    ck = torch.tensor([0, 100, 160], dtype=torch.int32, device=DEV)
    torch.library.opcheck(_attn_fwd_bf16_varlen_op, (q, k, k, cq, ck, 56, 0.0, True, True))
    q8, qs = W.quantize_e4m3(q.float().cpu())
    k8, ks = W.quantize_e4m3(k.float().cpu())
    q8, k8 = q8.to(DEV), k8.to(DEV)
    torch.library.opcheck(_attn_fwd_fp8_varlen_op, (q8, k8, k8, cq, ck, 56, qs, ks, ks, 0.0, False, 1, True))

    def f(q, k, cq, ck):
        return flash_attn_varlen_func(q, k, k, cq, ck, 56, 100, causal=True).float() * 2

    eager = f(q, k, cq, ck)
    compiled = torch.compile(f, backend="aot_eager", fullgraph=True)(q, k, cq, ck)
    torch.cuda.synchronize()
    assert torch.equal(eager, compiled)


def test_fp8_wrapper_device_scales_match_and_compile():
    d, q8, k8, v8 = _fp8(S=333)
    qf, kf, vf = (t.view(torch.float8_e4m3fn) for t in (q8, k8, v8))
    ds = [torch.tensor([d[n]], dtype=torch.float32, device=DEV) for n in ("q_scale", "k_scale", "v_scale")]
    ref = flash_attn_func(qf, kf, vf, causal=True, q_descale=d["q_scale"], k_descale=d["k_scale"],
                          v_descale=d["v_scale"])

    def f(q, k, v, a, b, c):
        return flash_attn_func(q, k, v, causal=True, q_descale=a, k_descale=b, v_descale=c)

    out = f(qf, kf, vf, *ds)
    comp = torch.compile(f, backend="aot_eager", fullgraph=True)(qf, kf, vf, *ds)
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), ref.view(torch.int16))
    assert torch.equal(comp.view(torch.int16), ref.view(torch.int16))
    torch.library.opcheck(_attn_fwd_fp8_dscale_op, (q8, k8, v8, *ds, 0.0, True, 1, True))

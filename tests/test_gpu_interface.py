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


# ------------------------------------------------------------- the wrapper against the oracle

import numpy as np  # noqa: E402

from parity import (check_fp8, check_lse_fp8, gpu_select, lse_select, oracle_bf16, oracle_fp8, rel_rms,  # noqa: E402
                    row_rel_rms, TOL_BF16, TOL_BF16_ROW)


def _maybe_compiled(f, compiled):
    return torch.compile(f, backend="aot_eager", fullgraph=True) if compiled else f


@pytest.mark.parametrize("compiled", [False, True])
@pytest.mark.parametrize("scales", ["host", "device"])
@pytest.mark.parametrize("mode", ["exact", "lean"])
@pytest.mark.parametrize("dqk", [128, 192])
def test_flash_attn_func_fp8_against_oracle(dqk, mode, scales, compiled):
    d = W.make_fp8(W.Workload("iface_oracle", 1, 4, 2, 700, dqk, 128), seed=70 + dqk)
    q8, k8, v8 = (d[n].to(DEV).view(torch.float8_e4m3fn) for n in ("q8", "k8", "v8"))
    if scales == "host":
        sc = (d["q_scale"], d["k_scale"], d["v_scale"])
    else:
        sc = tuple(torch.tensor([d[n]], dtype=torch.float32, device=DEV) for n in ("q_scale", "k_scale", "v_scale"))

    def f(q, k, v, a, b, c):
        return flash_attn_func(q, k, v, causal=True, return_attn_probs=True, q_descale=a, k_descale=b, v_descale=c,
                               p_mode=mode)

    out, lse, _ = _maybe_compiled(f, compiled)(q8, k8, v8, *sc)
    torch.cuda.synchronize()
    emu, ref, lemu, lref = oracle_fp8(d, mode, with_lse=True)
    label = f"flash_attn_func fp8 d{dqk} {mode} {scales} scales{' compiled' if compiled else ''}"
    check_fp8(gpu_select(out), emu, ref, label, d=d, mode=mode)
    check_lse_fp8(lse_select(lse), lemu, lref, mode, label, d=d)


@pytest.mark.parametrize("compiled", [False, True])
@pytest.mark.parametrize("causal", [True, False])
def test_flash_attn_func_bf16_against_oracle(causal, compiled):
    d = W.make_bf16(W.Workload("iface_oracle", 2, 4, 2, 333, 192, 128), seed=71)
    q, k, v = (d[n].to(DEV) for n in ("q", "k", "v"))

    def f(q, k, v):
        return flash_attn_func(q, k, v, causal=causal, return_attn_probs=True)

    out, lse, _ = _maybe_compiled(f, compiled)(q, k, v)
    torch.cuda.synchronize()
    ref, lref = oracle_bf16(d, causal=causal, with_lse=True)
    got = gpu_select(out)
    e, er = rel_rms(got, ref), row_rel_rms(got, ref)
    dl = np.abs(lse_select(lse) - lref).max()
    print(f"[parity] flash_attn_func bf16 causal={causal} compiled={compiled}: vs fp64 {e:.2e}, per row max "
          f"{er.max():.2e}, lse {dl:.2e}")
    assert e <= TOL_BF16 and er.max() <= TOL_BF16_ROW and dl <= 2e-4


def _varlen_case(seed=72):
    """Three sequences with (queries, keys) = (50, 300), (180, 180), (7, 0): bottom-right causal
    alignment, one sequence with no keys."""
    pairs = [(50, 300), (180, 180), (7, 0)]
    g = torch.Generator().manual_seed(seed)
    tq, tk = sum(p[0] for p in pairs), sum(p[1] for p in pairs)
    x = {"q": torch.randn((tq, 4, 128), generator=g), "k": torch.randn((tk, 2, 128), generator=g),
         "v": torch.randn((tk, 2, 128), generator=g)}
    cq = np.cumsum([0] + [p[0] for p in pairs])
    ck = np.cumsum([0] + [p[1] for p in pairs])
    return pairs, x, cq, ck


@pytest.mark.parametrize("compiled", [False, True])
@pytest.mark.parametrize("dtype", ["lean", "exact", "bf16"])
def test_flash_attn_varlen_func_against_oracle(dtype, compiled):
    pairs, x, cq, ck = _varlen_case()
    cqd = torch.tensor(cq, dtype=torch.int32, device=DEV)
    ckd = torch.tensor(ck, dtype=torch.int32, device=DEV)
    maxq = max(p[0] for p in pairs)
    if dtype == "bf16":
        t = {n: x[n].to(torch.bfloat16) for n in x}
        args = [t[n].to(DEV) for n in ("q", "k", "v")]
        kw = {}
    else:
        t = {}
        for n in x:
            t[n + "8"], t[n + "_scale"] = W.quantize_e4m3(x[n])
        args = [t[n + "8"].to(DEV).view(torch.float8_e4m3fn) for n in ("q", "k", "v")]
        kw = dict(q_descale=t["q_scale"], k_descale=t["k_scale"], v_descale=t["v_scale"], p_mode=dtype)

    def f(q, k, v, cq_, ck_):
        return flash_attn_varlen_func(q, k, v, cq_, ck_, maxq, causal=True, **kw)

    from fp8_causal_prefill_tiled_amd.interface import flash_attn_varlen_func
    out = _maybe_compiled(f, compiled)(*args, cqd, ckd)
    torch.cuda.synchronize()
    got_all = out.float().cpu().numpy().astype(np.float64)
    for b, (nq, nk) in enumerate(pairs):
        got = got_all[None, cq[b]:cq[b + 1]]
        if nk == 0:
            assert np.all(got == 0.0)
            continue
        if dtype == "bf16":
            sq = {n: t[n][None, (cq if n == "q" else ck)[b]:(cq if n == "q" else ck)[b + 1]] for n in ("q", "k", "v")}
            ref = oracle_bf16(sq)
            e, er = rel_rms(got, ref), row_rel_rms(got, ref)
            assert e <= TOL_BF16 and er.max() <= TOL_BF16_ROW, (b, e, er.max())
        else:
            sd = {n + "8": t[n + "8"][None, (cq if n == "q" else ck)[b]:(cq if n == "q" else ck)[b + 1]].contiguous()
                  for n in ("q", "k", "v")}
            sd.update({n + "_scale": t[n + "_scale"] for n in ("q", "k", "v")})
            emu, ref = oracle_fp8(sd, dtype)
            check_fp8(got, emu, ref, f"varlen wrapper seq {b} ({nq} q, {nk} k) {dtype}", d=sd, mode=dtype)

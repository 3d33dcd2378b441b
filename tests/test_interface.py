"""Host-side checks of the flash_attn_func-style wrapper and the torch custom operators
(fp8_causal_prefill_tiled_amd/interface.py): option validation, and shape inference
through the fake implementations, which is what torch.compile traces (no GPU needed)."""
import pytest
import torch
from torch._subclasses.fake_tensor import FakeTensorMode
from torch.fx.experimental.proxy_tensor import make_fx

from fp8_causal_prefill_tiled_amd.interface import flash_attn_func


def _fake_inputs(dtype, B=2, S=100, Hq=4, Hkv=2, dqk=128, dv=128):
    q = torch.empty(B, S, Hq, dqk, dtype=dtype, device="cuda")
    k = torch.empty(B, S, Hkv, dqk, dtype=dtype, device="cuda")
    v = torch.empty(B, S, Hkv, dv, dtype=dtype, device="cuda")
    return q, k, v


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float8_e4m3fn])
@pytest.mark.parametrize("dqk", [128, 192])
def test_fake_shapes(dtype, dqk):
    kw = dict(q_descale=0.5, k_descale=0.25, v_descale=1.0) if dtype != torch.bfloat16 else {}
    with FakeTensorMode():
        q, k, v = _fake_inputs(dtype, dqk=dqk)
        out, lse, probs = flash_attn_func(q, k, v, causal=True, return_attn_probs=True, **kw)
        assert out.shape == (2, 100, 4, 128) and out.dtype == torch.bfloat16
        assert lse.shape == (2, 4, 100) and lse.dtype == torch.float32 and probs is None
        out2 = flash_attn_func(q, k, v, **kw)
        assert out2.shape == (2, 100, 4, 128)


@pytest.mark.parametrize("dtype,op", [(torch.bfloat16, "fp8_prefill.attn_fwd_bf16"),
                                      (torch.float8_e4m3fn, "fp8_prefill.attn_fwd_fp8")])
def test_traces_as_one_custom_op_node(dtype, op):
    kw = dict(q_descale=0.5, k_descale=0.25, v_descale=1.0) if dtype != torch.bfloat16 else {}

    def f(q, k, v):
        return flash_attn_func(q, k, v, causal=True, **kw) * 2

    with FakeTensorMode():
        q, k, v = _fake_inputs(dtype)
        g = make_fx(f, tracing_mode="fake")(q, k, v)
    targets = [str(n.target) for n in g.graph.nodes if n.op == "call_function"]
    assert sum(t.startswith(op) for t in targets) == 1, targets


@pytest.mark.parametrize("kw,exc", [
    (dict(dropout_p=0.1), NotImplementedError), (dict(window_size=(128, 0)), NotImplementedError),
    (dict(softcap=30.0), NotImplementedError), (dict(alibi_slopes=torch.zeros(4)), NotImplementedError),
])
def test_out_of_scope_options_raise(kw, exc):
    with FakeTensorMode():
        q, k, v = _fake_inputs(torch.bfloat16)
        with pytest.raises(exc):
            flash_attn_func(q, k, v, **kw)


def test_dtype_and_scale_errors():
    with FakeTensorMode():
        q, k, v = _fake_inputs(torch.float8_e4m3fn)
        with pytest.raises(ValueError, match="q_descale"):
            flash_attn_func(q, k, v, k_descale=1.0, v_descale=1.0)
        qb, kb, vb = _fake_inputs(torch.bfloat16)
        with pytest.raises(TypeError):
            flash_attn_func(q, kb, vb)
        with pytest.raises(TypeError):
            flash_attn_func(qb.half(), kb.half(), vb.half())


@pytest.mark.parametrize("dtype,op", [(torch.bfloat16, "fp8_prefill.attn_fwd_bf16_varlen"),
                                      (torch.float8_e4m3fn, "fp8_prefill.attn_fwd_fp8_varlen")])
def test_varlen_traces_as_one_custom_op_node(dtype, op):
    from fp8_causal_prefill_tiled_amd.interface import flash_attn_varlen_func
    kw = dict(q_descale=0.5, k_descale=0.25, v_descale=1.0) if dtype != torch.bfloat16 else {}

    def f(q, k, v, cq, ck):
        out, lse, _ = flash_attn_varlen_func(q, k, v, cq, ck, 64, 96, causal=True, return_attn_probs=True, **kw)
        return out, lse

    with FakeTensorMode():
        q = torch.empty(100, 4, 128, dtype=dtype, device="cuda")
        k = torch.empty(150, 2, 128, dtype=dtype, device="cuda")
        cq = torch.empty(3, dtype=torch.int32, device="cuda")
        g = make_fx(f, tracing_mode="fake")(q, k, k, cq, cq)
        out, lse = f(q, k, k, cq, cq)
    assert out.shape == (100, 4, 128) and out.dtype == torch.bfloat16 and lse.shape == (4, 100)
    targets = [str(n.target) for n in g.graph.nodes if n.op == "call_function"]
    assert sum(t.startswith(op) for t in targets) == 1, targets

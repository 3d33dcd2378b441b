"""The C-ABI library loads, exports every entry point include/attn_fwd.h declares,
and rejects every malformed or unsupported request on the host, before any HIP
call (so these run without a GPU)."""
import math
import os
import re

import pytest

from fp8_causal_prefill_tiled_amd import binding

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
OK, INVALID, UNSUPPORTED = binding.ATTN_OK, binding.ATTN_E_INVALID_ARG, binding.ATTN_E_UNSUPPORTED


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(binding.library_path()):
        from fp8_causal_prefill_tiled_amd import build
        build.build()
    return binding.load_library()


def declared_functions():
    names = set()
    for fn in os.listdir(os.path.join(ROOT, "include")):
        if fn.endswith(".h"):
            text = open(os.path.join(ROOT, "include", fn)).read()
            text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
            names |= set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(attn_\w+)\s*\(", text, flags=re.M))
    return names


def test_exports_every_declared_symbol(lib):
    decl = declared_functions()
    assert {"attn_fwd_fp8", "attn_fwd_fp8_lse", "attn_fwd_fp8_varlen", "attn_fwd_fp8_dscale", "attn_fwd_bf16",
            "attn_fwd_bf16_lse",
            "attn_fwd_bf16_varlen", "attn_last_error", "attn_abi_version"} <= decl
    assert decl <= binding.exported_symbols()
    assert lib.attn_abi_version() == 105


# fake, never-dereferenced, 16-byte aligned device addresses of disjoint buffers
Q, K, V, O = 0x10000000, 0x20000000, 0x30000000, 0x40000000


def fp8(**kw):
    a = dict(q=Q, k=K, v=V, o=O, q_scale=1.0, k_scale=1.0, v_scale=1.0, softmax_scale=0.0,
             B=1, Hq=4, Hkv=2, S=128, d_qk=128, d_v=128, causal=1, p_mode=0)
    a.update(kw)
    return binding.attn_fwd_fp8_raw(**a)


def bf16(**kw):
    a = dict(q=Q, k=K, v=V, o=O, softmax_scale=0.0, B=1, Hq=4, Hkv=2, S=128, d_qk=128, d_v=128, causal=1)
    a.update(kw)
    return binding.attn_fwd_bf16_raw(**a)


@pytest.mark.parametrize("kw,status", [
    (dict(q=0), INVALID), (dict(o=0), INVALID), (dict(v=0), INVALID),
    (dict(Hq=3), INVALID), (dict(Hkv=0), INVALID), (dict(S=-1), INVALID), (dict(B=-2), INVALID),
    (dict(d_qk=64), UNSUPPORTED), (dict(d_qk=0), INVALID), (dict(d_v=192), UNSUPPORTED),
    (dict(causal=-1), INVALID), (dict(causal=2), INVALID),
    (dict(p_mode=2), INVALID), (dict(p_mode=-1), INVALID),
    (dict(q_scale=0.0), INVALID), (dict(k_scale=-1.0), INVALID), (dict(v_scale=math.nan), INVALID),
    (dict(v_scale=math.inf), INVALID), (dict(softmax_scale=math.nan), INVALID),
    (dict(q_scale=1e-30, k_scale=1e-30), INVALID),
    (dict(q=Q + 8), INVALID), (dict(o=O + 2), INVALID),
    (dict(o=Q + 4096), INVALID),                      # output overlaps Q
    (dict(Hq=262144, Hkv=262144), UNSUPPORTED),       # a 64-key block of K past 2 GiB (32-bit offsets)
    (dict(Hq=174763, Hkv=174763, d_qk=192), UNSUPPORTED),
    (dict(S=0, q=0, k=0, v=0, o=0), OK), (dict(B=0, q=0, k=0, v=0, o=0), OK),  # empty: nothing launched
])
def test_fp8_host_validation(lib, kw, status):
    assert fp8(**kw) == status
    msg = binding.attn_last_error()
    assert (msg == "") == (status == OK)
    if status != OK:
        assert msg.startswith("attn_fwd_fp8")


@pytest.mark.parametrize("kw,status", [
    (dict(k=0), INVALID), (dict(Hq=5, Hkv=2), INVALID), (dict(d_qk=256), UNSUPPORTED),
    (dict(causal=3), INVALID), (dict(softmax_scale=math.inf), INVALID), (dict(k=K + 1), INVALID),
    (dict(o=V + 64), INVALID), (dict(S=0, q=0, k=0, v=0, o=0), OK),
    (dict(Hq=131072, Hkv=131072), UNSUPPORTED),       # bf16: a 64-key block of K past 2 GiB
])
def test_bf16_host_validation(lib, kw, status):
    assert bf16(**kw) == status
    assert (binding.attn_last_error() == "") == (status == OK)


def test_python_binding_rejects_bad_tensors(lib):
    import torch
    x = torch.zeros((1, 8, 2, 128), dtype=torch.uint8)
    with pytest.raises(ValueError, match="GPU tensor"):
        binding.attn_fwd_fp8(x, x, x, 1.0, 1.0, 1.0)
    with pytest.raises(TypeError):
        binding.attn_fwd_fp8(x.float(), x, x, 1.0, 1.0, 1.0)
    with pytest.raises(TypeError):
        binding.attn_fwd_bf16(x, x, x)


LSE = 0x50000000


@pytest.mark.parametrize("entry", ["fp8", "bf16"])
@pytest.mark.parametrize("kw,status", [
    (dict(lse=LSE + 2), INVALID),                 # misaligned
    (dict(lse=Q + 1024), INVALID),                # inside Q
    (dict(lse=O + 64), INVALID),                  # inside O
    (dict(lse=LSE, d_qk=64), UNSUPPORTED),
    (dict(lse=LSE, S=0, q=0, k=0, v=0, o=0), OK),  # empty: nothing launched
])
def test_lse_host_validation(lib, entry, kw, status):
    if entry == "fp8":
        a = dict(q=Q, k=K, v=V, o=O, lse=LSE, q_scale=1.0, k_scale=1.0, v_scale=1.0, softmax_scale=0.0,
                 B=1, Hq=4, Hkv=2, S=128, d_qk=128, d_v=128, causal=0, p_mode=1)
        a.update(kw)
        st = binding.attn_fwd_fp8_lse_raw(**a)
    else:
        a = dict(q=Q, k=K, v=V, o=O, lse=LSE, softmax_scale=0.0, B=1, Hq=4, Hkv=2, S=128, d_qk=128, d_v=128,
                 causal=1)
        a.update(kw)
        st = binding.attn_fwd_bf16_lse_raw(**a)
    assert st == status
    msg = binding.attn_last_error()
    assert (msg == "") == (status == OK)
    if status != OK:
        assert msg.startswith(f"attn_fwd_{entry}_lse")


CU = 0x60000000
OK_IF_NULL_K = "ok-if-null-k"


@pytest.mark.parametrize("entry", ["fp8", "bf16"])
@pytest.mark.parametrize("kw,status", [
    (dict(cu_seqlens_q=0), INVALID),                        # null offsets with sequences
    (dict(cu_seqlens_q=CU + 2), INVALID),                   # misaligned offsets
    (dict(cu_seqlens_k=CU + 6), INVALID),
    (dict(total_q=-1), INVALID), (dict(total_k=-1), INVALID), (dict(max_seqlen_q=-1), INVALID),
    (dict(n_seqs=-1), INVALID),
    (dict(total_q=(1 << 30) + 1), UNSUPPORTED), (dict(total_k=(1 << 30) + 1), UNSUPPORTED),
    (dict(n_seqs=1 << 22, max_seqlen_q=1 << 12, Hq=64, Hkv=2), UNSUPPORTED),   # grid beyond 2^31 workgroups
    (dict(cu_seqlens_k=0, total_k=-5), OK_IF_NULL_K),       # null key offsets: total_k ignored
    (dict(k=O + 4096), INVALID),                            # K starting inside O
    (dict(d_qk=64), UNSUPPORTED), (dict(Hq=3), INVALID), (dict(causal=2), INVALID),
    (dict(lse=Q + 64), INVALID),                            # lse inside Q
    (dict(o=Q + 4096), INVALID),                            # output overlaps Q
    (dict(n_seqs=0, cu_seqlens_q=0, cu_seqlens_k=0, q=0, k=0, v=0, o=0), OK),  # empty: nothing launched
    (dict(total_q=0, q=0, k=0, v=0, o=0), OK),
    (dict(max_seqlen_q=0, q=0, k=0, v=0, o=0), OK),
])
def test_varlen_host_validation(lib, entry, kw, status):
    if status == OK_IF_NULL_K:
        # a null cu_seqlens_k with a garbage total_k is accepted; check it on an empty problem
        kw = dict(kw, n_seqs=0, cu_seqlens_q=0, q=0, k=0, v=0, o=0)
        status = OK
    a = dict(q=Q, k=K, v=V, o=O, lse=LSE, cu_seqlens_q=CU, cu_seqlens_k=CU + 64, n_seqs=3, max_seqlen_q=100,
             total_q=200, total_k=300, softmax_scale=0.0, Hq=4, Hkv=2, d_qk=128, d_v=128, causal=1)
    if entry == "fp8":
        a.update(q_scale=1.0, k_scale=1.0, v_scale=1.0, p_mode=1)
    a.update(kw)
    st = (binding.attn_fwd_fp8_varlen_raw if entry == "fp8" else binding.attn_fwd_bf16_varlen_raw)(**a)
    assert st == status
    msg = binding.attn_last_error()
    assert (msg == "") == (status == OK)
    if status != OK:
        assert msg.startswith(f"attn_fwd_{entry}_varlen")


SC = 0x70000000


@pytest.mark.parametrize("kw,status", [
    (dict(q_scale=0), INVALID), (dict(v_scale=0), INVALID), (dict(k_scale=SC + 2), INVALID),
    (dict(d_qk=64), UNSUPPORTED), (dict(p_mode=3), INVALID), (dict(o=Q + 64), INVALID),
    (dict(S=0, q=0, k=0, v=0, o=0), OK),
])
def test_dscale_host_validation(lib, kw, status):
    a = dict(q=Q, k=K, v=V, o=O, lse=0, q_scale=SC, k_scale=SC + 4, v_scale=SC + 8, softmax_scale=0.0,
             B=1, Hq=4, Hkv=2, S=128, d_qk=128, d_v=128, causal=1, p_mode=1)
    a.update(kw)
    assert binding.attn_fwd_fp8_dscale_raw(**a) == status
    msg = binding.attn_last_error()
    assert (msg == "") == (status == OK)
    if status != OK:
        assert msg.startswith("attn_fwd_fp8_dscale")


def rotp(**kw):
    a = dict(x=Q, x8=K, scale=V, amax=O, B=1, S=64, H=2, d=128)
    a.update(kw)
    return binding.attn_rotate_quant_bf16_prescaled_raw(**a)


@pytest.mark.parametrize("kw,status", [
    (dict(scale=0), INVALID), (dict(amax=O + 2), INVALID), (dict(scale=V + 1), INVALID),
    (dict(d=96), UNSUPPORTED), (dict(x=0), INVALID), (dict(amax=Q + 64), INVALID),
    (dict(x8=Q + 4096), INVALID), (dict(B=0, x=0, x8=0, amax=0), OK),   # empty, no amax: nothing launched
])
def test_rotate_quant_prescaled_validation(lib, kw, status):
    assert rotp(**kw) == status
    assert (binding.attn_last_error() == "") == (status == OK)


def rotq(**kw):
    a = dict(x=Q, x8=K, scale=V, B=1, S=64, H=2, d=128)
    a.update(kw)
    return binding.attn_rotate_quant_bf16_raw(**a)


@pytest.mark.parametrize("kw,status", [
    (dict(x=0), INVALID), (dict(x8=0), INVALID), (dict(scale=0), INVALID),
    (dict(B=-1), INVALID), (dict(S=-3), INVALID), (dict(H=0), INVALID),
    (dict(d=96), UNSUPPORTED), (dict(d=64), UNSUPPORTED), (dict(d=256), UNSUPPORTED),
    (dict(x=Q + 8), INVALID), (dict(x8=K + 4), INVALID),
    (dict(x8=Q + 4096), INVALID),               # codes overlap the input
    (dict(scale=Q + 64), INVALID),              # scale inside the input
    (dict(B=1 << 20, S=1 << 10, H=8), UNSUPPORTED),
])
def test_rotate_quant_rejects(lib, kw, status):
    assert rotq(**kw) == status
    assert binding.attn_last_error()

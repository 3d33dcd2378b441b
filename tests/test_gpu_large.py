"""GPU parity at tensor sizes whose byte offsets pass 2^31 and 2^32.

Every kernel address is a 64-bit offset from the tensor base; these tests put
batches at offsets past 2 GiB (K, V) and 4 GiB (Q, O) and check them.  The big
tensors repeat one small seeded batch, with other seeded batches planted in the
middle and at the end, so every batch's output is known from a call on that
batch alone: equal bytes where the kernel runs the same code over the same
bytes, and the small calls are tied to the oracle.  The variable-length entry
points run over the same buffers packed as one sequence per batch.
"""
import sys

import pytest
import torch

from parity import (W, binding, check_fp8, gpu_select, oracle_bf16, oracle_fp8, rel_rms, TOL_BF16)

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
S, HQ, HKV = 300, 4, 2          # two query tiles, the second ragged; GQA 2:1


def _note(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _big(small, B, special):
    """(B, ...) GPU copy of the one-batch CPU tensor `small`, with special[b] (CPU,
    one batch) planted at batch b."""
    x = small.to(DEV).expand(B, *small.shape[1:]).contiguous()
    for b, t in special.items():
        x[b].copy_(t[0].to(DEV))
    return x


def _same_as(out, ref, skip, chunk=2048):
    """Batches of `out` (B, ...) other than `skip` whose bytes differ from `ref` (one batch)."""
    B = out.shape[0]
    o = out.view(B, -1).view(torch.int16)
    r = ref.reshape(1, -1).view(torch.int16)
    bad = []
    for b0 in range(0, B, chunk):
        diff = (o[b0:b0 + chunk] != r).any(dim=1).nonzero().flatten().cpu().tolist()
        bad += [b0 + i for i in diff if b0 + i not in skip]
    return bad


@pytest.mark.parametrize("mode,dqk", [("lean", 128), ("exact", 128), ("lean", 192)])
def test_fp8_batches_past_4gib(mode, dqk):
    B = 30000
    _note(f"[large] fp8 {mode} d_qk={dqk} B={B} S={S} H={HQ}x{HKV}")
    w = W.Workload(f"large_fp8_d{dqk}", 1, HQ, HKV, S, dqk, 128)
    base = W.make_fp8(w, seed=4100)
    plant = {B // 2 + 1: W.make_fp8(w, seed=4200), B - 1: W.make_fp8(w, seed=4300)}
    qs, ks, vs = base["q_scale"], base["k_scale"], base["v_scale"]
    q8, k8, v8 = (_big(base[n], B, {b: d[n] for b, d in plant.items()}) for n in ("q8", "k8", "v8"))
    assert q8.numel() > 1 << 32 and k8.numel() > 1 << 31     # offsets past 4 GiB (Q) and 2 GiB (K, V)

    def one(d):                        # a call on one batch alone, with the big tensors' scales
        o, l = binding.attn_fwd_fp8(d["q8"].to(DEV), d["k8"].to(DEV), d["v8"].to(DEV), qs, ks, vs,
                                    p_mode=mode, return_lse=True)
        torch.cuda.synchronize()
        return o[0], l[0]

    refs = {b: one(d) for b, d in plant.items()}
    base_o, base_l = one(base)
    for label, d, o in [("base", base, base_o)] + [(f"batch {b}", plant[b], refs[b][0]) for b in plant]:
        dd = dict(d, q_scale=qs, k_scale=ks, v_scale=vs)
        emu, ref = oracle_fp8(dd, mode)
        check_fp8(gpu_select(o[None]), emu, ref, f"large fp8 {mode} d{dqk} {label}")

    out, lse = binding.attn_fwd_fp8(q8, k8, v8, qs, ks, vs, p_mode=mode, return_lse=True)
    torch.cuda.synchronize()
    assert out.numel() * 2 > 1 << 33
    for b, (o, l) in refs.items():
        assert torch.equal(out[b].view(torch.int16), o.view(torch.int16)), b
        assert torch.equal(lse[b], l), b
    assert _same_as(out, base_o, set(plant)) == []
    assert torch.equal(lse[0], base_l) and torch.equal(lse[B - 2], base_l)

    # the same buffers as one packed variable-length batch, a sequence per batch
    cu = torch.arange(0, (B + 1) * S, S, dtype=torch.int32, device=DEV)
    out.fill_(0)
    ov, lv = binding.attn_fwd_fp8_varlen(q8.view(B * S, HQ, dqk), k8.view(B * S, HKV, dqk),
                                         v8.view(B * S, HKV, 128), cu, S, qs, ks, vs, p_mode=mode,
                                         out=out.view(B * S, HQ, 128), return_lse=True)
    torch.cuda.synchronize()
    for b, (o, l) in refs.items():
        assert torch.equal(out[b].view(torch.int16), o.view(torch.int16)), ("varlen", b)
        assert torch.equal(lv[:, b * S:(b + 1) * S], l), ("varlen", b)
    assert _same_as(out, base_o, set(plant)) == []


def test_bf16_batches_past_4gib():
    B = 15000
    _note(f"[large] bf16 B={B} S={S} H={HQ}x{HKV}")
    w = W.Workload("large_bf16", 1, HQ, HKV, S, 128, 128)
    base = W.make_bf16(w, seed=4400)
    plant = {B // 2 + 1: W.make_bf16(w, seed=4500), B - 1: W.make_bf16(w, seed=4600)}
    q, k, v = (_big(base[n], B, {b: d[n] for b, d in plant.items()}) for n in ("q", "k", "v"))
    assert q.numel() * 2 > 1 << 32 and k.numel() * 2 > 1 << 31

    def one(d):
        o, l = binding.attn_fwd_bf16(d["q"].to(DEV), d["k"].to(DEV), d["v"].to(DEV), return_lse=True)
        torch.cuda.synchronize()
        return o[0], l[0]

    refs = {b: one(d) for b, d in plant.items()}
    base_o, base_l = one(base)
    for label, d, o in [("base", base, base_o)] + [(f"batch {b}", plant[b], refs[b][0]) for b in plant]:
        e = rel_rms(gpu_select(o[None]), oracle_bf16(d))
        _note(f"[parity] large bf16 {label}: vs fp64 {e:.2e}")
        assert e <= TOL_BF16, (label, e)

    out, lse = binding.attn_fwd_bf16(q, k, v, return_lse=True)
    torch.cuda.synchronize()
    for b, (o, l) in refs.items():
        assert torch.equal(out[b].view(torch.int16), o.view(torch.int16)), b
        assert torch.equal(lse[b], l), b
    assert _same_as(out, base_o, set(plant)) == []

    cu = torch.arange(0, (B + 1) * S, S, dtype=torch.int32, device=DEV)
    out.fill_(0)
    ov, lv = binding.attn_fwd_bf16_varlen(q.view(B * S, HQ, 128), k.view(B * S, HKV, 128), v.view(B * S, HKV, 128),
                                          cu, S, out=out.view(B * S, HQ, 128), return_lse=True)
    torch.cuda.synchronize()
    for b, (o, l) in refs.items():
        assert torch.equal(out[b].view(torch.int16), o.view(torch.int16)), ("varlen", b)
        assert torch.equal(lv[:, b * S:(b + 1) * S], l), ("varlen", b)
    assert _same_as(out, base_o, set(plant)) == []

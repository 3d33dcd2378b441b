"""The FP8 kernel variants compute the same bits (GPU).

The log-sum-exp store and scales read from device memory are template switches: each
combination is its own kernel with its own register allocation and instruction schedule,
but the arithmetic of the output is the same, so the outputs must be byte-identical.  A
difference means a schedule-dependent fault: it caught a matrix instruction reading a
register that a vector move had written just before it (no wait states in between), which
changed rows of one variant only.
"""
import pytest
import torch

from fp8_causal_prefill_tiled_amd import binding
from fp8_causal_prefill_tiled_amd import workloads as W

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("mode", ["lean", "exact"])
@pytest.mark.parametrize("dqk", [128, 192])
def test_lse_and_device_scale_variants_same_bytes(dqk, mode, causal):
    d = W.make_fp8(W.Workload("variants", 2, 8, 2, 700, dqk, 128), seed=700 + dqk)
    q8, k8, v8 = (d[n].to(DEV) for n in ("q8", "k8", "v8"))
    host = (d["q_scale"], d["k_scale"], d["v_scale"])
    dev = [torch.tensor([x], dtype=torch.float32, device=DEV) for x in host]
    outs = {
        "plain": binding.attn_fwd_fp8(q8, k8, v8, *host, p_mode=mode, causal=causal),
        "lse": binding.attn_fwd_fp8(q8, k8, v8, *host, p_mode=mode, causal=causal, return_lse=True)[0],
        "dscale": binding.attn_fwd_fp8(q8, k8, v8, *dev, p_mode=mode, causal=causal),
        "dscale_lse": binding.attn_fwd_fp8(q8, k8, v8, *dev, p_mode=mode, causal=causal, return_lse=True)[0],
    }
    again = binding.attn_fwd_fp8(q8, k8, v8, *host, p_mode=mode, causal=causal)
    torch.cuda.synchronize()
    ref = outs["plain"].view(torch.int16)
    assert torch.equal(again.view(torch.int16), ref)
    for name, o in outs.items():
        same = torch.equal(o.view(torch.int16), ref)
        if not same:
            rows = ((o.float() - outs["plain"].float()).abs() > 0).any(-1).any(-1).nonzero()[:, 1].unique()
            pytest.fail(f"{name} differs from the plain kernel in {rows.numel()} rows, e.g. {rows[:8].tolist()}")

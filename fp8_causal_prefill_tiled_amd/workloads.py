"""Seeded synthetic inputs for causal prefill attention (shared by tests and the benchmark).

This module holds no attention arithmetic: it draws fp32 Gaussian tensors on the
CPU with ``torch.Generator`` and quantises them with torch's own float8_e4m3fn /
bfloat16 conversions (per-tensor scale amax/448, the e4m3fn maximum).  The CPU
oracle and the HIP path both receive exactly these bytes.

Workloads (the pages measure on real-model activations, which need trained
weights; these seeded synthetic tensors of the same shapes stand in for them):

* ``tiny``     B=1, Hq=Hkv=2,  S=256,   d=128/128, N(0,1).
* ``mistral``  B=1, Hq=32, Hkv=8, S=16384, d=128: N(0,1) with 4 fixed outlier
               channels per KV head scaled x8 in K and in every Q head that
               reads that KV head.
* ``qwen``     B=1, Hq=32, Hkv=8, S=16384, d=128, N(0,1) (FP8 and BF16 runs).
* ``gauss32k`` B=1, Hq=Hkv=32, S=32768, d=128/128, N(0,1) - the kernel benchmark
               shape of the pages (Gaussian inputs, 32K tokens, head dim 128).
* ``mla``      B=1, Hq=Hkv=16, S=32768, d_qk=192, d_v=128, N(0,1) with Q/K
               dims 128..191 (the rotary part) scaled x2.
"""
from dataclasses import dataclass, replace

import torch

BASE_SEED = 20261202
E4M3_MAX = 448.0


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    Hq: int
    Hkv: int
    S: int
    d_qk: int
    d_v: int
    outlier_channels: int = 0      # per KV head, x outlier_gain in Q and K
    outlier_gain: float = 8.0
    rope_dims: int = 0             # trailing Q/K dims scaled x rope_gain
    rope_gain: float = 2.0

    def with_(self, **kw):
        return replace(self, **kw)

    @property
    def causal_flops(self):
        """2*B*Hq*S^2*(d_qk+d_v)/2: two matmuls over the S^2/2 causal pairs."""
        return 2.0 * self.B * self.Hq * self.S * self.S * (self.d_qk + self.d_v) / 2.0


WORKLOADS = {
    "tiny": Workload("tiny", 1, 2, 2, 256, 128, 128),
    "mistral": Workload("mistral", 1, 32, 8, 16384, 128, 128, outlier_channels=4),
    "qwen": Workload("qwen", 1, 32, 8, 16384, 128, 128),
    "gauss32k": Workload("gauss32k", 1, 32, 32, 32768, 128, 128),
    "mla": Workload("mla", 1, 16, 16, 32768, 192, 128, rope_dims=64),
}


def _gen(seed):
    g = torch.Generator(device="cpu")
    g.manual_seed(int(seed))
    return g


def draw_fp32(w: Workload, seed=BASE_SEED):
    """fp32 Q, K, V of shapes (B,S,Hq,d_qk), (B,S,Hkv,d_qk), (B,S,Hkv,d_v)."""
    q = torch.randn((w.B, w.S, w.Hq, w.d_qk), generator=_gen(seed + 0), dtype=torch.float32)
    k = torch.randn((w.B, w.S, w.Hkv, w.d_qk), generator=_gen(seed + 1), dtype=torch.float32)
    v = torch.randn((w.B, w.S, w.Hkv, w.d_v), generator=_gen(seed + 2), dtype=torch.float32)
    if w.outlier_channels:
        gch = _gen(seed + 3)
        group = w.Hq // w.Hkv
        for g in range(w.Hkv):
            ch = torch.randperm(w.d_qk, generator=gch)[: w.outlier_channels]
            k[:, :, g, ch] *= w.outlier_gain
            for h in range(g * group, (g + 1) * group):
                q[:, :, h, ch] *= w.outlier_gain
    if w.rope_dims:
        q[..., w.d_qk - w.rope_dims:] *= w.rope_gain
        k[..., w.d_qk - w.rope_dims:] *= w.rope_gain
    return q, k, v


def quantize_e4m3(x: torch.Tensor):
    """Per-tensor quantisation: scale = amax/448, codes = e4m3fn(x/scale) (torch's RNE cast).

    Returns (codes as uint8 tensor, scale as float).  amax == 0 gives scale 1.
    """
    amax = float(x.abs().max())
    scale = amax / E4M3_MAX if amax > 0 else 1.0
    codes = (x / scale).clamp_(-E4M3_MAX, E4M3_MAX).to(torch.float8_e4m3fn).view(torch.uint8)
    return codes, float(scale)


def make_fp8(w: Workload, seed=BASE_SEED):
    """Dict with uint8 e4m3 codes q8/k8/v8 (CPU, contiguous) and their fp32 scales."""
    q, k, v = draw_fp32(w, seed)
    q8, qs = quantize_e4m3(q)
    del q
    k8, ks = quantize_e4m3(k)
    del k
    v8, vs = quantize_e4m3(v)
    return {"q8": q8, "k8": k8, "v8": v8, "q_scale": qs, "k_scale": ks, "v_scale": vs}


def make_bf16(w: Workload, seed=BASE_SEED):
    """Dict with bfloat16 q/k/v (CPU): the same fp32 draws rounded to bf16."""
    q, k, v = draw_fp32(w, seed)
    return {"q": q.to(torch.bfloat16), "k": k.to(torch.bfloat16), "v": v.to(torch.bfloat16)}


def sample_rows(S, n, seed=BASE_SEED + 7):
    """A seeded sorted sample of n query rows that always holds 0, 1, 63, 64, S-1."""
    fixed = {0, 1, 63, 64, S - 1}
    fixed = {r for r in fixed if 0 <= r < S}
    if n >= S:
        return torch.arange(S)
    perm = torch.randperm(S, generator=_gen(seed))[:n]
    rows = sorted(fixed | set(int(r) for r in perm[: max(0, n - len(fixed))]))
    return torch.tensor(rows, dtype=torch.int64)


def sample_rows_long(S, n, seed=BASE_SEED + 11):
    """A seeded sorted sample of about n distinct query rows weighted towards long causal rows:
    rows 0, 1, 63, 64 and S-1, then n/8 rows drawn uniformly from 0..S-1 and the rest from
    the second half S/2..S-1 (where almost all of a causal launch's work is)."""
    if n >= S:
        return torch.arange(S)
    fixed = {r for r in (0, 1, 63, 64, S - 1) if 0 <= r < S}
    g = _gen(seed)
    spread = torch.randperm(S, generator=g)[: max(1, n // 8)]
    half = S // 2
    late = half + torch.randperm(S - half, generator=g)
    rows = fixed | set(int(r) for r in spread)
    for r in late.tolist():
        if len(rows) >= n:
            break
        rows.add(int(r))
    return torch.tensor(sorted(rows), dtype=torch.int64)


def sample_rows_strata(S, n_first=256, n_rest=1024, seed=BASE_SEED + 13):
    """Rows for estimating a whole-tensor sum over query rows: every row below n_first, plus a
    seeded uniform sample of n_rest rows from n_first..S-1.  Returns (rows, weights): the weight
    of a row is the number of rows it stands for (1 for the first stratum)."""
    first = torch.arange(min(n_first, S))
    if S <= n_first + n_rest:
        return torch.arange(S), torch.ones(S, dtype=torch.float64)
    rest = n_first + torch.randperm(S - n_first, generator=_gen(seed))[:n_rest]
    rest = torch.sort(rest).values
    rows = torch.cat([first, rest])
    weights = torch.cat([torch.ones(len(first), dtype=torch.float64),
                         torch.full((n_rest,), (S - n_first) / n_rest, dtype=torch.float64)])
    return rows, weights

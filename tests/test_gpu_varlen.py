"""GPU parity of variable-length batches (attn_fwd_fp8_varlen / attn_fwd_bf16_varlen)
through the C ABI.

Each packed sequence runs the same kernel code over the same key blocks as an
equal-length call on that sequence alone, so its output and log-sum-exp must be
byte-identical to that call's (which the other parity tests tie to the oracle);
the oracle is also run on every sequence of one mixed batch directly.  Rows
outside every sequence must stay untouched, and offsets outside the tensors are
clamped by the kernels (documented behaviour), not read out of bounds.
"""
import numpy as np
import pytest
import torch

from parity import W, binding, check_fp8, oracle_bf16, oracle_fp8, rel_rms, TOL_BF16

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
LENS = [1, 63, 64, 65, 300, 0, 257, 1000]


def _draws(lens, Hq, Hkv, dqk, seed):
    """Seeded fp32 Q, K, V of every sequence, concatenated along the rows: (T, H, d) each."""
    xs = [W.draw_fp32(W.Workload(f"seq{i}", 1, Hq, Hkv, max(n, 1), dqk, 128), seed=seed + i)
          for i, n in enumerate(lens)]
    return tuple(torch.cat([x[t][0, :n] for x, n in zip(xs, lens)]) for t in range(3))


def _packed_fp8(lens, Hq, Hkv, dqk, seed):
    """e4m3 codes of the packed batch with one per-tensor scale each (CPU), and the scales."""
    (q8, qs), (k8, ks), (v8, vs) = (W.quantize_e4m3(x) for x in _draws(lens, Hq, Hkv, dqk, seed))
    return q8, k8, v8, qs, ks, vs


def _cu(lens):
    return torch.tensor(np.concatenate([[0], np.cumsum(lens)]), dtype=torch.int32, device=DEV)


@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("mode", ["lean", "exact"])
@pytest.mark.parametrize("dqk", [128, 192])
def test_fp8_varlen_equals_per_sequence_calls(dqk, mode, causal):
    q8, k8, v8, qs, ks, vs = _packed_fp8(LENS, 4, 2, dqk, 500)
    q8, k8, v8 = q8.to(DEV), k8.to(DEV), v8.to(DEV)
    out, lse = binding.attn_fwd_fp8_varlen(q8, k8, v8, _cu(LENS), max(LENS), qs, ks, vs, p_mode=mode,
                                           causal=causal, return_lse=True)
    torch.cuda.synchronize()
    off = 0
    for n in LENS:
        if n:
            o1, l1 = binding.attn_fwd_fp8(q8[None, off:off + n].contiguous(), k8[None, off:off + n].contiguous(),
                                          v8[None, off:off + n].contiguous(), qs, ks, vs, p_mode=mode,
                                          causal=causal, return_lse=True)
            torch.cuda.synchronize()
            assert torch.equal(out[off:off + n].view(torch.int16), o1[0].view(torch.int16)), (n, off)
            assert torch.equal(lse[:, off:off + n], l1[0]), (n, off)
        off += n


@pytest.mark.parametrize("mode", ["lean", "exact"])
def test_fp8_varlen_against_oracle(mode):
    lens = [130, 0, 64, 513, 1]
    q8, k8, v8, qs, ks, vs = _packed_fp8(lens, 4, 1, 128, 900)
    out = binding.attn_fwd_fp8_varlen(q8.to(DEV), k8.to(DEV), v8.to(DEV), _cu(lens), max(lens), qs, ks, vs,
                                      p_mode=mode)
    torch.cuda.synchronize()
    got = out.float().cpu().numpy().astype(np.float64)[None]
    # the oracle per sequence, packed the same way; the bars apply to the call's whole output
    emus, refs, off = [], [], 0
    for n in lens:
        if n:
            d = {"q8": q8[None, off:off + n], "k8": k8[None, off:off + n], "v8": v8[None, off:off + n],
                 "q_scale": qs, "k_scale": ks, "v_scale": vs}
            emu, ref = oracle_fp8(d, mode)
            emus.append(emu)
            refs.append(ref)
        off += n
    check_fp8(got, np.concatenate(emus, axis=1), np.concatenate(refs, axis=1), f"varlen {lens} {mode}")


def test_bf16_varlen_equals_per_sequence_calls_and_oracle():
    lens = [65, 0, 1, 300, 129]
    qc, kc, vc = (x.to(torch.bfloat16) for x in _draws(lens, 4, 2, 192, 77))
    q, k, v = qc.to(DEV), kc.to(DEV), vc.to(DEV)
    for causal in (True, False):
        out, lse = binding.attn_fwd_bf16_varlen(q, k, v, _cu(lens), max(lens), causal=causal, return_lse=True)
        torch.cuda.synchronize()
        off = 0
        for n in lens:
            if n:
                o1, l1 = binding.attn_fwd_bf16(q[None, off:off + n].contiguous(), k[None, off:off + n].contiguous(),
                                               v[None, off:off + n].contiguous(), causal=causal, return_lse=True)
                torch.cuda.synchronize()
                assert torch.equal(out[off:off + n].view(torch.int16), o1[0].view(torch.int16))
                assert torch.equal(lse[:, off:off + n], l1[0])
                d = {"q": qc[None, off:off + n], "k": kc[None, off:off + n], "v": vc[None, off:off + n]}
                e = rel_rms(o1.float().cpu().numpy(), oracle_bf16(d, causal=causal))
                assert e <= TOL_BF16, (n, e)
            off += n


@pytest.mark.parametrize("entry", ["fp8", "bf16"])
def test_rows_outside_sequences_untouched_and_offsets_clamped(entry):
    T, Hq, Hkv = 300, 2, 2
    g = torch.Generator().manual_seed(3)
    if entry == "fp8":
        q, k, v = (torch.randint(0, 120, (T, H, 128), generator=g, dtype=torch.uint8).to(DEV)
                   for H in (Hq, Hkv, Hkv))
        run = lambda cu, n_max, o, lse_: binding.attn_fwd_fp8_varlen(q, k, v, cu, n_max, 0.01, 0.01, 0.01, out=o,
                                                                    return_lse=True, p_mode="lean")
    else:
        q, k, v = (torch.randn((T, H, 128), generator=g).to(torch.bfloat16).to(DEV) for H in (Hq, Hkv, Hkv))
        run = lambda cu, n_max, o, lse_: binding.attn_fwd_bf16_varlen(q, k, v, cu, n_max, out=o, return_lse=True)
    sentinel = torch.full((T, Hq, 128), 7.0, dtype=torch.bfloat16, device=DEV)
    # sequences cover rows [0, 100) and [100, 250); rows 250..299 belong to none
    o = sentinel.clone()
    out, _ = run(torch.tensor([0, 100, 100, 250], dtype=torch.int32, device=DEV), 150, o, None)
    torch.cuda.synchronize()
    assert torch.equal(out[250:], sentinel[250:]) and not torch.equal(out[:250], sentinel[:250])
    # offsets outside [0, T] and decreasing ones are clamped: sequence 0 -> rows [0, 300) capped at
    # max_seqlen=120 rows, sequence 1 -> empty, sequence 2 -> empty; nothing past row 119 is written
    o = sentinel.clone()
    out, lse = run(torch.tensor([-40, 5000, 200, -7], dtype=torch.int32, device=DEV), 120, o, None)
    torch.cuda.synchronize()
    assert torch.equal(out[120:], sentinel[120:])
    assert bool(torch.isfinite(out[:120].float()).all()) and bool(torch.isfinite(lse[:, :120]).all())


# ------------------------------------------------- unequal query and key lengths

PAIRS = [(64, 300), (1, 257), (200, 200), (130, 1000), (256, 513)]   # (Sq, Sk), Sq <= Sk


def _cu_from(lens):
    return _cu(list(lens))


@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("mode", ["lean", "exact"])
@pytest.mark.parametrize("dqk", [128, 192])
def test_fp8_fewer_queries_than_keys_is_the_tail_of_the_full_call(dqk, mode, causal):
    # A sequence with Sq queries over Sk >= Sq keys (bottom-right aligned) is, row for row, the
    # last Sq rows of the equal-length call whose queries end with these: same key blocks, same
    # masks, same order, so the bytes must match.
    Sks = [sk for _, sk in PAIRS]
    qf8, k8, v8, qs, ks, vs = _packed_fp8(Sks, 4, 2, dqk, 1300)
    qf8, k8, v8 = qf8.to(DEV), k8.to(DEV), v8.to(DEV)
    offs = np.concatenate([[0], np.cumsum(Sks)])
    q8 = torch.cat([qf8[offs[i] + sk - sq:offs[i] + sk] for i, (sq, sk) in enumerate(PAIRS)])
    out, lse = binding.attn_fwd_fp8_varlen(q8, k8, v8, _cu_from(sq for sq, _ in PAIRS), max(sq for sq, _ in PAIRS),
                                           qs, ks, vs, p_mode=mode, causal=causal, return_lse=True,
                                           cu_seqlens_k=_cu_from(Sks))
    torch.cuda.synchronize()
    qo = 0
    for i, (sq, sk) in enumerate(PAIRS):
        sl = slice(offs[i], offs[i] + sk)
        of, lf = binding.attn_fwd_fp8(qf8[None, sl].contiguous(), k8[None, sl].contiguous(), v8[None, sl].contiguous(),
                                      qs, ks, vs, p_mode=mode, causal=causal, return_lse=True)
        torch.cuda.synchronize()
        assert torch.equal(out[qo:qo + sq].view(torch.int16), of[0, sk - sq:].view(torch.int16)), (sq, sk)
        assert torch.equal(lse[:, qo:qo + sq], lf[0, :, sk - sq:]), (sq, sk)
        qo += sq


@pytest.mark.parametrize("mode", ["lean", "exact"])
def test_fp8_unequal_lengths_against_oracle(mode):
    # includes more queries than keys: the first Sq - Sk queries see nothing (O = 0, lse = -inf)
    pairs = [(100, 300), (300, 100), (65, 64), (1, 1), (40, 0)]
    g = torch.Generator().manual_seed(77)
    qf = torch.randn((sum(p[0] for p in pairs), 2, 128), generator=g)
    kf = torch.randn((sum(p[1] for p in pairs), 1, 128), generator=g)
    vf = torch.randn((sum(p[1] for p in pairs), 1, 128), generator=g)
    (q8, qs), (k8, ks), (v8, vs) = (W.quantize_e4m3(x) for x in (qf, kf, vf))
    cq, ck = _cu_from(p[0] for p in pairs), _cu_from(p[1] for p in pairs)
    out, lse = binding.attn_fwd_fp8_varlen(q8.to(DEV), k8.to(DEV), v8.to(DEV), cq, max(p[0] for p in pairs),
                                           qs, ks, vs, p_mode=mode, return_lse=True, cu_seqlens_k=ck)
    torch.cuda.synchronize()
    got = out.float().cpu().numpy().astype(np.float64)
    gl = lse.cpu().numpy().astype(np.float64)
    emus, refs, lemus, qo, ko = [], [], [], 0, 0
    for sq, sk in pairs:
        d = {"q8": q8[None, qo:qo + sq], "k8": k8[None, ko:ko + sk], "v8": v8[None, ko:ko + sk],
             "q_scale": qs, "k_scale": ks, "v_scale": vs}
        emu, ref, lemu, lref = oracle_fp8(d, mode, with_lse=True)
        emus.append(emu)
        refs.append(ref)
        lemus.append(lemu)
        blind = max(sq - sk, 0)                  # queries that see no key
        assert np.all(got[qo:qo + blind] == 0) and np.all(np.isneginf(gl[:, qo:qo + blind]))
        fin = np.isfinite(lemu[0])
        assert np.array_equal(np.isfinite(gl[:, qo:qo + sq]), fin)
        if fin.any():
            assert np.max(np.abs(gl[:, qo:qo + sq][fin] - lemu[0][fin])) < np.log(1.125)
        qo += sq
        ko += sk
    check_fp8(got[None], np.concatenate(emus, axis=1), np.concatenate(refs, axis=1), f"unequal {pairs} {mode}")


def test_bf16_fewer_queries_than_keys_is_the_tail_of_the_full_call():
    Sks = [sk for _, sk in PAIRS]
    qf, kf, vf = (x.to(torch.bfloat16).to(DEV) for x in _draws(Sks, 4, 2, 128, 41))
    offs = np.concatenate([[0], np.cumsum(Sks)])
    q = torch.cat([qf[offs[i] + sk - sq:offs[i] + sk] for i, (sq, sk) in enumerate(PAIRS)])
    for causal in (True, False):
        out, lse = binding.attn_fwd_bf16_varlen(q, kf, vf, _cu_from(sq for sq, _ in PAIRS),
                                                max(sq for sq, _ in PAIRS), causal=causal, return_lse=True,
                                                cu_seqlens_k=_cu_from(Sks))
        torch.cuda.synchronize()
        qo = 0
        for i, (sq, sk) in enumerate(PAIRS):
            sl = slice(offs[i], offs[i] + sk)
            of, lf = binding.attn_fwd_bf16(qf[None, sl].contiguous(), kf[None, sl].contiguous(),
                                           vf[None, sl].contiguous(), causal=causal, return_lse=True)
            torch.cuda.synchronize()
            assert torch.equal(out[qo:qo + sq].view(torch.int16), of[0, sk - sq:].view(torch.int16)), (sq, sk)
            assert torch.equal(lse[:, qo:qo + sq], lf[0, :, sk - sq:]), (sq, sk)
            qo += sq

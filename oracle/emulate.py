"""Step-by-step CPU emulation of the FP8 method (block-scaled, rounded-sum softmax).

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

The method approximates ``attention64.attention_fp64``: the probabilities P are
rounded to FP8 e4m3 before the P.V product.  This module takes the pages' steps
in their order, in fp64 except where the method itself rounds:

1. Scores.  s_ij = sum_c decode(Q8[i,c]) * decode(K8[j,c]) - the product of the
   FP8 codes' values that the FP8 matrix instruction forms (exact in fp64: each
   product has at most 8 significant bits and the sum spans < 53 bits).
   t_ij = s_ij * q_scale * k_scale * sm * log2(e) is the score in log2 units.
2. Causal mask: keys j > i are excluded ([KG-en] §"Application Boundaries").
3. Per-64-key-block power-of-2 scale.  Every block of 64 keys gets its own
   power-of-two factor, applied to its probabilities ahead of the e4m3 rounding
   and undone again by the block scale of the matrix instruction ([MTP] §"Per-block scaling and a rounded row sum";
   [KG-en] §"ZYFA's Technical Solutions").  Reading: the power is chosen per
   (query row, 64-key block) from M_ib = ceil(max_{j in block b, j<=i} t_ij),
   so that the block's largest probability lands in (128, 256] - the top binade
   of e4m3 below its 448 maximum - and the probability is taken relative to
   the block's own integer maximum (independent of block order).
4. Probabilities, one of two paths:
   * exact: p~_ij = e4m3_RNE(2^(t_ij - M_ib + 8)) - a true exponential, rounded;
   * Lean P: the e4m3 code of 2^x is about 8x + const because doubling a value
     adds 8 to its code ([MTP] §"Lean P: one multiply-add instead of an
     exponential"; [KG-en] §"ZYFA's Technical Solutions").  With
     x = t_ij - M_ib + 8 and code(2^n) = 8n + 56 the code is the single
     multiply-add A*s_ij + B_ib, A = 8*q_scale*k_scale*sm*log2(e),
     B_ib = 120 - 8*M_ib, followed by one conversion to an integer.  Reading:
     the conversion rounds to nearest, ties to even, and saturates to [0, 126]
     (codes below 0 are probability 0; 126 = 448 is never reached since the
     block maximum maps to code <= 120).  p~_ij = decode(code).
5. Rounded row sum: l_ib = sum_j p~_ij, the sum of the rounded probabilities,
   not of the unrounded ones ([MTP] ibid.; [KG-zh] §技术解法 gives the reason:
   values that round to zero would otherwise still count in the denominator).
6. Combination over blocks (the online-softmax recurrence written in closed
   form; it is exact because every block factor is a power of two):
       O_i = v_scale * sum_b 2^(M_ib - R_i) sum_j p~_ij decode(V8_j)
                     / sum_b 2^(M_ib - R_i) l_ib,        R_i = max_b M_ib.
   The common 2^-8 of step 3 and the choice of R_i cancel between numerator and
   denominator; R_i only keeps 2^(.) in range.

``rounding=False`` (exact path only) skips the e4m3 rounding in step 4; the
result is then the plain definition, which pins this module to
``attention64`` (tests/test_oracle_emulate.py).

Rounding decisions near a boundary.  Step 4 turns a real number into an integer
code, so a score that lies very close to a rounding boundary has two valid
codes: the pages fix neither the precision of the scores nor the order of the
matrix instruction's sums.  ``rounding_alternatives`` lists, for one query row,
every key whose code changes when its log2-domain score moves by at most
eps_j = kappa * c * sum_m max_{k in step m} |q_k k_jk| (an error scale of a dot
product summed in steps of 64 products, each step accurate to a fraction of its
largest product), and the code it would take then.  Reading: a result that differs from the
emulation only by such alternative codes is as correct as the emulation.
"""
import numpy as np

from .e4m3 import decode_e4m3, encode_e4m3_rne, round_to_e4m3
from .attention64 import kv_head, visible_keys, _rows_of

LOG2E = 1.4426950408889634
BLOCK_KEYS = 64


def _block_probs(t, valid, p_mode, rounding, s=None, A=None):
    """Steps 3-5 for one chunk of rows.

    t, valid: (R, nb, 64) log2-domain scores and the causal/tail validity mask.
    Returns (p~ (R, nb, 64) float64, M (R, nb) float64, block_has_keys (R, nb)).
    """
    tm = np.where(valid, t, -np.inf)
    has = valid.any(axis=2)
    bmax = tm.max(axis=2)
    M = np.where(has, np.ceil(np.where(has, bmax, 0.0)), 0.0)
    if p_mode == "exact":
        x = t - M[:, :, None] + 8.0
        p = np.exp2(np.where(valid, x, -np.inf))
        if rounding:
            p = round_to_e4m3(p)
    elif p_mode == "lean":
        if not rounding:
            raise ValueError("Lean P always produces integer codes")
        B = 120.0 - 8.0 * M
        code = np.rint(A * s + B[:, :, None])
        code = np.clip(code, 0, 126)
        code = np.where(valid, code, 0).astype(np.uint8)
        p = decode_e4m3(code)
    else:
        raise ValueError(p_mode)
    p = np.where(valid, p, 0.0)
    return p, M, has


def emulate_fp8(q8, k8, v8, q_scale, k_scale, v_scale, sm_scale=None, p_mode="exact",
                causal=True, rows=None, rounding=True, chunk=256, return_lse=False):
    """Emulate the FP8 method on e4m3 codes (uint8 arrays, (B, S, H, d) layout; K and V may
    have their own length Sk, with the causal mask and the no-key convention of
    attention64.attention_fp64).

    Returns O (B, len(rows), Hq, d_v) float64.  With ``return_lse`` also returns
    log2L (B, len(rows), Hq) = log2(sum_b 2^(M_ib - 8) l_ib), the base-2 log of the
    denominator step 6 divides by (the sum of the rounded probabilities, each block
    at its own power of two).  Without rounding it is log2 sum_j 2^(t_ij), so
    ln(2) * log2L is the row's log-sum-exp of the logits sm * <q_i, k_j>.
    """
    q8 = np.asarray(q8, dtype=np.uint8)
    k8 = np.asarray(k8, dtype=np.uint8)
    v8 = np.asarray(v8, dtype=np.uint8)
    B, S, Hq, dqk = q8.shape
    Sk, Hkv = k8.shape[1], k8.shape[2]
    dv = v8.shape[3]
    sm = 1.0 / np.sqrt(dqk) if sm_scale is None else float(sm_scale)
    C = float(q_scale) * float(k_scale) * sm * LOG2E
    A = np.float64(np.float32(8.0 * C))
    rows = _rows_of(rows, S)
    out = np.zeros((B, len(rows), Hq, dv))
    log2L = np.full((B, len(rows), Hq), -np.inf)
    qd = decode_e4m3(q8)
    kd = decode_e4m3(k8)
    vd = decode_e4m3(v8)
    for b in range(B):
        for h in range(Hq):
            g = kv_head(h, Hq, Hkv)
            for c0 in range(0, len(rows), chunk):
                r_all = rows[c0:c0 + chunk]
                nvis_all = visible_keys(r_all, S, Sk, causal)
                live = np.flatnonzero(nvis_all > 0)       # rows that see no key keep O = 0
                if len(live) == 0:
                    continue
                r, nvis = r_all[live], nvis_all[live]
                n = int(nvis.max())
                nb = (n + BLOCK_KEYS - 1) // BLOCK_KEYS
                npad = nb * BLOCK_KEYS
                s = np.zeros((len(r), npad))
                s[:, :n] = qd[b, r, h, :] @ kd[b, :n, g, :].T
                keys = np.arange(npad)
                valid = keys[None, :] < nvis[:, None]
                s3 = s.reshape(len(r), nb, BLOCK_KEYS)
                v3 = valid.reshape(len(r), nb, BLOCK_KEYS)
                p, M, has = _block_probs(s3 * C, v3, p_mode, rounding, s=s3, A=A)
                Rref = np.max(np.where(has, M, -np.inf), axis=1)
                fac = np.where(has, np.exp2(M - Rref[:, None]), 0.0)
                l = p.sum(axis=2)
                den = (fac * l).sum(axis=1)
                W = (p * fac[:, :, None]).reshape(len(r), npad)[:, :n]
                num = W @ vd[b, :n, g, :]
                out[b, c0 + live, h, :] = float(v_scale) * (num / den[:, None])
                log2L[b, c0 + live, h] = np.log2(den) + Rref - 8.0
    if return_lse:
        return out, log2L
    return out


def block_probabilities(q8, k8, q_scale, k_scale, sm_scale=None, p_mode="exact", i=0, b=0, h=0,
                        Hkv=None):
    """The rounded probabilities p~ (nb, 64) and exponents M (nb,) of one query row.

    For tests of the per-block structure on small inputs.
    """
    q8 = np.asarray(q8, dtype=np.uint8)
    k8 = np.asarray(k8, dtype=np.uint8)
    B, S, Hq, dqk = q8.shape
    Hkv = k8.shape[2] if Hkv is None else Hkv
    sm = 1.0 / np.sqrt(dqk) if sm_scale is None else float(sm_scale)
    C = float(q_scale) * float(k_scale) * sm * LOG2E
    A = np.float64(np.float32(8.0 * C))
    g = kv_head(h, Hq, Hkv)
    n = i + 1
    nb = (n + BLOCK_KEYS - 1) // BLOCK_KEYS
    s = np.zeros((1, nb * BLOCK_KEYS))
    s[:, :n] = decode_e4m3(q8[b, i:i + 1, h, :]) @ decode_e4m3(k8[b, :n, g, :]).T
    valid = (np.arange(nb * BLOCK_KEYS) < n)[None, :]
    s3 = s.reshape(1, nb, BLOCK_KEYS)
    p, M, has = _block_probs(s3 * C, valid.reshape(1, nb, BLOCK_KEYS), p_mode, True, s=s3, A=A)
    return p[0], M[0]


def encode_probability_lean(y):
    """Lean-P code for a log2-domain value y = t - M + 8 (y <= 8): rint(8y + 56) in [0, 126]."""
    return np.clip(np.rint(8.0 * np.asarray(y, dtype=np.float64) + 56.0), 0, 126).astype(np.uint8)


def encode_probability_exact(y):
    """Exact-path code for y: e4m3_RNE(2^y)."""
    return encode_e4m3_rne(np.exp2(np.asarray(y, dtype=np.float64)))


def rounding_alternatives(q8, k8, v8, q_scale, k_scale, v_scale, sm_scale=None, p_mode="exact", b=0, i=0, h=0,
                          causal=True, kappa=2.0 ** -10):
    """One query row of the emulation together with its ambiguous rounding decisions.

    Returns a dict with
      ``out``    O_i (d_v,), as emulate_fp8 returns it;
      ``vhat``   the dequantised value rows of the visible keys (n, d_v);
      ``weight`` W_j = p~_j * 2^(M_b(j) - R_i) of every visible key (n,), so that
                 O_i = sum_j W_j vhat_j / sum_j W_j (steps 3-6);
      ``alt``    a list of (j, W_alt): keys whose code differs when the log2-domain score
                 t_j moves anywhere within [t_j - eps_j, t_j + eps_j] (block exponents held
                 fixed), with the weight each other code gives.
    eps_j = kappa * c * sum_m max_{k in [64m, 64m+64)} |decode(Q8[i,k]) * decode(K8[j,k])| in
    log2 units (c = the log2-domain score factor).  kappa = 0 lists nothing.
    """
    q8 = np.asarray(q8, dtype=np.uint8)
    k8 = np.asarray(k8, dtype=np.uint8)
    v8 = np.asarray(v8, dtype=np.uint8)
    B, S, Hq, dqk = q8.shape
    Sk, Hkv = k8.shape[1], k8.shape[2]
    sm = 1.0 / np.sqrt(dqk) if sm_scale is None else float(sm_scale)
    C = float(q_scale) * float(k_scale) * sm * LOG2E
    A = np.float64(np.float32(8.0 * C))
    g = kv_head(h, Hq, Hkv)
    n = int(visible_keys(np.array([i]), S, Sk, causal)[0])
    if n == 0:
        return {"out": np.zeros(v8.shape[3]), "vhat": np.zeros((0, v8.shape[3])), "weight": np.zeros(0), "alt": []}
    nb = (n + BLOCK_KEYS - 1) // BLOCK_KEYS
    npad = nb * BLOCK_KEYS
    qd = decode_e4m3(q8[b, i, h, :])
    kd = decode_e4m3(k8[b, :n, g, :])
    s = np.zeros(npad)
    s[:n] = kd @ qd
    sabs = np.zeros(npad)
    prod = np.abs(kd * qd[None, :])
    for m0 in range(0, dqk, 64):
        sabs[:n] += prod[:, m0:m0 + 64].max(axis=1)
    valid = (np.arange(npad) < n).reshape(1, nb, BLOCK_KEYS)
    s3 = s.reshape(1, nb, BLOCK_KEYS)
    p, M, has = _block_probs(s3 * C, valid, p_mode, True, s=s3, A=A)
    R = np.max(np.where(has, M, -np.inf))
    fac = np.repeat(np.exp2(M[0] - R), BLOCK_KEYS)[:n]
    weight = p.reshape(-1)[:n] * fac
    vhat = float(v_scale) * decode_e4m3(v8[b, :n, g, :])
    out = weight @ vhat / weight.sum()
    eps = (kappa * C * sabs[:n])
    Mk = np.repeat(M[0], BLOCK_KEYS)[:n]
    t = s[:n] * C
    cands = []
    for sign in (-1.0, 1.0):
        if p_mode == "exact":
            palt = round_to_e4m3(np.exp2(t + sign * eps - Mk + 8.0))
        else:
            code = np.clip(np.rint(A * s[:n] + (120.0 - 8.0 * Mk) + sign * 8.0 * eps), 0, 126)
            palt = decode_e4m3(code.astype(np.uint8))
        cands.append(palt)
    alt = []
    base = p.reshape(-1)[:n]
    for j in np.flatnonzero((cands[0] != base) | (cands[1] != base)):
        for palt in sorted({float(cands[0][j]), float(cands[1][j])} - {float(base[j])}):
            alt.append((int(j), palt * fac[j]))
    return {"out": out, "vhat": vhat, "weight": weight, "alt": alt}

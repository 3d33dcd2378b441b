"""Plain causal softmax attention in fp64 - the quantity the method approximates.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

The operation is forward prefill attention with equal query and key lengths and
a causal mask ([KG-en] §"Application Boundaries and Engineering Decisions";
[MTP] §TL;DR and its comparison table, row "Scope"): for every batch b, query
head h and query position i,

    O[b,i,h,:] = sum_{j<=i} w_ij V[b,j,g,:],
    w_ij = exp(sm * <Q[b,i,h,:], K[b,j,g,:]> - m_i) / sum_{j'<=i} exp(sm * <Q_i, K_j'> - m_i),

with m_i the row maximum (it cancels; it only keeps exp in range), sm the
softmax scale (1/sqrt(d_qk) unless given) and g the key/value head of query head
h.  The pages measure accuracy as RMS error against fp64 for a single attention
call ([KG-en] §"Performance Benchmarks"; [MTP] §"How accurate is ZYFA's FP8
attention?"), so this is evaluated in fp64.

Readings (the pages are silent): grouped-query attention maps query head h to
key/value head floor(h / (Hq / Hkv)) (consecutive groups, the flash_attn
convention behind the "drop-in flash_attn_func interface", [MTP] §TL;DR);
tensors are (B, S, H, d), contiguous in d.

Unequal query and key lengths (Sq queries, Sk keys; outside the pages' scope, for
chunked prefill and variable-length batches): reading - the causal mask is aligned
at the bottom right, as in FlashAttention 2.1 and later, so query i sees keys
j <= i + (Sk - Sq); a query that sees no key gets O = 0 and a log-sum-exp of -inf.
With Sq == Sk this is the causal mask above.

Every query row is computed independently from the definition; rows are only
grouped into chunks to bound memory.
"""
import numpy as np

from .e4m3 import decode_e4m3


def dequantize(codes, scale):
    """x_hat = scale * decode(code), as float64."""
    return float(scale) * decode_e4m3(codes)


def kv_head(h, Hq, Hkv):
    """Key/value head used by query head h (consecutive groups)."""
    return h // (Hq // Hkv)


def _rows_of(rows, S):
    if rows is None:
        return np.arange(S)
    return np.asarray(rows, dtype=np.int64)


def visible_keys(rows, Sq, Sk, causal):
    """Number of keys each query row sees: keys 0 .. n-1 with n = clip(i + 1 + Sk - Sq, 0, Sk)
    when causal (bottom-right aligned), all Sk keys otherwise."""
    rows = np.asarray(rows, dtype=np.int64)
    if not causal:
        return np.full(rows.shape, Sk, dtype=np.int64)
    return np.clip(rows + 1 + (Sk - Sq), 0, Sk)


def attention_fp64(q, k, v, sm_scale=None, causal=True, rows=None, chunk=512):
    """Causal (or full) softmax attention in fp64.

    q: (B, Sq, Hq, d_qk), k: (B, Sk, Hkv, d_qk), v: (B, Sk, Hkv, d_v), any real dtype
    (Sq == Sk for the pages' equal-length case).
    rows: optional 1-D array of query positions to evaluate (default: all).
    Returns O of shape (B, len(rows), Hq, d_v), float64.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    B, Sq, Hq, dqk = q.shape
    Sk, Hkv = k.shape[1], k.shape[2]
    dv = v.shape[3]
    assert k.shape == (B, Sk, Hkv, dqk) and v.shape == (B, Sk, Hkv, dv)
    assert Hq % Hkv == 0
    sm = 1.0 / np.sqrt(dqk) if sm_scale is None else float(sm_scale)
    rows = _rows_of(rows, Sq)
    out = np.zeros((B, len(rows), Hq, dv), dtype=np.float64)
    keys = np.arange(Sk)
    for b in range(B):
        for h in range(Hq):
            g = kv_head(h, Hq, Hkv)
            kk = k[b, :, g, :]
            vv = v[b, :, g, :]
            for c0 in range(0, len(rows), chunk):
                r = rows[c0:c0 + chunk]
                nvis = visible_keys(r, Sq, Sk, causal)
                n = int(nvis.max())                    # keys any row here can see
                live = nvis > 0                        # rows that see no key keep O = 0
                if n == 0:
                    continue
                logits = sm * (q[b, r[live], h, :] @ kk[:n].T)
                logits = np.where(keys[None, :n] < nvis[live][:, None], logits, -np.inf)
                m = logits.max(axis=1, keepdims=True)
                w = np.exp(logits - m)
                w /= w.sum(axis=1, keepdims=True)
                out[b, c0 + np.flatnonzero(live), h, :] = w @ vv[:n]
    return out


def lse_fp64(q, k, sm_scale=None, causal=True, rows=None, chunk=512):
    """Natural-log softmax normaliser of each query row, ln sum_j exp(sm <q_i, k_j>) over
    the keys the row sees (all keys, or the causal ones as in attention_fp64), in fp64;
    -inf for a row that sees no key.  Returns (B, Hq, len(rows)): the layout attention
    libraries return it in."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    B, Sq, Hq, dqk = q.shape
    Sk, Hkv = k.shape[1], k.shape[2]
    sm = 1.0 / np.sqrt(dqk) if sm_scale is None else float(sm_scale)
    rows = _rows_of(rows, Sq)
    out = np.full((B, Hq, len(rows)), -np.inf, dtype=np.float64)
    keys = np.arange(Sk)
    for b in range(B):
        for h in range(Hq):
            kk = k[b, :, kv_head(h, Hq, Hkv), :]
            for c0 in range(0, len(rows), chunk):
                r = rows[c0:c0 + chunk]
                nvis = visible_keys(r, Sq, Sk, causal)
                n = int(nvis.max())
                live = nvis > 0
                if n == 0:
                    continue
                logits = sm * (q[b, r[live], h, :] @ kk[:n].T)
                logits = np.where(keys[None, :n] < nvis[live][:, None], logits, -np.inf)
                m = logits.max(axis=1)
                out[b, h, c0 + np.flatnonzero(live)] = m + np.log(np.exp(logits - m[:, None]).sum(axis=1))
    return out


def attention_weights_fp64(q, k, sm_scale=None, causal=True):
    """The full weight matrix w[b, h, i, j] (small shapes only)."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    B, S, Hq, dqk = q.shape
    Hkv = k.shape[2]
    sm = 1.0 / np.sqrt(dqk) if sm_scale is None else float(sm_scale)
    w = np.empty((B, Hq, S, S))
    mask = np.tril(np.ones((S, S), dtype=bool)) if causal else np.ones((S, S), dtype=bool)
    for b in range(B):
        for h in range(Hq):
            g = kv_head(h, Hq, Hkv)
            logits = np.where(mask, sm * (q[b, :, h, :] @ k[b, :, g, :].T), -np.inf)
            e = np.exp(logits - logits.max(axis=1, keepdims=True))
            w[b, h] = e / e.sum(axis=1, keepdims=True)
    return w


def rel_rms(x, ref):
    """Relative RMS error ||x - ref||_2 / ||ref||_2 over all elements."""
    x = np.asarray(x, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    return float(np.sqrt(np.sum((x - ref) ** 2)) / np.sqrt(np.sum(ref ** 2)))

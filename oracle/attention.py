"""Single-token decode attention in float64 (test infrastructure only).

[KVL] section "01 · Conceito": during causal decode only the newest position
needs an output; its query attends to the cached keys and mixes the cached
values, and this is exact causal attention, not an approximation of it.
[KVC] section "Attention Sinks e o StreamingLLM…" and [SINK] "a ideia": the
attention weights are a softmax, so they sum to one.

Readings (the per-head equation is lost from [KVL]'s text): logits are the query
/ key inner products times ``scale`` (default 1/sqrt(D)); the softmax subtracts
the row maximum before exponentiating (this changes nothing mathematically).
Grouped-query attention ([KVL] "01 · Conceito": 24 query heads share 4 K/V
heads; [KVC] notes n_kv = n_q / 8 in GQA models) maps query head h to KV head
floor(h / G) with G = H_q / H_kv.
"""
import numpy as np

from .rope import apply_rope


def softmax(x: np.ndarray, axis: int = -1) -> np.ndarray:
    x = np.asarray(x, dtype=np.float64)
    m = np.max(x, axis=axis, keepdims=True)
    e = np.exp(x - m)
    return e / np.sum(e, axis=axis, keepdims=True)


def attend_one(q: np.ndarray, k: np.ndarray, v: np.ndarray, scale: float):
    """One query q[D] over keys k[n][D] and values v[n][Dv]: returns (out[Dv], p[n])."""
    logits = (k @ q) * scale
    p = softmax(logits)
    return p @ v, p


def _default_scale(D: int, scale):
    return 1.0 / np.sqrt(D) if scale is None else float(scale)


def decode_gqa(q: np.ndarray, k: np.ndarray, v: np.ndarray, scale=None, return_probs=False):
    """q[Hq][D], k[Hkv][n][D], v[Hkv][n][D] -> out[Hq][D] (and probs[Hq][n])."""
    Hq, D = q.shape
    Hkv = k.shape[0]
    if Hq % Hkv:
        raise ValueError("query heads must be a multiple of kv heads")
    G = Hq // Hkv
    sc = _default_scale(D, scale)
    out = np.empty((Hq, v.shape[-1]), dtype=np.float64)
    probs = np.empty((Hq, k.shape[1]), dtype=np.float64)
    for h in range(Hq):
        g = h // G
        out[h], probs[h] = attend_one(q[h], k[g], v[g], sc)
    return (out, probs) if return_probs else out


def decode_gqa_rope(q, k, v, q_pos, k_pos, base, scale=None, pairs="half"):
    """Decode with keys stored un-rotated: rotate q at ``q_pos`` and every key at
    its own entry of ``k_pos`` ([SINK] "como funciona"), then attend."""
    qr = apply_rope(q, q_pos, base, pairs)
    kr = apply_rope(k, np.asarray(k_pos)[None, :], base, pairs)
    return decode_gqa(qr, kr, v, scale)


def causal_attention(Q, K, V, positions, base=None, scale=None, pairs="half"):
    """Full causal self-attention over a whole sequence, every row at once.

    Q[T][Hq][D], K[T][Hkv][D], V[T][Hkv][D]; row t attends keys 0..t.  RoPE (if
    ``base``) is applied at ``positions[t]``.  Written as a masked score matrix so
    that it shares no decode-path code: used to pin the decode path ([KVL]
    "01 · Conceito": cached decode equals exact causal attention).
    """
    Q = np.asarray(Q, np.float64)
    K = np.asarray(K, np.float64)
    V = np.asarray(V, np.float64)
    T, Hq, D = Q.shape
    Hkv = K.shape[1]
    G = Hq // Hkv
    sc = _default_scale(D, scale)
    pos = np.asarray(positions, np.float64)
    if base is not None:
        Q = apply_rope(Q, pos[:, None], base, pairs)
        K = apply_rope(K, pos[:, None], base, pairs)
    mask = np.tril(np.ones((T, T), dtype=bool))
    out = np.empty((T, Hq, V.shape[-1]))
    for h in range(Hq):
        S = (Q[:, h, :] @ K[:, h // G, :].T) * sc
        S = np.where(mask, S, -np.inf)
        S = S - S.max(axis=1, keepdims=True)
        P = np.exp(S)
        P /= P.sum(axis=1, keepdims=True)
        out[:, h, :] = P @ V[:, h // G, :]
    return out

"""DuoAttention mixed-head decode (test infrastructure only).

[KVC] "Decomposição funcional com o DuoAttention": a minority of heads (retrieval
heads, gamma = 1) need the whole history and keep a full cache; the others
(streaming heads, gamma = 0) keep a constant buffer of the 4 attention sinks and the
64 most recent tokens.  The gammas come from an L1-regularised calibration before
deployment; here they are an input (one per layer and KV head: the query heads of a
group share their KV head's cache).

Readings:
* A streaming head's buffer is the StreamingLLM sink + window cache of the same page
  ("Attention Sinks e o StreamingLLM..."), the window counting the token being
  decoded, which is written before its query attends.
* Keys and values are used as given (already position-encoded upstream), as for the
  other compressed caches; no rotation at in-cache positions.
"""
import numpy as np

from .attention import decode_gqa
from .streaming import retained_tokens


def duo_attended_tokens(t: int, retrieval: bool, n_sink: int, window: int) -> np.ndarray:
    """Ascending ids of the tokens one KV head attends at decode step ``t``."""
    if retrieval:
        return np.arange(0, t + 1, dtype=np.int64)
    return retained_tokens(t, n_sink, window)


def duo_decode(q_t, kv_of_tokens, t, gamma, n_sink, window, scale=None):
    """Decode output [Hq][D] of token ``t``.

    q_t[Hq][D] is the token's query; gamma[Hkv] the head kinds (1 retrieval, 0
    streaming); ``kv_of_tokens(g, tokens)`` returns KV head g's keys and values of
    those tokens as ([n][D], [n][D]).  Each KV head attends its own token set; the
    G query heads of group g use KV head g.
    """
    q_t = np.asarray(q_t, np.float64)
    Hq, D = q_t.shape
    Hkv = len(gamma)
    G = Hq // Hkv
    out = np.empty((Hq, D), dtype=np.float64)
    for g in range(Hkv):
        toks = duo_attended_tokens(t, bool(gamma[g]), n_sink, window)
        k, v = kv_of_tokens(g, toks)
        out[g * G:(g + 1) * G] = decode_gqa(q_t[g * G:(g + 1) * G], np.asarray(k, np.float64)[None],
                                            np.asarray(v, np.float64)[None], scale)
    return out

"""StreamingLLM sink + rolling-window cache (test infrastructure only).

[KVC] section "Attention Sinks e o StreamingLLM para fluxos contínuos": the cache
is split into two contiguous partitions, the first four tokens kept fixed as
attention sinks and the most recent W tokens kept in a circular buffer, so the
cache size is constant, O(W + 4).
[SINK] section "como funciona": the four initial tokens never leave, only the
window rolls, and positions are assigned inside the cache rather than in the
original text; the worked example holds tokens [0,1,2,3,6,7,8] while decoding the
next token and uses positions 0..7.  With RoPE this means keys are cached
before rotation and rotated at every step.

Readings:
* The window count W includes the token being decoded: a token's K/V are
  written into the cache (evicting the oldest window entry when full) before
  its query attends, so the query attends itself.  In the worked example this
  is n_sink = 4, W = 4: after writing token 9 the cache holds
  {0,1,2,3} + {6,7,8,9}, i.e. positions 0..7 with the query at 7.
* "Position inside the cache" is a token's rank among the cached tokens, oldest
  first.
"""
import numpy as np

from .attention import decode_gqa_rope


def retained_tokens(t: int, n_sink: int, window: int) -> np.ndarray:
    """Ascending ids of the tokens cached right after token ``t`` (0-based) was written."""
    if t < 0:
        raise ValueError("t must be >= 0")
    sinks = np.arange(0, min(n_sink, t + 1), dtype=np.int64)
    recent = np.arange(max(n_sink, t - window + 1), t + 1, dtype=np.int64)
    return np.concatenate([sinks, recent])


def in_cache_positions(tokens) -> np.ndarray:
    """Position of each cached token = number of cached tokens older than it."""
    tokens = np.asarray(tokens, dtype=np.int64)
    return np.array([int(np.sum(tokens < a)) for a in tokens], dtype=np.int64)


def ring_slot(token: int, n_sink: int, window: int) -> int:
    """Buffer slot of a token: sinks fill slots 0..n_sink-1; later tokens enter a
    circular buffer of ``window`` slots after them in arrival order."""
    if token < n_sink:
        return int(token)
    return int(n_sink + (token - n_sink) % window)


def streaming_decode(q_t, kv_of_tokens, t, n_sink, window, base, scale=None, pairs="half"):
    """Decode output of token ``t`` over a sink + window cache.

    q_t[Hq][D] is the token's query; ``kv_of_tokens(tokens)`` returns the
    un-rotated keys and values of those tokens as ([Hkv][n][D], [Hkv][n][D]).
    ``base=None`` attends without any rotation.
    """
    tokens = retained_tokens(t, n_sink, window)
    pos = in_cache_positions(tokens)
    k, v = kv_of_tokens(tokens)
    if base is None:
        from .attention import decode_gqa

        return decode_gqa(np.asarray(q_t, np.float64), k, v, scale)
    q_pos = pos[list(tokens).index(t)]
    return decode_gqa_rope(q_t, k, v, q_pos, pos, base, scale, pairs)

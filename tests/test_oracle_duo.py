"""Pins of oracle.duo_decode ([KVC] "Decomposição funcional com o DuoAttention")."""
import collections

import numpy as np
import pytest

import oracle


def _seq(T, Hq, Hkv, D, seed):
    rng = np.random.default_rng(seed)
    return (rng.standard_normal((T, Hq, D)), rng.standard_normal((T, Hkv, D)), rng.standard_normal((T, Hkv, D)))


def _kv(K, V):
    return lambda g, toks: (K[toks, g], V[toks, g])


def test_retrieval_heads_equal_full_causal_attention():
    """All heads retrieval: every decode step equals the last row of exact causal
    attention over the prefix (computed as a masked score matrix)."""
    T, Hq, Hkv, D = 40, 4, 2, 8
    Q, K, V = _seq(T, Hq, Hkv, D, 1)
    full = oracle.causal_attention(Q, K, V, np.arange(T))
    for t in (0, 5, 39):
        got = oracle.duo_decode(Q[t], _kv(K, V), t, [1, 1], n_sink=4, window=8)
        np.testing.assert_allclose(got, full[t], rtol=1e-12, atol=1e-12)


def test_streaming_heads_equal_attention_over_a_literal_deque():
    """Streaming heads: the attended set is the 4 sinks plus a bounded deque of the
    most recent tokens, simulated literally; attention over that set by brute force."""
    T, Hq, Hkv, D, S, W = 30, 2, 1, 8, 4, 6
    Q, K, V = _seq(T, Hq, Hkv, D, 2)
    dq = collections.deque(maxlen=W)
    for t in range(T):
        if t >= S:
            dq.append(t)
        toks = list(range(min(S, t + 1))) + list(dq)
        got = oracle.duo_decode(Q[t], _kv(K, V), t, [0], n_sink=S, window=W)
        x = np.array([[Q[t, h] @ K[j, 0] for j in toks] for h in range(Hq)]) / np.sqrt(D)
        p = np.exp(x - x.max(axis=1, keepdims=True))
        p /= p.sum(axis=1, keepdims=True)
        want = p @ V[toks, 0]
        np.testing.assert_allclose(got, want, rtol=1e-12, atol=1e-12)


def test_mixed_heads_are_independent_and_reduce_to_each_kind():
    """A mixed layer is head-wise the all-retrieval or all-streaming result; before
    the window fills both kinds agree."""
    T, Hq, Hkv, D, S, W = 50, 6, 3, 8, 4, 10
    Q, K, V = _seq(T, Hq, Hkv, D, 3)
    gamma = [1, 0, 1]
    for t in (3, 13, 14, 49):
        mixed = oracle.duo_decode(Q[t], _kv(K, V), t, gamma, S, W)
        ret = oracle.duo_decode(Q[t], _kv(K, V), t, [1, 1, 1], S, W)
        stm = oracle.duo_decode(Q[t], _kv(K, V), t, [0, 0, 0], S, W)
        for g in range(Hkv):
            want = ret if gamma[g] else stm
            np.testing.assert_array_equal(mixed[2 * g:2 * g + 2], want[2 * g:2 * g + 2])
        if t + 1 <= S + W:
            np.testing.assert_allclose(stm, ret, rtol=1e-12, atol=1e-12)
    assert not np.allclose(oracle.duo_decode(Q[49], _kv(K, V), 49, [0, 0, 0], S, W),
                           oracle.duo_decode(Q[49], _kv(K, V), 49, [1, 1, 1], S, W))


def test_attended_sets():
    assert list(oracle.duo_attended_tokens(9, True, 4, 4)) == list(range(10))
    assert list(oracle.duo_attended_tokens(9, False, 4, 4)) == [0, 1, 2, 3, 6, 7, 8, 9]
    assert len(oracle.duo_attended_tokens(100000, False, 4, 64)) == 68  # the page's 4 sinks + 64 local

"""Pins of the oracle's sink + window cache (CPU only)."""
import collections
import json
import os

import numpy as np
import pytest

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_worked_example_positions_inside_cache():
    with open(os.path.join(GOLDEN, "in_cache_positions_example.json")) as f:
        g = json.load(f)
    before = g["cached_tokens_before_decoding"]
    t = max(before) + 1  # "decoding the next token"
    toks = oracle.retained_tokens(t, n_sink=4, window=4)
    assert list(toks[:-1]) == before and toks[-1] == t
    pos = oracle.in_cache_positions(toks)
    assert list(pos) == g["positions_used"]
    assert list(pos) != g["positions_never_used"]
    assert pos[-1] == 7  # the query's own position


def _simulate(T, S, W):
    """Literal simulation: sinks list + a bounded deque for the window."""
    sinks, win = [], collections.deque(maxlen=W)
    states = []
    for t in range(T):
        if len(sinks) < S:
            sinks.append(t)
        else:
            win.append(t)  # deque drops the oldest entry when full
        states.append(sinks + list(win))
    return states


@pytest.mark.parametrize("S,W", [(4, 4), (4, 60), (0, 5), (1, 1), (3, 7)])
def test_retained_tokens_match_literal_simulation(S, W):
    states = _simulate(150, S, W)
    for t, st in enumerate(states):
        assert list(oracle.retained_tokens(t, S, W)) == st
        assert len(st) == min(t + 1, S + W)  # constant O(W + S) once full


def _ring_slots(T, S, W):
    """Literal circular buffer: a write pointer that wraps inside the window slots."""
    slot_of, ptr = [], 0
    for t in range(T):
        if t < S:
            slot_of.append(t)
        else:
            slot_of.append(S + ptr)
            ptr = (ptr + 1) % W
    return slot_of


@pytest.mark.parametrize("S,W", [(4, 60), (4, 2044), (0, 7), (4, 1)])
def test_ring_slot_matches_pointer_simulation(S, W):
    sim = _ring_slots(20000, S, W)
    for t in range(0, 20000, 7):
        assert oracle.ring_slot(t, S, W) == sim[t]


def test_ring_slot_long_streams_and_int64():
    # 4 million tokens (KVC: StreamingLLM sustains more than 4M tokens) and beyond int32
    S, W = 4, 2044
    for t in [4_000_000, 2**31 + 5, 2**40 + 3]:
        s = oracle.ring_slot(t, S, W)
        assert S <= s < S + W and (s - S) == (t - S) % W
    # every slot of the current cache holds a distinct retained token
    t = 4_000_000
    toks = oracle.retained_tokens(t, S, W)
    slots = [oracle.ring_slot(a, S, W) for a in toks]
    assert sorted(slots) == list(range(S + W))


def _kv(rng, T, Hkv, D):
    return rng.standard_normal((T, Hkv, D)), rng.standard_normal((T, Hkv, D))


def test_streaming_equals_full_causal_attention_before_eviction():
    # while nothing is evicted, decode over the cache is exact causal attention at the
    # original positions (KVL "01 · Conceito"), computed here by a separate full-matrix path
    rng = np.random.default_rng(10)
    T, Hq, Hkv, D, S, W = 40, 4, 1, 64, 4, 60
    Q = rng.standard_normal((T, Hq, D))
    K, V = _kv(rng, T, Hkv, D)
    full = oracle.causal_attention(Q, K, V, np.arange(T), base=10000.0)
    lookup = lambda toks: (K[toks].transpose(1, 0, 2), V[toks].transpose(1, 0, 2))
    for t in range(T):
        o = oracle.streaming_decode(Q[t], lookup, t, S, W, 10000.0)
        np.testing.assert_allclose(o, full[t], rtol=0, atol=1e-12)


@pytest.mark.parametrize("S,W", [(4, 8), (0, 6), (2, 3)])
def test_streaming_after_eviction_equals_attention_over_compacted_sequence(S, W):
    # positions inside the cache: decoding token t is the last row of causal attention over
    # the retained tokens laid out contiguously at positions 0..n-1 (SINK "como funciona")
    rng = np.random.default_rng(11)
    T, Hq, Hkv, D = 50, 6, 2, 32
    Q = rng.standard_normal((T, Hq, D))
    K, V = _kv(rng, T, Hkv, D)
    lookup = lambda toks: (K[toks].transpose(1, 0, 2), V[toks].transpose(1, 0, 2))
    for t in [S + W, S + W + 1, 23, T - 1]:
        toks = oracle.retained_tokens(t, S, W)
        full = oracle.causal_attention(Q[toks], K[toks], V[toks], np.arange(len(toks)), base=500.0)
        o = oracle.streaming_decode(Q[t], lookup, t, S, W, 500.0)
        np.testing.assert_allclose(o, full[-1], rtol=0, atol=1e-12)
        # and, once the retained ids have a gap, it differs from rotating at the ids
        if S > 0 and toks[S] > S:
            wrong = oracle.causal_attention(Q[toks], K[toks], V[toks], toks, base=500.0)
            assert np.max(np.abs(wrong[-1] - o)) > 1e-6


def test_window_without_sinks_keeps_only_recent():
    toks = oracle.retained_tokens(100, 0, 10)
    assert list(toks) == list(range(91, 101))

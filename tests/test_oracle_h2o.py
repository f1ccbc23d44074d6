"""Pins of the oracle's H2O budgeted decode (CPU only).

Includes a second, independently written simulation (a full matrix over all
positions with an alive mask) that must agree with the oracle's set-based one.
"""
import numpy as np
import pytest
import scipy.special

import oracle


def _stream(seed, T, G, D):
    rng = np.random.default_rng(seed)
    return rng.standard_normal((T, G, D)), rng.standard_normal((T, D)), rng.standard_normal((T, D))


def _mask_simulation(Q, K, V, budget, n_recent, scale):
    """Alive mask over every position; scores in a dense array; argmin by lexsort."""
    T, G, D = Q.shape
    alive = np.zeros(T, dtype=bool)
    s = np.zeros(T)
    outs, evicted = [], []
    for t in range(T):
        ev = None
        if alive.sum() == budget:
            cand = np.flatnonzero(alive & (np.arange(T) <= t - n_recent))
            s32 = s[cand].astype(np.float32)
            order = np.lexsort((-cand, s32))  # primary: s (ascending), then newer first
            ev = int(cand[order[0]])
            alive[ev] = False
            s[ev] = 0.0
        alive[t] = True
        idx = np.flatnonzero(alive)
        logits = (Q[t] @ K[idx].T) * scale  # [G][n]
        P = scipy.special.softmax(logits, axis=1)
        outs.append(P @ V[idx])
        s[idx] += P.sum(axis=0)
        evicted.append(ev)
    return np.array(outs), evicted


@pytest.mark.parametrize("budget,n_recent,G", [(8, 3, 1), (12, 4, 4), (6, 1, 2), (5, 5, 3)])
def test_two_independent_simulations_agree(budget, n_recent, G):
    T, D = 40, 16
    Q, K, V = _stream(budget * 10 + G, T, G, D)
    head = oracle.H2OHead(budget, n_recent)
    outs, evs = [], []
    for t in range(T):
        o, ev = head.step(t, Q[t], K[t], V[t])
        outs.append(o)
        evs.append(ev)
    ref_out, ref_ev = _mask_simulation(Q, K, V, budget, n_recent, 1 / np.sqrt(D))
    assert evs == ref_ev
    np.testing.assert_allclose(np.array(outs), ref_out, atol=1e-13)


def test_scores_gain_G_per_step():
    G, D, T = 3, 8, 20
    Q, K, V = _stream(1, T, G, D)
    head = oracle.H2OHead(6, 2)
    for t in range(T):
        before = sum(head.s)
        lost = head.s[head.victim_index(t)] if len(head.pos) == head.budget else 0.0
        head.step(t, Q[t], K[t], V[t])
        assert abs((sum(head.s) - (before - lost)) - G) < 1e-12
    assert len(head.pos) == 6


def test_budget_above_stream_is_full_attention():
    G, D, T = 2, 16, 25
    Q, K, V = _stream(2, T, G, D)
    head = oracle.H2OHead(64, 4)
    for t in range(T):
        o, ev = head.step(t, Q[t], K[t], V[t])
        assert ev is None
        ref = oracle.decode_gqa(Q[t], K[None, : t + 1], V[None, : t + 1])
        np.testing.assert_allclose(o, ref, atol=1e-13)


def test_all_recent_budget_is_a_sliding_window():
    # n_recent == budget: only the oldest token is ever a candidate
    G, D, T, B = 1, 8, 30, 5
    Q, K, V = _stream(3, T, G, D)
    head = oracle.H2OHead(B, B)
    for t in range(T):
        o, ev = head.step(t, Q[t], K[t], V[t])
        assert ev == (t - B if t >= B else None)
        assert head.pos == list(range(max(0, t - B + 1), t + 1))


def test_victim_ties_evict_the_newer_token():
    head = oracle.H2OHead(3, 1, positions=[0, 1, 2], keys=np.zeros((3, 4)), values=np.zeros((3, 4)),
                          scores=[0.5, 0.25, 0.25])
    assert head.pos[head.victim_index(3)] == 2
    head.s = [0.1, 0.25, 0.25]
    assert head.pos[head.victim_index(3)] == 0
    # the recent partition includes the new token: with n_recent = 2 token 2 is protected at t = 3
    head2 = oracle.H2OHead(3, 2, positions=[0, 1, 2], keys=np.zeros((3, 4)), values=np.zeros((3, 4)),
                           scores=[0.5, 0.25, 0.0])
    assert head2.pos[head2.victim_index(3)] == 1


def test_prompt_selection_pins():
    T, G, D = 20, 2, 8
    rng = np.random.default_rng(4)
    Q, K = rng.standard_normal((T, G, D)), rng.standard_normal((T, D))
    keep, s = oracle.h2o_prompt_select(Q, K, budget=T, n_recent=2)
    assert list(keep) == list(range(T))
    np.testing.assert_allclose(s.sum(), G * T, atol=1e-11)  # each causal row sums to one
    # column sums of the causal attention matrices, written with library softmax
    ref = np.zeros(T)
    for h in range(G):
        L = (Q[:, h] @ K.T) / np.sqrt(D)
        L[np.triu_indices(T, 1)] = -np.inf
        ref += scipy.special.softmax(L, axis=1).sum(axis=0)
    np.testing.assert_allclose(s, ref, atol=1e-12)
    keep, _ = oracle.h2o_prompt_select(Q, K, budget=8, n_recent=3)
    assert list(keep[-3:]) == [17, 18, 19] and len(keep) == 8
    top = np.lexsort((np.arange(17), -ref[:17].astype(np.float32)))[:5]
    assert sorted(top) == list(keep[:5])

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
            order = np.lexsort((-cand, s[cand]))  # primary: s (ascending), then newer first
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
    top = np.lexsort((np.arange(17), -ref[:17]))[:5]
    assert sorted(top) == list(keep[:5])


# ---------------------------------------------------------------- block-level eviction
def _bstream(T, G, D, seed):
    rng = np.random.default_rng(seed)
    return rng.standard_normal((T, G, D)), rng.standard_normal((T, D)), rng.standard_normal((T, D))


def test_block_size_one_is_token_level_h2o():
    """With blocks of one token, block eviction is H2O's token eviction (no recent block
    can be a candidate either way)."""
    T, G, D, C, R = 60, 2, 8, 12, 3
    Q, K, V = _bstream(T, G, D, 11)
    a, b = oracle.H2OHead(C, R), oracle.H2OBlockHead(C, 1, R)
    for t in range(T):
        oa, ea = a.step(t, Q[t], K[t], V[t])
        ob, eb = b.step(t, Q[t], K[t], V[t])
        np.testing.assert_allclose(oa, ob, rtol=1e-12, atol=1e-12)
        assert (ea is None and eb is None) or [ea] == eb
        assert sorted(a.pos) == sorted(b.tokens())


def test_block_eviction_frees_whole_blocks_by_summed_score():
    """Literal pin of the rule: at each boundary with the budget full, the freed block is
    the candidate with the smallest sum of its tokens' s (ties: newer block),
    computed here from a separately tracked per-token score table."""
    T, G, D, NB, BS, R = 120, 2, 8, 4, 8, 5
    Q, K, V = _bstream(T, G, D, 12)
    head = oracle.H2OBlockHead(NB, BS, R)
    s_tab = {}  # position -> accumulated weight, tracked independently
    for t in range(T):
        before = [list(b["pos"]) for b in head.blocks]
        out, freed = head.step(t, Q[t], K[t], V[t])
        toks = head.tokens()
        assert len(toks) <= NB * BS and len(head.blocks) <= NB
        if freed is not None:
            cands = [blk for blk in before if max(blk) <= t - R]
            want = min(cands, key=lambda blk: (sum(s_tab[p] for p in blk), -max(blk)))
            assert freed == want and len(freed) == BS
            for p in freed:
                del s_tab[p]
        # brute-force attention over the cached tokens and the score update
        Ks, Vs = K[toks], V[toks]
        w = np.zeros(len(toks))
        for h in range(G):
            x = Ks @ Q[t, h] / np.sqrt(D)
            a = np.exp(x - x.max())
            a /= a.sum()
            np.testing.assert_allclose(out[h], a @ Vs, rtol=1e-12, atol=1e-12)
            w += a
        s_tab[t] = 0.0
        for p, x in zip(toks, w):
            s_tab[p] += x
    # blocks fill in arrival order; once the budget is reached every boundary frees one block
    assert len(head.blocks) == NB


def test_block_recent_protection():
    """The blocks holding any of the n_recent newest tokens are never freed."""
    T, G, D, NB, BS, R = 90, 1, 4, 3, 8, 9  # 9 recent tokens span two blocks at each boundary
    Q, K, V = _bstream(T, G, D, 13)
    head = oracle.H2OBlockHead(NB, BS, R)
    for t in range(T):
        _, freed = head.step(t, Q[t], K[t], V[t])
        if freed is not None:
            assert max(freed) <= t - R


def test_prompt_scores_equal_a_scalar_brute_force():
    """s_j written out element by element with math.exp (no arrays, no softmax helper):
    for every head h and row t >= j, exp(x_tj) / sum_{i <= t} exp(x_ti), summed."""
    import math

    rng = np.random.default_rng(21)
    T, G, D = 7, 3, 4
    Q, K = rng.standard_normal((T, G, D)), rng.standard_normal((T, D))
    sc = 0.7
    want = [0.0] * T
    for h in range(G):
        for t in range(T):
            x = [sc * sum(float(Q[t, h, d]) * float(K[i, d]) for d in range(D)) for i in range(t + 1)]
            den = sum(math.exp(v) for v in x)
            for j in range(t + 1):
                want[j] += math.exp(x[j]) / den
    got = oracle.h2o_prompt_scores(Q, K, scale=sc, rows_per_group=2)  # row groups split the rows
    np.testing.assert_allclose(got, want, rtol=1e-13, atol=0)
    np.testing.assert_allclose(oracle.h2o_prompt_scores(Q, K, scale=sc, rows_per_group=T), want, rtol=1e-13, atol=0)
    # rows from t = 4 on: exact for keys 4.. (no earlier row sees them)
    tail = oracle.h2o_prompt_scores(Q, K, scale=sc, rows_per_group=2, first_row=4)
    np.testing.assert_allclose(tail[4:], want[4:], rtol=1e-13, atol=0)
    assert np.all(tail[:4] < np.array(want[:4]))

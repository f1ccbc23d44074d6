"""Planted mistakes in the oracle must be caught by its pins (CPU only).

Each mutant replaces one oracle function with a plausibly wrong variant (a wrong
sign, index, exponent, tie rule or step order); the test runs the pins of that
function under the mutant and requires at least one of them to fail.
"""
import numpy as np
import pytest

import oracle
import oracle.attention as att
import oracle.h2o as h2o
import oracle.rope as rope
import oracle.snapkv as snap
import oracle.streaming as stream
from tests import test_oracle_core as core
from tests import test_oracle_h2o as th2o
from tests import test_oracle_snapkv as tsnap
from tests import test_oracle_streaming as tstream


def _rope_variant(sign=1.0, exp=2.0, pairs_default="half"):
    def apply(x, pos, base, pairs=pairs_default):
        x = np.asarray(x, np.float64)
        D = x.shape[-1]
        f = float(base) ** (-exp * np.arange(D // 2) / D)
        phi = np.asarray(pos, np.float64)[..., None] * f
        c, s = np.cos(phi), sign * np.sin(phi)
        if pairs == "half":
            a, b = x[..., : D // 2], x[..., D // 2:]
        else:
            a, b = x[..., 0::2], x[..., 1::2]
        out = np.empty(np.broadcast_shapes(x.shape, phi.shape[:-1] + (D,)))
        if pairs == "half":
            out[..., : D // 2], out[..., D // 2:] = a * c - b * s, a * s + b * c
        else:
            out[..., 0::2], out[..., 1::2] = a * c - b * s, a * s + b * c
        return out

    def inv_freq(D, base):
        return float(base) ** (-exp * np.arange(D // 2) / D)

    return apply, inv_freq


def _patch_rope(mp, apply, inv_freq):
    for mod in (oracle, rope, att):
        mp.setattr(mod, "apply_rope", apply, raising=False)
    mp.setattr(oracle, "rope_inv_freq", inv_freq)
    mp.setattr(rope, "rope_inv_freq", inv_freq)


def _gqa_modulo(q, k, v, scale=None, return_probs=False):
    Hq, D = q.shape
    Hkv = k.shape[0]
    if Hq % Hkv:
        raise ValueError
    sc = 1 / np.sqrt(D) if scale is None else scale
    out = np.stack([att.attend_one(q[h], k[h % Hkv], v[h % Hkv], sc)[0] for h in range(Hq)])
    return out


def _scale_over_d(q, k, v, scale=None, return_probs=False):
    return att.__dict__["_orig_decode"](q, k, v, 1.0 / q.shape[1] if scale is None else scale)


def _retained_excluding_current(t, n_sink, window):
    S, W = n_sink, window
    sinks = np.arange(0, min(S, t + 1))
    recent = np.arange(max(S, t - W), t + 1)
    return np.concatenate([sinks, recent]).astype(np.int64)


def _positions_are_ids(tokens):
    return np.asarray(tokens, dtype=np.int64)


def _obs_mask_off_by_one(q_obs, k, scale=None):
    L, D = q_obs.shape
    N = k.shape[0]
    A = np.zeros((L, N))
    for t in range(L):
        last = min(N - 1, N - L + t + 1)
        A[t, : last + 1] = att.softmax((k[: last + 1] @ q_obs[t]) / np.sqrt(D))
    return A


def _pool_inrange_divisor(s, kernel_size, mode="avg"):
    s = np.asarray(s, np.float64)
    r = kernel_size // 2
    return np.array([s[max(0, i - r): i + r + 1].mean() for i in range(len(s))])


def _topk_ties_high(S, k):
    S = np.asarray(S, np.float64)
    order = sorted(range(len(S)), key=lambda i: (-float(S[i]), -i))
    return np.array(sorted(order[:k]), dtype=np.int64)


def _victim_ties_old(self, t):
    c = [i for i, p in enumerate(self.pos) if p <= t - self.n_recent]
    return min(c, key=lambda i: (self.s[i], self.pos[i]))


def _victim_recent_excludes_new(self, t):
    c = [i for i, p in enumerate(self.pos) if p < t - self.n_recent]
    if not c:
        c = list(range(len(self.pos)))
    return min(c, key=lambda i: (self.s[i], -self.pos[i]))


def _run_all(tests):
    failures = 0
    for fn, args in tests:
        try:
            fn(*args)
        except (AssertionError, ValueError, IndexError):
            failures += 1
    return failures


ROPE_PINS = [(core.test_rope_two_dims_is_textbook_plane_rotation, ()),
             (core.test_rope_pairs_and_frequencies_half_layout, ()),
             (core.test_rope_inv_freq_closed_form, ()),
             (tstream.test_streaming_after_eviction_equals_attention_over_compacted_sequence, (4, 8))]


@pytest.mark.parametrize("variant", [dict(sign=-1.0), dict(exp=1.0), dict(pairs_default="interleaved")])
def test_rope_mutants_are_caught(monkeypatch, variant):
    _patch_rope(monkeypatch, *_rope_variant(**variant))
    assert _run_all(ROPE_PINS) >= 1


def test_gqa_grouping_mutant_is_caught(monkeypatch):
    monkeypatch.setattr(att, "decode_gqa", _gqa_modulo)
    monkeypatch.setattr(oracle, "decode_gqa", _gqa_modulo)
    assert _run_all([(core.test_gqa_equals_mha_with_repeated_kv, ())]) == 1


def test_scale_mutant_is_caught(monkeypatch):
    monkeypatch.setitem(att.__dict__, "_orig_decode", att.decode_gqa)
    monkeypatch.setattr(oracle, "decode_gqa", _scale_over_d)
    assert _run_all([(core.test_two_keys_logistic_weights_and_default_scale, ())]) == 1


@pytest.mark.parametrize("which", ["window", "positions"])
def test_streaming_mutants_are_caught(monkeypatch, which):
    if which == "window":
        monkeypatch.setattr(stream, "retained_tokens", _retained_excluding_current)
        monkeypatch.setattr(oracle, "retained_tokens", _retained_excluding_current)
    else:
        monkeypatch.setattr(stream, "in_cache_positions", _positions_are_ids)
        monkeypatch.setattr(oracle, "in_cache_positions", _positions_are_ids)
    pins = [(tstream.test_worked_example_positions_inside_cache, ()),
            (tstream.test_retained_tokens_match_literal_simulation, (4, 4))]
    assert _run_all(pins) >= 1


def test_snapkv_mutants_are_caught(monkeypatch):
    monkeypatch.setattr(snap, "observation_attention", _obs_mask_off_by_one)
    monkeypatch.setattr(oracle, "observation_attention", _obs_mask_off_by_one)
    assert _run_all([(tsnap.test_observation_rows_are_causal_softmax_rows, ()),
                     (tsnap.test_whole_prompt_as_window_is_textbook_causal_attention, ())]) >= 1
    monkeypatch.undo()
    monkeypatch.setattr(oracle, "pool1d", _pool_inrange_divisor)
    assert _run_all([(tsnap.test_avg_pool_matches_numpy_convolve, ())]) == 1
    monkeypatch.undo()
    monkeypatch.setattr(oracle, "select_topk", _topk_ties_high)
    assert _run_all([(tsnap.test_topk_matches_brute_force_over_subsets, (s,)) for s in range(6)]) >= 1


@pytest.mark.parametrize("mut", [_victim_ties_old, _victim_recent_excludes_new])
def test_h2o_mutants_are_caught(monkeypatch, mut):
    monkeypatch.setattr(h2o.H2OHead, "victim_index", mut)
    pins = [(th2o.test_victim_ties_evict_the_newer_token, ()),
            (th2o.test_two_independent_simulations_agree, (8, 3, 1)),
            (th2o.test_two_independent_simulations_agree, (12, 4, 4))]
    assert _run_all(pins) >= 1


def _prompt_scores_mask_diagonal(Q, K, scale=None, rows_per_group=256):
    """Mutant: a row does not see its own key (strict causal mask)."""
    Q, K = np.asarray(Q, np.float64), np.asarray(K, np.float64)
    T, G, D = Q.shape
    sc = 1.0 / np.sqrt(D) if scale is None else float(scale)
    s = np.zeros(T)
    for h in range(G):
        X = (Q[:, h] @ K.T) * sc
        X[np.arange(T)[None, :] >= np.arange(T)[:, None]] = -np.inf
        X[0, 0] = 0.0  # row 0 would be empty
        s += att.softmax(X, axis=1).sum(axis=0)
    return s


def _prompt_scores_one_head(Q, K, scale=None, rows_per_group=256):
    """Mutant: only the first query head of the group is summed."""
    return h2o.__dict__["_orig_prompt_scores"](np.asarray(Q)[:, :1], K, scale, rows_per_group)


@pytest.mark.parametrize("mut", [_prompt_scores_mask_diagonal, _prompt_scores_one_head])
def test_h2o_prompt_score_mutants_are_caught(monkeypatch, mut):
    monkeypatch.setitem(h2o.__dict__, "_orig_prompt_scores", h2o.h2o_prompt_scores)
    monkeypatch.setattr(h2o, "h2o_prompt_scores", mut)
    monkeypatch.setattr(oracle, "h2o_prompt_scores", mut)
    assert _run_all([(th2o.test_prompt_scores_equal_a_scalar_brute_force, ())]) == 1

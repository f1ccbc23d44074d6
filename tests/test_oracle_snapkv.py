"""Pins of the oracle's SnapKV compression (CPU only)."""
import itertools

import numpy as np
import pytest
import scipy.ndimage
import scipy.special

import oracle
from oracle.snapkv import raw_scores


def _rand(seed, L, N, D):
    rng = np.random.default_rng(seed)
    return rng.standard_normal((L, D)), rng.standard_normal((N, D)), rng.standard_normal((N, D))


def test_observation_rows_are_causal_softmax_rows():
    q, k, _ = _rand(0, 4, 37, 16)
    A = oracle.observation_attention(q, k)
    np.testing.assert_allclose(A.sum(axis=1), 1.0, atol=1e-13)
    N, L = 37, 4
    for t in range(L):
        assert np.all(A[t, N - L + t + 1:] == 0)  # keys after the row's own token are masked
        assert np.all(A[t, : N - L + t + 1] > 0)
    # the mean over rows of unit rows sums to one over all N keys
    np.testing.assert_allclose(raw_scores(q, k).sum(), 1.0, atol=1e-13)


def test_whole_prompt_as_window_is_textbook_causal_attention():
    # L_obs = N: the rows are the full causal attention matrix of the prompt
    q, k, _ = _rand(1, 9, 9, 8)
    logits = (q @ k.T) / np.sqrt(8)
    logits[np.triu_indices(9, 1)] = -np.inf
    ref = scipy.special.softmax(logits, axis=1)
    np.testing.assert_allclose(oracle.observation_attention(q, k), ref, atol=1e-14)
    np.testing.assert_allclose(raw_scores(q, k), ref.mean(axis=0), atol=1e-14)


def test_avg_pool_matches_numpy_convolve():
    s = np.random.default_rng(2).random(101)
    for ks in [1, 3, 5, 7]:
        np.testing.assert_allclose(oracle.pool1d(s, ks), np.convolve(s, np.ones(ks) / ks, mode="same"),
                                   atol=1e-15)


def test_max_pool_matches_scipy_filter_for_nonnegative_scores():
    s = np.random.default_rng(3).random(64)
    ref = scipy.ndimage.maximum_filter1d(s, size=5, mode="constant", cval=0.0)
    np.testing.assert_array_equal(oracle.pool1d(s, 5, "max"), ref)


def test_pool_rejects_even_kernel():
    with pytest.raises(ValueError):
        oracle.pool1d(np.ones(4), 4)


def _dominates(S, i, j):
    return (S[i] > S[j]) or (S[i] == S[j] and i < j)


@pytest.mark.parametrize("seed", range(6))
def test_topk_matches_brute_force_over_subsets(seed):
    rng = np.random.default_rng(seed)
    n, k = 9, 4
    S = rng.integers(0, 4, n).astype(np.float64) / 3.0  # many exact ties
    winners = [set(c) for c in itertools.combinations(range(n), k)
               if all(_dominates(S, i, j) for i in c for j in set(range(n)) - set(c))]
    assert len(winners) == 1
    got = oracle.select_topk(S, k)
    assert set(got) == winners[0] and list(got) == sorted(got)


def test_topk_ranks_exact_scores():
    # two scores equal in float32 but not in float64: the higher exact score wins; an
    # exact tie keeps the lower index
    a = 1.0
    b = 1.0 + 2.0**-30
    assert np.float32(a) == np.float32(b)
    assert list(oracle.select_topk(np.array([a, b]), 1)) == [1]
    assert list(oracle.select_topk(np.array([b, b]), 1)) == [0]


def test_equal_keys_keep_lowest_indices():
    # identical keys: every prefix key gets the same pooled score away from the edges
    D, N, L, k = 8, 40, 4, 10
    rng = np.random.default_rng(4)
    key = rng.standard_normal(D)
    K = np.repeat(key[None], N, axis=0)
    q = rng.standard_normal((L, D))
    idx, *_ = oracle.snapkv_compress(q, K, K, k, kernel_size=1)
    assert list(idx[:k]) == list(range(k))


def test_single_row_single_kernel_is_topk_of_one_attention_row():
    D, N, k = 16, 50, 7
    q, K, V = _rand(5, 1, N, D)
    idx, Ko, Vo, S = oracle.snapkv_compress(q, K, V, k, kernel_size=1)
    row = scipy.special.softmax((K @ q[0]) / np.sqrt(D))  # L_obs = 1 sees every key
    order = np.argsort(-row[: N - 1], kind="stable")[:k]
    assert list(idx[:k]) == sorted(order) and idx[-1] == N - 1
    np.testing.assert_allclose(S, row[: N - 1], atol=1e-15)


def test_compress_output_layout():
    L, N, D, k = 4, 64, 16, 10
    q, K, V = _rand(6, L, N, D)
    idx, Ko, Vo, S = oracle.snapkv_compress(q, K, V, k)
    assert idx.shape == (k + L,) and S.shape == (N - L,)
    assert list(idx[k:]) == list(range(N - L, N))  # observation window always kept, last
    assert np.all(np.diff(idx) > 0) and idx[k - 1] < N - L
    np.testing.assert_array_equal(Ko, K[idx])
    np.testing.assert_array_equal(Vo, V[idx])
    # every kept prefix score is >= every dropped one
    dropped = np.setdiff1d(np.arange(N - L), idx[:k])
    assert S[idx[:k]].min() >= S[dropped].max()


def test_keep_fraction_of_the_32k_example():
    # SnapKV keeps 16% of the cache at 32k tokens (KVC, SnapKV section)
    assert int(np.floor(0.16 * 32768 + 0.5)) == 5243

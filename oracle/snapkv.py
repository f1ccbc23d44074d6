"""SnapKV prefill compression in float64 (test infrastructure only).

[KVC] section "SnapKV e a seleção de contexto no prefill": at the end of prefill,
before generation, the cache of each head is compressed in four steps:
  1. an observation window of the last L_obs prompt queries gives an attention
     matrix A[h] of L_obs rows over the N prompt keys;
  2. the raw score of key i is the mean of A[h, t, i] over the L_obs rows;
  3. a 1-D pooling of kernel size 5 smooths the scores (neighbours of a
     high-attention token carry context);
  4. each head keeps the positions with the highest smoothed score.
The same section quotes keeping 16% of the cache at 32k tokens.

Readings (the pages leave these open):
* Each observation row is a causal softmax over the prompt: row t (0-based)
  is the query of prompt token N - L_obs + t and sees keys 0 .. N - L_obs + t.
* Only the prefix [0, N - L_obs) competes in the top-k; the observation window
  itself is always kept and appended after the selected positions.
* Pooling is an average over a centred window of ``kernel_size`` with zero
  padding and divisor ``kernel_size`` at every position, over the prefix scores
  only; ``mode="max"`` takes the maximum over the in-range entries instead.
* The top-k ranks by (higher score, lower index) on the exact (float64) pooled
  scores, and the kept positions are returned in ascending order.  An
  implementation that decides on rounded scores can differ only where two scores
  agree to within its rounding (a near-tie).
"""
import numpy as np

from .attention import softmax


def observation_attention(q_obs: np.ndarray, k: np.ndarray, scale=None) -> np.ndarray:
    """A[L_obs][N]: causal softmax rows of the observation-window queries."""
    q_obs = np.asarray(q_obs, np.float64)
    k = np.asarray(k, np.float64)
    L, D = q_obs.shape
    N = k.shape[0]
    sc = 1.0 / np.sqrt(D) if scale is None else float(scale)
    A = np.zeros((L, N), dtype=np.float64)
    for t in range(L):
        last = N - L + t  # the row's own prompt position
        A[t, : last + 1] = softmax((k[: last + 1] @ q_obs[t]) * sc)
    return A


def raw_scores(q_obs, k, scale=None) -> np.ndarray:
    """Step 2: s[i] = mean over observation rows of A[t, i], for all N keys."""
    return observation_attention(q_obs, k, scale).mean(axis=0)


def pool1d(s: np.ndarray, kernel_size: int, mode: str = "avg") -> np.ndarray:
    """Step 3: centred 1-D pooling of odd ``kernel_size`` with zero padding."""
    if kernel_size < 1 or kernel_size % 2 == 0:
        raise ValueError("kernel_size must be odd and >= 1")
    s = np.asarray(s, np.float64)
    n, r = s.shape[0], kernel_size // 2
    out = np.empty(n, dtype=np.float64)
    for i in range(n):
        lo, hi = max(0, i - r), min(n, i + r + 1)
        if mode == "avg":
            out[i] = s[lo:hi].sum() / kernel_size
        elif mode == "max":
            out[i] = s[lo:hi].max()
        else:
            raise ValueError(mode)
    return out


def select_topk(S: np.ndarray, k: int) -> np.ndarray:
    """Step 4: ascending indices of the ``k`` best by (higher score, lower index)."""
    S = np.asarray(S, np.float64)
    order = sorted(range(len(S)), key=lambda i: (-float(S[i]), i))
    return np.array(sorted(order[:k]), dtype=np.int64)


def snapkv_compress(q_obs, k, v, k_keep, kernel_size=5, scale=None, pool="avg"):
    """One head: returns (kept indices [k_keep + L_obs], K_out, V_out, pooled scores).

    The kept indices are the selected prefix positions (ascending) followed by
    the observation window N - L_obs .. N - 1.
    """
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    L = np.asarray(q_obs).shape[0]
    N = k.shape[0]
    if not 0 <= k_keep <= N - L:
        raise ValueError("k_keep out of range")
    s = raw_scores(q_obs, k, scale)[: N - L]
    S = pool1d(s, kernel_size, pool)
    keep = select_topk(S, k_keep)
    idx = np.concatenate([keep, np.arange(N - L, N, dtype=np.int64)])
    return idx, k[idx], v[idx], S

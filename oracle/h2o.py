"""H2O (heavy-hitter) budgeted decode in float64 (test infrastructure only).

[KVC] section "Heavy-Hitter Oracle (H2O) e a esparsidade de cauda pesada": each
cached token j carries the attention it has received summed over decode steps,
s_j = sum_t alpha_{t,j}.  When the cache reaches its budget K_budget the manager
prunes: a recent partition keeps the L_local newest tokens, a heavy-hitter
partition keeps the K_HH historical tokens with the largest s_j, and the rest is
freed.

Readings (the pages leave these open):
* Order inside a step: evict one token if the cache is at its budget, write the
  new token (s = 0), attend over the cache, then add this step's attention
  weights to every cached token's s.  The span is therefore exactly the budget
  and the new token receives its own weight in the step it arrives.
* The recent partition includes the new token: at step t the tokens with
  position > t - L_local are protected; the victim is the smallest s among the
  others (exact float64 s), ties evicting the newer token (the same order as
  SnapKV's keep rule: higher score, then lower index, is kept).
* With grouped-query attention one s is kept per KV head and is the sum of the
  weights of the G query heads that share it.
* No positional rotation is applied: cached keys are used as given.
"""
import numpy as np

from .attention import attend_one, softmax


class H2OHead:
    """The H2O cache of one (batch row, KV head) shared by G query heads."""

    def __init__(self, budget: int, n_recent: int, positions=(), keys=(), values=(), scores=()):
        if not 0 < n_recent <= budget:
            raise ValueError("need 0 < n_recent <= budget")
        self.budget, self.n_recent = int(budget), int(n_recent)
        self.pos = [int(p) for p in positions]
        self.k = [np.asarray(x, np.float64) for x in keys]
        self.v = [np.asarray(x, np.float64) for x in values]
        self.s = [float(x) for x in scores]
        if not (len(self.pos) == len(self.k) == len(self.v) == len(self.s) <= budget):
            raise ValueError("inconsistent initial state")

    def victim_index(self, t: int) -> int:
        """Entry evicted before writing token ``t`` (the cache must be full)."""
        cands = [i for i, p in enumerate(self.pos) if p <= t - self.n_recent]
        if not cands:
            raise ValueError("no eviction candidate")
        return min(cands, key=lambda i: (self.s[i], -self.pos[i]))

    def step(self, t: int, q: np.ndarray, k_t: np.ndarray, v_t: np.ndarray, scale=None):
        """Decode token ``t`` with queries q[G][D]; returns (out[G][D], evicted position or None)."""
        q = np.asarray(q, np.float64)
        evicted = None
        if len(self.pos) == self.budget:
            i = self.victim_index(t)
            evicted = self.pos[i]
            for lst in (self.pos, self.k, self.v, self.s):
                del lst[i]
        self.pos.append(int(t))
        self.k.append(np.asarray(k_t, np.float64))
        self.v.append(np.asarray(v_t, np.float64))
        self.s.append(0.0)
        K, V = np.stack(self.k), np.stack(self.v)
        sc = 1.0 / np.sqrt(q.shape[-1]) if scale is None else float(scale)
        out = np.empty((q.shape[0], V.shape[1]))
        weights = np.zeros(len(self.pos))
        for h in range(q.shape[0]):
            out[h], p = attend_one(q[h], K, V, sc)
            weights += p
        self.s = [a + b for a, b in zip(self.s, weights)]
        return out, evicted


def h2o_prompt_scores(Q, K, scale=None, rows_per_group=256, first_row=0):
    """s_j of every prompt token for one KV head: the column sums, over the G query
    heads, of the causal attention matrices A_h[t, j] = softmax over j <= t of
    scale * <Q[t, h], K[j]> (zero for j > t).  Rows are formed ``rows_per_group`` at a
    time, each row a full causal softmax, so memory stays bounded.

    With ``first_row`` > 0 only rows t >= first_row are summed: the result is then exact
    for the keys j >= first_row (no earlier row attends them) and partial before."""
    Q = np.asarray(Q, np.float64)
    K = np.asarray(K, np.float64)
    T, G, D = Q.shape
    sc = 1.0 / np.sqrt(D) if scale is None else float(scale)
    s = np.zeros(T)
    for h in range(G):
        for r0 in range(first_row, T, rows_per_group):
            r1 = min(T, r0 + rows_per_group)
            X = (Q[r0:r1, h] @ K[:r1].T) * sc  # rows r0 .. r1-1 against keys 0 .. r1-1
            X[np.arange(r1)[None, :] > np.arange(r0, r1)[:, None]] = -np.inf  # key after row
            s[:r1] += softmax(X, axis=1).sum(axis=0)
    return s


def h2o_prompt_select(Q, K, budget: int, n_recent: int, scale=None):
    """Prompt-phase selection for one KV head.

    Q[T][G][D] are the prompt queries of the G heads sharing K[T][D].  Each prompt
    token j accumulates s_j = sum over rows t >= j and heads of the causal
    attention weight; the last ``n_recent`` tokens are kept, and of the older ones
    the ``budget - n_recent`` best by (higher s, lower position).
    Returns (kept positions ascending, s of every prompt token).
    """
    s = h2o_prompt_scores(Q, K, scale)
    T = s.shape[0]
    if budget >= T:
        return np.arange(T, dtype=np.int64), s
    old = T - n_recent
    order = sorted(range(old), key=lambda j: (-float(s[j]), j))
    keep = sorted(order[: budget - n_recent]) + list(range(old, T))
    return np.array(keep, dtype=np.int64), s


class H2OBlockHead:
    """Block-level H2O cache of one (batch row, KV head): [KVC] "Implementação prática em
    vLLM e SGLang" — memory is managed in blocks of 16 or 32 tokens, a block's score is the
    sum of its tokens' accumulated attention, Score(B_k) = sum_{t in B_k} s_t, and when
    memory runs out the lowest-scoring blocks are freed whole (and reused, no copies).

    Readings:
    * The budget is ``n_blocks`` blocks of ``block_size`` tokens.  Tokens fill an open
      block in arrival order; a new block is needed when the open one is full.  While the
      budget allows, a fresh block is opened; at the budget the lowest-scoring block is
      freed first and becomes the new open block.
    * A block is an eviction candidate only if none of its tokens is among the n_recent
      newest (positions <= t - n_recent for the arriving token t, as in H2OHead).  Its
      score is the float64 sum of its tokens' s; ties free the block
      holding the newer token.
    * Step order, scores and GQA as in H2OHead.
    """

    def __init__(self, n_blocks: int, block_size: int, n_recent: int):
        if n_blocks < 2 or block_size < 1 or not 0 < n_recent <= (n_blocks - 1) * block_size:
            raise ValueError("need >= 2 blocks and 0 < n_recent <= (n_blocks - 1) * block_size")
        self.n_blocks, self.block_size, self.n_recent = int(n_blocks), int(block_size), int(n_recent)
        self.blocks = []  # each: dict(pos=[...], k=[...], v=[...], s=[...]); the last is the open block

    def load(self, positions, keys, values, scores):
        """Seed a full cache: consecutive runs of block_size entries form the blocks."""
        n = len(positions)
        if n != self.n_blocks * self.block_size:
            raise ValueError("a seeded block cache must be full")
        bs = self.block_size
        self.blocks = [dict(pos=[int(x) for x in positions[i:i + bs]],
                            k=[np.asarray(x, np.float64) for x in keys[i:i + bs]],
                            v=[np.asarray(x, np.float64) for x in values[i:i + bs]],
                            s=[float(x) for x in scores[i:i + bs]]) for i in range(0, n, bs)]

    def tokens(self):
        return [p for blk in self.blocks for p in blk["pos"]]

    def block_score(self, blk) -> float:
        return float(sum(blk["s"]))

    def victim_block(self, t: int) -> int:
        """Index of the block freed before writing token ``t`` (budget full, open block full)."""
        cands = [i for i, blk in enumerate(self.blocks) if max(blk["pos"]) <= t - self.n_recent]
        if not cands:
            raise ValueError("no eviction candidate")
        return min(cands, key=lambda i: (self.block_score(self.blocks[i]), -max(self.blocks[i]["pos"])))

    def step(self, t: int, q: np.ndarray, k_t: np.ndarray, v_t: np.ndarray, scale=None):
        """Decode token ``t`` with queries q[G][D]; returns (out[G][D], freed positions or None)."""
        q = np.asarray(q, np.float64)
        freed = None
        if not self.blocks or len(self.blocks[-1]["pos"]) == self.block_size:
            if len(self.blocks) == self.n_blocks:
                i = self.victim_block(t)
                freed = list(self.blocks[i]["pos"])
                del self.blocks[i]
            self.blocks.append(dict(pos=[], k=[], v=[], s=[]))
        blk = self.blocks[-1]
        blk["pos"].append(int(t))
        blk["k"].append(np.asarray(k_t, np.float64))
        blk["v"].append(np.asarray(v_t, np.float64))
        blk["s"].append(0.0)
        K = np.stack([x for b in self.blocks for x in b["k"]])
        V = np.stack([x for b in self.blocks for x in b["v"]])
        sc = 1.0 / np.sqrt(q.shape[-1]) if scale is None else float(scale)
        out = np.empty((q.shape[0], V.shape[1]))
        weights = np.zeros(K.shape[0])
        for h in range(q.shape[0]):
            out[h], p = attend_one(q[h], K, V, sc)
            weights += p
        j = 0
        for b in self.blocks:
            for e in range(len(b["s"])):
                b["s"][e] += weights[j]
                j += 1
        return out, freed

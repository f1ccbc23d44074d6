"""The synthetic workloads and their seeded tensors.

Shapes follow the decode configurations of the pages' examples (a tiny streaming
case, a Llama-2-7B-shaped layer with a 4+2044 cache, a Qwen-like 24/4-head GQA
model with 16 attention layers, a 32k SnapKV prompt, a 128k H2O budget, its
128k prompt phase and a 128k DuoAttention mixed-head layer).
Tensors are virtual: each is a :class:`synth.gen.NormalStream` over a fixed
logical shape, so any slice can be produced on the CPU (numpy) or on the GPU
(torch) with identical bits.
"""
from __future__ import annotations

import dataclasses
import math

import numpy as np

from .gen import NormalStream, hash_positions, stream_key, uniform_bits

SEED = 0
# Elements per generation chunk on the device (int64 indices and hash temporaries of a
# chunk take a few GiB).
TORCH_CHUNK = 1 << 27


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    title: str
    kind: str  # "streaming" | "snapkv" | "h2o" | "duo" | "h2o_prompt"
    batch: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    dtype: str
    n_layers: int = 1
    rope_base: float = 10000.0
    # streaming (sink + ring window)
    n_sink: int = 0
    window: int = 0
    prefill: int = 0
    steps: int = 0
    sink_key_scale: float = 1.0
    # snapkv
    n_prompt: int = 0
    l_obs: int = 0
    kernel_size: int = 0
    k_keep: int = 0
    plant_frac: float = 0.0
    plant_scale: float = 1.0
    # h2o
    budget: int = 0
    n_recent: int = 0
    block_size: int = 0  # 0: token-level eviction; 16 / 32: block-level
    # duo: per layer, per KV head, 1 = retrieval head (full history), 0 = streaming
    # head (n_sink sinks + window recent tokens)
    retrieval: tuple = ()
    seed: int = SEED

    @property
    def group(self) -> int:
        return self.n_q_heads // self.n_kv_heads

    @property
    def capacity(self) -> int:
        if self.kind == "streaming":
            return self.n_sink + self.window
        if self.kind == "h2o":
            return self.budget
        if self.kind == "duo":
            return self.prefill + self.steps
        return self.k_keep + self.l_obs

    @property
    def esize(self) -> int:
        return 4 if self.dtype == "f32" else 2

    @property
    def total_tokens(self) -> int:
        return self.prefill + self.steps if self.kind != "h2o" else self.n_prompt + self.steps

    # ------------------------------------------------------------------ tensors
    def stream(self, tensor: str, layer: int = 0) -> NormalStream:
        return NormalStream(self.seed, f"{self.name}/L{layer}/{tensor}", self.dtype)

    def token_shape(self, tensor: str):
        h = self.n_q_heads if tensor == "q" else self.n_kv_heads
        return (self.total_tokens, self.batch, h, self.head_dim)

    def key_scale_of_tokens(self, tokens: np.ndarray) -> np.ndarray:
        """Per-token scale of keys before rounding (sink keys of the GQA workload)."""
        tokens = np.asarray(tokens, dtype=np.int64)
        s = np.ones(tokens.shape, dtype=np.float64)
        if self.sink_key_scale != 1.0:
            s[tokens < 4] = self.sink_key_scale
        return s

    def token_block(self, tensor: str, layer: int, tokens, batches=None, heads=None, *, f64=True):
        """Values of a token-major virtual tensor, returned as [b][h][token][d].

        ``tensor`` is one of "q", "k", "v"; the result is float64 (``f64=True``) or the
        stored representation (float32 or bf16 bits).
        """
        from .gen import flat_index_np

        shape = self.token_shape(tensor)
        tokens = np.atleast_1d(np.asarray(tokens, dtype=np.int64))
        batches = np.arange(self.batch) if batches is None else np.atleast_1d(batches)
        heads = np.arange(shape[2]) if heads is None else np.atleast_1d(heads)
        d = np.arange(self.head_dim)
        idx = flat_index_np(shape, [tokens, batches, heads, d])  # [t][b][h][d]
        scale = 1.0
        if tensor == "k" and self.sink_key_scale != 1.0:
            scale = self.key_scale_of_tokens(tokens)[:, None, None, None]
        st = self.stream(tensor, layer)
        out = st.values(idx, scale) if f64 else st.stored(idx, scale)
        return np.ascontiguousarray(np.transpose(out, (1, 2, 0, 3)))

    def token_block_torch(self, tensor: str, layer: int, t0: int, t1: int, device, max_elems=TORCH_CHUNK):
        """Tokens [t0, t1) of a token-major tensor on ``device`` as [b][h][token][d]
        (the bulk-append layout); generated in a few chunks of up to ``max_elems``
        elements, each a handful of whole-tensor operations."""
        import torch

        T, B, H, D = self.token_shape(tensor)
        st = self.stream(tensor, layer)
        out = torch.empty((B, H, t1 - t0, D), device=device,
                          dtype=torch.float32 if self.dtype == "f32" else torch.bfloat16)
        per = B * H * D  # elements of one token
        bhd = (torch.arange(B * H, device=device, dtype=torch.int64) * D).view(B, H, 1, 1) + \
            torch.arange(D, device=device, dtype=torch.int64).view(1, 1, 1, D)
        for a, e in _chunks(t0, t1, per, max_elems):
            idx = torch.arange(a, e, device=device, dtype=torch.int64).view(1, 1, -1, 1) * per + bhd
            out[:, :, a - t0:e - t0] = st.torch_stored(idx, span=(a * per, e * per))
            if tensor == "k" and self.sink_key_scale != 1.0 and a < 4:
                m = min(4, e) - a
                out[:, :, a - t0:a - t0 + m] = st.torch_stored(idx[:, :, :m], self.sink_key_scale,
                                                               span=(a * per, (a + m) * per))
            del idx
        return out

    def token_major_torch(self, tensor: str, layer: int, t0: int, t1: int, device, max_elems=TORCH_CHUNK):
        """Tokens [t0, t1) on ``device`` as [token][b][h][d]: each token's slice is a
        contiguous [b][h][d] block (the single-token append / query layout)."""
        import torch

        T, B, H, D = self.token_shape(tensor)
        per = B * H * D
        st = self.stream(tensor, layer)
        out = torch.empty((t1 - t0, B, H, D), device=device,
                          dtype=torch.float32 if self.dtype == "f32" else torch.bfloat16)
        for a, e in _chunks(t0, t1, per, max_elems):
            idx = torch.arange(a * per, e * per, device=device, dtype=torch.int64)
            out[a - t0: e - t0] = st.torch_stored(idx, span=(a * per, e * per)).view(e - a, B, H, D)
            if tensor == "k" and self.sink_key_scale != 1.0 and a < 4:
                m = min(4, e) - a
                out[a - t0: a - t0 + m] = st.torch_stored(idx[: m * per], self.sink_key_scale,
                                                          span=(a * per, (a + m) * per)).view(m, B, H, D)
            del idx
        return out

    # ------------------------------------------------------------------ snapkv
    def snapkv_plants(self, b: int, h: int) -> np.ndarray:
        count = int(round(self.plant_frac * self.n_prompt))
        return hash_positions(self.seed, f"{self.name}/plant/b{b}/h{h}", self.n_prompt, count)

    def snapkv_tensor(self, tensor: str, b: int, h: int, *, f64=True):
        """[rows][d] block of the prompt tensors: "q_obs" (L_obs rows), "k", "v" (N rows)."""
        rows = self.l_obs if tensor == "q_obs" else self.n_prompt
        shape = (self.batch, self.n_q_heads, rows, self.head_dim)
        base = (b * shape[1] + h) * rows * self.head_dim
        idx = base + np.arange(rows * self.head_dim, dtype=np.int64).reshape(rows, self.head_dim)
        scale = 1.0
        if tensor == "k" and self.plant_frac > 0:
            s = np.ones(rows, dtype=np.float64)
            s[self.snapkv_plants(b, h)] = self.plant_scale
            scale = s[:, None]
        st = NormalStream(self.seed, f"{self.name}/{tensor}", self.dtype)
        return st.values(idx, scale) if f64 else st.stored(idx, scale)

    def snapkv_tensor_torch(self, tensor: str, device):
        """The whole [B][H][rows][D] prompt tensor on ``device`` (planted keys included)."""
        import torch

        rows = self.l_obs if tensor == "q_obs" else self.n_prompt
        B, H, D = self.batch, self.n_q_heads, self.head_dim
        st = NormalStream(self.seed, f"{self.name}/{tensor}", self.dtype)
        out = _flat_stream_torch(st, B * H * rows * D, device).view(B, H, rows, D)
        if tensor == "k" and self.plant_frac > 0:
            # every planted row of every head in one call: flat row ids (b * H + h) * rows + p
            prow = np.concatenate([(b * H + h) * rows + self.snapkv_plants(b, h)
                                   for b in range(B) for h in range(H)])
            pr = torch.from_numpy(prow).to(device)
            idx = pr.view(-1, 1) * D + torch.arange(D, device=device, dtype=torch.int64).view(1, D)
            out.view(B * H * rows, D)[pr] = st.torch_stored(idx, self.plant_scale, span=(0, B * H * rows * D))
        return out

    # ------------------------------------------------------------------ h2o prompt phase
    def prompt_tensor(self, tensor: str, b: int, h: int, *, f64=True):
        """[N][d] prompt block of one head: "q" (query head h) or "k" / "v" (KV head h)."""
        heads = self.n_q_heads if tensor == "q" else self.n_kv_heads
        base = (b * heads + h) * self.n_prompt * self.head_dim
        idx = base + np.arange(self.n_prompt * self.head_dim, dtype=np.int64).reshape(self.n_prompt, self.head_dim)
        st = NormalStream(self.seed, f"{self.name}/prompt/{tensor}", self.dtype)
        return st.values(idx) if f64 else st.stored(idx)

    def prompt_tensor_torch(self, tensor: str, device):
        """The whole [B][H][N][D] prompt tensor on ``device`` (H = query or KV heads)."""
        heads = self.n_q_heads if tensor == "q" else self.n_kv_heads
        B, N, D = self.batch, self.n_prompt, self.head_dim
        st = NormalStream(self.seed, f"{self.name}/prompt/{tensor}", self.dtype)
        return _flat_stream_torch(st, B * heads * N * D, device).view(B, heads, N, D)

    # ------------------------------------------------------------------ h2o
    def h2o_initial_state(self, b: int, g: int):
        """Seeded post-compression H2O state of one (batch row, kv head).

        Returns (positions int64 [budget], initial scores float32 [budget],
        planted-mask bool [budget]).  Positions: the ``n_recent`` most recent
        prompt tokens, every planted heavy position of the older prompt, and a
        seeded fill of other old positions up to the budget; slots hold them in
        ascending position order.  Scores are Pareto(1.5)-distributed (seeded),
        multiplied by 4 on planted positions, as float32.
        """
        N, R, C = self.n_prompt, self.n_recent, self.budget
        old = N - R
        n_plant = int(round(self.plant_frac * old))
        plants = self.h2o_plants(b, g)
        if n_plant > C - R:
            raise ValueError("budget smaller than planted set")
        rest = np.setdiff1d(np.arange(old, dtype=np.int64), plants, assume_unique=True)
        key = stream_key(self.seed, f"{self.name}/fill/b{b}/g{g}")
        order = np.argsort(uniform_bits(key, rest), kind="stable")
        fill = np.sort(rest[order[: C - R - n_plant]])
        pos = np.sort(np.concatenate([plants, fill, np.arange(old, N, dtype=np.int64)]))
        planted = np.isin(pos, plants)
        ukey = stream_key(self.seed, f"{self.name}/score/b{b}/g{g}")
        u = (uniform_bits(ukey, pos).astype(np.float64) + 0.5) / 2.0**32
        s = (1.0 - u) ** (-1.0 / 1.5)
        s[planted] *= 4.0
        return pos, s.astype(np.float32), planted

    def h2o_plants(self, b: int, g: int) -> np.ndarray:
        old = self.n_prompt - self.n_recent
        n_plant = int(round(self.plant_frac * old))
        return hash_positions(self.seed, f"{self.name}/plant/b{b}/g{g}", old, n_plant)

    def h2o_kv(self, tensor: str, b: int, g: int, positions, *, f64=True):
        """[len(positions)][d] K or V rows of one (b, kv head); planted keys scaled."""
        from .gen import flat_index_np

        positions = np.asarray(positions, dtype=np.int64)
        idx = flat_index_np(self.token_shape(tensor), [positions, [b], [g], np.arange(self.head_dim)])
        idx = idx[:, 0, 0, :]
        scale = 1.0
        if tensor == "k":
            s = np.where(np.isin(positions, self.h2o_plants(b, g)), self.plant_scale, 1.0)
            scale = s[:, None]
        st = self.stream(tensor, 0)
        return st.values(idx, scale) if f64 else st.stored(idx, scale)


def h2o_state_torch(w: Workload, device):
    """The seeded H2O state of every (row, KV head) on ``device``.

    Returns (K, V [B][Hkv][C][D] in the cache dtype, positions int32 [B][Hkv][C],
    scores float32 [B][Hkv][C]) with slots in ascending position order, the layout an
    H2O cache holds after being seeded in place.  Positions and scores come from
    :meth:`Workload.h2o_initial_state` (host); the K / V rows of all heads are generated
    in one pass each.
    """
    import torch

    B, H, C, D = w.batch, w.n_kv_heads, w.budget, w.head_dim
    T = w.total_tokens
    pos = np.empty((B, H, C), np.int64)
    sc = np.empty((B, H, C), np.float32)
    planted = np.empty((B, H, C), bool)
    for b in range(B):
        for g in range(H):
            pos[b, g], sc[b, g], planted[b, g] = w.h2o_initial_state(b, g)
    assert T > int(pos.max())
    pt = torch.from_numpy(pos).to(device)
    bg = (torch.arange(B, device=device, dtype=torch.int64).view(B, 1, 1) * H +
          torch.arange(H, device=device, dtype=torch.int64).view(1, H, 1))
    rows = pt * (B * H) + bg  # token-major row index (t * B + b) * H + g
    idx = rows.unsqueeze(-1) * D + torch.arange(D, device=device, dtype=torch.int64)
    span = (0, T * B * H * D)
    K = w.stream("k", 0).torch_stored(idx, span=span)
    pl = torch.from_numpy(planted).to(device)
    K[pl] = w.stream("k", 0).torch_stored(idx[pl], w.plant_scale, span=span)
    V = w.stream("v", 0).torch_stored(idx, span=span)
    return K, V, pt.to(torch.int32), torch.from_numpy(sc).to(device)


def _chunks(t0, t1, per, max_elems):
    """Token ranges [a, e) covering [t0, t1), each of at most max(1, max_elems // per)
    tokens and never crossing a multiple of 2**32 elements (so each has one upper index
    word)."""
    step = max(1, max_elems // per)
    a = t0
    while a < t1:
        e = min(t1, a + step)
        wall = ((a * per >> 32) + 1) << 32  # next multiple of 2**32 elements
        if e * per > wall and (wall // per) > a:
            e = wall // per
        yield a, e
        a = e


def _flat_stream_torch(st, n, device, max_elems=TORCH_CHUNK):
    """Elements 0 .. n-1 of a stream as one flat tensor, in chunks of at most max_elems
    that never cross a multiple of 2**32."""
    import torch

    out = torch.empty(n, device=device, dtype=torch.float32 if st.dtype == "f32" else torch.bfloat16)
    a = 0
    while a < n:
        e = min(n, a + max_elems, ((a >> 32) + 1) << 32)
        out[a:e] = st.torch_stored(torch.arange(a, e, device=device, dtype=torch.int64), span=(a, e))
        a = e
    return out


def _streaming(name, title, **kw):
    return Workload(name=name, title=title, kind="streaming", **kw)


WORKLOADS = {
    "tiny_streaming": _streaming(
        "tiny_streaming",
        "tiny StreamingLLM decode: 1 layer, B=1, 4 q / 1 kv heads, D=64, fp32, 4 sinks + window 60, "
        "512 tokens streamed from empty",
        batch=1, n_q_heads=4, n_kv_heads=1, head_dim=64, dtype="f32",
        n_sink=4, window=60, prefill=0, steps=512),
    "llama2_7b_layer": _streaming(
        "llama2_7b_layer",
        "Llama-2-7B-shaped decode layer: B=16, 32 q / 32 kv heads, D=128, bf16, 4 sinks + 2044 ring, "
        "prefilled to 2048 then 8192 decode steps",
        batch=16, n_q_heads=32, n_kv_heads=32, head_dim=128, dtype="bf16",
        n_sink=4, window=2044, prefill=2048, steps=8192),
    "llama3_8b_layer": _streaming(
        "llama3_8b_layer",
        "Llama-3-8B-shaped decode layer: B=16, 32 q / 8 kv heads, D=128, bf16, 4 sinks + 8188 ring, "
        "prefilled to 8192 then 1024 decode steps",
        batch=16, n_q_heads=32, n_kv_heads=8, head_dim=128, dtype="bf16", rope_base=500000.0,
        n_sink=4, window=8188, prefill=8192, steps=1024),
    "gqa_long": _streaming(
        "gqa_long",
        "GQA long-cache decode: B=16, 24 q / 4 kv heads, D=256, bf16, 16 attention layers, "
        "4 sinks + 32764 ring, prefilled to 32768 then 1024 decode steps; sink keys x4",
        batch=16, n_q_heads=24, n_kv_heads=4, head_dim=256, dtype="bf16", n_layers=16,
        n_sink=4, window=32764, prefill=32768, steps=1024, sink_key_scale=4.0),
    "snapkv_32k": Workload(
        name="snapkv_32k",
        title="SnapKV prefill compression: B=1, 32 heads, D=128, bf16, N=32768, L_obs=32, "
              "avg pool 5, keep 5243 per head + the observation window; 2% of keys x3",
        kind="snapkv", batch=1, n_q_heads=32, n_kv_heads=32, head_dim=128, dtype="bf16",
        n_prompt=32768, l_obs=32, kernel_size=5, k_keep=5243, plant_frac=0.02, plant_scale=3.0),
    "duo_128k": Workload(
        name="duo_128k",
        title="DuoAttention mixed-head decode: B=16, 32 q / 8 kv heads, D=128, bf16, per layer 2 retrieval "
              "heads (full history) + 6 streaming heads (4 sinks + 64 recent), prefilled to 131072 then "
              "256 decode steps",
        kind="duo", batch=16, n_q_heads=32, n_kv_heads=8, head_dim=128, dtype="bf16",
        n_sink=4, window=64, prefill=131072, steps=256, retrieval=((1, 0, 0, 0, 0, 1, 0, 0),)),
    "h2o_prompt_128k": Workload(
        name="h2o_prompt_128k",
        title="H2O prompt-phase compression: B=16, 32 q / 8 kv heads, D=128, bf16, 131072-token prompt "
              "scored by its full causal attention, kept in a 4096 budget (512 recent + 3584 heavy)",
        kind="h2o_prompt", batch=16, n_q_heads=32, n_kv_heads=8, head_dim=128, dtype="bf16",
        n_prompt=131072, budget=4096, n_recent=512),
    "h2o_blocks_128k": Workload(
        name="h2o_128k",  # the same seeded tensors as h2o_128k
        title="H2O block-level decode: B=16, 32 q / 8 kv heads, D=128, bf16, 131072-token prompt held in "
              "a 4096 budget of 16-token blocks (512 recent + 3584 heavy), 1024 decode steps",
        kind="h2o", batch=16, n_q_heads=32, n_kv_heads=8, head_dim=128, dtype="bf16",
        n_prompt=131072, budget=4096, n_recent=512, steps=1024, plant_frac=0.02, plant_scale=3.0, block_size=16),
    "h2o_128k": Workload(
        name="h2o_128k",
        title="H2O budgeted decode: B=16, 32 q / 8 kv heads, D=128, bf16, 131072-token prompt held in "
              "a 4096 budget (512 recent + 3584 heavy), 1024 decode steps",
        kind="h2o", batch=16, n_q_heads=32, n_kv_heads=8, head_dim=128, dtype="bf16",
        n_prompt=131072, budget=4096, n_recent=512, steps=1024, plant_frac=0.02, plant_scale=3.0),
}


def scaled(w: Workload, **changes) -> Workload:
    """A copy of a workload with some fields changed (smaller parity cases)."""
    return dataclasses.replace(w, **changes)


def snapkv_keep_count(n_prompt: int, frac: float = 0.16) -> int:
    return int(math.floor(frac * n_prompt + 0.5))

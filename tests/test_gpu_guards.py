"""GPU: no entry point writes outside the memory it is given.

Every device buffer handed to the library (cache K/V and auxiliary memory, workspaces,
inputs, outputs, checkpoint buffers) sits inside a larger allocation whose guard regions
before and after it hold a canary byte pattern.  After a run of calls through every entry
point the guard regions must still hold the pattern; inputs must be unchanged entirely, and
output rows the documentation says are left untouched must keep their contents.
"""
import pytest

from synth import WORKLOADS
from synth.workloads import scaled

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

GUARD = 64 * 1024  # bytes of canary before and after each buffer (a multiple of 256)


@pytest.fixture(scope="module")
def L():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    import long_context_decode_amd as lib

    return lib


def _pattern(n, salt):
    i = torch.arange(n, dtype=torch.int64, device="cuda")
    return ((i * 131 + 7 + salt) & 255).to(torch.uint8)


class Guarded:
    """nbytes of device memory (256-byte aligned) between two canary regions."""

    def __init__(self, nbytes, salt=0):
        self.n = max(int(nbytes), 1)
        padded = (self.n + 255) // 256 * 256
        self.full = _pattern(GUARD + padded + GUARD, salt)
        self.ref = self.full.clone()
        assert self.full.data_ptr() % 256 == 0
        self.inner = self.full[GUARD: GUARD + self.n]

    def view(self, dtype, shape):
        return self.inner.view(dtype).view(shape)

    def fill_from(self, t):
        b = t.contiguous().view(torch.uint8).flatten()
        assert b.numel() == self.n
        self.inner.copy_(b)
        self.ref[GUARD: GUARD + self.n].copy_(b)
        return self

    def check(self, name, inner_unchanged=False, untouched_from=None):
        torch.cuda.synchronize()
        lo, hi = GUARD, GUARD + self.n
        assert torch.equal(self.full[:lo], self.ref[:lo]), f"{name}: bytes written before the buffer"
        assert torch.equal(self.full[hi:], self.ref[hi:]), f"{name}: bytes written after the buffer"
        if inner_unchanged:
            assert torch.equal(self.full[lo:hi], self.ref[lo:hi]), f"{name}: an input was modified"
        if untouched_from is not None:
            a = GUARD + untouched_from
            assert torch.equal(self.full[a:hi], self.ref[a:hi]), f"{name}: rows past the written ones changed"


def _input(t, salt):
    return Guarded(t.numel() * t.element_size(), salt).fill_from(t)


@pytest.mark.parametrize("policy", ["ring_rope", "append", "h2o_blocks", "duo"])
def test_cache_calls_stay_in_bounds(L, policy):
    G, D = 4, 128
    w = scaled(WORKLOADS["llama2_7b_layer"], name=f"guard_{policy}", batch=2, n_kv_heads=2, n_q_heads=2 * G,
               head_dim=D, n_layers=2, prefill=0, steps=200)
    kw = {"ring_rope": dict(policy=L.LCD_SINK_RING, n_sink=4, window=92, rope=1),
          "append": dict(policy=L.LCD_APPEND, capacity=160),
          "h2o_blocks": dict(policy=L.LCD_H2O, capacity=96, n_recent=16, block_size=16),
          "duo": dict(policy=L.LCD_DUO, capacity=160, n_sink=4, window=28, retrieval=[[1, 0], [0, 1]])}[policy]
    cfg = L.cache_config(w.batch, w.n_q_heads, w.n_kv_heads, D, L.LCD_BF16, n_layers=2, **kw)
    kvb, auxb, wsb = L.cache_sizes(cfg)
    print(f"[guards] {policy}: kv {kvb} aux {auxb} ws {wsb} bytes", flush=True)
    kv, aux, ws = Guarded(kvb, 1), Guarded(auxb, 2), Guarded(wsb, 3)
    h = L.kv_cache_init(cfg, kv.inner, kvb, aux.inner if auxb else None, auxb)
    dev = "cuda"
    n_steps = 150
    toks = {(l, x): w.token_major_torch(x, l, 0, n_steps, dev) for l in range(2) for x in "qkv"}
    inputs = {key: _input(t, 10 + i) for i, (key, t) in enumerate(toks.items())}
    out = Guarded(w.batch * w.n_q_heads * D * 4, 4)
    o = out.view(torch.float32, (w.batch, w.n_q_heads, D))
    fused = policy != "duo"
    shape = (n_steps, w.batch, w.n_kv_heads, D)
    try:
        for t in range(n_steps):
            for l in range(2):
                k = inputs[(l, "k")].view(torch.bfloat16, shape)[t]
                v = inputs[(l, "v")].view(torch.bfloat16, shape)[t]
                q = inputs[(l, "q")].view(torch.bfloat16, (n_steps, w.batch, w.n_q_heads, D))[t]
                if fused and t % 2 == 0:
                    L.decode_step(h, l, k, v, q, o, ws.inner, wsb)
                elif fused and t % 3 == 1:
                    L.decode_step_noalloc(h, l, k, v, q, o)
                else:
                    L.kv_append(h, l, k.unsqueeze(2), v.unsqueeze(2), 1)
                    L.decode_attn(h, l, q, o, ws.inner, wsb)
        # checkpoint both layers into guarded buffers and load them back
        nb = L.kv_layer_bytes(h, 1)
        bufs = {"k": Guarded(nb, 5), "v": Guarded(nb, 6)}
        if policy == "h2o_blocks":
            n = w.batch * w.n_kv_heads
            bufs |= {"pos": Guarded(n * 96 * 4, 7), "score": Guarded(n * 96 * 4, 8), "victim": Guarded(n * 4, 9),
                     "open": Guarded(n * 4, 10)}
        g = {x: b.inner for x, b in bufs.items()}
        st = L.kv_save(h, 1, g["k"], g["v"], g.get("pos"), g.get("score"), g.get("victim"), g.get("open"))
        L.kv_load(h, 1, g["k"], g["v"], g.get("pos"), g.get("score"), g.get("victim"), g.get("open"), st)
        if policy == "append":
            L.kv_set_filled(h, 0, 100, 100)
        torch.cuda.synchronize()
    finally:
        L.kv_cache_destroy(h)
    kv.check("K/V cache memory")
    aux.check("auxiliary memory")
    ws.check("decode workspace")
    out.check("decode output")
    for key, b in inputs.items():
        b.check(f"input {key}", inner_unchanged=True)
    for x, b in bufs.items():
        b.check(f"checkpoint {x}")


@pytest.mark.parametrize("l_obs", [40, 24])
def test_snapkv_stays_in_bounds(L, l_obs):
    """The compress writes k_keep + l_obs rows of out_rows and nothing else (a window of 40
    rows runs two 32-row blocks, one of 24 a single partial block)."""
    w = scaled(WORKLOADS["snapkv_32k"], name=f"guard_snapkv_{l_obs}", n_q_heads=3, n_kv_heads=3, n_prompt=2000,
               l_obs=l_obs, k_keep=300)
    B, H, D, N, Lo, K = w.batch, w.n_q_heads, w.head_dim, w.n_prompt, w.l_obs, w.k_keep
    out_rows = K + Lo + 17
    print(f"[guards] snapkv: N={N} l_obs={Lo} keep={K} out_rows={out_rows}", flush=True)
    p = L.snapkv_params(B, H, D, N, Lo, w.kernel_size, K, out_rows=out_rows)
    wsb = L.snapkv_sizes(p)
    q = _input(w.snapkv_tensor_torch("q_obs", "cuda"), 20)
    k = _input(w.snapkv_tensor_torch("k", "cuda"), 21)
    v = _input(w.snapkv_tensor_torch("v", "cuda"), 22)
    ko, vo = Guarded(B * H * out_rows * D * 2, 23), Guarded(B * H * out_rows * D * 2, 24)
    idx, sc, ws = Guarded(B * H * out_rows * 4, 25), Guarded(B * H * (N - Lo) * 4, 26), Guarded(wsb, 27)
    L.snapkv_compress(p, q.inner, k.inner, v.inner, ko.inner, vo.inner, idx.inner, sc.inner, ws.inner, wsb)
    torch.cuda.synchronize()
    for name, b in (("q_obs", q), ("k", k), ("v", v)):
        b.check(name, inner_unchanged=True)
    ws.check("workspace")
    sc.check("scores_out")
    # per head, rows k_keep + l_obs .. out_rows - 1 are left untouched
    kept = K + Lo
    for name, b, rb in (("k_out", ko, D * 2), ("v_out", vo, D * 2), ("idx_out", idx, 4)):
        b.check(name)
        full = b.full[GUARD: GUARD + b.n].view(B * H, out_rows * rb)
        ref = b.ref[GUARD: GUARD + b.n].view(B * H, out_rows * rb)
        assert torch.equal(full[:, kept * rb:], ref[:, kept * rb:]), f"{name}: rows past k_keep + l_obs changed"


def test_h2o_prompt_stays_in_bounds(L):
    """budget > N: rows N .. budget - 1 of the outputs are left untouched."""
    B, Hq, Hkv, D, N, C, R = 1, 4, 2, 128, 700, 800, 64
    base = WORKLOADS["h2o_prompt_128k"]
    w = scaled(base, name="guard_h2o_prompt", batch=B, n_q_heads=Hq, n_kv_heads=Hkv, head_dim=D, n_prompt=N,
               budget=C, n_recent=R)
    print(f"[guards] h2o prompt: N={N} budget={C}", flush=True)
    p = L.h2o_prompt_params(B, Hq, Hkv, D, N, C, R)
    wsb = L.h2o_prompt_sizes(p)
    q, k, v = (_input(w.prompt_tensor_torch(t, "cuda"), 30 + i) for i, t in enumerate("qkv"))
    ko, vo = Guarded(B * Hkv * C * D * 2, 33), Guarded(B * Hkv * C * D * 2, 34)
    pos, sco = Guarded(B * Hkv * C * 4, 35), Guarded(B * Hkv * C * 4, 36)
    sall, ws = Guarded(B * Hkv * N * 4, 37), Guarded(wsb, 38)
    L.h2o_prompt_compress(p, q.inner, k.inner, v.inner, ko.inner, vo.inner, pos.inner, sco.inner, sall.inner,
                          ws.inner, wsb)
    torch.cuda.synchronize()
    for name, b in (("q", q), ("k", k), ("v", v)):
        b.check(name, inner_unchanged=True)
    ws.check("workspace")
    sall.check("scores_all")
    for name, b, rb in (("k_out", ko, D * 2), ("v_out", vo, D * 2), ("pos_out", pos, 4), ("score_out", sco, 4)):
        b.check(name)
        full = b.full[GUARD: GUARD + b.n].view(B * Hkv, C * rb)
        ref = b.ref[GUARD: GUARD + b.n].view(B * Hkv, C * rb)
        assert torch.equal(full[:, N * rb:], ref[:, N * rb:]), f"{name}: rows past the prompt changed"

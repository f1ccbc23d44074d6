"""GPU: the fused decode step captured in a HIP graph.

A captured `lcd_decode_step` (or `lcd_decode_step_noalloc`, the entry point for callers
that cannot allocate) re-runs with the same arguments on every replay: the token is written
to the same slot again and the same slots are attended, so for a sink + ring or APPEND cache
every replay must reproduce the eager step's output bit for bit.  Each graph covers one
token over two layers and is replayed several times with the program's own eager work and
synchronisations in between; every replay is checked.
"""
import pytest

from synth import WORKLOADS
from synth.workloads import scaled

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def L():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    import long_context_decode_amd as lib

    return lib


@pytest.mark.parametrize("policy,G,noalloc", [("ring_rope", 4, False), ("ring_rope", 1, True),
                                              ("append", 2, False), ("ring_rope", 6, True)])
def test_captured_step_replays_bit_exact(L, policy, G, noalloc):
    D = 128 if G != 6 else 256
    w = scaled(WORKLOADS["llama2_7b_layer"], name=f"graph_{policy}_{G}", batch=2, n_kv_heads=2, n_q_heads=2 * G,
               head_dim=D, n_layers=2, prefill=700, steps=2)
    kw = dict(policy=L.LCD_SINK_RING, n_sink=4, window=508, rope=1) if policy == "ring_rope" else \
        dict(policy=L.LCD_APPEND, capacity=800)
    cfg = L.cache_config(w.batch, w.n_q_heads, w.n_kv_heads, D, L.LCD_BF16, n_layers=2, **kw)
    print(f"[graph] {policy} G={G} D={D} noalloc={noalloc}", flush=True)
    dev = "cuda"
    eager, graphed = L.KVCache(cfg), L.KVCache(cfg)
    pre = w.prefill
    for c in (eager, graphed):
        for l in range(2):
            c.append(l, w.token_block_torch("k", l, 0, pre, dev), w.token_block_torch("v", l, 0, pre, dev))
    toks = {(l, x): w.token_major_torch(x, l, pre, pre + 1, dev)[0] for l in range(2) for x in "qkv"}
    ref = [torch.empty((w.batch, w.n_q_heads, D), dtype=torch.float32, device=dev) for _ in range(2)]
    out = [torch.empty_like(r) for r in ref]

    def step(c, l, o, stream=None):
        k, v, q = toks[(l, "k")], toks[(l, "v")], toks[(l, "q")]
        if noalloc:
            L.decode_step_noalloc(c.handle, l, k, v, q, o, stream)
        else:
            L.decode_step(c.handle, l, k, v, q, o, c.ws, c.ws_bytes, stream)

    for l in range(2):
        step(eager, l, ref[l])
    torch.cuda.synchronize()

    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        s = torch.cuda.current_stream()
        for l in range(2):
            step(graphed, l, out[l], s)
    assert L.kv_tokens(graphed.handle, 0) == pre + 1  # the host counters advanced once, at capture
    filler = torch.randn(1 << 20, device=dev)
    for rep in range(4):
        for o in out:
            o.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        for l in range(2):
            assert torch.equal(out[l].view(torch.int32), ref[l].view(torch.int32)), f"replay {rep} layer {l}"
        # the program's own eager work between replays
        filler.mul_(0.5).add_(1.0)
        eager_out = torch.empty_like(ref[0])
        L.decode_attn(eager.handle, 0, toks[(0, "q")], eager_out, eager.ws, eager.ws_bytes)
        torch.cuda.synchronize()
        assert torch.equal(eager_out.view(torch.int32), ref[0].view(torch.int32))
    n = L.kv_filled(graphed.handle, 1)  # slots holding tokens (an APPEND cache has unwritten ones)
    assert n == L.kv_filled(eager.handle, 1)
    kg, vg = graphed.layer_tensors(1)
    ke, ve = eager.layer_tensors(1)
    assert torch.equal(kg[:, :, :n].view(torch.int16), ke[:, :, :n].view(torch.int16))
    assert torch.equal(vg[:, :, :n].view(torch.int16), ve[:, :, :n].view(torch.int16))

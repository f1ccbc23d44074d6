"""GPU: checkpoint / resume of a cache layer (lcd_kv_save, lcd_kv_load).

Two caches of one configuration take the same tokens.  At token 300 the second one's
layers are saved, the cache is destroyed, a fresh cache is built and the saved state is
loaded into it; both then continue to token 512.  Every decode output after the reload,
and the final device state and counters, must equal the uninterrupted cache's bit for bit:
sink + ring with RoPE, APPEND, H2O (token- and block-level, the fused step picking slots on
the device) and mixed retrieval / streaming heads, over two layers so that layer addressing
is covered.  Also the load-time checks of the saved counters (nothing copied on refusal).
"""
import pytest

from synth import WORKLOADS
from synth.workloads import scaled

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

SAVE_AT, END = 300, 512


@pytest.fixture(scope="module")
def L():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    import long_context_decode_amd as lib

    return lib


CASES = {
    # name: (policy name, G, D, dtype, extra config, fused step)
    "ring_rope_G4": ("LCD_SINK_RING", 4, 128, "bf16", dict(n_sink=4, window=252, rope=1), True),
    "ring_G1_f32": ("LCD_SINK_RING", 1, 64, "f32", dict(n_sink=2, window=190), True),
    "append_G2": ("LCD_APPEND", 2, 128, "bf16", dict(capacity=600), True),
    "h2o_token_G4": ("LCD_H2O", 4, 128, "bf16", dict(capacity=160, n_recent=20), True),
    "h2o_block16_G4": ("LCD_H2O", 4, 128, "bf16", dict(capacity=128, n_recent=16, block_size=16), True),
    "duo_G4": ("LCD_DUO", 4, 128, "bf16", dict(capacity=600, n_sink=4, window=124,
                                               retrieval=[[1, 0], [0, 1]]), False),
}


def _state(L, c, layer):
    """Everything the layer holds that later steps read, as host tensors."""
    torch.cuda.synchronize()
    filled = L.kv_filled(c.handle, layer)
    out = {"tokens": L.kv_tokens(c.handle, layer), "filled": filled}
    if c.cfg.policy == L.LCD_DUO:
        # the layer's K (and V) block: [B][R][C][D] retrieval heads, then [B][T][S + W][D]
        # streaming heads; the slots holding tokens are compared
        t, _ = c.save_state(layer)
        torch.cuda.synchronize()
        cf = c.cfg
        R = sum(c.retrieval[layer])
        T = cf.n_kv_heads - R
        C2 = cf.n_sink + cf.window
        for x in "kv":
            buf = t[x].cpu().view(torch.int16)
            ret = buf[: cf.batch * R * cf.capacity * cf.head_dim].view(cf.batch, R, cf.capacity, cf.head_dim)
            st = buf[cf.batch * R * cf.capacity * cf.head_dim:].view(cf.batch, T, C2, cf.head_dim)
            out[x + "_ret"] = ret[:, :, :filled].clone()
            out[x + "_str"] = st[:, :, :min(out["tokens"], C2)].clone()
        return out
    k, v = c.layer_tensors(layer)
    if c.cfg.policy == L.LCD_H2O:
        p, s = c.h2o_tensors(layer)
        live = (p[:, :, :filled] >= 0).cpu()
        out["pos"], out["score"] = p[:, :, :filled].cpu(), s[:, :, :filled].cpu()
        out["k"] = k[:, :, :filled].cpu().view(torch.int16)[live] if k.dtype == torch.bfloat16 else \
            k[:, :, :filled].cpu()[live]
        out["v"] = v[:, :, :filled].cpu().view(torch.int16)[live] if v.dtype == torch.bfloat16 else \
            v[:, :, :filled].cpu()[live]
    else:
        out["k"], out["v"] = k[:, :, :filled].cpu(), v[:, :, :filled].cpu()
    return out


def _same(a, b, where):
    assert a.keys() == b.keys()
    for key in a:
        if torch.is_tensor(a[key]):
            x, y = a[key], b[key]
            if x.dtype.is_floating_point:
                x, y = x.view(torch.int32 if x.element_size() == 4 else torch.int16), \
                    y.view(torch.int32 if y.element_size() == 4 else torch.int16)
            assert torch.equal(x, y), f"{where}: {key} differs"
        else:
            assert a[key] == b[key], f"{where}: {key} {a[key]} != {b[key]}"


@pytest.mark.parametrize("name", list(CASES))
def test_save_reload_continue_is_bit_exact(L, name):
    pol, G, D, dtype, extra, fused = CASES[name]
    n_layers = 2
    w = scaled(WORKLOADS["llama2_7b_layer"], name=f"ckpt_{name}", batch=2, n_kv_heads=2, n_q_heads=2 * G,
               head_dim=D, dtype=dtype, n_layers=n_layers, prefill=0, steps=END)
    print(f"[checkpoint] {name}: save at {SAVE_AT}, reload into a fresh cache, continue to {END}", flush=True)
    cfg = L.cache_config(w.batch, w.n_q_heads, w.n_kv_heads, D, L.LCD_F32 if dtype == "f32" else L.LCD_BF16,
                         getattr(L, pol), n_layers=n_layers, **extra)
    a, b = L.KVCache(cfg), L.KVCache(cfg)
    for x in (a, b):
        x.retrieval = extra.get("retrieval")
    dev = "cuda"
    toks = {(l, x): w.token_major_torch(x, l, 0, END, dev) for l in range(n_layers) for x in "qkv"}
    oa = torch.empty((w.batch, w.n_q_heads, D), dtype=torch.float32, device=dev)
    ob = torch.empty_like(oa)

    def step(c, l, t, o):
        k, v, q = toks[(l, "k")][t], toks[(l, "v")][t], toks[(l, "q")][t]
        if fused:
            c.step(l, k, v, q, o)
        else:
            c.append(l, k.unsqueeze(2), v.unsqueeze(2))
            c.decode(l, q, o)

    for t in range(SAVE_AT):
        for l in range(n_layers):
            step(a, l, t, oa)
            step(b, l, t, ob)
    saved = [b.save_state(l) for l in range(n_layers)]
    before = [_state(L, b, l) for l in range(n_layers)]
    for l, (_, st) in enumerate(saved):
        assert st.tokens == SAVE_AT and st.filled == L.kv_filled(b.handle, l)
    b.close()
    del b
    c = L.KVCache(cfg)
    c.retrieval = extra.get("retrieval")
    for l, (tensors, st) in enumerate(saved):
        c.load_state(l, tensors, st)
    for l in range(n_layers):
        _same(_state(L, c, l), before[l], f"layer {l} after reload")
    for t in range(SAVE_AT, END):
        for l in range(n_layers):
            step(a, l, t, oa)
            step(c, l, t, ob)
            assert torch.equal(oa, ob), f"token {t} layer {l}: outputs differ after the reload"
    for l in range(n_layers):
        _same(_state(L, a, l), _state(L, c, l), f"layer {l} at token {END}")


def test_load_refuses_inconsistent_counters(L):
    cfg = L.cache_config(1, 4, 1, 128, L.LCD_BF16, L.LCD_SINK_RING, n_sink=4, window=60, rope=1)
    c = L.KVCache(cfg)
    t, st = c.save_state(0)
    assert (st.tokens, st.filled, st.open_fill) == (0, 0, 0)
    for tokens, filled, open_fill in ((10, 11, 0), (100, 50, 0), (10, 10, 1), (10, 65, 0), (-1, 0, 0)):
        bad = L.LayerState(tokens, filled, open_fill, 0)
        with pytest.raises(L.LcdError) as e:
            c.load_state(0, t, bad)
        assert e.value.name == "LCD_EINVAL", (tokens, filled, open_fill)
        assert L.kv_tokens(c.handle, 0) == 0 and L.kv_filled(c.handle, 0) == 0
    with pytest.raises(L.LcdError) as e:  # H2O arrays on a sink + ring layer
        L.kv_load(c.handle, 0, t["k"], t["v"], t["k"], None, None, None, st)
    assert e.value.name == "LCD_EINVAL"
    hcfg = L.cache_config(1, 4, 1, 128, L.LCD_BF16, L.LCD_H2O, capacity=64, n_recent=8, block_size=16)
    h = L.KVCache(hcfg)
    ht, hst = h.save_state(0)
    with pytest.raises(L.LcdError) as e:  # open block fill beyond the block size
        h.load_state(0, ht, L.LayerState(5, 5, 17, 0))
    assert e.value.name == "LCD_EINVAL"
    with pytest.raises(L.LcdError) as e:  # an H2O layer needs its four arrays
        L.kv_load(h.handle, 0, ht["k"], ht["v"], None, None, None, None, hst)
    assert e.value.name == "LCD_EINVAL"
    h.load_state(0, ht, L.LayerState(5, 5, 5, 0))
    assert L.kv_tokens(h.handle, 0) == 5 and L.kv_filled(h.handle, 0) == 5

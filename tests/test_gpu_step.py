"""GPU: lcd_decode_step (append fused into the decode launch) against kv_append +
decode_attn on identical caches: outputs, cache contents and counters bit for bit,
and the error paths (nothing enqueued, counters unchanged)."""
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


def _pair(L, w, policy, **kw):
    dt = L.LCD_F32 if w.dtype == "f32" else L.LCD_BF16
    cfg = L.cache_config(w.batch, w.n_q_heads, w.n_kv_heads, w.head_dim, dt, policy, **kw)
    return L.KVCache(cfg), L.KVCache(cfg)


@pytest.mark.parametrize("G,D,dtype,S,W,pre,steps", [
    (1, 128, "bf16", 4, 500, 600, 40),    # one-pass kernel, wrapped ring, several splits
    (4, 128, "bf16", 4, 252, 100, 200),   # two-pass kernel, growth then wrap
    (6, 256, "bf16", 4, 1020, 1100, 8),
    (4, 64, "f32", 4, 60, 0, 150),        # fp32 from empty
])
def test_step_equals_append_then_decode_ring(L, G, D, dtype, S, W, pre, steps):
    w = scaled(WORKLOADS["llama2_7b_layer"], name=f"step_G{G}_D{D}", batch=2, n_kv_heads=2, n_q_heads=2 * G,
               head_dim=D, dtype=dtype, n_sink=S, window=W, prefill=pre, steps=steps)
    print(f"[step vs append+decode] G={G} D={D} {dtype} S={S} W={W} prefill={pre}", flush=True)
    a, b = _pair(L, w, L.LCD_SINK_RING, n_sink=S, window=W, rope=1)
    dev = "cuda"
    if pre:
        k = w.token_block_torch("k", 0, 0, pre, dev)
        v = w.token_block_torch("v", 0, 0, pre, dev)
        a.append(0, k, v)
        b.append(0, k, v)
    q_all = w.token_major_torch("q", 0, pre, pre + steps, dev)
    k_all = w.token_major_torch("k", 0, pre, pre + steps, dev)
    v_all = w.token_major_torch("v", 0, pre, pre + steps, dev)
    oa = torch.empty((w.batch, w.n_q_heads, D), dtype=torch.float32, device=dev)
    ob = torch.empty_like(oa)
    for s in range(steps):
        a.append(0, k_all[s].unsqueeze(2), v_all[s].unsqueeze(2))
        a.decode(0, q_all[s], oa)
        b.step(0, k_all[s], v_all[s], q_all[s], ob)
        assert torch.equal(oa, ob), f"step {s}: outputs differ"
    torch.cuda.synchronize()
    ka, va = a.layer_tensors(0)
    kb, vb = b.layer_tensors(0)
    assert torch.equal(ka, kb) and torch.equal(va, vb)
    assert L.kv_tokens(a.handle, 0) == L.kv_tokens(b.handle, 0) == pre + steps
    assert L.kv_filled(a.handle, 0) == L.kv_filled(b.handle, 0)


def test_step_equals_append_then_decode_append_policy(L):
    """APPEND cache (no rotation), G=2 bf16 (one-pass, dot2 path): fill to capacity."""
    w = scaled(WORKLOADS["llama2_7b_layer"], name="step_append", batch=2, n_kv_heads=2, n_q_heads=4,
               n_sink=0, window=300, prefill=0, steps=300)
    a, b = _pair(L, w, L.LCD_APPEND, capacity=300)
    dev = "cuda"
    q_all = w.token_major_torch("q", 0, 0, 300, dev)
    k_all = w.token_major_torch("k", 0, 0, 300, dev)
    v_all = w.token_major_torch("v", 0, 0, 300, dev)
    oa = torch.empty((2, 4, 128), dtype=torch.float32, device=dev)
    ob = torch.empty_like(oa)
    for s in range(300):
        a.append(0, k_all[s].unsqueeze(2), v_all[s].unsqueeze(2))
        a.decode(0, q_all[s], oa)
        b.step(0, k_all[s], v_all[s], q_all[s], ob)
        assert torch.equal(oa, ob), f"step {s}"
    ka, va = a.layer_tensors(0)
    kb, vb = b.layer_tensors(0)
    assert torch.equal(ka, kb) and torch.equal(va, vb)
    # the cache is full: a further step is refused and changes nothing
    with pytest.raises(L.LcdError) as e:
        b.step(0, k_all[0], v_all[0], q_all[0], ob)
    assert e.value.name == "LCD_ECAPACITY"
    assert L.kv_tokens(b.handle, 0) == 300 and L.kv_filled(b.handle, 0) == 300


def test_step_rejects_other_policies_and_bad_arguments(L):
    cfg = L.cache_config(1, 4, 1, 128, L.LCD_BF16, L.LCD_H2O, capacity=64, n_recent=8)
    c = L.KVCache(cfg)
    k = torch.zeros((1, 1, 128), dtype=torch.bfloat16, device="cuda")
    q = torch.zeros((1, 4, 128), dtype=torch.bfloat16, device="cuda")
    out = torch.empty((1, 4, 128), dtype=torch.float32, device="cuda")
    with pytest.raises(L.LcdError) as e:
        c.step(0, k, k, q, out)
    assert e.value.name == "LCD_EUNSUPPORTED"
    cfg = L.cache_config(1, 4, 1, 128, L.LCD_BF16, L.LCD_SINK_RING, n_sink=4, window=60, rope=1)
    c = L.KVCache(cfg)
    with pytest.raises(L.LcdError) as e:
        L.decode_step(c.handle, 0, None, k, q, out, c.ws, c.ws_bytes)
    assert e.value.name == "LCD_EINVAL"
    with pytest.raises(L.LcdError) as e:
        L.decode_step(c.handle, 0, k, k, q, out, c.ws, 1)
    assert e.value.name == "LCD_ESIZE"
    assert L.kv_tokens(c.handle, 0) == 0

"""GPU: lcd_decode_step (append fused into the decode launch) against kv_append +
decode_attn on identical caches -- sink + ring, APPEND and H2O (token- and block-level,
the slot of a full cache chosen on the device) -- outputs, cache contents, H2O state and
counters bit for bit, and the error paths (nothing enqueued, counters unchanged)."""
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
    cfg = L.cache_config(1, 4, 1, 128, L.LCD_BF16, L.LCD_DUO, capacity=64, n_sink=4, window=8, retrieval=[[1]])
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


@pytest.mark.parametrize("G,D,dtype,bs,budget,recent,seeded", [
    (4, 128, "bf16", 0, 96, 12, False),   # two-pass kernel, token-level: fill, then evict every step
    (2, 128, "bf16", 0, 80, 9, False),    # one-pass kernel
    (4, 128, "bf16", 16, 64, 10, False),  # blocks of 16: reopened blocks, masked slots
    (1, 64, "f32", 32, 128, 40, False),   # one-pass fp32, blocks of 32
    (4, 128, "bf16", 0, 4096, 512, True),  # the seeded 128k budget state (B=4 rows)
])
def test_step_equals_append_then_decode_h2o(L, G, D, dtype, bs, budget, recent, seeded):
    """H2O: one fused launch per token (the slot of a full cache chosen on the device) against
    lcd_kv_append + lcd_decode_attn: outputs, K / V rows, positions, scores, victims and open
    blocks bit for bit at every step."""
    from synth.workloads import h2o_state_torch

    base = WORKLOADS["h2o_128k"]
    w = scaled(base, name=f"h2o_step_G{G}_bs{bs}", batch=4 if seeded else 2, n_kv_heads=2, n_q_heads=2 * G,
               head_dim=D, dtype=dtype, n_prompt=base.n_prompt if seeded else 0, budget=budget, n_recent=recent,
               steps=120)
    print(f"[h2o step vs append+decode] G={G} D={D} {dtype} bs={bs} budget={budget} seeded={seeded}", flush=True)
    a, b = _pair(L, w, L.LCD_H2O, capacity=budget, n_recent=recent, block_size=bs)
    dev = "cuda"
    t0 = 0
    if seeded:
        K, V, P, S = h2o_state_torch(w, dev)
        for c in (a, b):
            kv, vv = c.layer_tensors(0)
            pv, sv = c.h2o_tensors(0)
            kv.copy_(K)
            vv.copy_(V)
            pv.copy_(P)
            sv.copy_(S)
            L.kv_set_filled(c.handle, 0, budget, w.n_prompt)
        t0 = w.n_prompt
    q_all = w.token_major_torch("q", 0, t0, t0 + w.steps, dev)
    k_all = w.token_major_torch("k", 0, t0, t0 + w.steps, dev)
    v_all = w.token_major_torch("v", 0, t0, t0 + w.steps, dev)
    oa = torch.empty((w.batch, w.n_q_heads, D), dtype=torch.float32, device=dev)
    ob = torch.empty_like(oa)

    def state(c):
        k, v = c.layer_tensors(0)
        p, s = c.h2o_tensors(0)
        return k, v, p, s

    for s in range(w.steps):
        a.append(0, k_all[s].unsqueeze(2), v_all[s].unsqueeze(2))
        a.decode(0, q_all[s], oa)
        b.step(0, k_all[s], v_all[s], q_all[s], ob)
        assert torch.equal(oa, ob), f"step {s}: outputs differ"
        ka, va, pa, sa = state(a)
        kb, vb, pb, sb = state(b)
        filled = min(budget, (w.n_prompt if seeded else 0) + s + 1)
        live = pa[:, :, :filled] >= 0  # slots holding a token (emptied block slots hold stale rows)
        assert torch.equal(pa[:, :, :filled], pb[:, :, :filled]), f"step {s}: positions differ"
        assert torch.equal(sa[:, :, :filled], sb[:, :, :filled]), f"step {s}: scores differ"
        ka16, kb16 = ka[:, :, :filled].view(torch.int16), kb[:, :, :filled].view(torch.int16)
        va16, vb16 = va[:, :, :filled].view(torch.int16), vb[:, :, :filled].view(torch.int16)
        assert torch.equal(ka16[live], kb16[live]) and torch.equal(va16[live], vb16[live]), f"step {s}: rows differ"
    torch.cuda.synchronize()
    assert L.kv_tokens(a.handle, 0) == L.kv_tokens(b.handle, 0) == t0 + w.steps
    assert L.kv_filled(a.handle, 0) == L.kv_filled(b.handle, 0)

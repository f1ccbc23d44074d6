"""GPU parity: StreamingLLM sink + ring cache, kv_append + decode_attn vs the oracle.

Inputs come from the seeded generators in synth/ (identical bits on CPU and GPU);
expected values come from the fp64 oracle.  Tolerances: bf16 inputs with fp32
accumulation must be within 2e-3 max abs and 1e-2 per-row relative L2 error; the
fp32 tiny case is held to 1e-4 abs (its expected error is ~1e-6).
Ring-slot contents are compared bit-exactly.
"""
import numpy as np
import pytest

import oracle
from synth import WORKLOADS
from synth.workloads import scaled

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

ATOL_BF16, RTOL_ROW = 2e-3, 1e-2
ATOL_F32 = 1e-4


@pytest.fixture(scope="module")
def L():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    import long_context_decode_amd as lib

    return lib


def _cfg(L, w):
    return L.cache_config(w.batch, w.n_q_heads, w.n_kv_heads, w.head_dim,
                          L.LCD_F32 if w.dtype == "f32" else L.LCD_BF16, L.LCD_SINK_RING,
                          n_layers=w.n_layers, n_sink=w.n_sink, window=w.window, rope=1,
                          rope_base=w.rope_base)


def _oracle_out(w, layer, t, b, g):
    """fp64 oracle output of the G query heads of (b, kv head g) at token t."""
    G = w.group
    q = w.token_block("q", layer, [t], batches=[b], heads=np.arange(g * G, g * G + G))[0, :, 0, :]

    def kv(tokens):
        k = w.token_block("k", layer, tokens, batches=[b], heads=[g])[0]
        v = w.token_block("v", layer, tokens, batches=[b], heads=[g])[0]
        return k, v

    return oracle.streaming_decode(q, kv, t, w.n_sink, w.window, w.rope_base)


def _assert_close(got, ref, atol, where):
    err = np.abs(got - ref)
    row = np.linalg.norm(got - ref, axis=-1) / np.maximum(np.linalg.norm(ref, axis=-1), 1e-30)
    assert err.max() <= atol, f"{where}: max abs err {err.max():.3e} > {atol}"
    assert row.max() <= RTOL_ROW, f"{where}: row rel err {row.max():.3e} > {RTOL_ROW}"
    return err.max(), row.max()


def _run_stream(L, w, check_steps, sample_bg, layers=None, check_slots=False, fused=False):
    """Prefill w.prefill tokens in one bulk append, then decode w.steps tokens (with
    fused=True each step is one lcd_decode_step instead of kv_append + decode_attn)."""
    dev = "cuda"
    layers = list(range(w.n_layers)) if layers is None else layers
    cache = L.KVCache(_cfg(L, w))
    tol = ATOL_F32 if w.dtype == "f32" else ATOL_BF16
    for layer in layers:
        if w.prefill:
            k = w.token_block_torch("k", layer, 0, w.prefill, dev)
            v = w.token_block_torch("v", layer, 0, w.prefill, dev)
            cache.append(layer, k, v)
            del k, v
    steps = max(check_steps) + 1
    q_all = {l: w.token_major_torch("q", l, w.prefill, w.prefill + steps, dev) for l in layers}
    k_all = {l: w.token_major_torch("k", l, w.prefill, w.prefill + steps, dev) for l in layers}
    v_all = {l: w.token_major_torch("v", l, w.prefill, w.prefill + steps, dev) for l in layers}
    out = torch.empty((w.batch, w.n_q_heads, w.head_dim), dtype=torch.float32, device=dev)
    worst = 0.0
    for s in range(steps):
        t = w.prefill + s
        for layer in layers:
            if fused:
                cache.step(layer, k_all[layer][s], v_all[layer][s], q_all[layer][s], out)
            else:
                cache.append(layer, k_all[layer][s].unsqueeze(2), v_all[layer][s].unsqueeze(2))
                cache.decode(layer, q_all[layer][s], out)
            if s in check_steps:
                got = out.cpu().numpy().astype(np.float64)
                G = w.group
                for (b, g) in sample_bg:
                    ref = _oracle_out(w, layer, t, b, g)
                    e, _ = _assert_close(got[b, g * G:(g + 1) * G], ref, tol, f"t={t} layer={layer} b={b} g={g}")
                    worst = max(worst, e)
                if check_slots:
                    _check_ring_slots(L, cache, w, layer, t)
    torch.cuda.synchronize()
    return worst


def _check_ring_slots(L, cache, w, layer, t):
    """Every retained token sits, bit for bit, in the slot the ring definition names."""
    K, V = cache.layer_tensors(layer)
    Kh = K.cpu()
    toks = oracle.retained_tokens(t, w.n_sink, w.window)
    ref = w.token_block("k", layer, toks, f64=False)  # [b][h][n][d] stored bits / f32
    for i, a in enumerate(toks):
        slot = oracle.ring_slot(int(a), w.n_sink, w.window)
        assert L.kv_slot_of(cache.handle, layer, int(a)) == slot
        got = Kh[:, :, slot, :]
        if w.dtype == "f32":
            assert np.array_equal(got.numpy(), ref[:, :, i, :]), f"slot {slot} token {a}"
        else:
            assert np.array_equal(got.view(torch.int16).numpy().view(np.uint16), ref[:, :, i, :])
    pos = oracle.in_cache_positions(toks)
    for i, a in enumerate(toks):
        assert L.kv_rank_of(cache.handle, layer, oracle.ring_slot(int(a), w.n_sink, w.window)) == pos[i]


def test_tiny_fp32_stream_every_step(L):
    """4 q / 1 kv head, D=64, fp32, 4 sinks + 60 window, 512 tokens from empty: all steps."""
    w = WORKLOADS["tiny_streaming"]
    print(f"[tiny_streaming] {w.title}", flush=True)
    worst = _run_stream(L, w, check_steps=set(range(w.steps)), sample_bg=[(0, 0)], check_slots=False)
    print(f"  worst abs err {worst:.2e}")


def test_tiny_fp32_ring_slots_bit_exact(L):
    w = scaled(WORKLOADS["tiny_streaming"], steps=140)
    _run_stream(L, w, check_steps={0, 3, 4, 63, 64, 65, 127, 128, 139}, sample_bg=[(0, 0)], check_slots=True)


@pytest.mark.parametrize("G,D,S,W,pre,steps", [
    (1, 128, 4, 300, 700, 40),    # multi-split, wrapped ring, MHA
    (4, 128, 4, 252, 100, 200),   # growth phase then wrap
    (6, 256, 4, 1020, 1100, 12),  # GQA 24/4 shape, D=256
    (8, 64, 2, 190, 0, 260),      # G=8, D=64, from empty
    (2, 128, 0, 130, 300, 10),    # no sinks: plain window attention
])
def test_bf16_shapes(L, G, D, S, W, pre, steps):
    w = scaled(WORKLOADS["llama2_7b_layer"], name=f"bf16_G{G}_D{D}", batch=2, n_kv_heads=2,
               n_q_heads=2 * G, head_dim=D, n_sink=S, window=W, prefill=pre, steps=steps)
    checks = {0, 1, steps - 1} | {s for s in range(steps) if (pre + s) % W in (0, 1, W - 1)}
    print(f"[bf16 G={G} D={D} S={S} W={W} prefill={pre}] checks {sorted(checks)}", flush=True)
    _run_stream(L, w, checks, sample_bg=[(0, 0), (1, 1)], check_slots=True)


def test_llama2_layer_full_size_fused_step(L):
    """The benchmarked step: one lcd_decode_step per token (append fused into the decode
    launch) on the full Llama-2-shaped layer, sampled heads against the oracle, ring slots
    checked bit for bit."""
    w = scaled(WORKLOADS["llama2_7b_layer"], steps=2050)
    checks = {0, 1, 2043, 2044, 2049}
    print(f"[llama2_7b_layer fused] checks {sorted(checks)}", flush=True)
    rng = np.random.default_rng(1)
    sample = [(0, 0), (15, 31)] + [tuple(x) for x in rng.integers(0, [16, 32], (2, 2))]
    worst = _run_stream(L, w, checks, sample_bg=sample, fused=True)
    print(f"  worst abs err {worst:.2e}")


@pytest.mark.parametrize("G,D,S,W,pre,steps", [
    (4, 128, 4, 252, 100, 200),   # growth phase then wrap, two-pass kernel
    (6, 256, 4, 1020, 1100, 12),  # D=256, several splits
    (1, 64, 2, 190, 0, 260),      # from empty
])
def test_fused_step_bf16_shapes(L, G, D, S, W, pre, steps):
    w = scaled(WORKLOADS["llama2_7b_layer"], name=f"fused_G{G}_D{D}", batch=2, n_kv_heads=2,
               n_q_heads=2 * G, head_dim=D, n_sink=S, window=W, prefill=pre, steps=steps)
    checks = {0, 1, steps - 1} | {s for s in range(steps) if (pre + s) % W in (0, 1, W - 1)}
    print(f"[fused bf16 G={G} D={D} S={S} W={W} prefill={pre}] checks {sorted(checks)}", flush=True)
    _run_stream(L, w, checks, sample_bg=[(0, 0), (1, 1)], check_slots=True, fused=True)


@pytest.mark.parametrize("G,D,steps", [
    (1, 128, 130),  # one-pass kernel: anchors every 128 keys of a lane group
    (4, 128, 200),  # two-pass, RoPE at G = 4: anchors every 192 keys
    (6, 256, 70),   # two-pass, G = 6, D = 256: anchors every 64 keys
    (8, 128, 40),   # two-pass, G = 8: a table row every iteration
])
def test_rope_rows_across_breakpoints(L, G, D, steps):
    """Keys' RoPE table rows are carried from key to key by angle addition and read only at
    anchors and where a rank breakpoint (the sink boundary, the ring's oldest slot) interrupts
    the sequence.  A wrapped 4 + 2044 ring of 16 rows x 8 KV heads (4 splits of 512 slots per
    row and head) is stepped while the oldest slot sweeps every phase of the anchor period
    inside a split, and every step is checked."""
    w = scaled(WORKLOADS["llama2_7b_layer"], name=f"rope_rows_G{G}_D{D}", batch=16, n_kv_heads=8,
               n_q_heads=8 * G, head_dim=D, n_sink=4, window=2044, prefill=2300, steps=steps)
    print(f"[rope rows G={G} D={D}] {steps} steps, every step checked", flush=True)
    _run_stream(L, w, set(range(steps)), sample_bg=[(0, 0), (9, 5)], fused=True)


def test_many_splits_grouped_merge(L):
    """B=1, 4/1 heads, D=128, 4+8188 wrapped: the plan gives more than 64 splits of one
    (row, KV head), so the merge stages its per-split weights in more than one group."""
    w = scaled(WORKLOADS["llama2_7b_layer"], name="bf16_many_splits", batch=1, n_kv_heads=1, n_q_heads=4,
               n_sink=4, window=8188, prefill=8200, steps=3)
    print("[many splits] B=1, 4/1 heads, 4+8188", flush=True)
    _run_stream(L, w, {0, 2}, sample_bg=[(0, 0)])


def test_llama2_layer_full_size_sampled(L):
    """B=16, 32/32 heads, D=128, 4+2044: prefill 2048, decode through two ring wraps."""
    w = WORKLOADS["llama2_7b_layer"]
    checks = {0, 1, 2043, 2044, 2045, 4088, 4100}
    print(f"[llama2_7b_layer] {w.title}; checks {sorted(checks)}", flush=True)
    rng = np.random.default_rng(0)
    sample = [(0, 0), (15, 31)] + [tuple(x) for x in rng.integers(0, [16, 32], (2, 2))]
    worst = _run_stream(L, w, checks, sample_bg=sample)
    print(f"  worst abs err {worst:.2e}")


def test_llama3_layer_full_size_sampled(L):
    """B=16, 32/8 heads (G=4), D=128, 4+8188, RoPE base 5e5: prefill 8192, then wrapped steps."""
    w = WORKLOADS["llama3_8b_layer"]
    checks = {0, 1, 37}
    print(f"[llama3_8b_layer] {w.title}; checks {sorted(checks)}", flush=True)
    worst = _run_stream(L, w, checks, sample_bg=[(0, 0), (15, 7), (9, 3)])
    print(f"  worst abs err {worst:.2e}")


def test_gqa_long_full_size_sampled(L):
    """B=16, 24/4 heads, D=256, 4+32764, 16 layers allocated; layers 0 and 15 checked."""
    w = WORKLOADS["gqa_long"]
    print(f"[gqa_long] {w.title}", flush=True)
    worst = _run_stream(L, w, check_steps={0, 2}, sample_bg=[(0, 0), (15, 3), (7, 2)], layers=[0, 15])
    print(f"  worst abs err {worst:.2e}")


def test_decode_is_deterministic(L):
    w = scaled(WORKLOADS["llama2_7b_layer"], batch=2, n_q_heads=8, n_kv_heads=2, window=700, prefill=900, steps=1)
    outs = []
    for _ in range(2):
        cache = L.KVCache(_cfg(L, w))
        cache.append(0, w.token_block_torch("k", 0, 0, 900, "cuda"), w.token_block_torch("v", 0, 0, 900, "cuda"))
        q = w.token_major_torch("q", 0, 899, 900, "cuda")[0]
        out = torch.empty((2, 8, 128), dtype=torch.float32, device="cuda")
        cache.decode(0, q, out)
        outs.append(out.cpu())
    assert torch.equal(outs[0], outs[1])


def test_gqa_long_full_size_bit_identical_reruns(L):
    """The full-size split merge is deterministic: one layer of the B=16, 24/4 heads,
    D=256, 4 + 32764 cache (the decode plan's full split count), decoded by two caches
    filled with the same tokens -- once with lcd_decode_attn after an append, once with
    the fused lcd_decode_step -- and re-decoded three times with different workspace
    buffers, gives bit-identical outputs every time."""
    w = scaled(WORKLOADS["gqa_long"], n_layers=1)
    dev = "cuda"
    pre = w.prefill
    print(f"[gqa_long determinism] one layer of {w.title}", flush=True)
    k = w.token_block_torch("k", 0, 0, pre, dev)
    v = w.token_block_torch("v", 0, 0, pre, dev)
    a, b = L.KVCache(_cfg(L, w)), L.KVCache(_cfg(L, w))
    a.append(0, k, v)
    b.append(0, k, v)
    del k, v
    q = w.token_major_torch("q", 0, pre, pre + 1, dev)[0]
    kn = w.token_major_torch("k", 0, pre, pre + 1, dev)[0]
    vn = w.token_major_torch("v", 0, pre, pre + 1, dev)[0]
    outs = []
    a.append(0, kn.unsqueeze(2), vn.unsqueeze(2))
    for i in range(3):
        ws = torch.empty(a.ws_bytes, dtype=torch.uint8, device=dev)  # a fresh workspace each time
        out = torch.empty((w.batch, w.n_q_heads, w.head_dim), dtype=torch.float32, device=dev)
        L.decode_attn(a.handle, 0, q, out, ws, a.ws_bytes)
        outs.append(out)
    ob = torch.empty((w.batch, w.n_q_heads, w.head_dim), dtype=torch.float32, device=dev)
    b.step(0, kn, vn, q, ob)
    outs.append(ob)
    torch.cuda.synchronize()
    for i, o in enumerate(outs[1:], 1):
        assert torch.equal(outs[0].view(torch.int32), o.view(torch.int32)), f"run {i} differs"
    assert torch.isfinite(outs[0]).all()

"""GPU parity: DuoAttention mixed retrieval / streaming heads in one decode launch
([KVC] "Decomposição funcional com o DuoAttention") vs the fp64 oracle.

Retrieval heads keep and attend every token; streaming heads keep their sinks and a
rolling window.  Inputs from synth/ (identical bits on CPU and GPU); expected values
from oracle.duo_decode.  Tolerances as for the other decode paths: bf16 inputs within
2e-3 max abs and 1e-2 per-row relative L2 error; fp32 inputs within 1e-4 abs.
"""
import numpy as np
import pytest

import oracle
from synth import WORKLOADS
from synth.workloads import scaled

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

ATOL_BF16, RTOL_ROW, ATOL_F32 = 2e-3, 1e-2, 1e-4
BASE = WORKLOADS["duo_128k"]


@pytest.fixture(scope="module")
def L():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    import long_context_decode_amd as lib

    return lib


def _cfg(L, w):
    return L.cache_config(w.batch, w.n_q_heads, w.n_kv_heads, w.head_dim,
                          L.LCD_F32 if w.dtype == "f32" else L.LCD_BF16, L.LCD_DUO, n_layers=w.n_layers,
                          n_sink=w.n_sink, window=w.window, capacity=w.capacity, retrieval=w.retrieval)


def _oracle(w, layer, t, b):
    q = w.token_block("q", layer, [t], batches=[b])[0, :, 0, :]

    def kv(g, toks):
        return (w.token_block("k", layer, toks, batches=[b], heads=[g])[0, 0],
                w.token_block("v", layer, toks, batches=[b], heads=[g])[0, 0])

    return oracle.duo_decode(q, kv, t, w.retrieval[layer], w.n_sink, w.window)


def _check(got, ref, atol, where):
    err = np.abs(got - ref)
    row = np.linalg.norm(got - ref, axis=-1) / np.maximum(np.linalg.norm(ref, axis=-1), 1e-30)
    assert err.max() <= atol, f"{where}: max abs err {err.max():.3e} > {atol}"
    assert row.max() <= RTOL_ROW, f"{where}: row rel err {row.max():.3e} > {RTOL_ROW}"


def _run(L, w, bulk, check_steps, rows=None):
    """Bulk-append `bulk` tokens per layer, then append + decode one token at a time."""
    dev = "cuda"
    cache = L.KVCache(_cfg(L, w))
    atol = ATOL_F32 if w.dtype == "f32" else ATOL_BF16
    rows = range(w.batch) if rows is None else rows
    for layer in range(w.n_layers):
        if bulk:
            cache.append(layer, w.token_block_torch("k", layer, 0, bulk, dev),
                         w.token_block_torch("v", layer, 0, bulk, dev))
    steps = max(check_steps) + 1
    q = {l: w.token_major_torch("q", l, bulk, bulk + steps, dev) for l in range(w.n_layers)}
    k = {l: w.token_major_torch("k", l, bulk, bulk + steps, dev) for l in range(w.n_layers)}
    v = {l: w.token_major_torch("v", l, bulk, bulk + steps, dev) for l in range(w.n_layers)}
    out = torch.empty((w.batch, w.n_q_heads, w.head_dim), dtype=torch.float32, device=dev)
    for s in range(steps):
        t = bulk + s
        for layer in range(w.n_layers):
            cache.append(layer, k[layer][s].unsqueeze(2), v[layer][s].unsqueeze(2))
            cache.decode(layer, q[layer][s], out)
            if s in check_steps:
                got = out.cpu().numpy()
                for b in rows:
                    _check(got[b], _oracle(w, layer, t, b), atol, f"t={t} layer={layer} b={b}")
    assert L.kv_tokens(cache.handle, 0) == bulk + steps
    cache.close()


def test_duo_small_every_step(L):
    """2 layers (mixed, all streaming), G=2 (one-pass kernel), 4 sinks + 16 window:
    from empty through the window filling and wrapping, every step checked."""
    w = scaled(BASE, name="duo_small", batch=2, n_q_heads=8, n_kv_heads=4, n_sink=4, window=16, prefill=0,
               steps=60, n_layers=2, retrieval=((1, 0, 0, 1), (0, 0, 0, 0)))
    print("[duo] small G=2", flush=True)
    _run(L, w, bulk=0, check_steps=set(range(60)))


def test_duo_bulk_prefill_two_pass(L):
    """G=4 (two-pass kernel), a bulk append that wraps the streaming window inside one
    call, then single steps; layers all-retrieval and mixed."""
    w = scaled(BASE, name="duo_bulk", batch=2, n_q_heads=16, n_kv_heads=4, n_sink=4, window=24, prefill=100,
               steps=12, n_layers=2, retrieval=((1, 1, 1, 1), (0, 1, 0, 0)))
    print("[duo] bulk G=4", flush=True)
    _run(L, w, bulk=100, check_steps={0, 1, 5, 11})


def test_duo_fp32_d64_and_splits(L):
    """fp32, D=64, G=8, one retrieval head of 8: the retrieval head spans several
    splits while streaming heads take one or two (early-exiting workgroups)."""
    w = scaled(BASE, name="duo_f32", batch=1, n_q_heads=16, n_kv_heads=2, head_dim=64, dtype="f32", n_sink=4,
               window=64, prefill=900, steps=4, n_layers=1, retrieval=((1, 0),))
    print("[duo] fp32 G=8", flush=True)
    _run(L, w, bulk=900, check_steps={0, 3})


def test_duo_d256_g6(L):
    w = scaled(BASE, name="duo_d256", batch=2, n_q_heads=12, n_kv_heads=2, head_dim=256, n_sink=4, window=64,
               prefill=700, steps=3, n_layers=1, retrieval=((0, 1),))
    print("[duo] D=256 G=6", flush=True)
    _run(L, w, bulk=700, check_steps={0, 2})


def test_duo_capacity_is_enforced(L):
    w = scaled(BASE, name="duo_cap", batch=1, n_q_heads=4, n_kv_heads=2, n_sink=4, window=8, prefill=10,
               steps=0, n_layers=1, retrieval=((1, 0),))
    cache = L.KVCache(_cfg(L, w))
    k = w.token_block_torch("k", 0, 0, 10, "cuda")
    cache.append(0, k, k)
    one = k[:, :, :1].contiguous()
    with pytest.raises(L.LcdError) as e:
        cache.append(0, one, one)
    assert e.value.name == "LCD_ECAPACITY"
    with pytest.raises(L.LcdError) as e:
        cache.layer_tensors(0)
    assert e.value.name == "LCD_EUNSUPPORTED"
    cache.close()


def test_duo_full_size_sampled(L):
    """The 128k workload (B=16, 32/8 heads, 2 retrieval heads per layer with the whole
    131072-token history, 6 streaming heads), prefilled in bulk chunks, two decode
    steps; sampled rows checked against the oracle."""
    w = BASE
    dev = "cuda"
    cache = L.KVCache(_cfg(L, w))
    chunk = 8192
    print("[duo] full size prefill", flush=True)
    for t0 in range(0, w.prefill, chunk):
        t1 = min(w.prefill, t0 + chunk)
        cache.append(0, w.token_block_torch("k", 0, t0, t1, dev), w.token_block_torch("v", 0, t0, t1, dev))
    q = w.token_major_torch("q", 0, w.prefill, w.prefill + 2, dev)
    k = w.token_major_torch("k", 0, w.prefill, w.prefill + 2, dev)
    v = w.token_major_torch("v", 0, w.prefill, w.prefill + 2, dev)
    out = torch.empty((w.batch, w.n_q_heads, w.head_dim), dtype=torch.float32, device=dev)
    for s in range(2):
        cache.append(0, k[s].unsqueeze(2), v[s].unsqueeze(2))
        cache.decode(0, q[s], out)
    got = out.cpu().numpy()
    t = w.prefill + 1
    for b in (0, 11):
        print(f"[duo] full size oracle b={b}", flush=True)
        _check(got[b], _oracle(w, 0, t, b), ATOL_BF16, f"full t={t} b={b}")
    cache.close()

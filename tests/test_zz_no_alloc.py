"""GPU: lcd_decode_step_noalloc (split partials in the library's device scratch, no
workspace argument) against lcd_decode_step with a caller workspace, bit for bit.

Two calls of the allocation-free entry point in a row, the second on a smaller cache,
each compared with lcd_decode_step on an identical cache: outputs and the cache contents
after the step.  A cache whose workspace exceeds the 32 MiB scratch is refused with
LCD_ESIZE and nothing enqueued (its token counter unchanged)."""
import numpy as np
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


def _pair(L, w):
    """Two identical prefilled caches and the inputs of the next step."""
    dt = L.LCD_F32 if w.dtype == "f32" else L.LCD_BF16
    cfg = L.cache_config(w.batch, w.n_q_heads, w.n_kv_heads, w.head_dim, dt, L.LCD_SINK_RING, n_sink=w.n_sink,
                         window=w.window, rope=1, rope_base=w.rope_base)
    caches = [L.KVCache(cfg, device="cuda") for _ in range(2)]
    if w.prefill:
        k = w.token_block_torch("k", 0, 0, w.prefill, "cuda")
        v = w.token_block_torch("v", 0, 0, w.prefill, "cuda")
        for c in caches:
            c.append(0, k, v)
    t = w.prefill
    step = [w.token_major_torch(x, 0, t, t + 1, "cuda")[0] for x in ("k", "v", "q")]
    return caches, step


def _compare(L, w):
    print(f"[no-alloc] {w.name}: B={w.batch} {w.n_q_heads}/{w.n_kv_heads} heads D={w.head_dim} "
          f"C={w.n_sink + w.window} prefill {w.prefill}", flush=True)
    (ref, mine), (k, v, q) = _pair(L, w)
    shape = (w.batch, w.n_q_heads, w.head_dim)
    out_ref = torch.full(shape, float("nan"), dtype=torch.float32, device="cuda")
    out = torch.full(shape, float("nan"), dtype=torch.float32, device="cuda")
    ref.step(0, k, v, q, out_ref)
    L.decode_step_noalloc(mine.handle, 0, k, v, q, out)
    torch.cuda.synchronize()
    assert torch.equal(out, out_ref), f"{w.name}: outputs differ"
    assert torch.isfinite(out).all()
    filled = min(w.prefill + 1, w.n_sink + w.window)  # slots written so far (the rest are uninitialised)
    for a, b in zip(ref.layer_tensors(0), mine.layer_tensors(0)):
        a, b = a[:, :, :filled], b[:, :, :filled]
        assert torch.equal(a.view(torch.int16) if a.dtype == torch.bfloat16 else a,
                           b.view(torch.int16) if b.dtype == torch.bfloat16 else b)
    assert L.kv_tokens(mine.handle, 0) == L.kv_tokens(ref.handle, 0) == w.prefill + 1
    for c in (ref, mine):
        c.close()


def test_noalloc_matches_decode_step_two_calls(L):
    # first call: the Llama-3-shaped layer (G = 4, two-pass kernel, 4 splits, ring wrapped)
    big = scaled(WORKLOADS["llama3_8b_layer"], name="noalloc_big", batch=8, prefill=9000, steps=1)
    _compare(L, big)
    # second call, smaller: tiny fp32 cache (G = 4, one split), growing phase
    small = scaled(WORKLOADS["tiny_streaming"], name="noalloc_small", prefill=37, steps=1)
    _compare(L, small)


def test_noalloc_refuses_a_workspace_above_the_scratch(L):
    # 64 rows x 64 query heads x D 256 over 16384 slots (9 splits): a 36 MiB workspace
    cfg = L.cache_config(64, 64, 8, 256, L.LCD_BF16, L.LCD_SINK_RING, n_sink=4, window=16380, rope=1)
    _, _, ws = L.cache_sizes(cfg)
    assert ws > 32 << 20
    c = L.KVCache(cfg, device="cuda")
    dev = "cuda"
    k = torch.zeros((64, 8, 256), dtype=torch.bfloat16, device=dev)
    q = torch.zeros((64, 64, 256), dtype=torch.bfloat16, device=dev)
    out = torch.zeros((64, 64, 256), dtype=torch.float32, device=dev)
    with pytest.raises(L.LcdError) as e:
        L.decode_step_noalloc(c.handle, 0, k, k, q, out)
    assert e.value.name == "LCD_ESIZE" and "32" in str(e.value)
    assert L.kv_tokens(c.handle, 0) == 0
    torch.cuda.synchronize()
    c.close()

"""GPU parity of the two-pass kernel's bf16 V pass at ragged range lengths.

The V pass runs on the matrix cores over tiles of 32 keys, each wave taking 64 dims of the
tiles of its key group (4, 2 or 1 key groups at D = 64, 128, 256).  Attended-slot counts
around the tile and key-group boundaries leave partial tiles, key groups with one tile or
none, and (with the split plan spreading a few rows over many workgroups) ragged last
splits.  One decode step after a prefill of n - 1 tokens (RoPE at in-cache ranks, growth
phase), every (row, KV head) against the fp64 oracle at the bf16 tolerances.
"""
import numpy as np
import pytest

import oracle
from synth import WORKLOADS
from synth.workloads import scaled

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

ATOL, RTOL_ROW = 2e-3, 1e-2


@pytest.fixture(scope="module")
def L():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    import long_context_decode_amd as lib

    return lib


@pytest.mark.parametrize("G,D", [(4, 64), (4, 128), (6, 256), (8, 128), (8, 256)])
@pytest.mark.parametrize("n", [1, 31, 32, 33, 95, 129, 257, 600, 1111])
def test_vpass_ragged_lengths(L, G, D, n):
    S, W = 4, 2044
    pre = n - 1
    w = scaled(WORKLOADS["llama2_7b_layer"], name=f"vtail_G{G}_D{D}_n{n}", batch=2, n_kv_heads=2,
               n_q_heads=2 * G, head_dim=D, n_sink=S, window=W, prefill=pre, steps=1)
    print(f"[vpass tails] G={G} D={D} n={n}", flush=True)
    cfg = L.cache_config(w.batch, w.n_q_heads, w.n_kv_heads, D, L.LCD_BF16, L.LCD_SINK_RING, n_sink=S, window=W,
                         rope=1, rope_base=w.rope_base)
    c = L.KVCache(cfg)
    dev = "cuda"
    c.append(0, w.token_block_torch("k", 0, 0, n, dev), w.token_block_torch("v", 0, 0, n, dev))
    q = w.token_major_torch("q", 0, pre, pre + 1, dev)[0]
    out = torch.empty((w.batch, w.n_q_heads, D), dtype=torch.float32, device=dev)
    c.decode(0, q, out)
    got = out.cpu().numpy()
    assert np.isfinite(got).all()
    for b in range(w.batch):
        for g in range(w.n_kv_heads):
            qq = w.token_block("q", 0, [pre], batches=[b], heads=np.arange(g * G, g * G + G))[0, :, 0, :]

            def kv(tokens, b=b, g=g):  # [1][tokens][D]: the KV head's rows
                return (w.token_block("k", 0, tokens, batches=[b], heads=[g])[0],
                        w.token_block("v", 0, tokens, batches=[b], heads=[g])[0])

            ref = oracle.streaming_decode(qq, kv, pre, S, W, w.rope_base)
            mine = got[b, g * G:(g + 1) * G]
            err = np.abs(mine - ref)
            row = np.linalg.norm(mine - ref, axis=-1) / np.maximum(np.linalg.norm(ref, axis=-1), 1e-30)
            assert err.max() <= ATOL, f"b={b} g={g}: max abs err {err.max():.3e}"
            assert row.max() <= RTOL_ROW, f"b={b} g={g}: row rel err {row.max():.3e}"

"""The seeded input generator: determinism, CPU/torch agreement, rounding (CPU only)."""
import numpy as np
import torch

from synth import NormalStream, WORKLOADS, bf16_bits_to_f32, f32_to_bf16_bits, hash_positions, mix32
from synth.gen import MASK32, mix32_np, uniform_bits


def test_hash_fast_path_equals_portable_path():
    x = np.random.default_rng(0).integers(0, 2**32, 200_000)
    assert np.array_equal(mix32(x), mix32_np(x))
    idx = np.array([0, 1, 2**32 - 1, 2**32, 2**33 + 17, 5 * 2**32 + 3], dtype=np.int64)
    ref = mix32((idx & MASK32) ^ mix32(((idx >> 32) + 99) & MASK32))
    assert np.array_equal(uniform_bits(99, idx), ref)


def test_torch_path_gives_identical_bits():
    for dtype in ("bf16", "f32"):
        st = NormalStream(3, "t/x", dtype)
        idx = np.arange(0, 300_000, 7, dtype=np.int64)
        a = st.stored(idx)
        b = st.torch_stored(torch.from_numpy(idx))
        if dtype == "bf16":
            b = b.view(torch.int16).numpy().view(np.uint16)
        else:
            b = b.numpy()
        assert np.array_equal(a, b)
    st = NormalStream(3, "t/y", "bf16")
    idx = np.arange(1000, dtype=np.int64)
    a = st.stored(idx, 3.0)
    b = st.torch_stored(torch.from_numpy(idx), 3.0).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(a, b)


def test_bf16_rounding_matches_torch():
    rng = np.random.default_rng(1)
    x = np.concatenate([rng.standard_normal(100_000).astype(np.float32) * 7,
                        np.array([1.0 + 2**-8, 1.0 + 3 * 2**-8, -1.0 - 2**-8, 0.0, 3.0e38], np.float32)])
    ours = f32_to_bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)
    np.testing.assert_array_equal(bf16_bits_to_f32(ours), torch.from_numpy(x).to(torch.bfloat16).float().numpy())


def test_streams_are_deterministic_and_distinct():
    a = NormalStream(0, "k", "bf16").values(np.arange(5000))
    b = NormalStream(0, "k", "bf16").values(np.arange(5000))
    c = NormalStream(0, "v", "bf16").values(np.arange(5000))
    d = NormalStream(1, "k", "bf16").values(np.arange(5000))
    assert np.array_equal(a, b) and not np.array_equal(a, c) and not np.array_equal(a, d)
    v = NormalStream(0, "big", "f32").values(np.arange(400_000))
    assert abs(v.mean()) < 0.01 and abs(v.std() - 1.0) < 0.01


def test_positions_and_workload_shapes():
    p = hash_positions(0, "x", 1000, 20)
    assert len(np.unique(p)) == 20 and p.min() >= 0 and p.max() < 1000 and np.all(np.diff(p) > 0)
    w = WORKLOADS["gqa_long"]
    k = w.token_block("k", 0, np.arange(6), batches=[1], heads=[2])
    k1 = WORKLOADS["llama2_7b_layer"].token_block("k", 0, np.arange(6), batches=[1], heads=[2])
    assert k.shape == (1, 1, 6, 256) and k1.shape == (1, 1, 6, 128)
    # sink keys are the base values scaled by 4 (exact in bf16)
    base = NormalStream(w.seed, "gqa_long/L0/k", "bf16")
    from synth.gen import flat_index_np
    idx = flat_index_np(w.token_shape("k"), [np.arange(6), [1], [2], np.arange(256)])
    raw = base.values(idx)[:, 0, 0, :]
    np.testing.assert_array_equal(k[0, 0, :4], 4 * raw[:4])
    np.testing.assert_array_equal(k[0, 0, 4:], raw[4:])
    s = WORKLOADS["snapkv_32k"]
    assert len(s.snapkv_plants(0, 3)) == 655 and s.k_keep == 5243


def test_token_block_torch_matches_numpy():
    w = WORKLOADS["gqa_long"]
    t = w.token_block_torch("k", 1, 2, 7, "cpu")  # [b][h][t][d]
    n = w.token_block("k", 1, np.arange(2, 7), f64=False)
    assert np.array_equal(t.view(torch.int16).numpy().view(np.uint16), n)

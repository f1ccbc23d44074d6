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


def test_chunked_torch_generators_match_numpy():
    """Whole-tensor torch generation (few large chunks) gives the numpy bits, across chunk
    edges, sink scaling, planted rows and seeded H2O state."""
    from synth.workloads import h2o_state_torch, scaled

    def u16(t):
        return t.view(torch.int16).numpy().view(np.uint16)

    w = WORKLOADS["gqa_long"]
    t = w.token_block_torch("k", 1, 0, 9, "cpu", max_elems=3 * 16 * 4 * 256)  # 3 chunks, sinks inside
    assert np.array_equal(u16(t), w.token_block("k", 1, np.arange(0, 9), f64=False))
    t = w.token_major_torch("k", 2, 0, 9, "cpu", max_elems=2 * 16 * 4 * 256)
    assert np.array_equal(u16(t), w.token_block("k", 2, np.arange(0, 9), f64=False).transpose(2, 0, 1, 3))
    s = scaled(WORKLOADS["snapkv_32k"], name="sk", n_q_heads=3, n_kv_heads=3, n_prompt=500, l_obs=8, k_keep=40)
    for tn in ("q_obs", "k", "v"):
        tt = u16(s.snapkv_tensor_torch(tn, "cpu"))
        for h in range(3):
            assert np.array_equal(tt[0, h], s.snapkv_tensor(tn, 0, h, f64=False)), tn
    p = scaled(WORKLOADS["h2o_prompt_128k"], name="pp", batch=2, n_q_heads=4, n_kv_heads=2, n_prompt=300)
    for tn in ("q", "k"):
        tt = u16(p.prompt_tensor_torch(tn, "cpu"))
        for b in range(2):
            for h in range(tt.shape[1]):
                assert np.array_equal(tt[b, h], p.prompt_tensor(tn, b, h, f64=False))
    hw = scaled(WORKLOADS["h2o_128k"], name="hh", batch=2, n_kv_heads=2, n_q_heads=8, n_prompt=3000, budget=256,
                n_recent=32, steps=10)
    K, V, P, S = h2o_state_torch(hw, "cpu")
    for b in range(2):
        for g in range(2):
            pos, sc, _ = hw.h2o_initial_state(b, g)
            assert np.array_equal(P[b, g].numpy(), pos) and np.array_equal(S[b, g].numpy(), sc)
            assert np.array_equal(u16(K[b, g]), hw.h2o_kv("k", b, g, pos, f64=False))
            assert np.array_equal(u16(V[b, g]), hw.h2o_kv("v", b, g, pos, f64=False))


def test_chunks_never_cross_a_2pow32_element_boundary():
    from synth.workloads import _chunks

    per = 2**30 + 7
    lst = list(_chunks(0, 100, per, 2**31))
    assert lst[0][0] == 0 and lst[-1][1] == 100
    assert all(lst[i][1] == lst[i + 1][0] for i in range(len(lst) - 1))
    for a, e in lst:
        assert e - a == 1 or (a * per) >> 32 == (e * per - 1) >> 32, (a, e)
    st = NormalStream(0, "x", "bf16")
    idx = torch.arange(2**32 - 50, 2**32 + 50)
    two = torch.cat([st.torch_stored(idx[:50], span=(2**32 - 50, 2**32)),
                     st.torch_stored(idx[50:], span=(2**32, 2**32 + 50))])
    assert np.array_equal(two.view(torch.int16).numpy().view(np.uint16), st.stored(idx.numpy()))

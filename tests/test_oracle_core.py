"""Pins of the oracle's KV sizing, RoPE and attention (CPU only).

Each test checks the oracle against something other than itself: a value printed
by the pages (tests/golden), a closed form, an invariant or a textbook special
case.
"""
import json
import os

import numpy as np
import pytest
import scipy.special

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


# ----------------------------------------------------------------------------- KV size
def test_kv_size_matches_worked_example():
    g = _golden("kv_size_qwen_example.json")
    per_tok = oracle.kv_cache_bytes(1, g["n_kv_heads"], g["head_dim"], 1, g["bytes_per_elem"])
    assert per_tok == g["per_token_per_layer_bytes"] == 4 * 1024
    assert oracle.kv_cache_bytes(g["all_layers"], g["n_kv_heads"], g["head_dim"], 1,
                                 g["bytes_per_elem"]) == g["per_token_all_layers_bytes"]
    assert oracle.kv_cache_bytes(g["all_layers"], g["n_kv_heads"], g["head_dim"], g["context_tokens"],
                                 g["bytes_per_elem"]) == g["full_context_all_layers_bytes"] == 64 * 2**30
    assert oracle.kv_cache_bytes(g["attention_layers"], g["n_kv_heads"], g["head_dim"],
                                 g["context_tokens"], g["bytes_per_elem"]) \
        == g["full_context_attention_layers_bytes"] == 16 * 2**30


def test_kv_size_batch_factor_hundreds_of_gb():
    # 16 requests at 128k tokens need "hundreds of gigabytes" (KVC introduction);
    # a Llama-3-8B-like shape (32 layers, 8 KV heads, D=128, fp16) is assumed.
    b = oracle.kv_cache_bytes(32, 8, 128, 131072, 2, batch=16)
    assert b == 256 * 2**30
    assert 100e9 <= b < 1000e9
    assert oracle.kv_cache_bytes(32, 8, 128, 131072, 2, batch=1) * 16 == b


# ----------------------------------------------------------------------------- RoPE
def test_rope_position_zero_is_identity():
    x = np.random.default_rng(0).standard_normal((5, 64))
    np.testing.assert_array_equal(oracle.apply_rope(x, 0, 10000.0), x)


def test_rope_two_dims_is_textbook_plane_rotation():
    # D = 2: a single pair with frequency base**0 = 1 rad per position.
    rng = np.random.default_rng(1)
    for p in [1, 2, 7, 1000]:
        x = rng.standard_normal(2)
        R = np.array([[np.cos(p), -np.sin(p)], [np.sin(p), np.cos(p)]])
        np.testing.assert_allclose(oracle.apply_rope(x, p, 10000.0), R @ x, rtol=0, atol=1e-14)


def test_rope_pairs_and_frequencies_half_layout():
    # D = 4, base 10000: pair i=0 is (x0, x2) at 1 rad/pos, pair i=1 is (x1, x3) at 0.01 rad/pos.
    e1 = np.array([0.0, 1.0, 0.0, 0.0])
    out = oracle.apply_rope(e1, 100, 10000.0)
    np.testing.assert_allclose(out, [0.0, np.cos(1.0), 0.0, np.sin(1.0)], atol=1e-14)
    e0 = np.array([1.0, 0.0, 0.0, 0.0])
    np.testing.assert_allclose(oracle.apply_rope(e0, 3, 10000.0), [np.cos(3), 0, np.sin(3), 0], atol=1e-14)
    # interleaved layout pairs (x0, x1) and (x2, x3)
    np.testing.assert_allclose(oracle.apply_rope(e0, 3, 10000.0, "interleaved"),
                               [np.cos(3), np.sin(3), 0, 0], atol=1e-14)


def test_rope_inv_freq_closed_form():
    f = oracle.rope_inv_freq(128, 10000.0)
    assert f[0] == 1.0
    np.testing.assert_allclose(f[32], 10000.0 ** -0.5, rtol=1e-15)
    np.testing.assert_allclose(f[-1], 10000.0 ** (-126 / 128), rtol=1e-15)


def test_rope_preserves_norm_and_composes():
    rng = np.random.default_rng(2)
    x = rng.standard_normal((16, 128))
    p = rng.integers(0, 40000, 16)
    y = oracle.apply_rope(x, p, 10000.0)
    np.testing.assert_allclose(np.linalg.norm(y, axis=1), np.linalg.norm(x, axis=1), rtol=1e-13)
    z = oracle.apply_rope(oracle.apply_rope(x, 17, 10000.0), 25, 10000.0)
    np.testing.assert_allclose(z, oracle.apply_rope(x, 42, 10000.0), atol=1e-12)


def test_rope_scores_depend_only_on_relative_position():
    rng = np.random.default_rng(3)
    q, k = rng.standard_normal(128), rng.standard_normal(128)
    for m, n, d in [(7, 3, 11), (100, 0, 2000), (5, 5, 31)]:
        a = oracle.apply_rope(q, m, 1e4) @ oracle.apply_rope(k, n, 1e4)
        b = oracle.apply_rope(q, m + d, 1e4) @ oracle.apply_rope(k, n + d, 1e4)
        assert abs(a - b) < 1e-11


# ----------------------------------------------------------------------------- attention
def test_softmax_rows_sum_to_one_and_match_library():
    x = np.random.default_rng(4).standard_normal((7, 33)) * 10
    p = oracle.softmax(x)
    np.testing.assert_allclose(p.sum(axis=1), 1.0, rtol=0, atol=1e-12)
    np.testing.assert_allclose(p, scipy.special.softmax(x, axis=1), rtol=1e-13, atol=0)


def test_single_key_returns_its_value():
    rng = np.random.default_rng(5)
    q, k, v = rng.standard_normal((4, 64)), rng.standard_normal((1, 1, 64)), rng.standard_normal((1, 1, 64))
    out = oracle.decode_gqa(q, k, v)
    np.testing.assert_allclose(out, np.repeat(v[0], 4, axis=0), atol=1e-15)


def test_equal_keys_give_mean_value():
    rng = np.random.default_rng(6)
    k = np.repeat(rng.standard_normal((1, 1, 32)), 9, axis=1)
    v = rng.standard_normal((1, 9, 32))
    out = oracle.decode_gqa(rng.standard_normal((2, 32)), k, v)
    np.testing.assert_allclose(out[0], v[0].mean(axis=0), atol=1e-14)


def test_two_keys_logistic_weights_and_default_scale():
    # two keys: softmax of two logits is the logistic function of their difference
    D = 64
    q = np.zeros(D); q[0] = 1.0
    k = np.zeros((1, 2, D)); k[0, 0, 0] = 3.0; k[0, 1, 0] = -1.0
    v = np.zeros((1, 2, D)); v[0, 0, 1] = 1.0; v[0, 1, 2] = 1.0
    out = oracle.decode_gqa(q[None], k, v)
    w = scipy.special.expit((3.0 - (-1.0)) / np.sqrt(D))
    np.testing.assert_allclose(out[0, 1:3], [w, 1 - w], rtol=1e-14)
    out2 = oracle.decode_gqa(q[None], k, v, scale=1.0)
    np.testing.assert_allclose(out2[0, 1], scipy.special.expit(4.0), rtol=1e-14)


def test_gqa_equals_mha_with_repeated_kv():
    rng = np.random.default_rng(7)
    Hq, Hkv, n, D = 24, 4, 19, 32
    q = rng.standard_normal((Hq, D))
    k, v = rng.standard_normal((Hkv, n, D)), rng.standard_normal((Hkv, n, D))
    G = Hq // Hkv
    gqa = oracle.decode_gqa(q, k, v)
    mha = oracle.decode_gqa(q, np.repeat(k, G, axis=0), np.repeat(v, G, axis=0))
    np.testing.assert_allclose(gqa, mha, atol=1e-14)
    # contiguous grouping: query head h uses kv head h // G
    one = oracle.decode_gqa(q[13:14], k[2:3], v[2:3])
    np.testing.assert_allclose(gqa[13], one[0], atol=1e-14)


def test_causal_attention_last_row_is_decode_and_first_row_is_v0():
    rng = np.random.default_rng(8)
    T, Hq, Hkv, D = 11, 4, 2, 16
    Q, K, V = rng.standard_normal((T, Hq, D)), rng.standard_normal((T, Hkv, D)), rng.standard_normal((T, Hkv, D))
    full = oracle.causal_attention(Q, K, V, np.arange(T), base=None)
    np.testing.assert_allclose(full[0], np.repeat(V[0], 2, axis=0), atol=1e-14)
    last = oracle.decode_gqa(Q[-1], K.transpose(1, 0, 2), V.transpose(1, 0, 2))
    np.testing.assert_allclose(full[-1], last, atol=1e-13)


@pytest.mark.parametrize("bad", ["scale", "group"])
def test_decode_rejects_or_detects_wrong_scale_group(bad):
    # guards against silently accepting an inconsistent head grouping
    rng = np.random.default_rng(9)
    if bad == "group":
        with pytest.raises(ValueError):
            oracle.decode_gqa(rng.standard_normal((5, 8)), rng.standard_normal((2, 3, 8)),
                              rng.standard_normal((2, 3, 8)))
    else:
        q, k, v = rng.standard_normal((1, 8)), rng.standard_normal((1, 3, 8)), rng.standard_normal((1, 3, 8))
        a = oracle.decode_gqa(q, k, v)
        b = oracle.decode_gqa(q, k, v, scale=1 / np.sqrt(8))
        np.testing.assert_array_equal(a, b)

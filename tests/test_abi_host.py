"""C ABI host-side checks that need no GPU: the library loads, exports every entry
point include/lcd.h declares, sizes its buffers by the KV size model, validates
arguments before any HIP call and keeps its slot / position bookkeeping."""
import ctypes
import os
import re

import numpy as np
import pytest

import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def L():
    import long_context_decode_amd as lib

    return lib


def _declared():
    text = open(os.path.join(ROOT, "include", "lcd.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(lcd_[a-z0-9_]+)\s*\(", text)))


def test_every_declared_symbol_is_exported(L):
    declared = _declared()
    assert len(declared) >= 15
    for name in declared:
        assert hasattr(L.lib, name), name
    assert set(declared) == set(L._lib.EXPORTED)
    assert L.abi_version() == 5


def test_sizes_follow_the_kv_size_model(L):
    for (B, Hq, Hkv, D, dt, S, W, layers) in [(16, 32, 32, 128, 1, 4, 2044, 1), (16, 24, 4, 256, 1, 4, 32764, 16),
                                              (1, 4, 1, 64, 0, 4, 60, 1)]:
        cfg = L.cache_config(B, Hq, Hkv, D, dt, L.LCD_SINK_RING, n_layers=layers, n_sink=S, window=W, rope=1)
        kv, aux, ws = L.cache_sizes(cfg)
        assert kv == oracle.kv_cache_bytes(layers, Hkv, D, S + W, 4 if dt == 0 else 2, batch=B)
        assert aux >= 2 * (S + W) * (D // 2) * 4  # cos + sin table
        assert ws > 0
    # the two full-size decode configurations
    cfg = L.cache_config(16, 32, 32, 128, 1, L.LCD_SINK_RING, n_sink=4, window=2044, rope=1)
    assert L.cache_sizes(cfg)[0] == 512 * 2**20
    cfg = L.cache_config(16, 24, 4, 256, 1, L.LCD_SINK_RING, n_layers=16, n_sink=4, window=32764, rope=1)
    assert L.cache_sizes(cfg)[0] == 32 * 2**30


@pytest.mark.parametrize("kw,status", [
    (dict(n_q_heads=5, n_kv_heads=2), "LCD_ESHAPE"),
    (dict(head_dim=96), "LCD_ESHAPE"),
    (dict(n_q_heads=12, n_kv_heads=4), "LCD_EUNSUPPORTED"),  # G = 3
    (dict(window=0), "LCD_ESHAPE"),
    (dict(dtype=7), "LCD_EINVAL"),
    (dict(policy=9), "LCD_EINVAL"),
    (dict(policy=1, capacity=0), "LCD_ESHAPE"),
    (dict(policy=2, capacity=16, n_recent=0), "LCD_ESHAPE"),
    (dict(policy=2, capacity=16, n_recent=17), "LCD_ESHAPE"),
    (dict(policy=1, capacity=16, rope=1), "LCD_EUNSUPPORTED"),
    (dict(rope=1, rope_base=1.0), "LCD_EINVAL"),
    (dict(scale=-1.0), "LCD_EINVAL"),
    (dict(window=1 << 25), "LCD_ESHAPE"),
])
def test_config_validation(L, kw, status):
    base = dict(batch=2, n_q_heads=4, n_kv_heads=2, head_dim=128, dtype=1, policy=0, n_sink=4, window=60,
                rope=0)
    base.update(kw)
    cfg = L.cache_config(**base)
    with pytest.raises(L.LcdError) as e:
        L.cache_sizes(cfg)
    assert e.value.name == status
    assert L.last_error()


def test_init_validation(L):
    cfg = L.cache_config(1, 4, 1, 64, 0, L.LCD_SINK_RING, n_sink=4, window=60)
    kv, aux, _ = L.cache_sizes(cfg)
    assert aux > 0  # split-merge arrival counters
    fake = 1 << 20  # never dereferenced: every case fails validation before any HIP call
    for args, status in [(((1 << 20) + 8, kv, fake, aux), "LCD_EALIGN"), ((fake, kv - 1, fake, aux), "LCD_ESIZE"),
                         ((None, kv, fake, aux), "LCD_EINVAL"), ((fake, kv, None, aux), "LCD_EINVAL"),
                         ((fake, kv, fake + 8, aux), "LCD_EALIGN"), ((fake, kv, fake, aux - 1), "LCD_ESIZE")]:
        with pytest.raises(L.LcdError) as e:
            L.kv_cache_init(cfg, *args, 0)
        assert e.value.name == status, args


def test_null_handle_calls_fail_cleanly(L):
    fake = 1 << 20
    with pytest.raises(L.LcdError) as e:
        L.kv_append(None, 0, fake, fake, 1, 0)
    assert e.value.name == "LCD_EINVAL"
    with pytest.raises(L.LcdError) as e:
        L.decode_attn(None, 0, fake, fake, fake, 1 << 30, 0)
    assert e.value.name == "LCD_EINVAL"
    assert L.kv_tokens(None, 0) == -1 and L.kv_slot_of(None, 0, 5) == -1 and L.kv_rank_of(None, 0, 1) == -1
    with pytest.raises(L.LcdError):
        L.kv_set_filled(None, 0, 1, 1, 0)
    assert L.lib.lcd_decode_step(None, 0, None, None, None, None, None, 0, None) == 1  # LCD_EINVAL
    assert L.lib.lcd_decode_step_noalloc(None, 0, None, None, None, None, None) == 1  # LCD_EINVAL


def test_snapkv_param_validation(L):
    ok = dict(batch=1, n_heads=32, head_dim=128, n_prompt=32768, l_obs=32, kernel_size=5, k_keep=5243)
    assert L.snapkv_sizes(L.snapkv_params(**ok)) > 0
    for l_obs, D in [(65, 128), (256, 128), (256, 64), (128, 256)]:  # windows up to 256 rows (128 at D = 256)
        assert L.snapkv_sizes(L.snapkv_params(**(ok | dict(l_obs=l_obs, head_dim=D)))) > 0
    for kw, status in [(dict(kernel_size=4), "LCD_ESHAPE"), (dict(l_obs=257), "LCD_ESHAPE"),
                       (dict(l_obs=129, head_dim=256), "LCD_ESHAPE"),
                       (dict(k_keep=32768 - 31), "LCD_ESHAPE"), (dict(dtype=0), "LCD_EUNSUPPORTED"),
                       (dict(pool=2), "LCD_EINVAL"), (dict(out_rows=100), "LCD_ESHAPE"),
                       (dict(head_dim=80), "LCD_ESHAPE")]:
        p = dict(ok)
        p.update(kw)
        with pytest.raises(L.LcdError) as e:
            L.snapkv_sizes(L.snapkv_params(**p))
        assert e.value.name == status


def test_duo_sizes_follow_the_mixed_layout(L):
    """DuoAttention caches: per layer, R_l retrieval heads of `capacity` slots and T_l
    streaming heads of n_sink + window slots, K and V each."""
    B, Hq, Hkv, D, C, S, W = 3, 16, 8, 128, 1000, 4, 64
    gamma = [[1, 0, 0, 0, 0, 1, 0, 0], [0] * 8, [1] * 8]
    cfg = L.cache_config(B, Hq, Hkv, D, L.LCD_BF16, L.LCD_DUO, n_layers=3, n_sink=S, window=W, capacity=C,
                         retrieval=gamma)
    kv, aux, ws = L.cache_sizes(cfg)
    want = sum(2 * B * (sum(r) * C + (Hkv - sum(r)) * (S + W)) * D * 2 for r in gamma)
    assert kv == want
    assert aux >= 3 * B * Hkv * 4 and ws > 0
    # the 128k workload: 2 of 8 heads keep the whole history
    from synth import WORKLOADS

    w = WORKLOADS["duo_128k"]
    cfg = L.cache_config(w.batch, w.n_q_heads, w.n_kv_heads, w.head_dim, L.LCD_BF16, L.LCD_DUO,
                         n_sink=w.n_sink, window=w.window, capacity=w.capacity, retrieval=w.retrieval)
    full = oracle.kv_cache_bytes(1, w.n_kv_heads, w.head_dim, w.capacity, 2, batch=w.batch)
    assert L.cache_sizes(cfg)[0] == 2 * w.batch * (2 * w.capacity + 6 * 68) * w.head_dim * 2 < full / 3


@pytest.mark.parametrize("kw,status", [
    (dict(retrieval=None), "LCD_EINVAL"),
    (dict(retrieval=[[1, 2]]), "LCD_EINVAL"),
    (dict(capacity=0), "LCD_ESHAPE"),
    (dict(window=0), "LCD_ESHAPE"),
    (dict(rope=1), "LCD_EUNSUPPORTED"),
])
def test_duo_config_validation(L, kw, status):
    base = dict(batch=2, n_q_heads=4, n_kv_heads=2, head_dim=128, dtype=1, policy=L.LCD_DUO, n_sink=4, window=64,
                capacity=100, retrieval=[[1, 0]])
    base.update(kw)
    with pytest.raises(L.LcdError) as e:
        L.cache_sizes(L.cache_config(**base))
    assert e.value.name == status


def test_duo_too_many_heads(L):
    cfg = L.cache_config(1, 129, 129, 64, 0, L.LCD_DUO, n_sink=4, window=64, capacity=10,
                         retrieval=[[0] * 129])
    with pytest.raises(L.LcdError) as e:
        L.cache_sizes(cfg)
    assert e.value.name == "LCD_EUNSUPPORTED"


def test_destroy_null_is_ignored(L):
    L.lib.lcd_kv_cache_destroy(None)
    assert isinstance(L.last_error(), str)
    assert ctypes.sizeof(L._lib.CacheConfig) == 12 * 4 + 2 * 8 + 8 + 8  # + DUO map pointer, block size (padded)


# ---------------------------------------------------------------- PyramidKV budgets (host-only)
@pytest.mark.parametrize("n_layers,b_base,b_target", [
    (1, 10, 77), (2, 0, 3), (4, 64, 128), (32, 128, 2048), (32, 0, 1000), (7, 100, 100), (80, 512, 5275),
    (3, 9, 7), (4096, 1 << 24, 1 << 24), (4096, 0, 1 << 24), (97, 5, 1 << 20),
])
def test_pyramid_budgets_match_oracle(L, n_layers, b_base, b_target):
    assert L.pyramid_budgets(n_layers, b_base, b_target) == oracle.pyramid_budgets(n_layers, b_base, b_target)


@pytest.mark.parametrize("args", [(0, 1, 1), (4097, 1, 1), (3, -1, 4), (3, 4, -1), (3, 300, 100),
                                  (2, (1 << 24) + 1, 5)])
def test_pyramid_budgets_rejects(L, args):
    with pytest.raises(L.LcdError):
        L.pyramid_budgets(*args)
    import ctypes
    assert L.lib.lcd_pyramid_budgets(3, 1, 2, None) == 1  # LCD_EINVAL for a null output


def test_h2o_prompt_param_validation(L):
    ok = dict(batch=16, n_q_heads=32, n_kv_heads=8, head_dim=128, n_prompt=131072, budget=4096, n_recent=512)
    assert L.h2o_prompt_sizes(L.h2o_prompt_params(**ok)) > 16 * 32 * 131072 * 8
    for kw, status in [(dict(n_q_heads=12, n_kv_heads=8), "LCD_ESHAPE"), (dict(head_dim=96), "LCD_ESHAPE"),
                       (dict(n_prompt=262145), "LCD_ESHAPE"), (dict(n_recent=0), "LCD_ESHAPE"),
                       (dict(budget=100, n_recent=200), "LCD_ESHAPE"), (dict(dtype=0), "LCD_EUNSUPPORTED"),
                       (dict(scale=-1.0), "LCD_EINVAL")]:
        p = dict(ok)
        p.update(kw)
        with pytest.raises(L.LcdError) as e:
            L.h2o_prompt_sizes(L.h2o_prompt_params(**p))
        assert e.value.name == status, kw


@pytest.mark.parametrize("kw,status", [
    (dict(block_size=8), "LCD_ESHAPE"), (dict(block_size=16, capacity=100), "LCD_ESHAPE"),
    (dict(block_size=16, capacity=64, n_recent=60), "LCD_ESHAPE"), (dict(block_size=-1), "LCD_ESHAPE"),
])
def test_h2o_block_validation(L, kw, status):
    base = dict(batch=1, n_q_heads=4, n_kv_heads=1, head_dim=128, dtype=1, policy=L.LCD_H2O, capacity=64,
                n_recent=8)
    base.update(kw)
    with pytest.raises(L.LcdError) as e:
        L.cache_sizes(L.cache_config(**base))
    assert e.value.name == status
    ok = dict(base, block_size=32, capacity=128, n_recent=96)
    assert L.cache_sizes(L.cache_config(**ok))[0] > 0


def test_header_compiles_as_c_and_links(tmp_path):
    """A plain C99 client (tests/c/abi_smoke.c) compiles against include/lcd.h with
    -pedantic -Werror, links against the library and gets error statuses back from
    calls that fail validation, with no GPU present."""
    import shutil
    import subprocess

    cc = shutil.which("gcc") or shutil.which("cc")
    if cc is None:
        pytest.skip("no C compiler")
    lib_dir = os.path.join(ROOT, "long_context_decode_amd")
    exe = str(tmp_path / "abi_smoke")
    r = subprocess.run([cc, "-std=c99", "-Wall", "-Wextra", "-Werror", "-pedantic", f"-I{os.path.join(ROOT, 'include')}",
                        os.path.join(ROOT, "tests", "c", "abi_smoke.c"), f"-L{lib_dir}", "-llcd",
                        f"-Wl,-rpath,{lib_dir}", "-o", exe], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    r = subprocess.run([exe], capture_output=True, text=True, timeout=60)
    assert r.returncode == 0, (r.returncode, r.stdout, r.stderr)
    assert r.stdout.startswith("ok: abi ")


def test_kv_save_load_validation_without_a_gpu(L):
    """Argument checks of the checkpoint calls run before any HIP call."""
    fake = 1 << 20
    st = L.LayerState(0, 0, 0, 0)
    assert L.kv_layer_bytes(None, 0) == -1
    for fn in (L.lib.lcd_kv_save, L.lib.lcd_kv_load):
        assert fn(None, 0, fake, fake, None, None, None, None, ctypes.byref(st), None) == 1  # LCD_EINVAL
    assert L.LayerState.reserved.offset == 20 and ctypes.sizeof(L.LayerState) == 24

"""ctypes binding of liblcd.so.  Names follow the C entry points without the
``lcd_`` prefix.  Tensor arguments are torch tensors (device memory); they are
passed as raw pointers after dtype/shape/contiguity checks.  The library itself
validates everything again and never allocates device memory.
"""
from __future__ import annotations

import ctypes
import os

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "liblcd.so")  # the in-tree build, the only library this binding loads

LCD_F32, LCD_BF16 = 0, 1
LCD_SINK_RING, LCD_APPEND, LCD_H2O, LCD_DUO = 0, 1, 2, 3

_STATUS = {0: "LCD_OK", 1: "LCD_EINVAL", 2: "LCD_ESHAPE", 3: "LCD_EALIGN", 4: "LCD_ECAPACITY",
           5: "LCD_ESIZE", 6: "LCD_EHIP", 7: "LCD_EUNSUPPORTED"}


class LcdError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{_STATUS.get(status, status)}: {message}")
        self.status = status
        self.name = _STATUS.get(status, str(status))


class CacheConfig(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("n_layers", ctypes.c_int32), ("n_q_heads", ctypes.c_int32),
                ("n_kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32), ("dtype", ctypes.c_int32),
                ("policy", ctypes.c_int32), ("n_sink", ctypes.c_int32), ("window", ctypes.c_int32),
                ("capacity", ctypes.c_int32), ("n_recent", ctypes.c_int32), ("rope", ctypes.c_int32),
                ("rope_base", ctypes.c_double), ("scale", ctypes.c_double),
                ("retrieval", ctypes.POINTER(ctypes.c_int32)), ("block_size", ctypes.c_int32)]


class LayerState(ctypes.Structure):
    _fields_ = [("tokens", ctypes.c_int64), ("filled", ctypes.c_int64), ("open_fill", ctypes.c_int32),
                ("reserved", ctypes.c_int32)]


class SnapkvParams(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("n_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("n_prompt", ctypes.c_int32), ("l_obs", ctypes.c_int32), ("kernel_size", ctypes.c_int32),
                ("k_keep", ctypes.c_int32), ("pool", ctypes.c_int32), ("dtype", ctypes.c_int32),
                ("out_rows", ctypes.c_int32), ("scale", ctypes.c_double)]


class H2oPromptParams(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("n_q_heads", ctypes.c_int32), ("n_kv_heads", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("n_prompt", ctypes.c_int32), ("budget", ctypes.c_int32),
                ("n_recent", ctypes.c_int32), ("dtype", ctypes.c_int32), ("scale", ctypes.c_double)]


def _load():
    # torch supplies the device memory and streams handed to the library, so the
    # library must run on torch's HIP runtime: importing torch first makes the
    # dynamic linker resolve liblcd's libamdhip64 dependency to torch's copy.
    import torch  # noqa: F401

    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"{LIB_PATH} is missing: build it with `python long_context_decode_amd/build.py` "
            "(there is no fallback implementation)")
    return ctypes.CDLL(LIB_PATH)


lib = _load()

_P = ctypes.c_void_p
_U64 = ctypes.c_uint64
_I32 = ctypes.c_int32
_I64 = ctypes.c_int64
_S = ctypes.c_int

_SIGS = {
    "lcd_abi_version": (_S, []),
    "lcd_last_error": (ctypes.c_char_p, []),
    "lcd_cache_sizes": (_S, [ctypes.POINTER(CacheConfig), ctypes.POINTER(_U64), ctypes.POINTER(_U64),
                             ctypes.POINTER(_U64)]),
    "lcd_kv_cache_init": (_S, [ctypes.POINTER(CacheConfig), _P, _U64, _P, _U64, _P, ctypes.POINTER(_P)]),
    "lcd_kv_cache_destroy": (None, [_P]),
    "lcd_kv_append": (_S, [_P, _I32, _P, _P, _I32, _P]),
    "lcd_decode_attn": (_S, [_P, _I32, _P, _P, _P, _U64, _P]),
    "lcd_decode_step": (_S, [_P, _I32, _P, _P, _P, _P, _P, _U64, _P]),
    "lcd_decode_step_noalloc": (_S, [_P, _I32, _P, _P, _P, _P, _P]),
    "lcd_kv_tokens": (_I64, [_P, _I32]),
    "lcd_kv_filled": (_I64, [_P, _I32]),
    "lcd_kv_slot_of": (_I64, [_P, _I32, _I64]),
    "lcd_kv_rank_of": (_I64, [_P, _I32, _I64]),
    "lcd_kv_layer_view": (_S, [_P, _I32, ctypes.POINTER(_P), ctypes.POINTER(_P), ctypes.POINTER(_P),
                               ctypes.POINTER(_P)]),
    "lcd_kv_set_filled": (_S, [_P, _I32, _I32, _I64, _P]),
    "lcd_kv_layer_bytes": (_I64, [_P, _I32]),
    "lcd_kv_save": (_S, [_P, _I32, _P, _P, _P, _P, _P, _P, ctypes.POINTER(LayerState), _P]),
    "lcd_kv_load": (_S, [_P, _I32, _P, _P, _P, _P, _P, _P, ctypes.POINTER(LayerState), _P]),
    "lcd_snapkv_sizes": (_S, [ctypes.POINTER(SnapkvParams), ctypes.POINTER(_U64)]),
    "lcd_snapkv_compress": (_S, [ctypes.POINTER(SnapkvParams), _P, _P, _P, _P, _P, _P, _P, _P, _U64, _P]),
    "lcd_pyramid_budgets": (_S, [_I32, _I32, _I32, ctypes.POINTER(_I32)]),
    "lcd_h2o_prompt_sizes": (_S, [ctypes.POINTER(H2oPromptParams), ctypes.POINTER(_U64)]),
    "lcd_h2o_prompt_compress": (_S, [ctypes.POINTER(H2oPromptParams), _P, _P, _P, _P, _P, _P, _P, _P, _P, _U64,
                                     _P]),
}
for _name, (_res, _args) in _SIGS.items():
    _f = getattr(lib, _name)
    _f.restype = _res
    _f.argtypes = _args

EXPORTED = tuple(_SIGS)


def abi_version() -> int:
    return lib.lcd_abi_version()


def last_error() -> str:
    return lib.lcd_last_error().decode()


def _check(status: int):
    if status != 0:
        raise LcdError(status, last_error())


def _ptr(t):
    """Raw address of a torch tensor (or an int / None)."""
    if t is None:
        return None
    if isinstance(t, int):
        return t
    if not t.is_contiguous():
        raise ValueError("tensor must be contiguous")
    return t.data_ptr()


def _stream(stream):
    if stream is None:
        import torch

        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def cache_config(batch, n_q_heads, n_kv_heads, head_dim, dtype=LCD_BF16, policy=LCD_SINK_RING, n_layers=1,
                 n_sink=0, window=0, capacity=0, n_recent=0, rope=0, rope_base=10000.0, scale=0.0,
                 retrieval=None, block_size=0):
    """``retrieval``: DUO head kinds, [n_layers][n_kv_heads] of 0/1 (any nested sequence)."""
    cfg = CacheConfig(batch, n_layers, n_q_heads, n_kv_heads, head_dim, dtype, policy, n_sink, window,
                      capacity, n_recent, rope, rope_base, scale, None, block_size)
    if retrieval is not None:
        flat = [int(x) for row in retrieval for x in row]
        arr = (ctypes.c_int32 * len(flat))(*flat)
        cfg._retrieval_keepalive = arr  # the library reads it during sizes / init only
        cfg.retrieval = ctypes.cast(arr, ctypes.POINTER(ctypes.c_int32))
    return cfg


def cache_sizes(cfg: CacheConfig):
    kv, aux, ws = _U64(), _U64(), _U64()
    _check(lib.lcd_cache_sizes(ctypes.byref(cfg), ctypes.byref(kv), ctypes.byref(aux), ctypes.byref(ws)))
    return kv.value, aux.value, ws.value


def kv_cache_init(cfg: CacheConfig, kv_mem, kv_bytes, aux_mem, aux_bytes, stream=None):
    h = _P()
    _check(lib.lcd_kv_cache_init(ctypes.byref(cfg), _ptr(kv_mem), kv_bytes, _ptr(aux_mem), aux_bytes,
                                 _stream(stream), ctypes.byref(h)))
    return h


def kv_cache_destroy(h):
    lib.lcd_kv_cache_destroy(h)


def kv_append(h, layer, k, v, n_new, stream=None):
    _check(lib.lcd_kv_append(h, layer, _ptr(k), _ptr(v), n_new, _stream(stream)))


def decode_attn(h, layer, q, out, ws, ws_bytes, stream=None):
    _check(lib.lcd_decode_attn(h, layer, _ptr(q), _ptr(out), _ptr(ws), ws_bytes, _stream(stream)))


def decode_step(h, layer, k, v, q, out, ws, ws_bytes, stream=None):
    """Append one token (k, v: [B][H_kv][D]) and attend q over the cache, one launch."""
    _check(lib.lcd_decode_step(h, layer, _ptr(k), _ptr(v), _ptr(q), _ptr(out), _ptr(ws), ws_bytes,
                               _stream(stream)))


def decode_step_noalloc(h, layer, k, v, q, out, stream=None):
    """decode_step with the split partials in the library's device scratch (no workspace)."""
    _check(lib.lcd_decode_step_noalloc(h, layer, _ptr(k), _ptr(v), _ptr(q), _ptr(out), _stream(stream)))


def kv_tokens(h, layer):
    return lib.lcd_kv_tokens(h, layer)


def kv_filled(h, layer):
    return lib.lcd_kv_filled(h, layer)


def kv_slot_of(h, layer, token):
    return lib.lcd_kv_slot_of(h, layer, token)


def kv_rank_of(h, layer, slot):
    return lib.lcd_kv_rank_of(h, layer, slot)


def kv_layer_view(h, layer):
    k, v, pos, score = _P(), _P(), _P(), _P()
    _check(lib.lcd_kv_layer_view(h, layer, ctypes.byref(k), ctypes.byref(v), ctypes.byref(pos),
                                 ctypes.byref(score)))
    return k.value, v.value, pos.value, score.value


def kv_set_filled(h, layer, n, next_token, stream=None):
    _check(lib.lcd_kv_set_filled(h, layer, n, next_token, _stream(stream)))


def kv_layer_bytes(h, layer):
    return lib.lcd_kv_layer_bytes(h, layer)


def kv_save(h, layer, k, v, pos=None, score=None, victim=None, open_=None, stream=None) -> LayerState:
    st = LayerState()
    _check(lib.lcd_kv_save(h, layer, _ptr(k), _ptr(v), _ptr(pos), _ptr(score), _ptr(victim), _ptr(open_),
                           ctypes.byref(st), _stream(stream)))
    return st


def kv_load(h, layer, k, v, pos, score, victim, open_, state: LayerState, stream=None):
    _check(lib.lcd_kv_load(h, layer, _ptr(k), _ptr(v), _ptr(pos), _ptr(score), _ptr(victim), _ptr(open_),
                           ctypes.byref(state), _stream(stream)))


def snapkv_params(batch, n_heads, head_dim, n_prompt, l_obs, kernel_size, k_keep, pool=0, dtype=LCD_BF16,
                  out_rows=0, scale=0.0):
    return SnapkvParams(batch, n_heads, head_dim, n_prompt, l_obs, kernel_size, k_keep, pool, dtype, out_rows,
                        scale)


def snapkv_sizes(p: SnapkvParams) -> int:
    ws = _U64()
    _check(lib.lcd_snapkv_sizes(ctypes.byref(p), ctypes.byref(ws)))
    return ws.value


def snapkv_compress(p: SnapkvParams, q_obs, k, v, k_out, v_out, idx_out, scores_out, ws, ws_bytes, stream=None):
    _check(lib.lcd_snapkv_compress(ctypes.byref(p), _ptr(q_obs), _ptr(k), _ptr(v), _ptr(k_out), _ptr(v_out),
                                   _ptr(idx_out), _ptr(scores_out), _ptr(ws), ws_bytes, _stream(stream)))


def h2o_prompt_params(batch, n_q_heads, n_kv_heads, head_dim, n_prompt, budget, n_recent, dtype=LCD_BF16,
                      scale=0.0):
    return H2oPromptParams(batch, n_q_heads, n_kv_heads, head_dim, n_prompt, budget, n_recent, dtype, scale)


def h2o_prompt_sizes(p: H2oPromptParams) -> int:
    ws = _U64()
    _check(lib.lcd_h2o_prompt_sizes(ctypes.byref(p), ctypes.byref(ws)))
    return ws.value


def h2o_prompt_compress(p: H2oPromptParams, q, k, v, k_out, v_out, pos_out, score_out, scores_all, ws, ws_bytes,
                        stream=None):
    _check(lib.lcd_h2o_prompt_compress(ctypes.byref(p), _ptr(q), _ptr(k), _ptr(v), _ptr(k_out), _ptr(v_out),
                                       _ptr(pos_out), _ptr(score_out), _ptr(scores_all), _ptr(ws), ws_bytes,
                                       _stream(stream)))


def pyramid_budgets(n_layers, b_base, b_target):
    """Per-layer PyramidKV budgets (layer 0 lowest), computed by the library."""
    out = (_I32 * max(n_layers, 1))()
    _check(lib.lcd_pyramid_budgets(n_layers, b_base, b_target, out))
    return list(out[:n_layers])


class KVCache:
    """A cache whose K/V, auxiliary state and decode workspace live in torch tensors.

    Allocation only; every operation calls the C ABI.
    """

    def __init__(self, cfg: CacheConfig, device="cuda", stream=None):
        import torch

        self.cfg = cfg
        self.kv_bytes, self.aux_bytes, self.ws_bytes = cache_sizes(cfg)
        self.kv_mem = torch.empty(max(self.kv_bytes, 16), dtype=torch.uint8, device=device)
        self.aux_mem = torch.empty(max(self.aux_bytes, 16), dtype=torch.uint8, device=device)
        self.ws = torch.empty(max(self.ws_bytes, 16), dtype=torch.uint8, device=device)
        self.handle = kv_cache_init(cfg, self.kv_mem, self.kv_bytes, self.aux_mem if self.aux_bytes else None,
                                    self.aux_bytes, stream)

    def append(self, layer, k, v, stream=None):
        kv_append(self.handle, layer, k, v, k.shape[-2], stream)

    def decode(self, layer, q, out, stream=None):
        decode_attn(self.handle, layer, q, out, self.ws, self.ws_bytes, stream)

    def step(self, layer, k, v, q, out, stream=None):
        """Fused append of one token (k, v: [B][H_kv][D]) and decode."""
        decode_step(self.handle, layer, k, v, q, out, self.ws, self.ws_bytes, stream)

    def layer_tensors(self, layer):
        """(K, V) views of one layer as [B][H_kv][C][D] torch tensors, at the addresses
        lcd_kv_layer_view reports (LcdError for a mixed-head layer)."""
        import torch

        c = self.cfg
        k, v, _, _ = kv_layer_view(self.handle, layer)
        C = c.n_sink + c.window if c.policy == LCD_SINK_RING else c.capacity
        dt = torch.float32 if c.dtype == LCD_F32 else torch.bfloat16
        es = 4 if c.dtype == LCD_F32 else 2
        per = c.batch * c.n_kv_heads * C * c.head_dim
        base = self.kv_mem.data_ptr()
        ko, vo = k - base, v - base
        K = self.kv_mem[ko: ko + per * es].view(dt).view(c.batch, c.n_kv_heads, C, c.head_dim)
        V = self.kv_mem[vo: vo + per * es].view(dt).view(c.batch, c.n_kv_heads, C, c.head_dim)
        return K, V

    def h2o_tensors(self, layer):
        """(positions int32, scores float32) views of one H2O layer as [B][H_kv][C]."""
        import torch

        c = self.cfg
        _, _, pos, score = kv_layer_view(self.handle, layer)
        n = c.batch * c.n_kv_heads * c.capacity
        base = self.aux_mem.data_ptr()
        po, so = pos - base, score - base
        P = self.aux_mem[po: po + 4 * n].view(torch.int32).view(c.batch, c.n_kv_heads, c.capacity)
        S = self.aux_mem[so: so + 4 * n].view(torch.float32).view(c.batch, c.n_kv_heads, c.capacity)
        return P, S

    def save_state(self, layer, device=None):
        """Copy one layer's state into new device tensors; returns (tensors dict, LayerState)."""
        import torch

        dev = device or self.kv_mem.device
        nb = kv_layer_bytes(self.handle, layer)
        t = {"k": torch.empty(nb, dtype=torch.uint8, device=dev), "v": torch.empty(nb, dtype=torch.uint8, device=dev)}
        c = self.cfg
        if c.policy == LCD_H2O:
            n = c.batch * c.n_kv_heads
            t["pos"] = torch.empty(n * c.capacity, dtype=torch.int32, device=dev)
            t["score"] = torch.empty(n * c.capacity, dtype=torch.float32, device=dev)
            t["victim"] = torch.empty(n, dtype=torch.int32, device=dev)
            t["open"] = torch.empty(n, dtype=torch.int32, device=dev)
        st = kv_save(self.handle, layer, t["k"], t["v"], t.get("pos"), t.get("score"), t.get("victim"),
                     t.get("open"))
        return t, st

    def load_state(self, layer, tensors, state):
        kv_load(self.handle, layer, tensors["k"], tensors["v"], tensors.get("pos"), tensors.get("score"),
                tensors.get("victim"), tensors.get("open"), state)

    def close(self):
        if self.handle:
            kv_cache_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

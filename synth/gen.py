"""Counter-based generator of approximately standard-normal values.

value(seed, tag, i) = round_dtype(scale * Q[u(i) >> 16])

* ``u(i)`` is a 32-bit hash of the element index ``i`` keyed by (seed, tag).  The
  mixing function is Chris Wellons' ``lowbias32`` ("Prospecting for Hash
  Functions", 2018): xor-shift 16, multiply 0x7feb352d, xor-shift 15, multiply
  0x846ca68b, xor-shift 16.
* ``Q[j] = Phi^-1((j + 0.5) / 65536)`` is a table of 65536 standard-normal
  quantiles computed once in float64 (mean 0, standard deviation 0.99999).
* ``round_dtype`` is float64 -> float32 (round to nearest even) and, for bf16,
  float32 -> bf16 (round to nearest even).

All integer work stays below 2**49, so numpy int64 arrays and torch int64 tensors
(on any device) give the same bits, and because the float part is a table lookup
the CPU and GPU copies of a tensor are identical element for element.
"""
from __future__ import annotations

import functools
import hashlib

import numpy as np

MASK32 = 0xFFFFFFFF
TABLE_BITS = 16
TABLE_SIZE = 1 << TABLE_BITS


def _mul32(x, c: int):
    """(x * c) mod 2**32 for 0 <= x < 2**32 without leaving 49-bit range."""
    c_hi, c_lo = c >> 16, c & 0xFFFF
    return ((((x * c_hi) & 0xFFFF) << 16) + x * c_lo) & MASK32


def mix32(x):
    """lowbias32 integer hash on values in [0, 2**32); works on numpy and torch int64."""
    x = x ^ (x >> 16)
    x = _mul32(x, 0x7FEB352D)
    x = x ^ (x >> 15)
    x = _mul32(x, 0x846CA68B)
    x = x ^ (x >> 16)
    return x


def stream_key(seed: int, tag: str) -> int:
    """32-bit key of one named tensor of one seed."""
    h = hashlib.blake2b(f"{int(seed)}:{tag}".encode(), digest_size=4).digest()
    return int.from_bytes(h, "little")


def mix32_np(x: np.ndarray) -> np.ndarray:
    """numpy fast path of :func:`mix32` (uint64 products wrap mod 2**64; same low bits)."""
    x = np.asarray(x).astype(np.uint64)
    x ^= x >> np.uint64(16)
    x = (x * np.uint64(0x7FEB352D)) & np.uint64(MASK32)
    x ^= x >> np.uint64(15)
    x = (x * np.uint64(0x846CA68B)) & np.uint64(MASK32)
    x ^= x >> np.uint64(16)
    return x.astype(np.int64)


def uniform_bits(key: int, index):
    """32-bit hash of 64-bit element indices (numpy or torch int64, all >= 0)."""
    hi = index >> 32
    lo = index & MASK32
    if isinstance(index, np.ndarray):
        if hi.size == 0 or hi.min() == hi.max():
            inner = int(mix32_np(np.array([(int(hi.flat[0]) if hi.size else 0) + key]) & MASK32)[0])
        else:
            hu, inv = np.unique(hi, return_inverse=True)
            inner = mix32_np((hu + key) & MASK32)[inv].reshape(hi.shape)
        return mix32_np(lo ^ inner)
    return mix32(lo ^ mix32((hi + key) & MASK32))


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to bf16 with round-to-nearest-even; returns the uint16 bit patterns."""
    b = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    b = (b + 0x7FFF + ((b >> 16) & 1)) >> 16
    return b.astype(np.uint16)


def bf16_bits_to_f32(u: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns (uint16) to float32."""
    return (np.asarray(u, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


@functools.lru_cache(maxsize=None)
def _base_quantiles() -> np.ndarray:
    from scipy.special import ndtri

    return ndtri((np.arange(TABLE_SIZE, dtype=np.float64) + 0.5) / TABLE_SIZE)


@functools.lru_cache(maxsize=None)
def quantile_table(scale: float, dtype: str) -> np.ndarray:
    """The 65536 stored values for one (scale, dtype): float32, or bf16 bits as uint16."""
    v = (float(scale) * _base_quantiles()).astype(np.float32)
    if dtype == "f32":
        return v
    if dtype == "bf16":
        return f32_to_bf16_bits(v)
    raise ValueError(f"unknown dtype {dtype!r}")


def hash_positions(seed: int, tag: str, n: int, count: int) -> np.ndarray:
    """``count`` distinct positions of [0, n) drawn without replacement, ascending.

    The draw keeps the ``count`` positions with the smallest keyed hash; the hash is
    a bijection on 32-bit inputs, so there are no ties for n <= 2**32.
    """
    if not 0 <= count <= n:
        raise ValueError("count out of range")
    key = stream_key(seed, tag)
    h = uniform_bits(key, np.arange(n, dtype=np.int64))
    pick = np.argpartition(h, count - 1)[:count] if count else np.zeros(0, np.int64)
    return np.sort(pick.astype(np.int64))


def flat_index_np(shape, ranges) -> np.ndarray:
    """Row-major flat indices of the sub-block ``ranges`` (one index array per axis)."""
    if len(shape) != len(ranges):
        raise ValueError("rank mismatch")
    grids = np.ix_(*[np.asarray(r, dtype=np.int64) for r in ranges])
    idx = np.zeros((1,) * len(shape), dtype=np.int64)
    for ax, g in enumerate(grids):
        idx = idx * int(shape[ax]) + g
    return idx


class NormalStream:
    """One named virtual tensor of approximately N(0,1) values."""

    def __init__(self, seed: int, tag: str, dtype: str):
        if dtype not in ("f32", "bf16"):
            raise ValueError(dtype)
        self.seed, self.tag, self.dtype = int(seed), tag, dtype
        self.key = stream_key(seed, tag)

    # -- CPU --------------------------------------------------------------------------
    def table_index(self, index: np.ndarray) -> np.ndarray:
        return uniform_bits(self.key, np.asarray(index, dtype=np.int64)) >> (32 - TABLE_BITS)

    def stored(self, index: np.ndarray, scale=1.0) -> np.ndarray:
        """Stored representation: float32 values, or bf16 bit patterns (uint16).

        ``scale`` may be a scalar or an array broadcastable to ``index`` holding
        per-element scales (planted values use the same table index, scaled before
        rounding).
        """
        j = self.table_index(index)
        scales = np.unique(np.asarray(scale, dtype=np.float64))
        if scales.size == 1:
            return quantile_table(float(scales[0]), self.dtype)[j]
        s = np.broadcast_to(np.asarray(scale, dtype=np.float64), j.shape)
        out = np.empty(j.shape, dtype=np.float32 if self.dtype == "f32" else np.uint16)
        for sc in scales:
            m = s == sc
            out[m] = quantile_table(float(sc), self.dtype)[j[m]]
        return out

    def values(self, index: np.ndarray, scale=1.0) -> np.ndarray:
        """Exact float64 copies of the stored values."""
        st = self.stored(index, scale)
        if self.dtype == "bf16":
            st = bf16_bits_to_f32(st)
        return st.astype(np.float64)

    # -- GPU (torch) ----------------------------------------------------------------
    def torch_stored(self, index, scale=1.0, *, span=None):
        """Same bits as :meth:`stored`, computed by torch on ``index.device``.

        Returns a torch tensor of dtype float32 or bfloat16.  ``scale`` must be a
        python scalar here (planting is done by the caller with a second call).
        ``span = (lo, hi)`` promises lo <= index < hi; when the whole span shares its
        upper 32 index bits the keyed inner hash of those bits is one host constant, so
        the tensor goes through one hash pass instead of two (same bits).
        """
        import torch

        index = index.to(torch.int64)
        if span is not None and span[1] > span[0] and (span[0] >> 32) == ((span[1] - 1) >> 32):
            inner = int(mix32((int(span[0] >> 32) + self.key) & MASK32))
            u = mix32((index & MASK32) ^ inner)
        else:
            u = uniform_bits(self.key, index)
        tab = _torch_table(float(scale), self.dtype, str(index.device))
        return tab[u >> (32 - TABLE_BITS)]


@functools.lru_cache(maxsize=None)
def _torch_table(scale: float, dtype: str, device: str):
    import torch

    t = quantile_table(scale, dtype)
    if dtype == "f32":
        return torch.from_numpy(t.copy()).to(device)
    return torch.from_numpy(t.view(np.int16).copy()).to(device).view(torch.bfloat16)

"""Seeded synthetic inputs shared by the GPU path's tests/bench and the CPU oracle.

This module draws random numbers and nothing else: it holds none of the
attention arithmetic.  Every value is produced by a counter-based generator so
any element (or any row of a large tensor) can be regenerated on its own, on the
CPU or on the GPU, with bit-identical results:

* a 32-bit integer hash (the "lowbias32" mixer: xor-shift / odd-constant
  multiply rounds, published by C. Wellons, "Prospecting for Hash Functions")
  of (stream key, row, column), done in int64 torch arithmetic whose every
  intermediate fits in 48 bits, so CPU and GPU agree exactly;
* the top 16 bits of the hash index a table of 65536 standard-normal
  quantiles, Phi^-1((k + 0.5) / 65536), computed once in fp64 on the host
  (``statistics.NormalDist``), multiplied by the tensor's scale in fp64 and
  rounded once to the tensor's dtype.  The device gathers from a copy of that
  table, so no floating-point arithmetic happens on the device.

N(0, s^2) samples are therefore quantised to 65536 levels (|x| <= 4.3 s), which
is plenty for synthetic activations, weights and latents.

Small host-side draws (ragged sequence lengths, page permutations) use numpy's
PCG64 generator.
"""
from __future__ import annotations

import functools
import statistics
import zlib

import numpy as np
import torch

_M32 = 0xFFFFFFFF


def _mul32_t(x: torch.Tensor, c: int) -> torch.Tensor:
    """(x * c) mod 2^32 for int64 tensors holding values in [0, 2^32)."""
    lo, hi = c & 0xFFFF, c >> 16
    return (x * lo + (((x * hi) & 0xFFFF) << 16)) & _M32


def _mix32_t(x: torch.Tensor) -> torch.Tensor:
    x = x ^ (x >> 16)
    x = _mul32_t(x, 0x7FEB352D)
    x = x ^ (x >> 15)
    x = _mul32_t(x, 0x846CA68B)
    x = x ^ (x >> 16)
    return x


def _mix32(x: int) -> int:
    x &= _M32
    x ^= x >> 16
    x = (x * 0x7FEB352D) & _M32
    x ^= x >> 15
    x = (x * 0x846CA68B) & _M32
    x ^= x >> 16
    return x


def stream_key(seed: int, name: str, layer: int = 0) -> int:
    """32-bit key of one named tensor of one layer under one seed."""
    k = _mix32(seed ^ 0x5BD1E995)
    k = _mix32(k ^ zlib.crc32(name.encode()))
    return _mix32(k + layer * 0x9E3779B9)


@functools.lru_cache(maxsize=None)
def _quantiles() -> np.ndarray:
    nd = statistics.NormalDist()
    return np.array([nd.inv_cdf((k + 0.5) / 65536.0) for k in range(65536)], dtype=np.float64)


@functools.lru_cache(maxsize=64)
def _table_cpu(scale: float, dtype: torch.dtype) -> torch.Tensor:
    return torch.from_numpy(_quantiles() * scale).to(dtype)


_table_dev_cache: dict = {}


def _table(scale: float, dtype: torch.dtype, device) -> torch.Tensor:
    device = torch.device(device)
    if device.type == "cpu":
        return _table_cpu(scale, dtype)
    key = (scale, dtype, str(device))
    t = _table_dev_cache.get(key)
    if t is None:
        t = _table_cpu(scale, dtype).to(device)
        _table_dev_cache[key] = t
    return t


def normal_rows(key: int, rows, n_cols: int, scale: float = 1.0, dtype=torch.float32,
                device="cpu", chunk_elems: int = 1 << 27) -> torch.Tensor:
    """Rows ``rows`` (1-D int tensor or range) of the N(0, scale^2) matrix with
    ``n_cols`` columns named by ``key``.  Row r of the full matrix is the same
    wherever and however it is generated."""
    device = torch.device(device)
    if isinstance(rows, range):
        rows = torch.arange(rows.start, rows.stop, rows.step, dtype=torch.int64, device=device)
    else:
        rows = torch.as_tensor(rows, dtype=torch.int64, device=device)
    table = _table(float(scale), dtype, device)
    out = torch.empty((rows.numel(), n_cols), dtype=dtype, device=device)
    cols = torch.arange(n_cols, dtype=torch.int64, device=device).unsqueeze(0)
    step = max(1, chunk_elems // max(1, n_cols))
    for r0 in range(0, rows.numel(), step):
        r = rows[r0:r0 + step].unsqueeze(1)
        a = _mix32_t((r ^ key) & _M32)
        x = _mix32_t((a + cols) & _M32)
        out[r0:r0 + step] = table[x >> 16]
    return out


def normal(key: int, shape, scale: float = 1.0, dtype=torch.float32, device="cpu") -> torch.Tensor:
    """Whole N(0, scale^2) tensor; its last dimension is the column index."""
    shape = tuple(shape)
    n_cols = shape[-1]
    n_rows = int(np.prod(shape[:-1])) if len(shape) > 1 else 1
    return normal_rows(key, range(n_rows), n_cols, scale, dtype, device).reshape(shape)


def uniform_ints(seed: int, name: str, n: int, lo: int, hi: int) -> np.ndarray:
    """n integers uniform on [lo, hi] (inclusive)."""
    g = np.random.Generator(np.random.PCG64([seed, zlib.crc32(name.encode())]))
    return g.integers(lo, hi + 1, size=n, dtype=np.int64)


def permutation(seed: int, name: str, n: int) -> np.ndarray:
    """A uniformly random permutation of range(n) (Fisher-Yates, PCG64)."""
    g = np.random.Generator(np.random.PCG64([seed, zlib.crc32(name.encode())]))
    return g.permutation(n)

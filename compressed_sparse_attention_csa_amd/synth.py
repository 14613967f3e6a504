"""Seeded synthetic inputs, reproducible bit-for-bit on the CPU and on the GPU.

This module holds no arithmetic of the attention method. It only turns
(seed, stream, element index) into numbers, so that the CPU oracle and the
HIP path can be fed identical inputs without generating a whole tensor on one
side and copying it: either side can regenerate any slice (a few rows of a
1M-token sequence, say) on its own device.

Generator
---------
* ``h = mix(mix(idx ^ key) + key2)`` where ``mix`` is the 32-bit
  "lowbias32" integer finaliser (xor-shift / multiply), ``idx`` is the flat
  element index inside the stream and ``key``/``key2`` are derived from
  ``(seed, stream)``. All of it is integer arithmetic done with torch int64
  tensors (every product is split so that it stays below 2**48), so CPU and
  GPU produce the same bits.
* ``normal``: ``TABLE[h >> 16]`` where ``TABLE[i]`` is the standard-normal
  quantile at ``(i + 0.5) / 65536`` (Python's ``statistics.NormalDist``, a
  pure-Python computation in IEEE doubles, rounded to float32). This is a
  65,536-level discretisation of N(0, 1) with support +-4.32.
* ``uniform``: ``(h >> 8) * 2**-24``, exactly representable in float32, in
  [0, 1).

Rounding to bf16 uses torch's round-to-nearest-even conversion, which is the
same on both devices.

Streams
-------
``stream_id(kind, layer, seq)`` packs the array kind and its coordinates into
one integer; every config draws each array from its own stream, so arrays can
be generated lazily and in any order.
"""
from __future__ import annotations

import statistics

import torch

_MASK32 = 0xFFFFFFFF

# array kinds (part of the stream id)
KIND_K = 1        # raw keys      [rows, D]
KIND_V = 2        # raw values    [rows, D]
KIND_Z = 3        # gate logits   [rows, D]
KIND_PROJ = 4     # indexer projection [D, D_I]
KIND_Q = 5        # attention query   [tokens, H_q, D]
KIND_QI = 6       # indexer query     [tokens, H_I, D_I]
KIND_W = 7        # indexer head weights [tokens, H_I] (uniform)
KIND_KI = 8       # indexer keys drawn directly (isolated index tests)
KIND_KBAR = 9     # compressed keys drawn directly (isolated attend tests)
KIND_VBAR = 10    # compressed values drawn directly
KIND_MISC = 11


def stream_id(kind: int, layer: int = 0, seq: int = 0) -> int:
    return (kind << 24) ^ (layer << 16) ^ seq


def _mul32(x: torch.Tensor, c: int) -> torch.Tensor:
    """(x * c) mod 2**32 for int64 tensors holding uint32 values, overflow-free."""
    lo = x * (c & 0xFFFF)
    hi = ((x * (c >> 16)) & 0xFFFF) << 16
    return (lo + hi) & _MASK32


def _mix(x: torch.Tensor) -> torch.Tensor:
    x = x ^ (x >> 16)
    x = _mul32(x, 0x7FEB352D)
    x = x ^ (x >> 15)
    x = _mul32(x, 0x846CA68B)
    x = x ^ (x >> 16)
    return x


def _mix_int(x: int) -> int:
    x &= _MASK32
    x ^= x >> 16
    x = (x * 0x7FEB352D) & _MASK32
    x ^= x >> 15
    x = (x * 0x846CA68B) & _MASK32
    x ^= x >> 16
    return x


def _keys(seed: int, stream: int) -> tuple[int, int]:
    k1 = _mix_int(_mix_int(seed * 0x9E3779B9 + 0x632BE5AB) ^ stream)
    k2 = _mix_int(k1 + 0x85EBCA77)
    return k1, k2


_TABLES: dict[str, torch.Tensor] = {}


def _normal_table(device) -> torch.Tensor:
    key = str(device)
    t = _TABLES.get(key)
    if t is None:
        nd = statistics.NormalDist()
        vals = [nd.inv_cdf((i + 0.5) / 65536.0) for i in range(65536)]
        t = torch.tensor(vals, dtype=torch.float64).to(torch.float32).to(device)
        _TABLES[key] = t
    return t


def _hash(seed: int, stream: int, idx: torch.Tensor) -> torch.Tensor:
    k1, k2 = _keys(seed, stream)
    lo = idx & _MASK32
    hi = idx >> 32
    h = _mix(lo ^ k1)
    h = _mix((h + k2 + _mul32(hi, 0x27D4EB2F)) & _MASK32)
    return h


def normal_flat(seed: int, stream: int, start: int, count: int, device="cpu") -> torch.Tensor:
    """float32 N(0,1)-like values for flat indices [start, start+count) of a stream."""
    idx = torch.arange(start, start + count, dtype=torch.int64, device=device)
    h = _hash(seed, stream, idx)
    return _normal_table(device)[h >> 16]


def uniform_flat(seed: int, stream: int, start: int, count: int, device="cpu") -> torch.Tensor:
    """float32 U[0,1) values for flat indices [start, start+count) of a stream."""
    idx = torch.arange(start, start + count, dtype=torch.int64, device=device)
    h = _hash(seed, stream, idx)
    return (h >> 8).to(torch.float32) * (2.0 ** -24)


def normal_rows(seed: int, stream: int, row0: int, nrows: int, width: int,
                device="cpu", dtype=torch.float32, chunk_rows: int = 1 << 18) -> torch.Tensor:
    """Rows [row0, row0+nrows) of a [*, width] matrix drawn from one stream.

    Element (row, col) has flat index row*width + col. The result is rounded
    to ``dtype`` (float32 or bfloat16) after drawing.
    """
    out = torch.empty((nrows, width), dtype=dtype, device=device)
    for r in range(0, nrows, chunk_rows):
        n = min(chunk_rows, nrows - r)
        v = normal_flat(seed, stream, (row0 + r) * width, n * width, device)
        out[r:r + n] = v.view(n, width).to(dtype)
    return out


def uniform_rows(seed: int, stream: int, row0: int, nrows: int, width: int,
                 device="cpu") -> torch.Tensor:
    v = uniform_flat(seed, stream, row0 * width, nrows * width, device)
    return v.view(nrows, width)


def proj_matrix(seed: int, d: int, d_i: int, device="cpu") -> torch.Tensor:
    """Indexer projection P_I [d, d_i] in float32: N(0,1) scaled by 1/sqrt(d)."""
    p = normal_rows(seed, stream_id(KIND_PROJ), 0, d, d_i, device)
    return p * torch.tensor(1.0 / (d ** 0.5), dtype=torch.float32, device=device)


def log_uniform_lengths(seed: int, n: int, lo: int, hi: int) -> list[int]:
    """Ragged context lengths floor(lo * (hi/lo)**u), u ~ U[0,1), one per request."""
    u = uniform_flat(seed, stream_id(KIND_MISC, 0, 1), 0, n).double()
    ratio = hi / lo
    return [int(lo * (ratio ** float(x))) for x in u]


def permutation(seed: int, n: int, salt: int = 0) -> list[int]:
    """A seeded permutation of range(n) (used for physical page placement)."""
    u = uniform_flat(seed, stream_id(KIND_MISC, 1, salt), 0, n)
    keys = u.double() + torch.arange(n, dtype=torch.float64) * 1e-12
    return torch.argsort(keys).tolist()

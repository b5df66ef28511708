"""Seeded synthetic inputs shared by the tests, the smoke check and the benchmark.

This module holds none of the method's arithmetic: it only draws numbers.
Both the HIP path and the oracle receive the arrays it returns.

Generator: SplitMix64 (Steele, Lea and Flood, "Fast splittable pseudorandom
number generators", OOPSLA 2014; the 64-bit finaliser constants are the ones
Vigna publishes with his public-domain ``splitmix64.c``).  It is counter based:
element ``i`` of stream ``(seed, stream_id)`` is

    z_i = mix(key + (i + 1) * GAMMA),   key = seed * 2^48 + stream_id * 2^40

so any element can be drawn on its own, and element 0 of (0, 0) is the first
output of a SplitMix64 generator seeded with 0.  From z:

    u = (z >> 11) * 2^-53                       uniform on [0, 1), 53 bits
    uniform value  = fp16(2u - 1)               round-to-nearest-even, [-1, 1]
    integer value  = floor(5u) - 2              in {-2, -1, 0, 1, 2}

Stream ids: 0 for A (GEMM) or W (GEMV), 1 for B (GEMM) or x (GEMV), 2 for
the 2:4 sparsity pattern of A.

2:4-sparse A (``sparse24``): values as above; along the last axis every group
of 4 consecutive entries keeps one of its 6 index pairs, pair floor(6u) in the
order (0,1) (0,2) (0,3) (1,2) (1,3) (2,3), u drawn from stream 2 (one draw per
group), and its other two entries are set to +0.
"""
from __future__ import annotations

import numpy as np

GAMMA = np.uint64(0x9E3779B97F4A7C15)
_M1 = np.uint64(0xBF58476D1CE4E5B9)
_M2 = np.uint64(0x94D049BB133111EB)

STREAM_A = 0
STREAM_B = 1
STREAM_MASK = 2

_PAIRS = np.array([(0, 1), (0, 2), (0, 3), (1, 2), (1, 3), (2, 3)])


_CHUNK = 1 << 20


def _mix_inplace(z: np.ndarray, t: np.ndarray) -> None:
    """SplitMix64 finaliser applied to z in place (t is scratch of z's size)."""
    np.right_shift(z, np.uint64(30), out=t)
    np.bitwise_xor(z, t, out=z)
    np.multiply(z, _M1, out=z)
    np.right_shift(z, np.uint64(27), out=t)
    np.bitwise_xor(z, t, out=z)
    np.multiply(z, _M2, out=z)
    np.right_shift(z, np.uint64(31), out=t)
    np.bitwise_xor(z, t, out=z)


def _fill(seed: int, stream_id: int, count: int, start: int, emit) -> None:
    """Draw outputs start .. start+count-1 chunk by chunk; emit(lo, hi, z)."""
    key = np.uint64(((seed << 48) + (stream_id << 40)) & 0xFFFFFFFFFFFFFFFF)
    z = np.empty(min(count, _CHUNK), dtype=np.uint64)
    t = np.empty_like(z)
    for lo in range(0, count, _CHUNK):
        hi = min(count, lo + _CHUNK)
        zz, tt = z[: hi - lo], t[: hi - lo]
        zz[:] = np.arange(start + lo + 1, start + hi + 1, dtype=np.uint64)
        np.multiply(zz, GAMMA, out=zz)          # (i + 1) * GAMMA mod 2^64
        np.add(zz, key, out=zz)
        _mix_inplace(zz, tt)
        emit(lo, hi, zz)


def splitmix64(seed: int, stream_id: int, count: int, start: int = 0) -> np.ndarray:
    """``count`` 64-bit outputs of stream (seed, stream_id) from index ``start``."""
    out = np.empty(count, dtype=np.uint64)

    def emit(lo, hi, z):
        out[lo:hi] = z

    _fill(seed, stream_id, count, start, emit)
    return out


def _draw(seed: int, stream_id: int, count: int, integer: bool, start: int = 0) -> np.ndarray:
    out = np.empty(count, dtype=np.float16)
    u = np.empty(min(count, _CHUNK), dtype=np.float64)

    def emit(lo, hi, z):
        uu = u[: hi - lo]
        np.right_shift(z, np.uint64(11), out=z)
        uu[:] = z                                # exact: 53-bit integers
        np.multiply(uu, 2.0 ** -53, out=uu)      # u in [0, 1)
        if integer:
            np.multiply(uu, 5.0, out=uu)
            np.floor(uu, out=uu)
            np.subtract(uu, 2.0, out=uu)         # floor(5u) - 2
        else:
            np.multiply(uu, 2.0, out=uu)
            np.subtract(uu, 1.0, out=uu)         # 2u - 1
        out[lo:hi] = uu                          # round-to-nearest-even to fp16

    _fill(seed, stream_id, count, start, emit)
    return out


def uniform01(seed: int, stream_id: int, count: int, start: int = 0) -> np.ndarray:
    z = splitmix64(seed, stream_id, count, start)
    return (z >> np.uint64(11)).astype(np.float64) * (2.0 ** -53)


def uniform_f16(shape, seed: int = 0, stream_id: int = STREAM_A) -> np.ndarray:
    """fp16 values, uniform on [-1, 1], as a float16 array of ``shape``."""
    n = int(np.prod(shape)) if len(shape) else 1
    return _draw(seed, stream_id, n, integer=False).reshape(shape)


def integer_f16(shape, seed: int = 0, stream_id: int = STREAM_A) -> np.ndarray:
    """fp16 values drawn from {-2, -1, 0, 1, 2}, as a float16 array of ``shape``."""
    n = int(np.prod(shape)) if len(shape) else 1
    return _draw(seed, stream_id, n, integer=True).reshape(shape)


def rows_f16(kind: str, shape, rows, seed: int = 0, stream_id: int = STREAM_A) -> np.ndarray:
    """Rows ``rows`` of ``make(kind, shape, seed, stream_id)`` (a 2-D shape),
    drawn on their own: the generator is counter based, so row r is elements
    r * shape[1] .. of the stream."""
    if kind not in ("uniform", "integer"):
        raise ValueError("kind must be 'uniform' or 'integer'")
    n = int(shape[1])
    out = np.empty((len(rows), n), dtype=np.float16)
    for t, r in enumerate(rows):
        if not 0 <= int(r) < int(shape[0]):
            raise IndexError("row %d outside %d rows" % (int(r), int(shape[0])))
        out[t] = _draw(seed, stream_id, n, kind == "integer", start=int(r) * n)
    return out


def make(kind: str, shape, seed: int = 0, stream_id: int = STREAM_A) -> np.ndarray:
    if kind == "uniform":
        return uniform_f16(shape, seed, stream_id)
    if kind == "integer":
        return integer_f16(shape, seed, stream_id)
    raise ValueError("kind must be 'uniform' or 'integer'")


def sparse24(kind: str, shape, seed: int = 0, stream_id: int = STREAM_A) -> np.ndarray:
    """A ``make(kind, ...)`` array with at most 2 nonzeros in each group of 4
    along the last axis (whose length must be a multiple of 4)."""
    a = make(kind, shape, seed, stream_id)
    if shape[-1] % 4:
        raise ValueError("the last axis must be a multiple of 4")
    groups = a.size // 4
    pick = np.minimum((uniform01(seed, STREAM_MASK, groups) * 6.0).astype(np.int64), 5)
    keep = np.zeros((groups, 4), dtype=bool)
    rows = np.arange(groups)
    keep[rows, _PAIRS[pick, 0]] = True
    keep[rows, _PAIRS[pick, 1]] = True
    g = a.reshape(groups, 4)
    g[~keep] = np.float16(0.0)
    return a


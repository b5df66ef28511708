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

Stream ids: 0 for A (GEMM) or W (GEMV), 1 for B (GEMM) or x (GEMV).
"""
from __future__ import annotations

import numpy as np

GAMMA = np.uint64(0x9E3779B97F4A7C15)
_M1 = np.uint64(0xBF58476D1CE4E5B9)
_M2 = np.uint64(0x94D049BB133111EB)

STREAM_A = 0
STREAM_B = 1


def _mix(z: np.ndarray) -> np.ndarray:
    z = (z ^ (z >> np.uint64(30))) * _M1
    z = (z ^ (z >> np.uint64(27))) * _M2
    return z ^ (z >> np.uint64(31))


def splitmix64(seed: int, stream_id: int, count: int, start: int = 0) -> np.ndarray:
    """``count`` 64-bit outputs of stream (seed, stream_id) from index ``start``."""
    key = np.uint64(((seed << 48) + (stream_id << 40)) & 0xFFFFFFFFFFFFFFFF)
    idx = np.arange(start + 1, start + count + 1, dtype=np.uint64)
    with np.errstate(over="ignore"):
        return _mix(key + idx * GAMMA)


def uniform01(seed: int, stream_id: int, count: int, start: int = 0) -> np.ndarray:
    z = splitmix64(seed, stream_id, count, start)
    return (z >> np.uint64(11)).astype(np.float64) * (2.0 ** -53)


def uniform_f16(shape, seed: int = 0, stream_id: int = STREAM_A) -> np.ndarray:
    """fp16 values, uniform on [-1, 1], as a float16 array of ``shape``."""
    n = int(np.prod(shape)) if len(shape) else 1
    u = uniform01(seed, stream_id, n)
    return (2.0 * u - 1.0).astype(np.float16).reshape(shape)


def integer_f16(shape, seed: int = 0, stream_id: int = STREAM_A) -> np.ndarray:
    """fp16 values drawn from {-2, -1, 0, 1, 2}, as a float16 array of ``shape``."""
    n = int(np.prod(shape)) if len(shape) else 1
    u = uniform01(seed, stream_id, n)
    return (np.floor(5.0 * u) - 2.0).astype(np.float16).reshape(shape)


def make(kind: str, shape, seed: int = 0, stream_id: int = STREAM_A) -> np.ndarray:
    if kind == "uniform":
        return uniform_f16(shape, seed, stream_id)
    if kind == "integer":
        return integer_f16(shape, seed, stream_id)
    raise ValueError("kind must be 'uniform' or 'integer'")

"""CPU oracle (double precision) for fp16 GEMM-NT, split-K GEMM and GEMV.

TEST INFRASTRUCTURE ONLY: the test suite, the smoke check and the benchmark's
CPU-baseline leg are the only callers.  The HIP library never imports, links
or calls anything here, and nothing here reads a value the GPU produced.

The arithmetic lives in ``oracle.c`` (plain C, built with the host compiler,
no HIP headers); this module only builds it and marshals numpy arrays.
fp16 tensors travel as ``numpy.uint16`` bit patterns.

Functions and the passages they follow:

* ``gemm_nt_f16(A, B)``  -- C = round_f16(A . B^T) from an exact-product,
  ascending-k double sum.  TileLang FP16 matmul autotune benchmark page,
  sections 1-2 (C = A B^T, fp16 operands, fp32 accumulate, A(M,K), B(N,K),
  C(M,N), transpose_B); autotune tutorial page, ``reference()``.
* ``gemm_nt_f32(A, B)``  -- the same sum rounded to fp32, the split-K output.
  Basic-GEMM-to-SplitK page, SplitK section (slice partials are summed into a
  float32 C).
* ``gemv_f16(W, x)``     -- y = round_f16(W . x).  TileLang GEMV page, problem
  statement and kernel signatures A(K,), B(N,K), C(N,) with x = A, W = B.
* ``gemm_nt_entries``    -- single entries of the above, for sampled checks of
  full-size outputs.
* ``sp24_compress(A)`` / ``sp24_decompress(A_sparse, E)`` -- 2:4 structured
  sparsity: each group of 4 consecutive k keeps its two largest-magnitude
  entries (ties to the lower index); A_sparse is (M, K/2), E is (M, K/16)
  16-bit words of 4-bit fields i0 | i1 << 2.  TileLang FP16 matmul autotune
  benchmark page, section 6 (A_sparse (M, K/2), metadata E (M, K/e_factor));
  the selection rule and the bit layout are readings (see ``oracle.c``).
* ``gemm_sp_nt_f16(A_sparse, E, B)`` -- round_f16(decompress(A_sparse, E) .
  B^T), the GEMM above with the A that the compressed form describes.
* ``f16_from_double`` / ``f16_to_double`` -- IEEE binary16 round-to-nearest-
  even encode and exact decode.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
_lib = None


def build(force: bool = False) -> str:
    """Compile oracle.c with gcc (OpenMP over output rows) into liboracle.so."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        cmd = ["gcc", "-O2", "-fno-fast-math", "-ffp-contract=off", "-fopenmp", "-fPIC",
               "-shared", "-std=c11", _SRC, "-o", tmp, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is not None:
        return _lib
    lib = ctypes.CDLL(build())
    u16p = ctypes.POINTER(ctypes.c_uint16)
    f32p = ctypes.POINTER(ctypes.c_float)
    i64p = ctypes.POINTER(ctypes.c_int64)
    c_int = ctypes.c_int
    lib.oracle_f16_to_double.argtypes = [ctypes.c_uint16]
    lib.oracle_f16_to_double.restype = ctypes.c_double
    lib.oracle_f16_from_double.argtypes = [ctypes.c_double]
    lib.oracle_f16_from_double.restype = ctypes.c_uint16
    lib.oracle_gemm_nt_f16_rows.argtypes = [u16p, u16p, u16p, c_int, c_int, c_int, c_int, c_int]
    lib.oracle_gemm_nt_f16.argtypes = [u16p, u16p, u16p, c_int, c_int, c_int]
    lib.oracle_gemm_nt_f32.argtypes = [u16p, u16p, f32p, c_int, c_int, c_int]
    lib.oracle_gemm_nt_entries.argtypes = [u16p, u16p, c_int, c_int, c_int, i64p,
                                           ctypes.c_int64, u16p, f32p]
    lib.oracle_gemv_f16.argtypes = [u16p, u16p, u16p, c_int, c_int]
    f64p = ctypes.POINTER(ctypes.c_double)
    lib.oracle_f16_encode_array.argtypes = [f64p, u16p, ctypes.c_int64]
    lib.oracle_f16_encode_array.restype = None
    lib.oracle_f16_decode_array.argtypes = [u16p, f64p, ctypes.c_int64]
    lib.oracle_f16_decode_array.restype = None
    lib.oracle_sp24_compress.argtypes = [u16p, u16p, u16p, c_int, c_int]
    lib.oracle_sp24_decompress.argtypes = [u16p, u16p, u16p, c_int, c_int]
    lib.oracle_set_threads.argtypes = [c_int]
    lib.oracle_set_threads.restype = None
    for name in ("oracle_gemm_nt_f16_rows", "oracle_gemm_nt_f16", "oracle_gemm_nt_f32",
                 "oracle_gemm_nt_entries", "oracle_gemv_f16", "oracle_threads",
                 "oracle_sp24_compress", "oracle_sp24_decompress"):
        getattr(lib, name).restype = c_int
    _lib = lib
    return lib


def _p(a, ctype):
    return a.ctypes.data_as(ctypes.POINTER(ctype))


def _u16(a) -> np.ndarray:
    a = np.ascontiguousarray(a)
    if a.dtype == np.float16:
        a = a.view(np.uint16)
    if a.dtype != np.uint16:
        raise TypeError("fp16 operands are passed as float16 or uint16 bit patterns")
    return a


def threads() -> int:
    """OpenMP threads the oracle's parallel loops use."""
    return int(_load().oracle_threads())


def set_threads(n: int) -> None:
    """Use n OpenMP threads in the oracle's parallel loops from now on."""
    _load().oracle_set_threads(int(n))


def f16_to_double(h: int) -> float:
    return float(_load().oracle_f16_to_double(int(h)))


def f16_from_double(v: float) -> int:
    return int(_load().oracle_f16_from_double(float(v)))


def f16_from_double_array(v) -> np.ndarray:
    """Vector RNE encode of doubles to fp16 bit patterns."""
    v = np.ascontiguousarray(v, dtype=np.float64).ravel()
    out = np.zeros(v.shape[0], dtype=np.uint16)
    _load().oracle_f16_encode_array(_p(v, ctypes.c_double), _p(out, ctypes.c_uint16), v.shape[0])
    return out


def gemm_nt_f16(A, B, rows: tuple[int, int] | None = None) -> np.ndarray:
    """C = round_f16(A . B^T); A is (M,K), B is (N,K); returns (M,N) uint16.

    ``rows=(r0, r1)`` computes only rows r0..r1-1 of C (shape (r1-r0, N))."""
    A, B = _u16(A), _u16(B)
    M, K = A.shape
    N, K2 = B.shape
    if K != K2:
        raise ValueError("A and B must share K")
    r0, r1 = rows if rows is not None else (0, M)
    C = np.zeros((r1 - r0, N), dtype=np.uint16)
    rc = _load().oracle_gemm_nt_f16_rows(_p(A, ctypes.c_uint16), _p(B, ctypes.c_uint16),
                                         _p(C, ctypes.c_uint16), M, N, K, r0, r1)
    if rc:
        raise RuntimeError("oracle_gemm_nt_f16_rows failed (%d)" % rc)
    return C


def gemm_nt_f32(A, B) -> np.ndarray:
    """C32 = round_f32(A . B^T); returns (M,N) float32."""
    A, B = _u16(A), _u16(B)
    M, K = A.shape
    N, K2 = B.shape
    if K != K2:
        raise ValueError("A and B must share K")
    C = np.zeros((M, N), dtype=np.float32)
    rc = _load().oracle_gemm_nt_f32(_p(A, ctypes.c_uint16), _p(B, ctypes.c_uint16),
                                    _p(C, ctypes.c_float), M, N, K)
    if rc:
        raise RuntimeError("oracle_gemm_nt_f32 failed (%d)" % rc)
    return C


def gemm_nt_entries(A, B, ij) -> tuple[np.ndarray, np.ndarray]:
    """Entries C[i, j] for each row (i, j) of ``ij``: (fp16 bits, fp32 values)."""
    A, B = _u16(A), _u16(B)
    M, K = A.shape
    N, _ = B.shape
    ij = np.ascontiguousarray(ij, dtype=np.int64).reshape(-1, 2)
    n = ij.shape[0]
    o16 = np.zeros(n, dtype=np.uint16)
    o32 = np.zeros(n, dtype=np.float32)
    rc = _load().oracle_gemm_nt_entries(_p(A, ctypes.c_uint16), _p(B, ctypes.c_uint16),
                                        M, N, K, _p(ij, ctypes.c_int64), n,
                                        _p(o16, ctypes.c_uint16), _p(o32, ctypes.c_float))
    if rc:
        raise RuntimeError("oracle_gemm_nt_entries failed (%d)" % rc)
    return o16, o32


def gemv_f16(W, x) -> np.ndarray:
    """y = round_f16(W . x); W is (N,K), x is (K,); returns (N,) uint16."""
    W, x = _u16(W), _u16(x).ravel()
    N, K = W.shape
    if x.shape[0] != K:
        raise ValueError("x must have K entries")
    y = np.zeros(N, dtype=np.uint16)
    rc = _load().oracle_gemv_f16(_p(W, ctypes.c_uint16), _p(x, ctypes.c_uint16),
                                 _p(y, ctypes.c_uint16), N, K)
    if rc:
        raise RuntimeError("oracle_gemv_f16 failed (%d)" % rc)
    return y


def f16_bits_to_double(h) -> np.ndarray:
    """Vector exact decode of fp16 bit patterns to double."""
    h = np.ascontiguousarray(h, dtype=np.uint16).ravel()
    out = np.zeros(h.shape[0], dtype=np.float64)
    _load().oracle_f16_decode_array(_p(h, ctypes.c_uint16), _p(out, ctypes.c_double), h.shape[0])
    return out


def sp24_compress(A) -> tuple[np.ndarray, np.ndarray]:
    """2:4 compression of A (M, K), K a multiple of 16: returns A_sparse
    (M, K/2) uint16 fp16 bits and E (M, K/16) uint16 metadata words."""
    A = _u16(A)
    M, K = A.shape
    if K % 16:
        raise ValueError("K must be a multiple of 16")
    Asp = np.zeros((M, K // 2), dtype=np.uint16)
    E = np.zeros((M, K // 16), dtype=np.uint16)
    rc = _load().oracle_sp24_compress(_p(A, ctypes.c_uint16), _p(Asp, ctypes.c_uint16),
                                      _p(E, ctypes.c_uint16), M, K)
    if rc:
        raise RuntimeError("oracle_sp24_compress failed (%d)" % rc)
    return Asp, E


def sp24_decompress(Asp, E) -> np.ndarray:
    """The dense (M, K) uint16 A that A_sparse (M, K/2) and E (M, K/16) describe."""
    Asp = _u16(Asp)
    E = np.ascontiguousarray(E, dtype=np.uint16)
    M, K2 = Asp.shape
    K = 2 * K2
    if E.shape != (M, K // 16) or K % 16:
        raise ValueError("A_sparse must be (M, K/2) and E (M, K/16) with K a multiple of 16")
    A = np.zeros((M, K), dtype=np.uint16)
    rc = _load().oracle_sp24_decompress(_p(Asp, ctypes.c_uint16), _p(E, ctypes.c_uint16),
                                        _p(A, ctypes.c_uint16), M, K)
    if rc:
        raise RuntimeError("oracle_sp24_decompress failed (%d)" % rc)
    return A


def gemm_sp_nt_f16(Asp, E, B, rows: tuple[int, int] | None = None) -> np.ndarray:
    """C = round_f16(decompress(A_sparse, E) . B^T); returns (M, N) uint16."""
    return gemm_nt_f16(sp24_decompress(Asp, E), B, rows)


def gemm_sp_nt_entries(Asp, E, B, ij) -> np.ndarray:
    """Entries C[i, j] (fp16 bits) of the sparse product for each row of ``ij``."""
    return gemm_nt_entries(sp24_decompress(Asp, E), B, ij)[0]


"""Write the oracle's expected entries that gate the offline tile sweep.

    python tests/golden/make_sweep_expected.py [--m 8192 --n 8192 --k 8192] [--gemv-only]

For one workload shape it draws the sweep's seeded inputs (inputs/: uniform
[-1, 1] and integer {-2..2}, seed 0, streams A and B; 2:4-pruned A for the
sparse product) and computes, with the CPU oracle only, the expected fp16 bit
patterns of sampled entries of C = A . B^T (every first/last row and column
entry on a 16-step lattice plus 1024 random ones), of the sparse product on
the same entries, and of every output of the GEMV y = W . x at N x K.  The
sweep (gemv_fp16_amd/sweep.py --expected) reads these files and gates every
candidate on them before timing it: integer inputs bit for bit, uniform
inputs within 1 fp16 ulp + 1e-3.  Nothing here reads a value a GPU produced.

Output files, next to this script:
    sweep_expected_gemm_<M>x<N>x<K>.txt
    sweep_expected_sparse_<M>x<N>x<K>.txt
    sweep_expected_gemv_<N>x<K>.txt
each a '#' header (shape, seed, what the columns are) and one line per entry.
"""
from __future__ import annotations

import argparse
import os
import sys

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))

import inputs  # noqa: E402
import oracle  # noqa: E402


def entries(M, N, seed=1234, count=1024, step=16):
    rng = np.random.default_rng(seed)
    ij = [np.stack([rng.integers(0, M, count), rng.integers(0, N, count)], axis=1)]
    for i in (0, M - 1):
        js = np.arange(0, N, step)
        ij.append(np.stack([np.full(js.size, i), js], axis=1))
    for j in (0, N - 1):
        is_ = np.arange(0, M, step)
        ij.append(np.stack([is_, np.full(is_.size, j)], axis=1))
    ij.append(np.array([[M - 1, N - 1]]))
    return np.unique(np.concatenate(ij).astype(np.int64), axis=0)


def write(path, header, rows):
    with open(path, "w") as f:
        for h in header:
            f.write("# %s\n" % h)
        for r in rows:
            f.write(" ".join(str(int(v)) for v in r) + "\n")
    print("wrote", path, len(rows), "entries")


def main(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("--m", type=int, default=8192)
    ap.add_argument("--n", type=int, default=8192)
    ap.add_argument("--k", type=int, default=8192)
    ap.add_argument("--gemv-only", action="store_true", help="only the GEMV file, at N x K")
    a = ap.parse_args(argv)
    M, N, K = a.m, a.n, a.k
    if a.gemv_only:
        write_gemv(N, K)
        return
    ij = entries(M, N)
    Au = inputs.uniform_f16((M, K), 0, inputs.STREAM_A)
    Bu = inputs.uniform_f16((N, K), 0, inputs.STREAM_B)
    Ai = inputs.integer_f16((M, K), 0, inputs.STREAM_A)
    Bi = inputs.integer_f16((N, K), 0, inputs.STREAM_B)
    u16, _ = oracle.gemm_nt_entries(Au, Bu, ij)
    i16, _ = oracle.gemm_nt_entries(Ai, Bi, ij)
    common = ["shape %d %d %d" % (M, N, K), "seed 0, stream 0 = A, stream 1 = B"]
    write(os.path.join(HERE, "sweep_expected_gemm_%dx%dx%d.txt" % (M, N, K)),
          ["oracle entries of C = A . B^T (TileLang FP16 matmul autotune benchmark page, sections 1-2)"]
          + common + ["columns: i j fp16-bits(uniform inputs) fp16-bits(integer inputs)"],
          np.column_stack([ij, u16, i16]))
    if K % 16 == 0:
        # 2:4 product: A pruned by the oracle's compression (the rule the
        # sweep's GPU compression is tested bit-exact against)
        Asp, E = oracle.sp24_compress(Au)
        su = oracle.gemm_sp_nt_entries(Asp, E, Bu, ij)
        Aspi, Ei = oracle.sp24_compress(inputs.sparse24("integer", (M, K), 0, inputs.STREAM_A))
        si = oracle.gemm_sp_nt_entries(Aspi, Ei, Bi, ij)
        write(os.path.join(HERE, "sweep_expected_sparse_%dx%dx%d.txt" % (M, N, K)),
              ["oracle entries of C = decompress(compress(A)) . B^T (TileLang FP16 matmul autotune "
               "benchmark page, section 6): uniform A pruned by the 2:4 compression, integer A drawn 2:4"]
              + common + ["columns: i j fp16-bits(uniform inputs) fp16-bits(integer inputs)"],
              np.column_stack([ij, su, si]))
    write_gemv(N, K)


def write_gemv(N, K):
    # GEMV y = W . x with W = the N x K B-shaped draw of stream 0 and x of stream 1
    Wu = inputs.uniform_f16((N, K), 0, inputs.STREAM_A)
    xu = inputs.uniform_f16((K,), 0, inputs.STREAM_B)
    Wi = inputs.integer_f16((N, K), 0, inputs.STREAM_A)
    xi = inputs.integer_f16((K,), 0, inputs.STREAM_B)
    yu = oracle.gemv_f16(Wu, xu)
    yi = oracle.gemv_f16(Wi, xi)
    write(os.path.join(HERE, "sweep_expected_gemv_%dx%d.txt" % (N, K)),
          ["oracle y = W . x, every output (TileLang GEMV page, kernel signatures A(K,), B(N,K), C(N,))",
           "shape %d %d" % (N, K), "seed 0, stream 0 = W, stream 1 = x",
           "columns: n fp16-bits(uniform inputs) fp16-bits(integer inputs)"],
          np.column_stack([np.arange(N), yu, yi]))


if __name__ == "__main__":
    main()

"""Pins for the oracle's 2:4 structured-sparsity functions.

Checked against things other than the oracle's own code:

* hand-worked rows (tests/golden/sp24_compress_worked.txt) covering every
  index pair, ties among equal magnitudes and among zeros, signed zeros, NaN,
  infinities and more than one metadata word per row;
* the round trip: on inputs with at most two nonzeros per group of 4,
  decompress(compress(A)) is A bit for bit;
* the selection property on dense inputs: every kept magnitude is at least
  every dropped one, equal magnitudes keep the lower index, and the kept
  entries are A's own bits;
* the sparse product, brute-forced in Python integers straight from the
  compressed form (value times the B entry its field names), with no
  decompression step;
* the metadata layout read back as bytes and 32-bit words (the e_factor 8 and
  32 views of the same memory).

Runs on the CPU; no test here touches a GPU.
"""
import os

import numpy as np
import pytest

import inputs
import oracle
from test_oracle import exact_f16_bits, f16_ints

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "sp24_compress_worked.txt")


def golden_cases():
    cases, cur = [], {}
    for line in open(GOLDEN):
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        key, val = line.split(":", 1)
        cur[key] = val.split()
        if key == "E":
            cases.append(cur)
            cur = {}
    return cases


def f16_row(tokens):
    return np.array([float(t) for t in tokens], dtype=np.float16).view(np.uint16)


@pytest.mark.parametrize("case", golden_cases(), ids=lambda c: " ".join(c["E"]))
def test_compress_worked_examples(case):
    A = f16_row(case["A"])[None, :]
    Asp, E = oracle.sp24_compress(A)
    assert Asp[0].tolist() == f16_row(case["Asp"]).tolist()
    assert E[0].tolist() == [int(w, 16) for w in case["E"]]
    back = oracle.sp24_decompress(Asp, E)
    kept = np.zeros(A.shape[1], dtype=bool)
    for g in range(A.shape[1] // 4):
        f = (int(E[0, g // 4]) >> (4 * (g % 4))) & 15
        kept[4 * g + (f & 3)] = kept[4 * g + (f >> 2)] = True
    assert np.array_equal(back[0][kept], A[0][kept])
    assert not back[0][~kept].any()


@pytest.mark.parametrize("M,K", [(1, 16), (3, 32), (17, 64), (64, 1024), (5, 4096)])
@pytest.mark.parametrize("kind", ["uniform", "integer"])
def test_roundtrip_on_24_sparse_inputs(M, K, kind):
    A = inputs.sparse24(kind, (M, K), seed=M + K).view(np.uint16)
    Asp, E = oracle.sp24_compress(A)
    assert Asp.shape == (M, K // 2) and E.shape == (M, K // 16)
    assert np.array_equal(oracle.sp24_decompress(Asp, E), A)


def keys(a):
    return (a & 0x7FFF).astype(np.int64)


@pytest.mark.parametrize("kind", ["uniform", "integer"])
def test_compress_keeps_the_two_largest(kind):
    A = inputs.make(kind, (33, 256), seed=7).view(np.uint16)
    Asp, E = oracle.sp24_compress(A)
    back = oracle.sp24_decompress(Asp, E)
    g = A.reshape(-1, 4)
    fields = ((E.astype(np.int64)[:, :, None] >> (4 * np.arange(4))) & 15).reshape(-1)
    i0, i1 = fields & 3, fields >> 2
    assert (i0 < i1).all()
    rows = np.arange(g.shape[0])
    kept = np.zeros(g.shape, dtype=bool)
    kept[rows, i0] = kept[rows, i1] = True
    k = keys(g)
    min_kept = np.where(kept, k, 1 << 20).min(axis=1)
    max_drop = np.where(kept, -1, k).max(axis=1)
    assert (min_kept >= max_drop).all()
    # equal magnitudes across the kept/dropped line: the kept index is the lower one
    for r in np.nonzero(min_kept == max_drop)[0]:
        lo_kept = min(t for t in range(4) if kept[r, t] and k[r, t] == min_kept[r])
        hi_drop = max(t for t in range(4) if not kept[r, t] and k[r, t] == max_drop[r])
        assert lo_kept < hi_drop
    assert np.array_equal(back.reshape(-1, 4)[kept], g[kept])
    assert not back.reshape(-1, 4)[~kept].any()


def test_compress_every_group_of_small_values():
    """Every group over {-2, -1, -0, 0, 1, 2, inf, nan}: the kept pair is the
    first two indices after a stable sort by decreasing magnitude."""
    vals = np.array([-2, -1, -0.0, 0, 1, 2, np.inf, np.nan], dtype=np.float16).view(np.uint16)
    idx = np.stack(np.meshgrid(*[np.arange(8)] * 4, indexing="ij"), -1).reshape(-1, 4)
    A = vals[idx].reshape(-1, 16)             # 4 groups per row
    Asp, E = oracle.sp24_compress(A)
    g = A.reshape(-1, 4)
    fields = ((E.astype(np.int64)[:, :, None] >> (4 * np.arange(4))) & 15).reshape(-1)
    for r in range(g.shape[0]):
        order = sorted(range(4), key=lambda t: (-(int(g[r, t]) & 0x7FFF), t))
        i0, i1 = sorted(order[:2])
        assert fields[r] == i0 | (i1 << 2), (g[r], fields[r])
        assert Asp.reshape(-1, 2)[r].tolist() == [g[r, i0], g[r, i1]]


def test_metadata_views_as_bytes_and_words():
    """e_dtype int8 / int32 are the same bytes: group g is nibble g % 2 of
    byte g / 2, and nibble g % 8 of 32-bit word g / 8."""
    A = inputs.make("uniform", (4, 128), seed=3).view(np.uint16)
    Asp, E = oracle.sp24_compress(A)
    b8 = E.view(np.uint8)
    b32 = E.view(np.uint32)
    assert b8.shape == (4, 128 // 8) and b32.shape == (4, 128 // 32)
    for i in range(4):
        for g in range(32):
            f16 = (int(E[i, g // 4]) >> (4 * (g % 4))) & 15
            assert (int(b8[i, g // 2]) >> (4 * (g % 2))) & 15 == f16
            assert (int(b32[i, g // 8]) >> (4 * (g % 8))) & 15 == f16


def test_decompress_rejects_bad_fields():
    Asp = np.zeros((1, 8), dtype=np.uint16)
    for bad in (0x0000, 0x0005, 0x000A, 0x0003):    # (0,0) (1,1) (2,2) (3,0)
        E = np.array([[bad]], dtype=np.uint16)
        with pytest.raises(RuntimeError):
            oracle.sp24_decompress(Asp, E)


def test_compress_rejects_k_not_multiple_of_16():
    with pytest.raises(ValueError):
        oracle.sp24_compress(np.zeros((2, 8), dtype=np.uint16))


def brute_sparse(Asp, E, B):
    """Exact integer sums straight from the compressed form: for each group,
    value times the B entry at the k its field names."""
    a, b = f16_ints(Asp.view(np.float16)), f16_ints(B.view(np.float16))
    M, N = len(a), len(b)
    S = [[0] * N for _ in range(M)]
    for i in range(M):
        for g in range(len(a[i]) // 2):
            f = (int(E[i, g // 4]) >> (4 * (g % 4))) & 15
            k0, k1 = 4 * g + (f & 3), 4 * g + (f >> 2)
            for j in range(N):
                S[i][j] += a[i][2 * g] * b[j][k0] + a[i][2 * g + 1] * b[j][k1]
    return S


@pytest.mark.parametrize("M,N,K", [(1, 1, 16), (3, 5, 32), (7, 9, 64), (16, 17, 128)])
@pytest.mark.parametrize("kind", ["uniform", "integer"])
def test_sparse_gemm_bruteforce(M, N, K, kind):
    A = inputs.make(kind, (M, K), seed=M * 100 + K).view(np.uint16)   # dense: pruned by compress
    B = inputs.make(kind, (N, K), seed=M * 100 + K, stream_id=1).view(np.uint16)
    Asp, E = oracle.sp24_compress(A)
    S = brute_sparse(Asp, E, B)
    want = np.array([[exact_f16_bits(s, 48) for s in row] for row in S], dtype=np.uint16)
    assert np.array_equal(oracle.gemm_sp_nt_f16(Asp, E, B), want)
    ij = np.array([[i, j] for i in range(M) for j in range(N)][::3])
    assert np.array_equal(oracle.gemm_sp_nt_entries(Asp, E, B, ij), want[ij[:, 0], ij[:, 1]])


def test_sparse_gemm_of_24_input_is_the_dense_gemm():
    A = inputs.sparse24("integer", (24, 256), seed=5).view(np.uint16)
    B = inputs.make("integer", (20, 256), seed=5, stream_id=1).view(np.uint16)
    Asp, E = oracle.sp24_compress(A)
    want = (A.view(np.float16).astype(np.int64) @ B.view(np.float16).astype(np.int64).T)
    got = oracle.gemm_sp_nt_f16(Asp, E, B).view(np.float16).astype(np.int64)
    assert np.array_equal(got, want)

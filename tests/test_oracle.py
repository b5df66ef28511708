"""Pins for the CPU oracle: checks against things other than the oracle itself.

* fp16 encode/decode: exhaustive over all 65,536 bit patterns against numpy's
  binary16 conversions (a library routine), plus the IEEE special cases
  (ties to even at every midpoint, overflow at 65520, the subnormal edge).
* GEMM / split-K / GEMV: an exact brute force in Python integers (every fp16
  value is an integer multiple of 2^-24, so a dot product is an integer times
  2^-48) rounded with integer round-to-nearest-even, bit-equal on every entry
  of random tiny shapes; closed forms (identity and permutation B, all-ones);
  the integer-input invariant against numpy's int64 matmul; transpose
  symmetry; power-of-two scaling; GEMV equal to the M = 1 GEMM.
* Generator: SplitMix64's published first outputs for seed 0.

Runs on the CPU; no test here touches a GPU.
"""
import struct

import numpy as np
import pytest

import inputs
import oracle

# ----------------------------------------------------------------------------
# Exact rounding written independently of oracle.c: integer arithmetic only.
# ----------------------------------------------------------------------------


def exact_f16_bits(S: int, shift: int) -> int:
    """fp16 bits of round-to-nearest-even(S * 2^-shift), S an exact integer."""
    if S == 0:
        return 0
    sign = 0x8000 if S < 0 else 0
    a = -S if S < 0 else S
    e = a.bit_length() - 1 - shift              # floor(log2 |value|)
    qexp = max(e, -14) - 10                     # quantum of that binade
    sh = shift + qexp
    if sh <= 0:
        n = a << (-sh)
    else:
        n = a >> sh
        rem = a - (n << sh)
        half = 1 << (sh - 1)
        if rem > half or (rem == half and (n & 1)):
            n += 1
    if e < -14:                                 # subnormal (n == 1024 is 2^-14)
        return sign | n
    if n == 2048:
        n, qexp = 1024, qexp + 1
    biased = qexp + 25
    if biased >= 31:
        return sign | 0x7C00
    return sign | (biased << 10) | (n - 1024)


def exact_f32_bits(S: int, shift: int) -> int:
    """fp32 bits of round-to-nearest-even(S * 2^-shift)."""
    if S == 0:
        return 0
    sign = 0x80000000 if S < 0 else 0
    a = -S if S < 0 else S
    e = a.bit_length() - 1 - shift
    qexp = max(e, -126) - 23
    sh = shift + qexp
    if sh <= 0:
        n = a << (-sh)
    else:
        n = a >> sh
        rem = a - (n << sh)
        half = 1 << (sh - 1)
        if rem > half or (rem == half and (n & 1)):
            n += 1
    if e < -126:
        return sign | n
    if n == 1 << 24:
        n, qexp = 1 << 23, qexp + 1
    biased = qexp + 150
    if biased >= 255:
        return sign | 0x7F800000
    return sign | (biased << 23) | (n - (1 << 23))


def f16_ints(a) -> list:
    """Each fp16 value as the exact integer m with value = m * 2^-24."""
    d = np.asarray(a, dtype=np.float16).astype(np.float64) * float(2 ** 24)
    return [[int(v) for v in row] for row in np.atleast_2d(d)]


def brute_gemm(A, B):
    """Exact integer sums S[i][j] with C[i][j] = S * 2^-48."""
    a, b = f16_ints(A), f16_ints(B)
    return [[sum(x * y for x, y in zip(ra, rb)) for rb in b] for ra in a]


def f32_bits(arr):
    return np.ascontiguousarray(arr, dtype=np.float32).view(np.uint32)


# ----------------------------------------------------------------------------
# fp16 conversions
# ----------------------------------------------------------------------------

ALL = np.arange(65536, dtype=np.uint16)
FINITE = ALL[(ALL & 0x7C00) != 0x7C00]


def test_decode_exhaustive_matches_numpy():
    got = oracle.f16_bits_to_double(ALL)
    ref = ALL.view(np.float16).astype(np.float64)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])
    # signs of zeros
    assert np.signbit(got[0x8000]) and not np.signbit(got[0])


def test_encode_roundtrip_every_finite_pattern():
    v = FINITE.view(np.float16).astype(np.float64)
    assert np.array_equal(oracle.f16_from_double_array(v), FINITE)


def test_encode_midpoints_tie_to_even_and_neighbours():
    pos = FINITE[FINITE < 0x7BFF]               # finite positives with a finite successor
    lo = pos.view(np.float16).astype(np.float64)
    hi = (pos + 1).astype(np.uint16).view(np.float16).astype(np.float64)
    mid = (lo + hi) / 2                          # exact in double
    even = np.where(pos % 2 == 0, pos, pos + 1).astype(np.uint16)
    assert np.array_equal(oracle.f16_from_double_array(mid), even)
    assert np.array_equal(oracle.f16_from_double_array(-mid), even | 0x8000)
    below = np.nextafter(mid, -np.inf)
    above = np.nextafter(mid, np.inf)
    assert np.array_equal(oracle.f16_from_double_array(below), pos)
    assert np.array_equal(oracle.f16_from_double_array(above), (pos + 1).astype(np.uint16))


def test_encode_random_doubles_match_numpy():
    rng = np.random.default_rng(1)
    v = np.concatenate([
        rng.uniform(-70000, 70000, 100000),
        rng.uniform(-1, 1, 100000) * 2.0 ** rng.integers(-30, 17, 100000),
        rng.standard_normal(100000),
    ])
    with np.errstate(over="ignore"):
        ref = v.astype(np.float16).view(np.uint16)
    assert np.array_equal(oracle.f16_from_double_array(v), ref)


@pytest.mark.parametrize("value,bits", [
    (65504.0, 0x7BFF), (65519.99, 0x7BFF), (65520.0, 0x7C00), (1e10, 0x7C00),
    (-65520.0, 0xFC00), (float("inf"), 0x7C00), (-0.0, 0x8000), (0.0, 0x0000),
    (2.0 ** -25, 0x0000), (-(2.0 ** -25), 0x8000), (1.5 * 2.0 ** -25, 0x0001),
    (np.nextafter(2.0 ** -25, 1.0), 0x0001), (2.0 ** -24, 0x0001), (2.0 ** -14, 0x0400),
    (2049.0, 0x6800), (2051.0, 0x6802), (1.0, 0x3C00), (-2.0, 0xC000),
])
def test_encode_special_cases(value, bits):
    assert oracle.f16_from_double(value) == bits


def test_encode_nan():
    h = oracle.f16_from_double(float("nan"))
    assert (h & 0x7C00) == 0x7C00 and (h & 0x3FF) != 0


def test_exact_rounders_agree_with_numpy():
    """The test's own integer rounders, checked before they are used as pins."""
    rng = np.random.default_rng(2)
    for _ in range(3000):
        S = int(rng.integers(-2 ** 62, 2 ** 62)) >> int(rng.integers(0, 60))
        shift = int(rng.integers(0, 80))
        v = S / 2.0 ** shift if abs(S) < 2 ** 53 else None
        if v is None:
            continue
        with np.errstate(over="ignore"):
            assert exact_f16_bits(S, shift) == int(np.float64(v).astype(np.float16).view(np.uint16))
            assert exact_f32_bits(S, shift) == int(np.float32(v).view(np.uint32))


# ----------------------------------------------------------------------------
# GEMM, split-K and GEMV against brute force
# ----------------------------------------------------------------------------

TINY = [(1, 1, 1), (1, 5, 3), (3, 1, 7), (4, 4, 4), (5, 7, 9), (17, 13, 11),
        (8, 16, 64), (16, 17, 33), (2, 3, 64), (7, 9, 1)]


@pytest.mark.parametrize("M,N,K", TINY)
@pytest.mark.parametrize("kind", ["uniform", "integer"])
def test_gemm_bruteforce_every_entry(M, N, K, kind):
    seed = M * 1000 + N * 10 + K
    A = inputs.make(kind, (M, K), seed, 0)
    B = inputs.make(kind, (N, K), seed, 1)
    S = brute_gemm(A, B)
    want16 = np.array([[exact_f16_bits(s, 48) for s in row] for row in S], dtype=np.uint16)
    want32 = np.array([[exact_f32_bits(s, 48) for s in row] for row in S], dtype=np.uint32)
    assert np.array_equal(oracle.gemm_nt_f16(A, B), want16)
    assert np.array_equal(f32_bits(oracle.gemm_nt_f32(A, B)), want32)


def test_gemm_bruteforce_wide_range_values():
    """Operands spanning subnormals to large values (results near overflow too)."""
    rng = np.random.default_rng(3)
    A = (rng.uniform(-1, 1, (6, 24)) * 2.0 ** rng.integers(-20, 8, (6, 24))).astype(np.float16)
    B = (rng.uniform(-1, 1, (5, 24)) * 2.0 ** rng.integers(-20, 8, (5, 24))).astype(np.float16)
    S = brute_gemm(A, B)
    want16 = np.array([[exact_f16_bits(s, 48) for s in row] for row in S], dtype=np.uint16)
    assert np.array_equal(oracle.gemm_nt_f16(A, B), want16)


def test_gemm_is_a_times_b_transposed_not_a_times_b():
    A = inputs.uniform_f16((4, 4), 9, 0)
    B = inputs.uniform_f16((4, 4), 9, 1)
    S_nt = brute_gemm(A, B)
    S_nn = brute_gemm(A, np.ascontiguousarray(B.T))
    nt = np.array([[exact_f16_bits(s, 48) for s in r] for r in S_nt], dtype=np.uint16)
    nn = np.array([[exact_f16_bits(s, 48) for s in r] for r in S_nn], dtype=np.uint16)
    got = oracle.gemm_nt_f16(A, B)
    assert np.array_equal(got, nt) and not np.array_equal(got, nn)


@pytest.mark.parametrize("N,K", [(1, 1), (7, 13), (33, 64), (16, 100)])
@pytest.mark.parametrize("kind", ["uniform", "integer"])
def test_gemv_bruteforce(N, K, kind):
    W = inputs.make(kind, (N, K), 5, 0)
    x = inputs.make(kind, (K,), 5, 1)
    S = brute_gemm(x[None, :], W)[0]
    want = np.array([exact_f16_bits(s, 48) for s in S], dtype=np.uint16)
    assert np.array_equal(oracle.gemv_f16(W, x), want)


def test_gemv_equals_gemm_with_one_row():
    W = inputs.uniform_f16((257, 300), 0, 0)
    x = inputs.uniform_f16((300,), 0, 1)
    assert np.array_equal(oracle.gemv_f16(W, x), oracle.gemm_nt_f16(x[None, :], W)[0])


def test_splitk_slices_add_up_exactly():
    """Cutting K into slices regroups one exact sum (the split-K reading)."""
    A = inputs.uniform_f16((3, 40), 4, 0)
    B = inputs.uniform_f16((2, 40), 4, 1)
    full = brute_gemm(A, B)
    for cuts in ([0, 40], [0, 10, 20, 30, 40], [0, 14, 28, 40], [0, 40, 40]):
        parts = [brute_gemm(A[:, a:b], B[:, a:b]) for a, b in zip(cuts[:-1], cuts[1:])]
        total = [[sum(p[i][j] for p in parts) for j in range(2)] for i in range(3)]
        assert total == full
    want = np.array([[exact_f32_bits(s, 48) for s in r] for r in full], dtype=np.uint32)
    assert np.array_equal(f32_bits(oracle.gemm_nt_f32(A, B)), want)


# ----------------------------------------------------------------------------
# Closed forms and invariants
# ----------------------------------------------------------------------------


def test_identity_b_returns_a():
    A = inputs.uniform_f16((37, 64), 0, 0)
    I = np.eye(64, dtype=np.float16)
    assert np.array_equal(oracle.gemm_nt_f16(A, I), A.view(np.uint16))


def test_permutation_b_permutes_columns():
    A = inputs.uniform_f16((19, 48), 1, 0)
    perm = np.random.default_rng(4).permutation(48)
    P = np.zeros((48, 48), dtype=np.float16)
    P[np.arange(48), perm] = 1          # row j of P picks column perm[j] of A
    C = oracle.gemm_nt_f16(A, P)
    assert np.array_equal(C, A.view(np.uint16)[:, perm])


@pytest.mark.parametrize("K", [1, 7, 100, 2047, 2048, 4096])
def test_all_ones_give_k(K):
    A = np.ones((3, K), dtype=np.float16)
    B = np.ones((5, K), dtype=np.float16)
    C = oracle.gemm_nt_f16(A, B)
    assert np.all(C == np.float16(K).view(np.uint16))
    assert np.all(oracle.gemm_nt_f32(A, B) == np.float32(K))


def test_all_ones_k_2049_rounds_to_even():
    A = np.ones((1, 2049), dtype=np.float16)
    assert oracle.gemm_nt_f16(A, A)[0, 0] == 0x6800      # 2049 is a tie -> 2048


def test_ones_a_gives_row_sums_of_b():
    B = inputs.uniform_f16((23, 64), 2, 1)
    A = np.ones((4, 64), dtype=np.float16)
    rowsum = B.astype(np.float64).sum(axis=1)            # exact: < 2^30 distinct bits
    want = rowsum.astype(np.float16).view(np.uint16)
    C = oracle.gemm_nt_f16(A, B)
    assert np.array_equal(C, np.broadcast_to(want, (4, 23)))


@pytest.mark.parametrize("M,N,K", [(64, 48, 128), (9, 130, 512), (32, 32, 2048)])
def test_integer_inputs_match_int64_matmul(M, N, K):
    A = inputs.integer_f16((M, K), 6, 0)
    B = inputs.integer_f16((N, K), 6, 1)
    exact = A.astype(np.int64) @ B.astype(np.int64).T
    assert np.abs(exact).max() <= 4 * K
    assert np.array_equal(oracle.gemm_nt_f32(A, B), exact.astype(np.float32))
    want16 = exact.astype(np.float64).astype(np.float16).view(np.uint16)
    assert np.array_equal(oracle.gemm_nt_f16(A, B), want16)
    if np.abs(exact).max() <= 2048:
        assert np.array_equal(oracle.gemm_nt_f16(A, B).view(np.float16).astype(np.int64), exact)


def test_transpose_symmetry():
    A = inputs.uniform_f16((29, 77), 7, 0)
    B = inputs.uniform_f16((31, 77), 7, 1)
    assert np.array_equal(oracle.gemm_nt_f16(A, B), oracle.gemm_nt_f16(B, A).T)
    assert np.array_equal(oracle.gemm_nt_f32(A, B), oracle.gemm_nt_f32(B, A).T)


def test_power_of_two_scaling():
    A = inputs.uniform_f16((40, 96), 8, 0)
    B = inputs.uniform_f16((24, 96), 8, 1)
    C = oracle.gemm_nt_f16(A, B).view(np.float16).astype(np.float64)
    C2 = oracle.gemm_nt_f16((A.astype(np.float32) * 2).astype(np.float16), B)
    C2 = C2.view(np.float16).astype(np.float64)
    normal = np.abs(C) >= 2.0 ** -13
    assert normal.mean() > 0.9
    assert np.array_equal(C2[normal], 2 * C[normal])
    C32 = oracle.gemm_nt_f32(A, B)
    C32_4 = oracle.gemm_nt_f32((A.astype(np.float32) * 4).astype(np.float16), B)
    assert np.array_equal(C32_4, 4 * C32)


def test_entries_match_full_product():
    A = inputs.uniform_f16((50, 70), 9, 0)
    B = inputs.uniform_f16((60, 70), 9, 1)
    ij = np.stack([np.random.default_rng(5).integers(0, 50, 300),
                   np.random.default_rng(6).integers(0, 60, 300)], axis=1)
    e16, e32 = oracle.gemm_nt_entries(A, B, ij)
    assert np.array_equal(e16, oracle.gemm_nt_f16(A, B)[ij[:, 0], ij[:, 1]])
    assert np.array_equal(e32, oracle.gemm_nt_f32(A, B)[ij[:, 0], ij[:, 1]])


def test_rows_subset_matches_full():
    A = inputs.uniform_f16((20, 33), 10, 0)
    B = inputs.uniform_f16((11, 33), 10, 1)
    assert np.array_equal(oracle.gemm_nt_f16(A, B, rows=(5, 12)), oracle.gemm_nt_f16(A, B)[5:12])


def test_degenerate_shapes():
    A = np.zeros((3, 0), dtype=np.float16)
    B = np.zeros((4, 0), dtype=np.float16)
    assert np.all(oracle.gemm_nt_f16(A, B) == 0)          # empty sum is +0
    assert oracle.gemm_nt_f16(np.zeros((0, 5), np.float16), np.zeros((2, 5), np.float16)).shape == (0, 2)
    assert np.all(oracle.gemv_f16(np.zeros((6, 0), np.float16), np.zeros(0, np.float16)) == 0)


# ----------------------------------------------------------------------------
# Generator
# ----------------------------------------------------------------------------


def test_splitmix64_published_outputs():
    # First outputs of SplitMix64 seeded with 0 (Vigna's reference splitmix64.c).
    want = [0xE220A8397B1DCDAF, 0x6E789E6AA1B965F4, 0x06C45D188009454F, 0xF88BB8A8724C81EC]
    assert [int(z) for z in inputs.splitmix64(0, 0, 4)] == want


def test_generator_counter_based_and_ranges():
    a = inputs.splitmix64(0, 1, 1000)
    b = inputs.splitmix64(0, 1, 10, start=500)
    assert np.array_equal(a[500:510], b)
    u = inputs.uniform_f16((100000,), 0, 0).astype(np.float64)
    assert u.min() >= -1 and u.max() <= 1 and abs(u.mean()) < 0.01
    z = inputs.integer_f16((100000,), 0, 0).astype(np.int64)
    assert set(np.unique(z)) == {-2, -1, 0, 1, 2}
    assert not np.array_equal(inputs.uniform_f16((64,), 0, 0), inputs.uniform_f16((64,), 0, 1))


# ----------------------------------------------------------------------------
# The double oracle against exact integer sums on the full-size workloads
# ----------------------------------------------------------------------------

def test_row_draws_match_the_full_draw():
    """inputs.rows_f16 (used below to draw only the rows that sampled
    entries need) gives exactly the rows of the full draw."""
    for kind in ("uniform", "integer"):
        full = inputs.make(kind, (37, 129), 5, 1)
        rows = [36, 0, 17, 17, 3]
        got = inputs.rows_f16(kind, (37, 129), rows, 5, 1)
        assert np.array_equal(got.view(np.uint16), full[rows].view(np.uint16))


@pytest.mark.parametrize("M,N,K", [(8192, 8192, 1024), (8192, 8192, 4096), (8192, 8192, 8192),
                                   (8192, 8192, 16384), (1024, 1024, 16384)])
def test_oracle_exact_on_workload_entries(M, N, K):
    """At least 10,000 entries of each large workload (the seeded uniform
    operands of the 8192^2 x K products and of the split-K product): the
    double oracle's fp16 and fp32 results equal, bit for bit, the exact sums
    rounded with integer round-to-nearest-even.  Uniform fp16 values in
    [-1, 1] are m * 2^-24 with |m| <= 2^24, so each product is below 2^48 and
    a sum of K <= 2^14 of them fits in int64: the exact sum is an int64
    matrix product of the scaled operands."""
    rng = np.random.default_rng(M + K)
    ri = np.sort(rng.choice(M, 100, replace=False))
    rj = np.sort(rng.choice(N, 101, replace=False))
    A = inputs.rows_f16("uniform", (M, K), ri, 0, inputs.STREAM_A)
    B = inputs.rows_f16("uniform", (N, K), rj, 0, inputs.STREAM_B)
    ia = (A.astype(np.float64) * float(2 ** 24)).astype(np.int64)
    ib = (B.astype(np.float64) * float(2 ** 24)).astype(np.int64)
    assert np.abs(ia).max() <= 2 ** 24 and np.abs(ib).max() <= 2 ** 24
    S = ia @ ib.T                                     # exact: |S| < 2^62
    ij = np.stack(np.meshgrid(np.arange(100), np.arange(101), indexing="ij"), -1).reshape(-1, 2)
    o16, o32 = oracle.gemm_nt_entries(A, B, ij)
    assert ij.shape[0] >= 10000
    want16 = np.array([exact_f16_bits(int(S[i, j]), 48) for i, j in ij], dtype=np.uint16)
    want32 = np.array([exact_f32_bits(int(S[i, j]), 48) for i, j in ij], dtype=np.uint32)
    assert np.array_equal(o16, want16)
    assert np.array_equal(f32_bits(o32), want32)

"""GPU parity: the HIP path (through the C ABI) against the CPU oracle.

Bars (fp16 outputs): integer inputs in {-2..2} bit-exact; uniform[-1,1]
inputs within 1 fp16 ulp(C_ref) + 1e-3.  Split-K fp32 outputs: integer
inputs bit-exact, uniform within 1e-5 * sqrt(K) * max|C_ref|.  Two-pass
split-K is bitwise reproducible.  Full-size shapes are checked on sampled
entries that the oracle computes one by one.
"""
import sys

import numpy as np
import pytest

import gemv_fp16_amd as gf
import inputs
import oracle
from tests.util import (check_f16_tolerance, check_f32_splitk_tolerance, dev, host_u16,
                        sample_ij)

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    gf.lib()                         # fail loudly if the HIP library is missing
    yield
    torch.cuda.synchronize()


_cache = {}


def operands(kind, M, N, K, seed=0):
    key = (kind, M, N, K, seed)
    if key not in _cache:
        A = inputs.make(kind, (M, K), seed, inputs.STREAM_A)
        B = inputs.make(kind, (N, K), seed, inputs.STREAM_B)
        _cache.clear()
        _cache[key] = (A, B)
    return _cache[key]


def run_gemm(A, B, cfg=None):
    C = gf.gemm_f16_nt(dev(A), dev(B), cfg=cfg)
    torch.cuda.synchronize()
    return host_u16(C)


def check_gemm_full(A, B, kind, what, cfg=None):
    got = run_gemm(A, B, cfg)
    ref = oracle.gemm_nt_f16(A, B)
    if kind == "integer":
        assert np.array_equal(got, ref), what + ": integer inputs not bit-exact"
    else:
        check_f16_tolerance(got, ref, what)


# ---------------------------------------------------------------------------
# fp16 GEMM-NT
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("kind", ["uniform", "integer"])
def test_gemm_256_cube(kind):
    """256^3, seed 0: uniform within tolerance, integers bit-exact."""
    A, B = operands(kind, 256, 256, 256)
    _say("gemm 256^3 %s" % kind)
    check_gemm_full(A, B, kind, "gemm 256^3 " + kind)


@pytest.mark.parametrize("M,N,K", [
    (1, 1, 1), (1, 1, 8), (17, 33, 65), (257, 129, 200), (64, 64, 64), (100, 300, 8),
    (129, 65, 1000), (3, 700, 24), (700, 3, 24), (256, 256, 7), (512, 384, 136),
])
@pytest.mark.parametrize("kind", ["uniform", "integer"])
def test_gemm_ragged_shapes(M, N, K, kind):
    A, B = operands(kind, M, N, K, seed=M + N + K)
    _say("gemm ragged %dx%dx%d %s" % (M, N, K, kind))
    check_gemm_full(A, B, kind, "gemm %dx%dx%d %s" % (M, N, K, kind))


def test_gemm_zero_k_writes_zeros():
    C = torch.full((5, 7), 3.0, dtype=torch.float16, device="cuda")
    gf.gemm_f16_nt(torch.empty((5, 0), dtype=torch.float16, device="cuda"),
                   torch.empty((7, 0), dtype=torch.float16, device="cuda"), C)
    torch.cuda.synchronize()
    assert np.all(host_u16(C) == 0)


def test_gemm_unaligned_pointers_take_masked_path():
    """Operands offset by one element (2-byte aligned only) still match."""
    A, B = operands("uniform", 96, 80, 128, seed=11)
    big_a = torch.zeros(96 * 128 + 1, dtype=torch.float16, device="cuda")
    big_b = torch.zeros(80 * 128 + 1, dtype=torch.float16, device="cuda")
    big_a[1:] = dev(A).reshape(-1)
    big_b[1:] = dev(B).reshape(-1)
    a_view = big_a[1:].view(96, 128)
    b_view = big_b[1:].view(80, 128)
    assert a_view.data_ptr() % 16 != 0
    C = gf.gemm_f16_nt(a_view, b_view)
    torch.cuda.synchronize()
    check_f16_tolerance(host_u16(C), oracle.gemm_nt_f16(A, B), "unaligned")


def test_gemm_every_compiled_config():
    """Every legal tile config, on a shape with ragged tails for all tiles."""
    M, N, K = 320, 192, 160
    Au, Bu = operands("uniform", M, N, K, seed=3)
    ref_u = oracle.gemm_nt_f16(Au, Bu)
    Ai = inputs.integer_f16((M, K), 3, 0)
    Bi = inputs.integer_f16((N, K), 3, 1)
    ref_i = oracle.gemm_nt_f16(Ai, Bi)
    dAu, dBu, dAi, dBi = dev(Au), dev(Bu), dev(Ai), dev(Bi)
    n = 0
    for cfg, ok in gf.gemm_configs():
        if not ok:
            continue
        for raster in (0, 1):
            c = dict(cfg, raster=raster)
            _say("cfg %s" % c)
            Cu = gf.gemm_f16_nt(dAu, dBu, cfg=c)
            Ci = gf.gemm_f16_nt(dAi, dBi, cfg=c)
            torch.cuda.synchronize()
            check_f16_tolerance(host_u16(Cu), ref_u, "cfg %s" % c)
            assert np.array_equal(host_u16(Ci), ref_i), "cfg %s integer" % c
            n += 1
    assert n >= 180


def test_gemm_every_config_masked_path():
    """Every tile config on operands the 128-bit path cannot take (K % 8 != 0,
    ragged M and N): a config compiled with its masked variant computes the
    product, any other one refuses with GF_ERR_UNSUPPORTED.  The configs
    the library picks by default all have the masked variant."""
    M, N, K = 140, 100, 1004
    Ai = inputs.integer_f16((M, K), 7, 0)
    Bi = inputs.integer_f16((N, K), 7, 1)
    ref = oracle.gemm_nt_f16(Ai, Bi)
    dA, dB = dev(Ai), dev(Bi)
    ran = []
    for cfg, ok in gf.gemm_configs():
        if not ok:
            continue
        c = dict(cfg, raster=0)
        try:
            C = gf.gemm_f16_nt(dA, dB, cfg=c)
        except RuntimeError as e:
            assert "UNSUPPORTED" in str(e), e
            continue
        _say("masked cfg %s" % c)
        torch.cuda.synchronize()
        assert np.array_equal(host_u16(C), ref), c
        ran.append(c)
    for shape in ((8192, 8192, 8192), (2048, 4096, 8192), (2048, 2048, 8192), (4096, 2048, 1024), (1024, 1024, 4096),
                  (300, 300, 64), (8192, 8192, 256), (4096, 4096, 512), (8192, 8192, 1024),
                  (2048, 2048, 256)):
        d = dict(gf.gemm_default_config(*shape), raster=0)
        assert d in ran, "default %s for %s has no masked variant" % (d, shape)
    for tail in ({"block_m": 128, "block_n": 128, "block_k": 64, "stages": 4, "threads": 256, "raster": 0, "schedule": 2},
                 {"block_m": 128, "block_n": 128, "block_k": 64, "stages": 2, "threads": 256, "raster": 0, "schedule": 2}):
        assert tail in ran, "row-split tail %s has no masked variant" % tail


def test_gemm_power_of_two_scaling_bit_exact():
    """Doubling A doubles every fp32 partial sum exactly, so C doubles."""
    A, B = operands("uniform", 384, 256, 512, seed=5)
    C1 = run_gemm(A, B).view(np.float16).astype(np.float64)
    C2 = run_gemm((A.astype(np.float32) * 2).astype(np.float16), B).view(np.float16).astype(np.float64)
    normal = np.abs(C1) >= 2.0 ** -13
    assert np.array_equal(C2[normal], 2 * C1[normal])


@pytest.mark.parametrize("K", [256, 512, 1024, 4096, 8192, 16384])
def test_gemm_8192_sampled(K):
    """M = N = 8192, K swept, default (bench) launch: sampled entries."""
    M = N = 8192
    A, B = operands("uniform", M, N, K)
    _say("gemm 8192x8192x%d uniform" % K)
    got = run_gemm(A, B)
    ij = sample_ij(M, N, 10000, seed=K)
    ref16, _ = oracle.gemm_nt_entries(A, B, ij)
    check_f16_tolerance(got[ij[:, 0], ij[:, 1]], ref16, "8192x8192x%d" % K)


def test_gemm_tile_order_leaves_every_output_unchanged():
    """The default at M = N = 8192, K = 16384 walks the tiles in panels of 4
    tile-rows; every tile is computed the same way in any order, so every
    output equals the plain order's bit for bit."""
    M = N = 8192
    K = 16384
    A, B = operands("uniform", M, N, K)
    d = gf.gemm_default_config(M, N, K)
    assert d["raster"] == 4
    _say("gemm 8192x8192x16384 default order against plain order")
    got = run_gemm(A, B)
    plain = run_gemm(A, B, cfg={**d, "raster": 0})
    assert np.array_equal(got, plain)


def test_gemm_8192_integer_sampled():
    M = N = K = 8192
    A, B = operands("integer", M, N, K)
    _say("gemm 8192^3 integer")
    got = run_gemm(A, B)
    ij = sample_ij(M, N, 10000, seed=1)
    ref16, _ = oracle.gemm_nt_entries(A, B, ij)
    assert np.array_equal(got[ij[:, 0], ij[:, 1]], ref16)


# ---------------------------------------------------------------------------
# wave-quantised shapes: the default launch runs the leading tile-rows in whole
# rounds of 256 x 256 tiles and the remaining rows as a second launch
# ---------------------------------------------------------------------------

def split_rows(M, N):
    """The row count of the first launch (M: no split), from the library's
    rule: the last round of 256 x 256 tiles over 256 CUs at most half full,
    a tail of at most 1024 rows."""
    tn = -(-N // 256)
    tiles = -(-M // 256) * tn
    rounds = -(-tiles // 256)
    if rounds < 2 or tiles - 256 * (rounds - 1) > 128:
        return M
    m1 = (256 * (rounds - 1) // tn) * 256
    return m1 if 256 <= m1 < M and M - m1 <= 1024 else M


# (M, N, K, tail form): a 256-row tail (one round of 128 x 128 tiles), a
# 768-row tail (two workgroups per CU), an 8-row and a 40-row tail (the
# skinny kernel), and ragged N and K; K where the default tile is 256 x 256 (one wave per SIMD at
# K = 2048, 8 waves at K <= 1536).
ROW_SPLIT_SHAPES = [(7168, 7168, 2048, "mfma"), (6144, 6144, 1024, "mfma"), (6920, 7168, 1024, "skinny"),
                    (7268, 7000, 1032, "mfma"), (6184, 8192, 4096, "skinny")]


@pytest.mark.parametrize("M,N,K,tail", ROW_SPLIT_SHAPES)
def test_gemm_row_split(M, N, K, tail):
    d = gf.gemm_default_config(M, N, K)
    assert (d["block_m"], d["block_n"]) == (256, 256), "the split applies to 256 x 256 tiles only"
    m1 = split_rows(M, N)
    assert m1 < M
    ij = sample_ij(M, N, 10000, seed=M + K)
    edge = [[r, c] for r in (0, m1 - 1, m1, min(m1 + 1, M - 1), M - 1) for c in (0, N // 2, N - 1)]
    ij = np.concatenate([ij, edge]).astype(np.int64)
    A, B = operands("integer", M, N, K, seed=3)
    _say("gemm row split %dx%dx%d (rows %d + %d) integer" % (M, N, K, m1, M - m1))
    got = run_gemm(A, B)
    ref16, _ = oracle.gemm_nt_entries(A, B, ij)
    assert np.array_equal(got[ij[:, 0], ij[:, 1]], ref16)
    A, B = operands("uniform", M, N, K, seed=3)
    _say("gemm row split %dx%dx%d uniform" % (M, N, K))
    got = run_gemm(A, B)
    ref16, _ = oracle.gemm_nt_entries(A, B, ij)
    check_f16_tolerance(got[ij[:, 0], ij[:, 1]], ref16, "row split %dx%dx%d" % (M, N, K))
    if tail == "mfma":
        # the same MFMAs over K in the same order: one launch of the big tile gives the same bits
        whole = run_gemm(A, B, cfg=gf.gemm_default_config(M, N, K))
        assert np.array_equal(got, whole), "row split changed the result"


# ---------------------------------------------------------------------------
# other operand layouts: A (M, K) or (K, M), B (N, K) or (K, N)
# ---------------------------------------------------------------------------

LAYOUTS = [(0, 1), (1, 1), (1, 0)]      # (a_kmajor, b_kmajor): NN, TN, and A^T . B^T


def stored(A, B, a_kmajor, b_kmajor):
    """The operands as the layout stores them (host arrays), from the (M, K)
    and (N, K) forms the oracle takes."""
    return (np.ascontiguousarray(A.T) if a_kmajor else A,
            np.ascontiguousarray(B.T) if b_kmajor else B)


def run_layout(A, B, a_kmajor, b_kmajor, cfg=None):
    As, Bs = stored(A, B, a_kmajor, b_kmajor)
    C = gf.gemm_f16(dev(As), dev(Bs), a_kmajor=a_kmajor, b_kmajor=b_kmajor, cfg=cfg)
    torch.cuda.synchronize()
    return host_u16(C)


@pytest.mark.parametrize("lay", LAYOUTS)
@pytest.mark.parametrize("M,N,K", [
    (256, 256, 256), (512, 384, 640), (640, 128, 1024),      # fast path, several tiles
    (100, 70, 1000), (130, 136, 72), (24, 40, 7),            # masked path (ragged extents)
    (8, 8, 8), (1, 1, 1), (16, 24, 0),
])
def test_gemm_layouts(M, N, K, lay):
    a_km, b_km = lay
    A, B = operands("integer", M, N, K, seed=7)
    assert np.array_equal(run_layout(A, B, a_km, b_km), oracle.gemm_nt_f16(A, B)), \
        "layout %s %dx%dx%d: integer inputs not bit-exact" % (lay, M, N, K)
    A, B = operands("uniform", M, N, K, seed=7)
    check_f16_tolerance(run_layout(A, B, a_km, b_km), oracle.gemm_nt_f16(A, B),
                        "layout %s %dx%dx%d" % (lay, M, N, K))


def test_gemm_layouts_every_config():
    """Every config that carries layout variants, each layout, two rasters."""
    M, N, K = 384, 512, 320
    A, B = operands("integer", M, N, K, seed=8)
    ref = oracle.gemm_nt_f16(A, B)
    n = 0
    for cfg, ok in gf.gemm_configs():
        if not ok or cfg["schedule"] != 2 or cfg["block_k"] != 64 or cfg["block_m"] % 128 or cfg["block_n"] % 128:
            continue
        for lay in LAYOUTS:
            for raster in (0, 1):
                c = dict(cfg, raster=raster)
                _say("layout %s cfg %s" % (lay, c))
                assert np.array_equal(run_layout(A, B, *lay, cfg=c), ref), (lay, c)
                n += 1
    assert n >= 24


@pytest.mark.parametrize("K,lay", [(8192, (0, 1)), (256, (0, 1)), (256, (1, 1))])
def test_gemm_layout_8192_sampled(K, lay):
    """K-major operands at M = N = 8192 with the library's tile (256 x 256;
    128 x 128 at K = 256), sampled."""
    M = N = 8192
    A, B = operands("uniform", M, N, K)
    _say("gemm layout %s 8192^2 x %d" % (lay, K))
    got = run_layout(A, B, *lay)
    ij = sample_ij(M, N, 10000, seed=11)
    ref16, _ = oracle.gemm_nt_entries(A, B, ij)
    check_f16_tolerance(got[ij[:, 0], ij[:, 1]], ref16, "gemm layout %s 8192^2 x %d sampled" % (lay, K))


# ---------------------------------------------------------------------------
# skinny GEMM (1 <= M <= 16 rows of A)
# ---------------------------------------------------------------------------

def run_skinny(A, B, cfg=None):
    C = gf.gemm_f16_nt_skinny(dev(A), dev(B), cfg=cfg)
    torch.cuda.synchronize()
    return host_u16(C)


@pytest.mark.parametrize("M", [1, 2, 3, 8, 15, 16])
@pytest.mark.parametrize("N,K", [(256, 512), (1000, 1032), (17, 8), (40, 24), (33, 0)])
def test_skinny(M, N, K):
    A, B = operands("integer", M, N, K, seed=5)
    assert np.array_equal(run_skinny(A, B), oracle.gemm_nt_f16(A, B)), \
        "skinny %dx%dx%d: integer inputs not bit-exact" % (M, N, K)
    A, B = operands("uniform", M, N, K, seed=5)
    check_f16_tolerance(run_skinny(A, B), oracle.gemm_nt_f16(A, B), "skinny %dx%dx%d" % (M, N, K))


def skinny_runs(cfg, M, K):
    """Whether a launch shape accepts M x K (its documented limits)."""
    if cfg["stages"] == 0:
        return True
    if cfg["stages"] >= 2:
        return K > 0 and K % 512 == 0
    if cfg["stages"] < 0:                              # split form
        return M <= 8 and K == 512 * cfg["unroll"] * cfg["waves"]
    mv = 1 if M <= 1 else (2 if M <= 2 else (4 if M <= 4 else 8))
    step = 64 * cfg["unroll"]                          # the last step of a row may be ragged
    npad = (K // 8 + step - 1) // step * step
    return M <= 8 and K > 0 and mv * npad * 16 <= 160 * 1024


@pytest.mark.parametrize("M,N,K", [(16, 520, 1536), (3, 1000, 512), (9, 77, 2048), (6, 300, 1024),
                                   (4, 1000, 4096), (8, 333, 2048), (1, 513, 2048), (2, 64, 8192),
                                   (7, 130, 16384), (5, 9000, 2048)])
def test_skinny_every_config(M, N, K):
    """Every launch shape: direct, LDS-staged (K a multiple of 512), vector
    form (M <= 8, A's rows padded to whole steps within 160 KiB; K not a
    multiple of 512 * unroll leaves a ragged last step; (5, 9000, 2048)
    gives waves more than one row group) and split form (M <= 8, K = 512 *
    unroll * waves: (2, 64, 8192) and (7, 130, 16384)); shapes outside a
    form's limits must be refused."""
    A, B = operands("integer", M, N, K, seed=6)
    ref = oracle.gemm_nt_f16(A, B)
    for cfg in gf.skinny_configs():
        _say("skinny cfg %s %dx%dx%d" % (cfg, M, N, K))
        if skinny_runs(cfg, M, K):
            assert np.array_equal(run_skinny(A, B, cfg), ref), cfg
        else:
            with pytest.raises(RuntimeError, match="UNSUPPORTED"):
                run_skinny(A, B, cfg)
    A, B = operands("uniform", M, N, K, seed=6)
    ref = oracle.gemm_nt_f16(A, B)
    for cfg in gf.skinny_configs():
        if skinny_runs(cfg, M, K):
            check_f16_tolerance(run_skinny(A, B, cfg), ref, "skinny %s %dx%dx%d" % (cfg, M, N, K))


def test_skinny_lds_form_needs_k_multiple_of_512():
    """K = 1000: the direct and vector forms run it (the vector form with a
    ragged last step), the LDS-staged and split forms refuse."""
    A, B = operands("integer", 4, 64, 1000, seed=6)
    ref = oracle.gemm_nt_f16(A, B)
    for cfg in gf.skinny_configs():
        if cfg["stages"] in (0, 1):
            assert np.array_equal(run_skinny(A, B, cfg), ref), cfg
        else:
            with pytest.raises(RuntimeError, match="UNSUPPORTED"):
                run_skinny(A, B, cfg)


def test_skinny_is_gemm_nt_for_small_m():
    """gemm_f16_nt takes the skinny kernel for M <= 16 (same bits), and
    agrees bit-exactly with the tiled kernel on integer inputs."""
    A, B = operands("integer", 6, 700, 2048, seed=9)
    got = run_gemm(A, B)
    assert np.array_equal(got, run_skinny(A, B))
    tiled = run_gemm(A, B, cfg=dict(block_m=64, block_n=64, block_k=64, stages=2, threads=256,
                                    raster=0, schedule=0))
    assert np.array_equal(got, tiled)


def lds_max_m(cfg):
    """Rows of A the LDS form of a launch shape takes: 16, or the largest of
    32, 48, 64 up to which its LDS ring (two or more 512-k chunks of
    16 * blocks + those rows, 1 KiB each, within 160 KiB) holds every count."""
    best = 16
    for ma in (32, 48, 64):
        rows = 16 * cfg["blocks"] + ma
        if not (rows % cfg["waves"] == 0 and cfg["stages"] * rows * 1024 <= 160 * 1024
                and (rows // cfg["waves"]) * cfg["stages"] < 64):
            break
        best = ma
    return best


@pytest.mark.parametrize("M", [17, 24, 32, 33, 48, 64])
@pytest.mark.parametrize("N,K", [(520, 1536), (77, 2048), (1000, 512)])
def test_skinny_wide_every_lds_config(M, N, K):
    """17 to 64 rows of A through the LDS form (A staged in 16-row blocks):
    every launch shape whose ring holds the rows, bit-exact on integers;
    the others, and the other forms, refused."""
    A, B = operands("integer", M, N, K, seed=12)
    ref = oracle.gemm_nt_f16(A, B)
    ran = 0
    for cfg in gf.skinny_configs():
        _say("skinny wide cfg %s %dx%dx%d" % (cfg, M, N, K))
        if cfg["stages"] >= 2 and M <= lds_max_m(cfg):
            assert np.array_equal(run_skinny(A, B, cfg), ref), cfg
            ran += 1
        else:
            with pytest.raises(RuntimeError, match="UNSUPPORTED"):
                run_skinny(A, B, cfg)
    assert ran >= 1                                                  # M = 64: one shape's ring holds it
    assert np.array_equal(run_skinny(A, B), ref)                     # the library's shape
    A, B = operands("uniform", M, N, K, seed=12)
    check_f16_tolerance(run_skinny(A, B), oracle.gemm_nt_f16(A, B), "skinny wide %dx%dx%d" % (M, N, K))


@pytest.mark.parametrize("M,N,K", [(24, 2048, 4096), (40, 8192, 4608), (64, 1000, 4096), (48, 9000, 4096),
                                   (32, 2048, 2048)])
def test_gemm_nt_takes_skinny_for_up_to_64_rows(M, N, K):
    """gemm_f16_nt routes 17 to 64 rows to the skinny kernel where B has at
    most 8192 rows and K >= 4096 (same bits as the explicit call), and to
    the tiles elsewhere; bit-exact on integers either way."""
    A, B = operands("integer", M, N, K, seed=13)
    _say("gemm nt %dx%dx%d (17..64 rows)" % (M, N, K))
    got = run_gemm(A, B)
    assert np.array_equal(got, oracle.gemm_nt_f16(A, B))
    if N <= 8192 and K >= 4096:
        assert np.array_equal(got, run_skinny(A, B))


@pytest.mark.parametrize("M", [32, 64])
def test_skinny_wide_8192(M):
    """17 to 64 rows against an 8192 x 8192 B, all outputs."""
    N = K = 8192
    A, B = operands("uniform", M, N, K)
    _say("skinny wide M=%d 8192^2" % M)
    check_f16_tolerance(run_skinny(A, B), oracle.gemm_nt_f16(A, B), "skinny wide M=%d 8192^2" % M)


@pytest.mark.parametrize("M", [1, 2, 4, 6, 16])
@pytest.mark.parametrize("N,K", [(4096, 14336), (6144, 6144), (2056, 4096), (12288, 6144), (16384, 2048),
                                 (8200, 4096)])
def test_skinny_default_shapes(M, N, K):
    """The library's launch shape where it depends on the size of B (16-wave
    vector workgroups, one or two 16-row blocks per LDS workgroup), all
    outputs."""
    A, B = operands("integer", M, N, K, seed=8)
    _say("skinny default %dx%dx%d cfg %s" % (M, N, K, gf.skinny_default_config(M, N, K)))
    assert np.array_equal(run_skinny(A, B), oracle.gemm_nt_f16(A, B))
    A, B = operands("uniform", M, N, K, seed=8)
    check_f16_tolerance(run_skinny(A, B), oracle.gemm_nt_f16(A, B), "skinny %dx%dx%d" % (M, N, K))


@pytest.mark.parametrize("M", [1, 3, 8])
@pytest.mark.parametrize("K", [11008, 1000, 13824, 8])
def test_skinny_vector_form_ragged_k(M, K):
    """The vector form on K with a ragged last step, every launch shape of
    it, all outputs; infinities in B's last chunks must not reach the
    padding lanes (an infinite B entry times a padded zero would be NaN)."""
    N = 300
    A, B = (x.copy() for x in operands("integer", M, N, K, seed=15))
    B[::7, -1] = np.float16(np.inf)
    B[1::7, -1] = np.float16(-np.inf)
    A[:, -1] = np.float16(1.0)
    ref = oracle.gemm_nt_f16(A, B)
    ran = 0
    for cfg in gf.skinny_configs():
        if cfg["stages"] != 1:
            continue
        _say("skinny vector ragged cfg %s %dx%dx%d" % (cfg, M, N, K))
        if skinny_runs(cfg, M, K):
            assert np.array_equal(run_skinny(A, B, cfg), ref), cfg
            ran += 1
        else:                                          # A's padded rows exceed the LDS
            with pytest.raises(RuntimeError, match="UNSUPPORTED"):
                run_skinny(A, B, cfg)
    mv = 1 if M <= 1 else (2 if M <= 2 else (4 if M <= 4 else 8))
    assert ran >= 1 or mv * (K // 8 + 63) // 64 * 64 * 16 > 160 * 1024


@pytest.mark.parametrize("M", [1, 2, 4])
@pytest.mark.parametrize("N,K", [(4096, 11008), (5120, 13824), (8200, 5120)])
def test_skinny_default_ragged_k(M, N, K):
    """The vector form where the library picks it with a ragged last step
    (K not a multiple of 2048), 16 and 8 waves, all outputs."""
    cfg = gf.skinny_default_config(M, N, K)
    assert cfg["stages"] == 1 and K % (512 * cfg["unroll"]) != 0
    A, B = operands("integer", M, N, K, seed=16)
    _say("skinny ragged default %dx%dx%d cfg %s" % (M, N, K, cfg))
    assert np.array_equal(run_skinny(A, B), oracle.gemm_nt_f16(A, B))
    A, B = operands("uniform", M, N, K, seed=16)
    check_f16_tolerance(run_skinny(A, B), oracle.gemm_nt_f16(A, B), "skinny ragged %dx%dx%d" % (M, N, K))


@pytest.mark.parametrize("M", [1, 2, 3, 5, 8])
@pytest.mark.parametrize("N,K", [(8192, 8192), (4100, 16384), (5000, 8192)])
def test_skinny_split_default_shapes(M, N, K):
    """The split form where the library picks it (M <= 8, K = 8192 or 16384,
    at least 4096 rows of B; 4100 and 5000 rows leave the grid-stride walk
    ragged), all outputs: integers bit-exact, uniform within tolerance."""
    assert gf.skinny_default_config(M, N, K)["stages"] == -1
    A, B = operands("integer", M, N, K, seed=14)
    _say("skinny split %dx%dx%d cfg %s" % (M, N, K, gf.skinny_default_config(M, N, K)))
    assert np.array_equal(run_skinny(A, B), oracle.gemm_nt_f16(A, B))
    A, B = operands("uniform", M, N, K, seed=14)
    check_f16_tolerance(run_skinny(A, B), oracle.gemm_nt_f16(A, B), "skinny split %dx%dx%d" % (M, N, K))


@pytest.mark.parametrize("M", [4, 16])
def test_skinny_decode_8192(M):
    """The decode-size case: M rows against an 8192 x 8192 B, all outputs."""
    N = K = 8192
    A, B = operands("uniform", M, N, K)
    _say("skinny decode M=%d 8192^2" % M)
    check_f16_tolerance(run_skinny(A, B), oracle.gemm_nt_f16(A, B), "skinny M=%d 8192^2" % M)


# ---------------------------------------------------------------------------
# split-K, fp32 out
# ---------------------------------------------------------------------------

def run_splitk(A, B, split_k, mode):
    dA, dB = dev(A), dev(B)
    if mode == "atomic":
        C = gf.gemm_f16_nt_splitk(dA, dB, split_k=split_k)
    else:
        C = gf.gemm_f16_nt_splitk_ex(dA, dB, split_k=split_k, mode=gf.GF_SPLITK_TWOPASS)
    torch.cuda.synchronize()
    return C.cpu().numpy()


@pytest.mark.parametrize("mode", ["atomic", "twopass"])
@pytest.mark.parametrize("split_k", [4, 8, 16])
def test_splitk_1024_16384(split_k, mode):
    """The split-K workload: M = N = 1024, K = 16384, sampled entries."""
    M = N = 1024
    K = 16384
    A, B = operands("uniform", M, N, K)
    _say("splitk 1024x1024x16384 s=%d %s" % (split_k, mode))
    got = run_splitk(A, B, split_k, mode)
    ij = sample_ij(M, N, 10000, seed=split_k)
    _, ref32 = oracle.gemm_nt_entries(A, B, ij)
    check_f32_splitk_tolerance(got[ij[:, 0], ij[:, 1]], ref32, K, "splitk s=%d %s" % (split_k, mode))
    Ai, Bi = operands("integer", M, N, K)
    got_i = run_splitk(Ai, Bi, split_k, mode)
    _, ref_i = oracle.gemm_nt_entries(Ai, Bi, ij)
    assert np.array_equal(got_i[ij[:, 0], ij[:, 1]], ref_i)


@pytest.mark.parametrize("mode", ["atomic", "twopass"])
@pytest.mark.parametrize("M,N,K,split_k", [
    (256, 256, 4096, 4), (100, 70, 1000, 3), (100, 70, 1000, 7), (65, 33, 64, 16),
    (17, 9, 1001, 5), (128, 128, 8, 1), (1, 1, 1, 1), (40, 24, 0, 4),
])
def test_splitk_full_small(M, N, K, split_k, mode):
    A, B = operands("uniform", M, N, K, seed=M * N + K)
    got = run_splitk(A, B, split_k, mode)
    ref = oracle.gemm_nt_f32(A, B)
    check_f32_splitk_tolerance(got, ref, K, "splitk %dx%dx%d s=%d %s" % (M, N, K, split_k, mode))
    Ai = inputs.integer_f16((M, K), 1, 0)
    Bi = inputs.integer_f16((N, K), 1, 1)
    assert np.array_equal(run_splitk(Ai, Bi, split_k, mode), oracle.gemm_nt_f32(Ai, Bi))


def test_splitk_every_config():
    """gemm_f16_nt_splitk_cfg on every config compiled with the fp32
    epilogues, all three combines, integer inputs (exact), a ragged shape."""
    M, N, K, split = 200, 136, 1000, 3
    Ai = inputs.integer_f16((M, K), 4, 0)
    Bi = inputs.integer_f16((N, K), 4, 1)
    ref32 = oracle.gemm_nt_f32(Ai, Bi)
    ref16 = oracle.gemm_nt_f16(Ai, Bi)
    dA, dB = dev(Ai), dev(Bi)
    ws = torch.empty(split * M * N, dtype=torch.float32, device="cuda")
    n = 0
    for cfg, ok in gf.gemm_configs():
        if not ok:
            continue
        for raster in (0, 1):
            c = dict(cfg, raster=raster)
            C32 = torch.empty((M, N), dtype=torch.float32, device="cuda")
            try:
                gf.gemm_f16_nt_splitk_cfg(dA, dB, C32, split, gf.GF_SPLITK_TWOPASS, c, ws)
            except RuntimeError as e:
                assert "unsupported" in str(e).lower(), e
                continue
            _say("splitk cfg %s" % c)
            torch.cuda.synchronize()
            assert np.array_equal(C32.cpu().numpy(), ref32), c
            gf.gemm_f16_nt_splitk_cfg(dA, dB, C32, split, gf.GF_SPLITK_ATOMIC, c, ws)
            torch.cuda.synchronize()
            assert np.array_equal(C32.cpu().numpy(), ref32), c
            C16 = torch.empty((M, N), dtype=torch.float16, device="cuda")
            gf.gemm_f16_nt_splitk_cfg(dA, dB, C16, split, gf.GF_SPLITK_F16, c, ws)
            torch.cuda.synchronize()
            assert np.array_equal(host_u16(C16), ref16), c
            n += 1
    assert n >= 20


def test_splitk_twopass_bitwise_deterministic():
    A, B = operands("uniform", 512, 512, 8192, seed=2)
    r1 = run_splitk(A, B, 16, "twopass")
    r2 = run_splitk(A, B, 16, "twopass")
    assert np.array_equal(r1.view(np.uint32), r2.view(np.uint32))


# ---------------------------------------------------------------------------
# split-K, fp16 out (slice partials summed in fp32, rounded once)
# ---------------------------------------------------------------------------

def run_splitk_f16(A, B, split_k):
    C = gf.gemm_f16_nt_splitk_f16(dev(A), dev(B), split_k=split_k)
    torch.cuda.synchronize()
    return host_u16(C)


@pytest.mark.parametrize("split_k", [4, 8, 16])
def test_splitk_f16_1024_16384(split_k):
    """fp16 output at the split-K workload: sampled entries against the
    oracle's fp16 result; integer inputs bit-exact."""
    M = N = 1024
    K = 16384
    A, B = operands("uniform", M, N, K)
    _say("splitk f16 1024x1024x16384 s=%d" % split_k)
    got = run_splitk_f16(A, B, split_k)
    ij = sample_ij(M, N, 10000, seed=100 + split_k)
    ref16, _ = oracle.gemm_nt_entries(A, B, ij)
    check_f16_tolerance(got[ij[:, 0], ij[:, 1]], ref16, "splitk f16 s=%d" % split_k)
    Ai, Bi = operands("integer", M, N, K)
    got_i = run_splitk_f16(Ai, Bi, split_k)
    ref_i, _ = oracle.gemm_nt_entries(Ai, Bi, ij)
    assert np.array_equal(got_i[ij[:, 0], ij[:, 1]], ref_i)


@pytest.mark.parametrize("M,N,K,split_k", [
    (256, 256, 4096, 4), (100, 70, 1000, 3), (100, 72, 1000, 7), (65, 33, 64, 16),
    (17, 9, 1001, 5), (128, 128, 8, 1), (1, 1, 1, 1), (40, 24, 0, 4),
])
def test_splitk_f16_full_small(M, N, K, split_k):
    A, B = operands("uniform", M, N, K, seed=M * N + K + 1)
    check_f16_tolerance(run_splitk_f16(A, B, split_k), oracle.gemm_nt_f16(A, B),
                        "splitk f16 %dx%dx%d s=%d" % (M, N, K, split_k))
    Ai = inputs.integer_f16((M, K), 2, 0)
    Bi = inputs.integer_f16((N, K), 2, 1)
    assert np.array_equal(run_splitk_f16(Ai, Bi, split_k), oracle.gemm_nt_f16(Ai, Bi))


@pytest.mark.parametrize("M,N,K,split_k", [(512, 512, 8192, 16), (100, 72, 1000, 7), (33, 17, 300, 3)])
def test_splitk_f16_is_twopass_rounded(M, N, K, split_k):
    """The fp16 output is the deterministic fp32 two-pass result rounded
    once to fp16 (numpy's float32 -> float16 cast is round-to-nearest-even),
    and it is the same from run to run."""
    A, B = operands("uniform", M, N, K, seed=3)
    f32 = run_splitk(A, B, split_k, "twopass")
    got = run_splitk_f16(A, B, split_k)
    assert np.array_equal(got, f32.astype(np.float16).view(np.uint16))
    assert np.array_equal(got, run_splitk_f16(A, B, split_k))


# ---------------------------------------------------------------------------
# GEMV
# ---------------------------------------------------------------------------

def run_gemv(W, x, cfg=None):
    y = gf.gemv_f16(dev(W), dev(x), cfg=cfg)
    torch.cuda.synchronize()
    return host_u16(y)


@pytest.mark.parametrize("NK", [1024, 8192])
@pytest.mark.parametrize("kind", ["uniform", "integer"])
def test_gemv_workloads(NK, kind):
    W = inputs.make(kind, (NK, NK), 0, inputs.STREAM_A)
    x = inputs.make(kind, (NK,), 0, inputs.STREAM_B)
    _say("gemv %d %s" % (NK, kind))
    got = run_gemv(W, x)
    ref = oracle.gemv_f16(W, x)
    if kind == "integer":
        assert np.array_equal(got, ref)
    else:
        check_f16_tolerance(got, ref, "gemv %d" % NK)


@pytest.mark.parametrize("N,K", [(1, 1), (1, 8), (7, 13), (1000, 1000), (1000, 1001),
                                 (33, 4104), (4097, 520), (5, 0)])
def test_gemv_ragged(N, K):
    W = inputs.uniform_f16((N, K), N + K, 0)
    x = inputs.uniform_f16((K,), N + K, 1)
    check_f16_tolerance(run_gemv(W, x), oracle.gemv_f16(W, x), "gemv %dx%d" % (N, K))


def test_gemv_every_config():
    N, K = 1000, 3000          # ragged rows and a ragged chunk tail
    W = inputs.uniform_f16((N, K), 4, 0)
    x = inputs.uniform_f16((K,), 4, 1)
    ref = oracle.gemv_f16(W, x)
    Wi = inputs.integer_f16((N, K), 4, 0)
    xi = inputs.integer_f16((K,), 4, 1)
    ref_i = oracle.gemv_f16(Wi, xi)
    dW, dx, dWi, dxi = dev(W), dev(x), dev(Wi), dev(xi)
    for cfg0 in gf.gemv_configs():
        for blocks in (0, 7, 256):        # one group per wave / grid-stride with x in LDS
            cfg = dict(cfg0, blocks=blocks)
            y = gf.gemv_f16(dW, dx, cfg=cfg)
            yi = gf.gemv_f16(dWi, dxi, cfg=cfg)
            torch.cuda.synchronize()
            check_f16_tolerance(host_u16(y), ref, "gemv cfg %s" % cfg)
            assert np.array_equal(host_u16(yi), ref_i), "gemv cfg %s integer" % cfg


@pytest.mark.parametrize("N,K", [(8192, 8192), (1001, 4096), (33, 1024), (1000, 1001),
                                 (3, 40000), (4097, 520)])
@pytest.mark.parametrize("kind", ["uniform", "integer"])
def test_gemv_bounded_grid(N, K, kind):
    """Bounded-grid launches: the waves-split-K kernel (K/8 a multiple of
    waves * 64 * unroll), the LDS-staged-x row-per-wave kernel, and the
    global-x fallback (K too large for LDS), on the workload and ragged
    shapes."""
    W = inputs.make(kind, (N, K), 11, 0)
    x = inputs.make(kind, (K,), 11, 1)
    ref = oracle.gemv_f16(W, x)
    for cfg in (dict(rows_per_wave=1, unroll=8, waves=4, blocks=512),
                dict(rows_per_wave=2, unroll=4, waves=4, blocks=256),
                dict(rows_per_wave=1, unroll=2, waves=8, blocks=3),
                dict(rows_per_wave=4, unroll=2, waves=2, blocks=100),
                dict(rows_per_wave=1, unroll=1, waves=2, blocks=5)):
        got = run_gemv(W, x, cfg)
        if kind == "integer":
            assert np.array_equal(got, ref), "gemv %dx%d %s" % (N, K, cfg)
        else:
            check_f16_tolerance(got, ref, "gemv %dx%d %s" % (N, K, cfg))


def test_gemv_matches_gemm_one_row_on_integers():
    W = inputs.integer_f16((300, 512), 8, 0)
    x = inputs.integer_f16((512,), 8, 1)
    assert np.array_equal(run_gemv(W, x), run_gemm(x[None, :], W)[0])

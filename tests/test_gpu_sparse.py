"""GPU parity of the 2:4 structured-sparse path against the CPU oracle.

* Compression (sp24_compress_f16) is byte work: bit-exact against
  oracle.sp24_compress on every input, special values included.
* The sparse product (gemm_sp_f16_nt): integer inputs in {-2..2} bit-exact;
  uniform[-1,1] inputs within 1 fp16 ulp(C_ref) + 1e-3, the dense GEMM's bar
  (the same fp32 accumulation of exact fp16 products, one fp16 rounding).
  Full-size shapes are checked on sampled entries the oracle computes one by
  one, in the launch configuration the benchmark times.
"""
import sys

import numpy as np
import pytest

import gemv_fp16_amd as gf
import inputs
import oracle
from tests.util import check_f16_tolerance, dev, host_u16, sample_ij

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


def dev_e(E):
    return dev(np.ascontiguousarray(E).view(np.int16))


def host_e(t):
    return t.cpu().numpy().view(np.uint16)


def gpu_compress(A):
    Asp, E = gf.sp24_compress_f16(dev(A))
    torch.cuda.synchronize()
    return host_u16(Asp), host_e(E)


def sp_run(Asp, E, B, cfg=None):
    C = gf.gemm_sp_f16_nt(dev(Asp.view(np.float16)), dev_e(E), dev(B), cfg=cfg)
    torch.cuda.synchronize()
    return host_u16(C)


def check(got, ref, kind, what):
    if kind == "integer":
        assert np.array_equal(got, ref), what + ": integer inputs not bit-exact"
    else:
        check_f16_tolerance(got, ref, what)


# ---------------------------------------------------------------------------
# compression
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("M,K", [(1, 16), (3, 48), (64, 64), (257, 1040), (1024, 4096)])
@pytest.mark.parametrize("kind", ["uniform", "integer"])
def test_compress_matches_oracle(M, K, kind):
    _say("compress %s %dx%d" % (kind, M, K))
    A = inputs.make(kind, (M, K), seed=M + K)
    Asp, E = gpu_compress(A)
    rAsp, rE = oracle.sp24_compress(A)
    assert np.array_equal(E, rE)
    assert np.array_equal(Asp, rAsp)


def test_compress_every_group_of_special_values():
    vals = np.array([0.0, -0.0, 1.0, -1.0, 2.0, np.inf, -np.inf, np.nan], dtype=np.float16)
    idx = np.stack(np.meshgrid(*[np.arange(8)] * 4, indexing="ij"), -1).reshape(-1)
    A = vals[idx].reshape(-1, 64)        # 4096 groups, 16 per row
    _say("compress special values %s" % (A.shape,))
    Asp, E = gpu_compress(A)
    rAsp, rE = oracle.sp24_compress(A)
    assert np.array_equal(E, rE)
    assert np.array_equal(Asp, rAsp)


def test_compress_unaligned_pointers():
    M, K = 33, 160
    A = inputs.make("uniform", (M, K), seed=11)
    flat = dev(np.concatenate([np.zeros(1, np.float16), A.ravel()]))
    At = flat[1:].view(M, K)                      # 2-byte aligned only
    asp_buf = torch.empty(M * K // 2 + 1, dtype=torch.float16, device="cuda")
    e_buf = torch.empty(M * K // 16 + 1, dtype=torch.int16, device="cuda")
    Asp, E = asp_buf[1:].view(M, K // 2), e_buf[1:].view(M, K // 16)
    _say("compress unaligned")
    gf.sp24_compress_f16(At, Asp, E)
    torch.cuda.synchronize()
    rAsp, rE = oracle.sp24_compress(A)
    assert np.array_equal(host_e(E), rE)
    assert np.array_equal(host_u16(Asp), rAsp)


def test_compress_8192_full():
    A = inputs.make("uniform", (8192, 8192), seed=1)
    _say("compress 8192x8192")
    Asp, E = gpu_compress(A)
    rAsp, rE = oracle.sp24_compress(A)
    assert np.array_equal(E, rE)
    assert np.array_equal(Asp, rAsp)


# ---------------------------------------------------------------------------
# the sparse product
# ---------------------------------------------------------------------------

# (M, N, K): several tiles with ragged M/N tails; K % 64 == 32 (the direct-
# to-LDS path with a ragged last K tile); K % 32 == 16 (the register-staged
# path); tiny shapes.
SP_SHAPES = [(256, 256, 256), (128, 128, 64), (1, 1, 16), (5, 7, 32), (300, 200, 352),
             (300, 200, 272), (513, 257, 1024), (64, 1000, 2048), (777, 555, 96)]


@pytest.mark.parametrize("M,N,K", SP_SHAPES)
@pytest.mark.parametrize("kind", ["integer", "uniform"])
def test_sparse_gemm_on_24_inputs(M, N, K, kind):
    _say("sparse gemm %s %dx%dx%d" % (kind, M, N, K))
    A = inputs.sparse24(kind, (M, K), seed=M + N + K)
    B = inputs.make(kind, (N, K), seed=M + N + K, stream_id=inputs.STREAM_B)
    Asp, E = oracle.sp24_compress(A)
    check(sp_run(Asp, E, B), oracle.gemm_sp_nt_f16(Asp, E, B), kind, "sparse %dx%dx%d" % (M, N, K))


@pytest.mark.parametrize("kind", ["integer", "uniform"])
def test_sparse_gemm_of_pruned_dense_a(kind):
    """Dense A: compression prunes it; the product is the pruned A's."""
    M, N, K = 384, 320, 512
    A = inputs.make(kind, (M, K), seed=3)
    B = inputs.make(kind, (N, K), seed=3, stream_id=inputs.STREAM_B)
    _say("sparse gemm pruned dense A %s" % kind)
    Asp, E = gpu_compress(A)
    ref = oracle.gemm_sp_nt_f16(*oracle.sp24_compress(A), B)
    check(sp_run(Asp, E, B), ref, kind, "pruned dense A")


def test_sparse_gemm_every_config():
    cfgs = gf.sp_configs()
    assert len(cfgs) >= 1
    for shape, kind in (((300, 520, 352), "integer"), ((512, 512, 1024), "uniform")):
        M, N, K = shape
        A = inputs.sparse24(kind, (M, K), seed=21)
        B = inputs.make(kind, (N, K), seed=21, stream_id=inputs.STREAM_B)
        Asp, E = oracle.sp24_compress(A)
        ref = oracle.gemm_sp_nt_f16(Asp, E, B)
        for cfg in cfgs:
            for raster in (0, 1):
                c = dict(cfg, raster=raster)
                _say("sparse cfg %s %s %s" % (c, shape, kind))
                check(sp_run(Asp, E, B, c), ref, kind, "cfg %s" % c)


# The paired form (stages = 0): A_sparse two K tiles per load, metadata eight.
# K spans the steady loop and the masked tail, several metadata slots, a
# ragged last K tile (K % 64 == 32) and an odd tile count; M and N are ragged.
PAIR_SHAPES = [((520, 264, 2080), "integer"), ((777, 300, 1056), "uniform"), ((256, 512, 4160), "integer"),
               ((300, 130, 96), "integer"), ((129, 257, 544), "uniform")]


@pytest.mark.parametrize("shape,kind", PAIR_SHAPES)
def test_sparse_paired_form(shape, kind):
    M, N, K = shape
    cfgs = [c for c in gf.sp_configs() if c["stages"] == 0]
    assert cfgs, "no paired-form config compiled"
    A = inputs.sparse24(kind, (M, K), seed=M + K)
    B = inputs.make(kind, (N, K), seed=N + K, stream_id=inputs.STREAM_B)
    Asp, E = oracle.sp24_compress(A)
    ref = oracle.gemm_sp_nt_f16(Asp, E, B)
    for cfg in cfgs:
        for raster in (0, 1):
            c = dict(cfg, raster=raster)
            _say("sparse paired %s %s %s" % (c, shape, kind))
            check(sp_run(Asp, E, B, c), ref, kind, "paired cfg %s %s" % (c, shape))


def test_sparse_gemm_zero_k_writes_zeros():
    M, N = 70, 90
    Asp = np.zeros((M, 0), np.uint16)
    E = np.zeros((M, 0), np.uint16)
    B = np.zeros((N, 0), np.float16)
    C = torch.full((M, N), 7.0, dtype=torch.float16, device="cuda")
    _say("sparse gemm K = 0")
    gf.gemm_sp_f16_nt(torch.empty((M, 0), dtype=torch.float16, device="cuda"),
                      torch.empty((M, 0), dtype=torch.int16, device="cuda"),
                      torch.empty((N, 0), dtype=torch.float16, device="cuda"), C)
    torch.cuda.synchronize()
    assert not host_u16(C).any()
    del Asp, E, B


def test_sparse_gemm_unaligned_pointers():
    M, N, K = 200, 136, 320
    A = inputs.sparse24("integer", (M, K), seed=8)
    B = inputs.make("integer", (N, K), seed=8, stream_id=inputs.STREAM_B)
    Asp, E = oracle.sp24_compress(A)

    def shifted(a, dtype):
        flat = dev(np.concatenate([np.zeros(1, a.dtype), a.ravel()]))
        return flat[1:].view(*a.shape)

    At = shifted(Asp.view(np.float16), torch.float16)
    Et = shifted(E.view(np.int16), torch.int16)
    Bt = shifted(B, torch.float16)
    cbuf = torch.empty(M * N + 1, dtype=torch.float16, device="cuda")
    C = cbuf[1:].view(M, N)
    _say("sparse gemm unaligned")
    gf.gemm_sp_f16_nt(At, Et, Bt, C)
    torch.cuda.synchronize()
    assert np.array_equal(host_u16(C), oracle.gemm_sp_nt_f16(Asp, E, B))


def test_sparse_end_to_end_8192_sampled():
    """The benchmark's workload and launch configuration: dense uniform A
    compressed on the GPU, then the sparse product with the default tile."""
    M = N = K = 8192
    A = inputs.make("uniform", (M, K), seed=0)
    B = inputs.make("uniform", (N, K), seed=0, stream_id=inputs.STREAM_B)
    _say("sparse end-to-end 8192")
    Asp_t, E_t = gf.sp24_compress_f16(dev(A))
    C = gf.gemm_sp_f16_nt(Asp_t, E_t, dev(B))
    torch.cuda.synchronize()
    rAsp, rE = oracle.sp24_compress(A)
    assert np.array_equal(host_e(E_t), rE)
    assert np.array_equal(host_u16(Asp_t), rAsp)
    ij = sample_ij(M, N, 10000, seed=5)
    got = host_u16(C)[ij[:, 0], ij[:, 1]]
    ref = oracle.gemm_sp_nt_entries(rAsp, rE, B, ij)
    check_f16_tolerance(got, ref, "sparse 8192 sampled")


def test_sparse_8192_integer_sampled():
    M = N = K = 8192
    A = inputs.sparse24("integer", (M, K), seed=2)
    B = inputs.make("integer", (N, K), seed=2, stream_id=inputs.STREAM_B)
    Asp, E = oracle.sp24_compress(A)
    _say("sparse 8192 integer")
    got = sp_run(Asp, E, B)
    ij = sample_ij(M, N, 10000, seed=6)
    assert np.array_equal(got[ij[:, 0], ij[:, 1]], oracle.gemm_sp_nt_entries(Asp, E, B, ij))


def test_sparse_default_half_tile_shape_sampled():
    """A shape whose default is the half-size tile (128 x 256, three
    stages): integer inputs, the library's own launch configuration, sampled
    entries."""
    M, N, K = 2048, 4096, 8192
    assert (gf.sp_default_config(M, N, K)["block_m"], gf.sp_default_config(M, N, K)["block_n"]) == (128, 256)
    A = inputs.sparse24("integer", (M, K), seed=9)
    B = inputs.make("integer", (N, K), seed=9, stream_id=inputs.STREAM_B)
    Asp, E = oracle.sp24_compress(A)
    _say("sparse default half tile %dx%dx%d" % (M, N, K))
    got = sp_run(Asp, E, B)
    ij = sample_ij(M, N, 10000, seed=13)
    ij = np.concatenate([ij, [[M - 1, N - 1], [0, N - 1], [M - 1, 0]]]).astype(np.int64)
    assert np.array_equal(got[ij[:, 0], ij[:, 1]], oracle.gemm_sp_nt_entries(Asp, E, B, ij))


@pytest.mark.parametrize("M,N,K", [(7168, 7168, 512), (6144, 6144, 256)])
def test_sparse_row_split(M, N, K):
    """Shapes whose last round of 256 x 256 tiles is at most half full: the
    default call splits the rows (7168: 6912 + 256, 6144: 5376 + 768).
    Integer inputs bit-exact on sampled entries around the split; uniform
    inputs give the same bits as one launch of the default tile."""
    m1 = {7168: 6912, 6144: 5376}[M]
    ij = sample_ij(M, N, 10000, seed=M + K)
    edge = [[r, c] for r in (0, m1 - 1, m1, M - 1) for c in (0, N // 2, N - 1)]
    ij = np.concatenate([ij, edge]).astype(np.int64)
    A = inputs.sparse24("integer", (M, K), seed=4)
    B = inputs.make("integer", (N, K), seed=4, stream_id=inputs.STREAM_B)
    Asp, E = oracle.sp24_compress(A)
    _say("sparse row split %dx%dx%d integer" % (M, N, K))
    got = sp_run(Asp, E, B)
    assert np.array_equal(got[ij[:, 0], ij[:, 1]], oracle.gemm_sp_nt_entries(Asp, E, B, ij))
    A = inputs.sparse24("uniform", (M, K), seed=4)
    B = inputs.make("uniform", (N, K), seed=4, stream_id=inputs.STREAM_B)
    Asp, E = oracle.sp24_compress(A)
    _say("sparse row split %dx%dx%d uniform" % (M, N, K))
    got = sp_run(Asp, E, B)
    check_f16_tolerance(got[ij[:, 0], ij[:, 1]], oracle.gemm_sp_nt_entries(Asp, E, B, ij), "sparse row split")
    whole = sp_run(Asp, E, B, gf.sp_default_config(M, N, K))
    assert np.array_equal(got, whole), "row split changed the sparse result"

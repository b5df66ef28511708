"""GPU parity at the largest operand the C ABI accepts (just under 2^31
elements, 4 GiB of fp16), where the kernels' 32-bit byte offsets reach their
largest values.

Inputs: a seeded integer block of 1024 rows, tiled down the rows, with one
entry per row changed so that rows 1024 apart differ (a row-offset mistake
shows up as a wrong product).  Integer inputs in {-2..2} make every result
exact, so the checks are bit-exact: GEMM on sampled entries including the last
rows and columns, GEMV on every output, the 2:4 sparse product (default tile
and the paired form) on sampled entries.
"""
import sys

import numpy as np
import pytest

import gemv_fp16_amd as gf
import inputs
import oracle
from tests.util import dev, host_u16, sample_ij

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

ROWS, K = 65535, 32768          # 65535 * 32768 = 2^31 - 2^15 elements
NG = 65528                      # GEMM's N: a multiple of 8, so the 128-bit (direct-to-LDS) path runs


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    gf.lib()
    yield
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def tall_integer(rows, k, seed):
    """rows x k fp16 integers: a seeded 1024-row block tiled down the rows;
    entry (r, 0) is ((r // 1024) % 5) - 2 so that tiled copies differ."""
    block = inputs.integer_f16((1024, k), seed, inputs.STREAM_B)
    out = np.tile(block, (-(-rows // 1024), 1))[:rows]
    out[:, 0] = (((np.arange(rows) // 1024) % 5) - 2).astype(np.float16)
    return out


def test_gemm_largest_b():
    M = 256
    A = inputs.integer_f16((M, K), 3, inputs.STREAM_A)
    B = tall_integer(NG, K, 3)
    _say("gemm %dx%dx%d (B of %d elements)" % (M, NG, K, NG * K))
    C = gf.gemm_f16_nt(dev(A), dev(B))
    torch.cuda.synchronize()
    got = host_u16(C)
    del C
    ij = sample_ij(M, NG, 10000, seed=11)
    ij = np.concatenate([ij, [[M - 1, NG - 1], [0, NG - 1], [M - 1, NG - 1024]]]).astype(np.int64)
    ref16, _ = oracle.gemm_nt_entries(A, B, ij)
    assert np.array_equal(got[ij[:, 0], ij[:, 1]], ref16)


def test_gemv_largest_w():
    W = tall_integer(ROWS, K, 4)
    x = inputs.integer_f16((K,), 4, inputs.STREAM_A)
    _say("gemv %dx%d (W of %d elements)" % (ROWS, K, ROWS * K))
    y = gf.gemv_f16(dev(W), dev(x))
    torch.cuda.synchronize()
    assert np.array_equal(host_u16(y), oracle.gemv_f16(W, x))


@pytest.mark.parametrize("cfg", [None, {"block_m": 256, "block_n": 128, "stages": 0, "raster": 1}],
                         ids=["default", "paired"])
def test_sparse_largest_a(cfg):
    N = 256
    block = inputs.sparse24("integer", (1024, K), 5, inputs.STREAM_A)
    bsp, be = oracle.sp24_compress(block)
    reps = -(-ROWS // 1024)
    Asp = np.tile(bsp, (reps, 1))[:ROWS]
    E = np.tile(be, (reps, 1))[:ROWS]
    Asp[:, 0] = (((np.arange(ROWS) // 1024) % 5) - 2).astype(np.float16).view(np.uint16)
    B = inputs.integer_f16((N, K), 5, inputs.STREAM_B)
    _say("sparse %dx%dx%d (A_sparse of %d elements) cfg %s" % (ROWS, N, K, Asp.size, cfg))
    C = gf.gemm_sp_f16_nt(dev(Asp.view(np.float16)), dev(E.view(np.int16)), dev(B), cfg=cfg)
    torch.cuda.synchronize()
    got = host_u16(C)
    del C
    ij = sample_ij(ROWS, N, 10000, seed=12)
    ij = np.concatenate([ij, [[ROWS - 1, N - 1], [ROWS - 1, 0], [ROWS - 1025, 7]]]).astype(np.int64)
    assert np.array_equal(got[ij[:, 0], ij[:, 1]], oracle.gemm_sp_nt_entries(Asp, E, B, ij))

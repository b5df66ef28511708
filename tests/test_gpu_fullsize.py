"""GPU parity on every output of the full-size workloads.

The oracle's full output of each workload is computed once per test session
(on all host threads) and kept in memory; every output of the HIP path is
then compared with it:

* the headline product C = A . B^T at M = N = K = 8192, uniform inputs
  (within 1 fp16 ulp + 1e-3) and integer inputs (bit-exact), and the NN and
  TN layouts of the same product against the same reference;
* M = N = 8192 with K = 1024, uniform inputs;
* split-K at M = N = 1024, K = 16384: every split (4, 8, 16) in every
  combine (fp32 atomic, fp32 two-pass, fp16 two-pass), uniform and integer
  inputs.

The other K of the 8192^2 products are checked on sampled entries in
test_gpu_parity.py.
"""
import sys
import time

import numpy as np
import pytest

import gemv_fp16_amd as gf
import inputs
import oracle
from tests.util import check_f16_tolerance, check_f32_splitk_tolerance, dev, host_u16

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


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


_ops = {}
_refs = {}


def operands(kind, M, N, K):
    key = (kind, M, N, K)
    if key not in _ops:
        _ops.clear()
        _ops[key] = (inputs.make(kind, (M, K), 0, inputs.STREAM_A),
                     inputs.make(kind, (N, K), 0, inputs.STREAM_B))
    return _ops[key]


def reference(kind, M, N, K, out):
    """The oracle's full fp16 (out = 16) or fp32 (out = 32) output, computed once."""
    key = (kind, M, N, K, out)
    if key not in _refs:
        A, B = operands(kind, M, N, K)
        t = time.time()
        _refs[key] = oracle.gemm_nt_f16(A, B) if out == 16 else oracle.gemm_nt_f32(A, B)
        _say("oracle %s %dx%dx%d fp%d: %.1f s on %d threads" % (kind, M, N, K, out, time.time() - t,
                                                                 oracle.threads()))
    return _refs[key]


def check16(got, ref, kind, what):
    if kind == "integer":
        bad = np.count_nonzero(got != ref)
        assert bad == 0, "%s: %d of %d entries differ" % (what, bad, got.size)
    else:
        check_f16_tolerance(got, ref, what)


@pytest.mark.parametrize("kind", ["uniform", "integer"])
def test_gemm_8192_cube_every_output(kind):
    M = N = K = 8192
    A, B = operands(kind, M, N, K)
    _say("gemm 8192^3 %s: every output" % kind)
    C = gf.gemm_f16_nt(dev(A), dev(B))
    torch.cuda.synchronize()
    check16(host_u16(C), reference(kind, M, N, K, 16), kind, "gemm 8192^3 " + kind)


@pytest.mark.parametrize("lay", ["nn", "tn"])
def test_gemm_layouts_8192_cube_every_output(lay):
    """B stored K x N (and A K x M for TN): the same product, every output."""
    M = N = K = 8192
    A, B = operands("uniform", M, N, K)
    _say("gemm 8192^3 %s: every output" % lay)
    Bt = dev(np.ascontiguousarray(B.T))
    if lay == "nn":
        C = gf.gemm_f16(dev(A), Bt, a_kmajor=False, b_kmajor=True)
    else:
        C = gf.gemm_f16(dev(np.ascontiguousarray(A.T)), Bt, a_kmajor=True, b_kmajor=True)
    torch.cuda.synchronize()
    check16(host_u16(C), reference("uniform", M, N, K, 16), "uniform", "gemm 8192^3 " + lay)


def test_gemm_8192_k1024_every_output():
    M = N = 8192
    K = 1024
    A, B = operands("uniform", M, N, K)
    _say("gemm 8192^2 x 1024: every output")
    C = gf.gemm_f16_nt(dev(A), dev(B))
    torch.cuda.synchronize()
    check16(host_u16(C), reference("uniform", M, N, K, 16), "uniform", "gemm 8192^2 x 1024")


@pytest.mark.parametrize("kind", ["uniform", "integer"])
def test_splitk_1024_16384_every_output(kind):
    """Every split and combine of the split-K workload, every output."""
    M = N = 1024
    K = 16384
    A, B = operands(kind, M, N, K)
    ref32 = reference(kind, M, N, K, 32)
    ref16 = reference(kind, M, N, K, 16)
    dA, dB = dev(A), dev(B)
    for split in (4, 8, 16):
        _say("splitk 1024^2 x 16384 %s s=%d: every output, three combines" % (kind, split))
        c_at = gf.gemm_f16_nt_splitk(dA, dB, split_k=split)
        c_tp = gf.gemm_f16_nt_splitk_ex(dA, dB, split_k=split, mode=gf.GF_SPLITK_TWOPASS)
        c16 = gf.gemm_f16_nt_splitk_f16(dA, dB, split_k=split)
        torch.cuda.synchronize()
        for name, c in (("atomic", c_at), ("twopass", c_tp)):
            got = c.cpu().numpy()
            if kind == "integer":
                assert np.array_equal(got, ref32), "splitk s=%d %s" % (split, name)
            else:
                check_f32_splitk_tolerance(got, ref32, K, "splitk s=%d %s" % (split, name))
        check16(host_u16(c16), ref16, kind, "splitk f16 s=%d" % split)

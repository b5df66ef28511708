"""The split-K entry point that allocates nothing (gemm_f16_nt_splitk_noalloc).

Called through the C ABI (ctypes, device pointers of tensors allocated up
front) twice in a row, the second call smaller than the first, and checked
bit for bit against the existing two-pass entry point
(gemm_f16_nt_splitk_ex, GF_SPLITK_TWOPASS) on the same inputs -- the same
slice partials summed in the same order -- and integer inputs against the
oracle exactly.  A problem whose partials exceed the scratch is refused on
the host.  torch's allocator must not move across the calls.
"""
import ctypes
import sys

import numpy as np
import pytest

import gemv_fp16_amd as gf
import inputs
import oracle
from tests.util import dev

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


def _p(t):
    return ctypes.c_void_p(t.data_ptr())


def test_noalloc_equals_two_pass_twice_then_smaller():
    L = gf.lib()
    assert L.gf_noalloc_scratch_bytes() == 64 << 20
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    # (M, N, K, split_k, kind): the first fills the scratch exactly (16 slices
    # of 1024 x 1024 fp32), the second is smaller and ragged
    cases = [(1024, 1024, 16384, 16, "uniform"), (300, 200, 2000, 5, "integer")]
    prepared = []
    for M, N, K, split, kind in cases:
        A = inputs.make(kind, (M, K), 31, inputs.STREAM_A)
        B = inputs.make(kind, (N, K), 31, inputs.STREAM_B)
        prepared.append((A, B, dev(A), dev(B), torch.full((M, N), 7.0, dtype=torch.float32, device="cuda")))
    torch.cuda.synchronize()
    for (M, N, K, split, kind), (A, B, dA, dB, C) in zip(cases, prepared):
        _say("noalloc %dx%dx%d split %d %s" % (M, N, K, split, kind))
        before = torch.cuda.memory_allocated()
        rc = L.gemm_f16_nt_splitk_noalloc(_p(dA), _p(dB), _p(C), M, N, K, split, stream)
        assert rc == gf.GF_OK, gf.status_string(rc)
        torch.cuda.synchronize()
        assert torch.cuda.memory_allocated() == before
        ref = gf.gemm_f16_nt_splitk_ex(dA, dB, split_k=split, mode=gf.GF_SPLITK_TWOPASS)
        torch.cuda.synchronize()
        got = C.cpu().numpy()
        assert np.array_equal(got.view(np.uint32), ref.cpu().numpy().view(np.uint32))
        if kind == "integer":
            assert np.array_equal(got, oracle.gemm_nt_f32(A, B))


def test_noalloc_on_a_side_stream():
    """On a stream other than the null stream the scratch is found through
    the stream's device; the result still equals the two-pass entry point's."""
    L = gf.lib()
    M, N, K, split = 256, 384, 4096, 8
    A = inputs.make("integer", (M, K), 32, inputs.STREAM_A)
    B = inputs.make("integer", (N, K), 32, inputs.STREAM_B)
    dA, dB = dev(A), dev(B)
    C = torch.zeros((M, N), dtype=torch.float32, device="cuda")
    side = torch.cuda.Stream()
    torch.cuda.synchronize()
    _say("noalloc %dx%dx%d split %d on a side stream" % (M, N, K, split))
    rc = L.gemm_f16_nt_splitk_noalloc(_p(dA), _p(dB), _p(C), M, N, K, split, ctypes.c_void_p(side.cuda_stream))
    assert rc == gf.GF_OK, gf.status_string(rc)
    side.synchronize()
    assert np.array_equal(C.cpu().numpy(), oracle.gemm_nt_f32(A, B))


def test_noalloc_refuses_more_than_its_scratch():
    L = gf.lib()
    dA = torch.zeros((1024, 64), dtype=torch.float16, device="cuda")
    dB = torch.zeros((1024, 64), dtype=torch.float16, device="cuda")
    C = torch.zeros((1024, 1024), dtype=torch.float32, device="cuda")
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    assert L.gemm_f16_nt_splitk_noalloc(_p(dA), _p(dB), _p(C), 1024, 1024, 64, 17, stream) == \
        gf.GF_ERR_TOO_LARGE
    assert L.gemm_f16_nt_splitk_noalloc(_p(dA), _p(dB), _p(C), 1024, 1024, 64, 0, stream) == \
        gf.GF_ERR_INVALID_ARG

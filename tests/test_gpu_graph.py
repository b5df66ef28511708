"""The library's calls under HIP graph capture and on concurrent streams.

Every entry point only launches kernels on the caller's stream: it allocates
nothing and records no memset (the atomic split-K clears its output with a
fill kernel), so a caller can capture it into a graph.  One graph here holds
the NT and NN products, split-K in all three modes, the GEMV, the skinny
GEMM in its split form and in its vector form with a ragged last step, the
2:4 compression and the sparse product.  It is replayed three times, with new
input contents copied into the captured buffers before each replay and the
same calls made eagerly (into other outputs) between replays; each replay's
outputs must equal the eager ones bit for bit.  Inputs are integers in
{-2..2}, so even the atomic split-K, whose order of additions varies, gives
exact and therefore identical sums.
"""
import sys

import numpy as np
import pytest

import gemv_fp16_amd as gf
import inputs
import oracle
from tests.util import dev, host_u16

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


# (M, N, K) of each call; several tiles each, ragged M and N
GM, GN, GK = 520, 392, 1024        # GEMM NT and NN
SM, SN, SK, SPLIT = 264, 200, 4096, 4
VN, VK = 4100, 2048                # GEMV
PM, PN, PK = 300, 264, 1024        # 2:4
KM, KN, KK = 4, 600, 8192          # skinny, split form
RM, RN, RK = 3, 300, 11008         # skinny, vector form with a ragged last step
SPLIT_CFG = {"blocks": 512, "unroll": 4, "waves": 4, "stages": -1}
RAGGED_CFG = {"blocks": 1, "unroll": 4, "waves": 16, "stages": 1}


class Buffers:
    """Device inputs (refilled between replays) and two sets of outputs."""

    def __init__(self):
        z = lambda shape, dt=torch.float16: torch.zeros(shape, dtype=dt, device="cuda")
        self.A, self.B, self.Bkn = z((GM, GK)), z((GN, GK)), z((GK, GN))
        self.SA, self.SB = z((SM, SK)), z((SN, SK))
        self.W, self.x = z((VN, VK)), z((VK,))
        self.PA, self.PB = z((PM, PK)), z((PN, PK))
        self.KA, self.KB = z((KM, KK)), z((KN, KK))
        self.RA, self.RB = z((RM, RK)), z((RN, RK))
        ws_elems = gf.gemm_f16_nt_splitk_workspace_bytes(SM, SN, SPLIT) // 4
        self.ws = [torch.empty(ws_elems, dtype=torch.float32, device="cuda") for _ in range(2)]
        self.out = [self._outputs() for _ in range(2)]     # [0]: graph, [1]: eager

    @staticmethod
    def _outputs():
        e = lambda shape, dt=torch.float16: torch.empty(shape, dtype=dt, device="cuda")
        return dict(nt=e((GM, GN)), nn=e((GM, GN)), atomic=e((SM, SN), torch.float32),
                    twopass=e((SM, SN), torch.float32), f16=e((SM, SN)), y=e((VN,)),
                    asp=e((PM, PK // 2)), meta=e((PM, PK // 16), torch.int16), sp=e((PM, PN)),
                    ks=e((KM, KN)), kr=e((RM, RN)))

    def fill(self, seed):
        host = {}
        for name, shape, stream in (("A", (GM, GK), 0), ("B", (GN, GK), 1), ("SA", (SM, SK), 0),
                                    ("SB", (SN, SK), 1), ("W", (VN, VK), 0), ("x", (VK,), 1),
                                    ("PA", (PM, PK), 0), ("PB", (PN, PK), 1), ("KA", (KM, KK), 0),
                                    ("KB", (KN, KK), 1), ("RA", (RM, RK), 0), ("RB", (RN, RK), 1)):
            host[name] = inputs.integer_f16(shape, seed, stream)
            getattr(self, name).copy_(dev(host[name]))
        self.Bkn.copy_(dev(np.ascontiguousarray(host["B"].T)))
        return host

    def run(self, k):
        """Every call once, into output set k."""
        o = self.out[k]
        gf.gemm_f16_nt(self.A, self.B, o["nt"])
        gf.gemm_f16_nn(self.A, self.Bkn, o["nn"])
        gf.gemm_f16_nt_splitk(self.SA, self.SB, o["atomic"], split_k=SPLIT)
        gf.gemm_f16_nt_splitk_ex(self.SA, self.SB, o["twopass"], split_k=SPLIT, mode=gf.GF_SPLITK_TWOPASS,
                                 workspace=self.ws[k])
        gf.gemm_f16_nt_splitk_f16(self.SA, self.SB, o["f16"], split_k=SPLIT, workspace=self.ws[k])
        gf.gemv_f16(self.W, self.x, o["y"])
        gf.gemm_f16_nt_skinny(self.KA, self.KB, o["ks"], cfg=SPLIT_CFG)
        gf.gemm_f16_nt_skinny(self.RA, self.RB, o["kr"], cfg=RAGGED_CFG)
        gf.sp24_compress_f16(self.PA, o["asp"], o["meta"])
        gf.gemm_sp_f16_nt(o["asp"], o["meta"], self.PB, o["sp"])


def _bits(t):
    return t.detach().cpu().contiguous().numpy().view(np.uint8)


def test_graph_capture_and_replay():
    b = Buffers()
    b.fill(seed=100)
    side = torch.cuda.Stream()                # default priority
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):             # warm-up outside capture (per-kernel set-up)
        b.run(0)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    _say("graph: capturing")
    with torch.cuda.graph(g):
        b.run(0)
    torch.cuda.synchronize()
    for rep in range(3):
        host = b.fill(seed=200 + rep)
        for t in b.out[0].values():           # stale outputs must not survive a replay
            t.fill_(7)
        torch.cuda.synchronize()
        _say("graph: replay %d" % rep)
        g.replay()
        torch.cuda.synchronize()
        b.run(1)                              # eager, between replays
        torch.cuda.synchronize()
        for name in b.out[0]:
            assert np.array_equal(_bits(b.out[0][name]), _bits(b.out[1][name])), \
                "replay %d: %s differs from the eager call" % (rep, name)
        # and the replay computed the new inputs' product, not a stale one
        assert np.array_equal(host_u16(b.out[0]["nt"]), oracle.gemm_nt_f16(host["A"], host["B"]))
        assert np.array_equal(host_u16(b.out[0]["y"]), oracle.gemv_f16(host["W"], host["x"]))
        assert np.array_equal(host_u16(b.out[0]["ks"]), oracle.gemm_nt_f16(host["KA"], host["KB"]))
        assert np.array_equal(host_u16(b.out[0]["kr"]), oracle.gemm_nt_f16(host["RA"], host["RB"]))


def test_concurrent_streams():
    """Calls on two streams at once write their own outputs correctly."""
    b = Buffers()
    host = b.fill(seed=300)
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    torch.cuda.synchronize()
    o = b.out[0]
    _say("two streams")
    for _ in range(3):
        with torch.cuda.stream(s1):
            gf.gemm_f16_nt(b.A, b.B, o["nt"])
            gf.gemm_f16_nt_splitk_f16(b.SA, b.SB, o["f16"], split_k=SPLIT, workspace=b.ws[0])
        with torch.cuda.stream(s2):
            gf.gemv_f16(b.W, b.x, o["y"])
            gf.sp24_compress_f16(b.PA, o["asp"], o["meta"])
            gf.gemm_sp_f16_nt(o["asp"], o["meta"], b.PB, o["sp"])
    torch.cuda.synchronize()
    assert np.array_equal(host_u16(o["nt"]), oracle.gemm_nt_f16(host["A"], host["B"]))
    assert np.array_equal(host_u16(o["f16"]), oracle.gemm_nt_f16(host["SA"], host["SB"]))
    assert np.array_equal(host_u16(o["y"]), oracle.gemv_f16(host["W"], host["x"]))
    rAsp, rE = oracle.sp24_compress(host["PA"])
    assert np.array_equal(host_u16(o["sp"]), oracle.gemm_sp_nt_f16(rAsp, rE, host["PB"]))


def test_binding_allocations_on_explicit_stream():
    """Outputs and two-pass workspaces that the binding allocates for a call
    on an explicit, non-current stream belong to that stream: while the
    side stream is still busy with the call, the current stream reallocates
    and overwrites freed memory, and the results must stay intact."""
    side = torch.cuda.Stream()
    A = inputs.integer_f16((SM, SK), 400, 0)
    B = inputs.integer_f16((SN, SK), 400, 1)
    dA, dB = dev(A), dev(B)
    torch.cuda.synchronize()
    outs = []
    _say("binding allocations on a side stream")
    for _ in range(4):
        # no workspace and no output passed: the binding allocates both
        outs.append(gf.gemm_f16_nt_splitk_ex(dA, dB, split_k=SPLIT, mode=gf.GF_SPLITK_TWOPASS,
                                             stream=side))
        outs.append(gf.gemm_f16_nt_splitk_f16(dA, dB, split_k=SPLIT, stream=side))
        # the current stream grabs and scribbles over whatever is free now
        junk = [torch.full((SPLIT * SM * SN,), 3.0, dtype=torch.float32, device="cuda") for _ in range(2)]
        del junk
    torch.cuda.synchronize()
    ref32 = oracle.gemm_nt_f32(A, B)
    ref16 = oracle.gemm_nt_f16(A, B)
    for i, o in enumerate(outs):
        if i % 2 == 0:
            assert np.array_equal(o.cpu().numpy(), ref32)
        else:
            assert np.array_equal(host_u16(o), ref16)

"""Launch one operation a fixed number of times, for an external profiler.

    rocprofv3 --kernel-trace --stats -- python3 -m gemv_fp16_amd.profile_run gemm
    rocprofv3 --pmc FETCH_SIZE -- python3 -m gemv_fp16_amd.profile_run gemv

Ops (inputs are the seeded uniform[-1,1] fp16 workloads):
  gemm    C = A . B^T at M = N = K = 8192 (default tile config); --layout nn / tn
          stores B as K x N (and A as K x M) and runs gemm_f16 on them
  gemv    y = W . x at N = K = 8192, rotating 5 W copies (640 MiB)
  splitk  M = N = 1024, K = 16384, split --split (default 8): fp32 atomic, fp32 two-pass, fp16
          two-pass, operands rotated over 4 copies (256 MiB)
  skinny  C = A . B^T with M = 4 and M = 16 rows of A against an 8192 x 8192 B (5 B copies
          rotated, 640 MiB); the library's default form for each M
  sparse  2:4 sparse C = decompress(A_sparse, E) . B^T at M = N = K = 8192 (A compressed
          once on the GPU from a dense uniform A; default tile config)
  compress  2:4 compression of an 8192 x 8192 A, rotating 3 copies (384 MiB)
  copy    torch copy of a 512 MiB buffer: a plain copy kernel of known size,
          the calibration for the HBM byte counters
"""
from __future__ import annotations

import argparse
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def main(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("op", choices=["gemm", "gemv", "splitk", "skinny", "sparse", "compress", "copy"])
    ap.add_argument("--iters", type=int, default=10)
    ap.add_argument("--m", type=int, default=8192)
    ap.add_argument("--n", type=int, default=8192)
    ap.add_argument("--k", type=int, default=8192)
    ap.add_argument("--layout", choices=["nt", "nn", "tn"], default="nt")
    ap.add_argument("--split", type=int, default=8, help="split-K slices (op splitk)")
    ap.add_argument("--cfg", default="",
                    help="gemm tile config block_m,block_n,block_k,stages,threads,raster[,schedule] "
                         "(default: the library's choice)")
    a = ap.parse_args(argv)

    import torch
    import gemv_fp16_amd as gf
    import inputs

    torch.cuda.set_device(0)
    if a.op == "gemm":
        A = torch.from_numpy(inputs.uniform_f16((a.m, a.k), 0, 0)).cuda()
        B = torch.from_numpy(inputs.uniform_f16((a.n, a.k), 0, 1)).cuda()
        C = torch.empty((a.m, a.n), dtype=torch.float16, device="cuda")
        cfg = None
        if a.cfg:
            v = [int(t) for t in a.cfg.split(",")]
            cfg = dict(zip(("block_m", "block_n", "block_k", "stages", "threads", "raster",
                            "schedule"), v + [0] * (7 - len(v))))
        if a.layout == "nt":
            call = gf.prepare_gemm_f16_nt(A, B, C, cfg=cfg)
        else:
            a_km = a.layout == "tn"
            As = A.t().contiguous() if a_km else A
            Bs = B.t().contiguous()
            del A, B
            def call():
                gf.gemm_f16(As, Bs, C, a_km, True, cfg=cfg)
        for _ in range(a.iters):
            call()
    elif a.op == "gemv":
        Ws = [torch.from_numpy(inputs.uniform_f16((a.n, a.k), i, 0)).cuda() for i in range(5)]
        x = torch.from_numpy(inputs.uniform_f16((a.k,), 0, 1)).cuda()
        y = torch.empty((a.n,), dtype=torch.float16, device="cuda")
        calls = [gf.prepare_gemv_f16(w, x, y) for w in Ws]
        for i in range(a.iters):
            calls[i % len(calls)]()
    elif a.op == "splitk":
        A = torch.from_numpy(inputs.uniform_f16((1024, 16384), 0, 0)).cuda()
        B = torch.from_numpy(inputs.uniform_f16((1024, 16384), 0, 1)).cuda()
        As, Bs = [A] + [A.clone() for _ in range(3)], [B] + [B.clone() for _ in range(3)]
        C = torch.empty((1024, 1024), dtype=torch.float32, device="cuda")
        C16 = torch.empty((1024, 1024), dtype=torch.float16, device="cuda")
        ws = torch.empty(a.split * 1024 * 1024, dtype=torch.float32, device="cuda")
        for i in range(a.iters):
            j = i % 4
            gf.gemm_f16_nt_splitk_ex(As[j], Bs[j], C, a.split, gf.GF_SPLITK_ATOMIC, ws)
            gf.gemm_f16_nt_splitk_ex(As[j], Bs[j], C, a.split, gf.GF_SPLITK_TWOPASS, ws)
            gf.gemm_f16_nt_splitk_f16(As[j], Bs[j], C16, a.split, ws)
    elif a.op == "skinny":
        Bs = [torch.from_numpy(inputs.uniform_f16((a.n, a.k), i, 1)).cuda() for i in range(5)]
        for m in (4, 16):
            A = torch.from_numpy(inputs.uniform_f16((m, a.k), 0, 0)).cuda()
            C = torch.empty((m, a.n), dtype=torch.float16, device="cuda")
            for i in range(a.iters):
                gf.gemm_f16_nt(A, Bs[i % len(Bs)], C)
    elif a.op == "sparse":
        A = torch.from_numpy(inputs.uniform_f16((a.m, a.k), 0, 0)).cuda()
        B = torch.from_numpy(inputs.uniform_f16((a.n, a.k), 0, 1)).cuda()
        Asp, E = gf.sp24_compress_f16(A)
        del A
        C = torch.empty((a.m, a.n), dtype=torch.float16, device="cuda")
        call = gf.prepare_gemm_sp_f16_nt(Asp, E, B, C)
        for _ in range(a.iters):
            call()
    elif a.op == "compress":
        As = [torch.from_numpy(inputs.uniform_f16((a.m, a.k), i, 0)).cuda() for i in range(3)]
        outs = [(torch.empty((a.m, a.k // 2), dtype=torch.float16, device="cuda"),
                 torch.empty((a.m, a.k // 16), dtype=torch.int16, device="cuda")) for _ in range(3)]
        for i in range(a.iters):
            gf.sp24_compress_f16(As[i % 3], *outs[i % 3])
    else:
        src = torch.ones(128 << 20, dtype=torch.float32, device="cuda")   # 512 MiB
        dst = torch.empty_like(src)
        for _ in range(a.iters):
            dst.copy_(src)
    torch.cuda.synchronize()
    print("profile_run %s: %d iterations done" % (a.op, a.iters), flush=True)


if __name__ == "__main__":
    main()

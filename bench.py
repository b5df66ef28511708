#!/usr/bin/env python3
"""Benchmark: fp16 GEMM-NT at M = N = K = 8192 on one MI355X, plus GEMV and
split-K on their workloads, with roofline fractions and the CPU oracle timed
on the host cores.

    python bench.py [--gpus 1] [--steps 20] [--warmup 5]

One step is one C = A . B^T call at 8192^3 (fp16 in, fp32 accumulate, fp16
out) on torch's current stream with A and B already resident in HBM.  The
headline value is whole-job TFLOP/s over the timed steps (wall clock,
bracketed by device synchronisation).  The GEMV (N = K = 8192 and 1024),
split-K (M = N = 1024, K = 16384) and 2:4 sparse GEMM (8192^3, plus the
compression of its A) figures are reported in "extra", each
timed with HIP events on the launching stream around batches of
back-to-back launches; GEMV rotates over enough W
copies (> 512 MiB) that every call streams W from HBM, not from the 256 MiB
MALL.  Prints exactly one JSON line on stdout; progress goes to stderr.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_F16_TFLOPS = 2500.0   # MI355X dense fp16 MFMA, published
PEAK_HBM_GBS = 8000.0      # MI355X HBM3E, published
PEAK_F16_SPARSE_TFLOPS = 5000.0   # MI355X fp16 MFMA with 2:4 structured sparsity, published


def log(msg):
    print("[bench] " + msg, file=sys.stderr, flush=True)


# The sources each timed kernel is built from: a traffic record taken on
# other sources is stale.
KERNEL_SOURCES = {
    "gemm_nt_kernel": ("common.hpp", "gemm_kernel.hpp", "gemm_configs.def", "configs.hpp",
                       "gemm_shard.hip", "api.hip"),
    "gemv_kernel": ("common.hpp", "gemv_kernel.hpp", "gemv_configs.def", "gemv.hip", "api.hip"),
    "sp_gemm_kernel": ("common.hpp", "sparse_kernel.hpp", "sparse.hip"),
    "sp24_compress_kernel": ("common.hpp", "sparse_kernel.hpp", "sparse.hip"),
}


def kernel_source_hash(kernel: str) -> str:
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "gemv_fp16_amd", "csrc")
    for name in sorted(KERNEL_SOURCES[kernel]):
        h.update(name.encode())
        h.update(open(os.path.join(csrc, name), "rb").read())
    return h.hexdigest()[:16]


def measured_traffic(kernel: str, workload: str):
    """HBM bytes per launch from the committed rocprofv3 --pmc summary, if it
    was taken on the current kernel sources; else None."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    try:
        rec = json.load(open(path)).get(kernel + "|" + workload)
    except (ValueError, OSError):
        return None
    if not rec or rec.get("source_hash") != kernel_source_hash(kernel):
        return None
    return rec.get("bytes_per_launch")


def time_batch(torch, fn, reps, warmup, trials=3):
    """Seconds per call: HIP events on the current stream around `reps`
    back-to-back calls (median of `trials` batches), after `warmup` calls."""
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    res = []
    for _ in range(trials):
        s = torch.cuda.Event(enable_timing=True)
        e = torch.cuda.Event(enable_timing=True)
        s.record(stream)
        for _ in range(reps):
            fn()
        e.record(stream)
        torch.cuda.synchronize()
        res.append(s.elapsed_time(e) * 1e-3 / reps)
    return float(np.median(res))


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--cpu-rows", type=int, default=6144,
                    help="rows of the 8192^3 product the CPU oracle computes")
    ap.add_argument("--no-extra", action="store_true", help="headline GEMM only")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    args = ap.parse_args()

    if args.gpus != 1:
        print("bench.py runs on one GPU only: this build has no multi-GPU path "
              "(--gpus %d requested)" % args.gpus, file=sys.stderr)
        sys.exit(2)

    import torch
    import gemv_fp16_amd as gf
    import inputs

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    gf.lib()
    torch.cuda.set_device(0)

    M = N = K = 8192
    log("generating A, B %dx%d fp16 uniform[-1,1] seed 0" % (M, K))
    A_np = inputs.uniform_f16((M, K), 0, inputs.STREAM_A)
    B_np = inputs.uniform_f16((N, K), 0, inputs.STREAM_B)
    A = torch.from_numpy(A_np).cuda()
    B = torch.from_numpy(B_np).cuda()
    C = torch.empty((M, N), dtype=torch.float16, device="cuda")
    cfg = gf.gemm_default_config(M, N, K)
    flops = 2.0 * M * N * K

    step = gf.prepare_gemm_f16_nt(A, B, C)

    log("warmup %d" % args.warmup)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    evs = []
    log("timing %d steps" % args.steps)
    t0 = time.perf_counter()
    for _ in range(args.steps):
        s = torch.cuda.Event(enable_timing=True)
        e = torch.cuda.Event(enable_timing=True)
        s.record(stream)
        step()
        e.record(stream)
        evs.append((s, e))
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    kern_s = float(np.mean([s.elapsed_time(e) for s, e in evs])) * 1e-3
    value = flops * args.steps / elapsed / 1e12
    achieved = flops / kern_s / 1e12
    log("gemm 8192^3: %.1f TFLOP/s wall, %.1f TFLOP/s per launch (%.3f ms)" %
        (value, achieved, kern_s * 1e3))

    out = {
        "metric": "fp16 GEMM TFLOP/s at M=N=K=8192 (% MFMA peak); GEMV GB/s (% HBM peak)",
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(elapsed / args.steps * 1e3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16",
        "data": "synthetic",
        "config": {"workload": "gemm_f16_nt C=A.B^T M=N=K=8192, A,B fp16 uniform[-1,1] seed 0",
                   "M": M, "N": N, "K": K, "tile": cfg},
        "roofline": {"bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_F16_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(achieved / PEAK_F16_TFLOPS, 4),
                     "traffic": measured_traffic("gemm_nt_kernel", "8192^3")},
    }

    extra = {}
    if not args.no_extra:
        # ---- GEMM, K swept ----
        sweep = {}
        for k2 in (256, 512, 1024, 4096, 16384):
            a2 = torch.from_numpy(inputs.uniform_f16((M, k2), 0, 0)).cuda()
            b2 = torch.from_numpy(inputs.uniform_f16((N, k2), 0, 1)).cuda()
            t2 = time_batch(torch, gf.prepare_gemm_f16_nt(a2, b2, C), 10, 3)
            sweep[str(k2)] = round(2.0 * M * N * k2 / t2 / 1e12, 1)
            log("gemm 8192x8192x%d: %.1f TFLOP/s" % (k2, sweep[str(k2)]))
            del a2, b2
        sweep[str(K)] = round(achieved, 1)
        extra["gemm_k_sweep_tflops"] = sweep

        # ---- GEMM at cube sizes whose 256 x 256 tiles leave the last round
        # of workgroups mostly empty: the default call (leading rows in whole
        # rounds, the rest with a smaller tile) vs one launch of the big tile
        quant = {}
        for n3 in (7168, 6144):
            a3 = torch.from_numpy(inputs.uniform_f16((n3, n3), 0, 0)).cuda()
            b3 = torch.from_numpy(inputs.uniform_f16((n3, n3), 0, 1)).cuda()
            c3 = torch.empty((n3, n3), dtype=torch.float16, device="cuda")
            f3 = 2.0 * n3 ** 3
            # the two launch plans alternate batch by batch, so that both see
            # the same clock and power state
            plans = (gf.prepare_gemm_f16_nt(a3, b3, c3),
                     gf.prepare_gemm_f16_nt(a3, b3, c3, cfg=gf.gemm_default_config(n3, n3, n3)))
            times = ([], [])
            for p in plans:
                time_batch(torch, p, 1, 5, trials=1)
            for _ in range(5):
                for i, p in enumerate(plans):
                    times[i].append(time_batch(torch, p, 10, 0, trials=1))
            t_def, t_one = float(np.median(times[0])), float(np.median(times[1]))
            quant["%d^3" % n3] = {"default_tflops": round(f3 / t_def / 1e12, 1),
                                  "one_launch_tflops": round(f3 / t_one / 1e12, 1)}
            del a3, b3, c3
        log("gemm wave-quantised cubes: %s" % quant)
        extra["gemm_row_split"] = quant

        # ---- GEMM at mid-size shapes (fewer than 256 tiles of 256 x 256)
        mid = {}
        for (m4, n4, k4) in ((2048, 4096, 8192), (2048, 2048, 8192), (1024, 4096, 8192)):
            a4 = torch.from_numpy(inputs.uniform_f16((m4, k4), 0, 0)).cuda()
            b4 = torch.from_numpy(inputs.uniform_f16((n4, k4), 0, 1)).cuda()
            c4 = torch.empty((m4, n4), dtype=torch.float16, device="cuda")
            t4 = time_batch(torch, gf.prepare_gemm_f16_nt(a4, b4, c4), 20, 5)
            d4 = gf.gemm_default_config(m4, n4, k4)
            mid["%dx%dx%d" % (m4, n4, k4)] = {"tflops": round(2.0 * m4 * n4 * k4 / t4 / 1e12, 1),
                                              "tile": "%dx%d/%d stages/schedule %d" % (
                                                  d4["block_m"], d4["block_n"], d4["stages"], d4["schedule"])}
            del a4, b4, c4
        log("gemm mid-size shapes: %s" % mid)
        extra["gemm_mid_shapes"] = mid

        # other operand layouts at 8192^3: B stored K x N (and A K x M)
        lay = {}
        Bt = B.t().contiguous()
        lay["nn"] = round(flops / time_batch(torch, lambda: gf.gemm_f16(A, Bt, C, False, True), 10, 3) / 1e12, 1)
        At = A.t().contiguous()
        lay["tn"] = round(flops / time_batch(torch, lambda: gf.gemm_f16(At, Bt, C, True, True), 10, 3) / 1e12, 1)
        del At, Bt
        log("gemm 8192^3 other layouts TFLOP/s: %s" % lay)
        extra["gemm_layouts_8192_tflops"] = lay

        # ---- GEMV ----
        gemv = {}
        for nk in (8192, 1024):
            wbytes = nk * nk * 2
            copies = max(1, -(-(640 << 20) // wbytes))
            copies = min(copies, 64)
            Ws = [torch.from_numpy(inputs.uniform_f16((nk, nk), i, 0)).cuda() for i in range(copies)]
            x = torch.from_numpy(inputs.uniform_f16((nk,), 0, 1)).cuda()
            y = torch.empty((nk,), dtype=torch.float16, device="cuda")
            calls = [gf.prepare_gemv_f16(w, x, y) for w in Ws]
            state = [0]

            def cold(calls=calls, state=state):
                calls[state[0] % len(calls)]()
                state[0] += 1

            t_cold = time_batch(torch, cold, 200, 20)
            t_warm = time_batch(torch, calls[0], 200, 20)
            bytes_ = 2.0 * nk * nk + 2.0 * nk + 2.0 * nk
            gbs = bytes_ / t_cold / 1e9
            gemv[str(nk)] = {
                "us": round(t_cold * 1e6, 3), "GB/s": round(gbs, 1),
                "frac_hbm_peak": round(gbs / PEAK_HBM_GBS, 4),
                "w_copies_rotated": copies,
                "cache_warm_GB/s_not_hbm": round(bytes_ / t_warm / 1e9, 1),
                "launch": gf.gemv_default_config(nk, nk),
            }
            log("gemv %d: %.2f us, %.1f GB/s (warm %.1f)" %
                (nk, t_cold * 1e6, gbs, gemv[str(nk)]["cache_warm_GB/s_not_hbm"]))
            del Ws
        g8 = gemv["8192"]
        gemv["roofline"] = {"bound": "hbm", "achieved": g8["GB/s"], "peak": PEAK_HBM_GBS,
                            "unit": "GB/s", "frac": g8["frac_hbm_peak"],
                            "traffic": measured_traffic("gemv_kernel", "8192^2")}
        extra["gemv"] = gemv

        # ---- skinny GEMM: M = 2..64 rows against an 8192 x 8192 B (decode batches;
        # gemm_f16_nt takes the skinny kernel for all of them) ----
        Bsk = [torch.from_numpy(inputs.uniform_f16((8192, 8192), i, 1)).cuda() for i in range(5)]
        sk_res = {}
        for mm in (2, 4, 8, 16, 32, 64):
            Ask = torch.from_numpy(inputs.uniform_f16((mm, 8192), 0, 0)).cuda()
            Csk = torch.empty((mm, 8192), dtype=torch.float16, device="cuda")
            state = [0]

            def skinny(Ask=Ask, Csk=Csk, state=state):
                gf.gemm_f16_nt(Ask, Bsk[state[0] % len(Bsk)], Csk)
                state[0] += 1

            t = time_batch(torch, skinny, 100, 10)
            byt = 2.0 * 8192 * 8192 + 2.0 * mm * 8192 * 2
            sk_res["M%d" % mm] = {"us": round(t * 1e6, 2), "GB/s": round(byt / t / 1e9, 1)}
        del Bsk
        log("skinny M x 8192 x 8192 (B from HBM): %s" % sk_res)
        extra["skinny_8192"] = sk_res

        # ---- split-K ----
        sm, sk_k = 1024, 16384
        a3 = torch.from_numpy(inputs.uniform_f16((sm, sk_k), 0, 0)).cuda()
        b3 = torch.from_numpy(inputs.uniform_f16((sm, sk_k), 0, 1)).cuda()
        c3 = torch.empty((sm, sm), dtype=torch.float32, device="cuda")
        ws = torch.empty(16 * sm * sm, dtype=torch.float32, device="cuda")
        sk = {}
        f3 = 2.0 * sm * sm * sk_k
        for split in (4, 8, 16):
            for mode, name in ((gf.GF_SPLITK_ATOMIC, "atomic"), (gf.GF_SPLITK_TWOPASS, "twopass")):
                t3 = time_batch(torch, lambda: gf.gemm_f16_nt_splitk_ex(
                    a3, b3, c3, split, mode, ws), 50, 5)
                sk["%s_s%d" % (name, split)] = round(f3 / t3 / 1e12, 1)
        c16 = torch.empty((sm, sm), dtype=torch.float16, device="cuda")
        for split in (4, 8, 16):
            t3 = time_batch(torch, lambda: gf.gemm_f16_nt_splitk_f16(a3, b3, c16, split, ws), 50, 5)
            sk["twopass_f16out_s%d" % split] = round(f3 / t3 / 1e12, 1)
        t3 = time_batch(torch, lambda: gf.gemm_f16_nt(a3, b3, c16), 50, 5)
        sk["no_split_fp16"] = round(f3 / t3 / 1e12, 1)
        log("splitk 1024x1024x16384 TFLOP/s: %s" % sk)
        extra["splitk_1024x1024x16384_tflops"] = sk
        del a3, b3, c3, ws

        # ---- 2:4 structured-sparse GEMM at 8192^3: the headline A compressed
        # (pruned to 2 of every 4 along K) on the GPU, then C = A_sparse . B^T ----
        Asp, E = gf.sp24_compress_f16(A)
        t_sp = time_batch(torch, gf.prepare_gemm_sp_f16_nt(Asp, E, B, C), 20, 5)
        sp_eff = flops / t_sp / 1e12
        # compression, rotating 3 inputs (384 MiB > the 256 MiB MALL)
        Acs = [A] + [torch.from_numpy(inputs.uniform_f16((M, K), i, 0)).cuda() for i in (1, 2)]
        outs = [(torch.empty_like(Asp), torch.empty_like(E)) for _ in range(3)]
        state = [0]

        def comp(state=state):
            j = state[0] % 3
            gf.sp24_compress_f16(Acs[j], *outs[j])
            state[0] += 1

        t_c = time_batch(torch, comp, 60, 6)
        c_bytes = 2.0 * M * K + 2.0 * M * K / 2 + 2.0 * M * K / 16
        extra["sparse24_8192"] = {
            "gemm_ms": round(t_sp * 1e3, 4),
            "gemm_tflops_effective": round(sp_eff, 1),
            "tile": gf.sp_default_config(M, N, K),
            "roofline": {"bound": "mfma", "achieved": round(sp_eff, 2), "peak": PEAK_F16_SPARSE_TFLOPS,
                         "unit": "TFLOP/s", "frac": round(sp_eff / PEAK_F16_SPARSE_TFLOPS, 4),
                         "traffic": measured_traffic("sp_gemm_kernel", "8192^3")},
            "compress_us": round(t_c * 1e6, 2),
            "compress_GB/s": round(c_bytes / t_c / 1e9, 1),
            "compress_frac_hbm_peak": round(c_bytes / t_c / 1e9 / PEAK_HBM_GBS, 4),
        }
        log("sparse 2:4 8192^3: %.1f effective TFLOP/s (%.3f ms); compress %.1f us, %.1f GB/s" %
            (sp_eff, t_sp * 1e3, t_c * 1e6, c_bytes / t_c / 1e9))
        del Asp, E, Acs, outs

    if not args.no_cpu:
        import oracle
        rows = max(1, min(args.cpu_rows, M))
        log("cpu oracle: %d rows of the 8192^3 product" % rows)
        t = time.perf_counter()
        oracle.gemm_nt_f16(A_np, B_np, rows=(0, rows))
        dt = time.perf_counter() - t
        out["cpu_baseline"] = {
            "value": round(2.0 * rows * N * K / dt / 1e12, 6), "unit": "TFLOP/s",
            "cores": oracle.threads(), "kind": "oracle",
            "sample": "rows 0..%d of C = A.B^T at M=N=K=8192 (%d x 8192 outputs, double "
                      "accumulation), %.1f s wall" % (rows - 1, rows, dt),
        }
        log("cpu oracle: %.3g TFLOP/s on %d threads (%.1f s)" %
            (out["cpu_baseline"]["value"], oracle.threads(), dt))

    if extra:
        out["extra"] = extra
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()

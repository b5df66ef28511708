"""Per-workgroup timeline of the split-K GEMM pass or of an fp16 GEMM
(diagnostic build).

    python -m gemv_fp16_amd.build --variant timeline     # once, on any machine
    python -m gemv_fp16_amd.timeline [--split 8 --cfg 256,128,64,3,256,2]
    python -m gemv_fp16_amd.timeline --gemm 8192,8192,8192 [--cfg ...,raster] [--per-xcd]

Loads gemv_fp16_amd/variants/timeline/libgemvfp16.so, in which every
workgroup of a two-pass split-K launch stamps the shader's 100 MHz real-time
counter at four points and writes the stamps over the first words of its own
partial tile (so that build's results are wrong by design; it is never the
library).  The split-K run is M = N = 1024, K = 16384 on the seeded
uniform[-1,1] operands, rotated over 4 copies (256 MiB, past the 256 MiB MALL
together with the workspace), 12 launches; the stamps of the last launch are
read back.  With --gemm the same stamps come from the first words of each
workgroup's fp16 output tile of a plain C = A . B^T (operands rotated over 3
copies, 12 launches; the library's default tile unless --cfg names one).

Per launch it prints, over the workgroups: the span from the first entry to
the last partial store, the skew of the entries (a second wave of workgroups
starts when the first one leaves), the prologue (entry until the first K tile
has landed: only the schedule-2 pipeline notes that point), the main loop,
the epilogue (partial stores until they have left the CU), the shader clock
over the main loop (shader-cycle counter over real time), the loop's shader
cycles per K tile, and its matrix-core share: its MFMA cycles (32 per
32 x 32 MFMA, per SIMD) over those cycles.
"""
from __future__ import annotations

import argparse
import os
import sys

_HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(_HERE)
VARIANT = os.path.join(_HERE, "variants", "timeline", "libgemvfp16.so")

CONFIGS = ((8, (256, 128, 64, 3, 256, 2)), (4, (256, 128, 64, 3, 256, 2)), (16, (256, 128, 64, 3, 256, 2)),
           (4, (128, 128, 64, 4, 256, 2)), (8, (128, 128, 64, 4, 256, 2)))


KEYS = ("block_m", "block_n", "block_k", "stages", "threads", "schedule")


def run(split, cfg, As, Bs, C32):
    import numpy as np
    import torch
    import gemv_fp16_amd as gf
    M, N, K = 1024, 1024, 16384
    c = dict(zip(KEYS, cfg), raster=1)
    ws = torch.zeros(split * M * N, dtype=torch.float32, device="cuda")
    for i in range(12):
        gf.gemm_f16_nt_splitk_cfg(As[i % 4], Bs[i % 4], C32, split, gf.GF_SPLITK_TWOPASS, c, ws)
    torch.cuda.synchronize()
    w = ws.view(split, M, N).cpu().numpy()
    bm, bn = cfg[0], cfg[1]
    rec = np.array([w[s, tm * bm, tn * bn:tn * bn + 16].view(np.uint64).astype(np.int64)
                    for s in range(split) for tm in range(M // bm) for tn in range(N // bn)])
    return row(str(split), cfg, rec, K // split)


def run_gemm(shape, cfg):
    """Stamps of a plain fp16 GEMM, read from each output tile's first 32 values."""
    import numpy as np
    import torch
    import gemv_fp16_amd as gf
    import inputs
    M, N, K = shape
    if cfg is None:
        d = gf.gemm_default_config(M, N, K)
        cfg = tuple(d[k] for k in KEYS) + (d["raster"],)
    c = dict(zip(KEYS + ("raster",), cfg))
    A0 = torch.from_numpy(inputs.uniform_f16((M, K), 0, inputs.STREAM_A)).cuda()
    B0 = torch.from_numpy(inputs.uniform_f16((N, K), 0, inputs.STREAM_B)).cuda()
    As, Bs = [A0] + [A0.clone() for _ in range(2)], [B0] + [B0.clone() for _ in range(2)]
    C = torch.empty((M, N), dtype=torch.float16, device="cuda")
    for i in range(12):
        gf.gemm_f16_nt(As[i % 3], Bs[i % 3], C, cfg=c)
    torch.cuda.synchronize()
    w = C.cpu().numpy().view(np.uint16)
    bm, bn = cfg[0], cfg[1]
    rec = np.array([w[tm * bm, tn * bn:tn * bn + 32].view(np.uint64).astype(np.int64)
                    for tm in range(M // bm) for tn in range(N // bn)])
    return row("-", cfg, rec, K), per_xcd(rec, K, cfg[2])


def per_xcd(rec, kext, bk):
    """Per-XCC lines from the same stamps: workgroups, last store, median main loop, median loop
    clock and median loop cycles per K tile."""
    import numpy as np
    t0 = rec[:, 0].min()
    start, first, mend, end = ((rec[:, j] - t0) / 100.0 for j in range(4))
    staged = rec[:, 1].min() > 0
    loop = mend - first if staged else mend - start
    cyc = (rec[:, 7] - rec[:, 6]) if staged else (rec[:, 7] - rec[:, 5])
    out = ["| XCC | WGs | last store us | main loop us (median) | loop clock GHz (median) | loop cycles per K tile (median) |",
           "|---|---|---|---|---|---|"]
    for x in range(8):
        m = rec[:, 4] == x
        if m.any():
            out.append("| %d | %d | %.1f | %.1f | %.3f | %.0f |" % (
                x, m.sum(), end[m].max(), np.median(loop[m]), np.median(cyc[m] / (loop[m] * 1e3)),
                np.median(cyc[m]) / (kext // bk)))
    return "\n".join(out)


def row(split, cfg, rec, kext):
    """One table row from the stamps rec[workgroup] = (entry, first tile landed, loop end, stores
    done, XCC id, cycles at entry, cycles at first tile, cycles at loop end)."""
    import numpy as np
    bm, bn, bk = cfg[0], cfg[1], cfg[2]
    t0 = rec[:, 0].min()
    start, first, mend, end = ((rec[:, j] - t0) / 100.0 for j in range(4))   # microseconds
    xcc = rec[:, 4]
    staged = rec[:, 1].min() > 0
    loop = mend - first if staged else mend - start
    loop_cycles = (rec[:, 7] - rec[:, 6]) if staged else (rec[:, 7] - rec[:, 5])
    clock = loop_cycles / (loop * 1e3)                                       # GHz
    ksteps = kext // bk
    # matrix-core cycles per SIMD and K tile: 2 bm bn bk flops at 1024 per cycle and SIMD, 4 SIMDs
    mfma_cycles = 2 * bm * bn * bk / 1024 / 4
    per_tile = np.median(loop_cycles) / ksteps
    return "| %s | %s | %d | %.1f | %.1f | %s | %.1f (%.1f-%.1f) | %.2f | %.2f (%.2f-%.2f) | %.0f | %.0f %% | %s |" % (
        split, "x".join(map(str, cfg[:3])) + " S%d sched %d" % (cfg[3], cfg[5]), len(rec), end.max(), start.max(),
        "%.2f" % np.median(first - start) if staged else "-", np.median(loop), loop.min(), loop.max(),
        np.median(end - mend), np.median(clock), clock.min(), clock.max(), per_tile, 100 * mfma_cycles / per_tile,
        " ".join("%d:%.1f" % (x, end[xcc == x].max()) for x in range(8) if (xcc == x).any()))


def main(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("--split", type=int, default=0, help="one run at this split (with --cfg)")
    ap.add_argument("--cfg", default="", help="block_m,block_n,block_k,stages,threads,schedule[,raster]")
    ap.add_argument("--gemm", default="", help="M,N,K: time a plain fp16 GEMM instead of the split-K pass")
    ap.add_argument("--per-xcd", action="store_true", help="with --gemm: also one line per XCC")
    a = ap.parse_args(argv)
    if not os.path.exists(VARIANT):
        raise SystemExit("build the diagnostic library first: python -m gemv_fp16_amd.build --variant timeline")
    sys.path.insert(0, ROOT)
    import torch
    import gemv_fp16_amd as gf
    import inputs
    # run as "python -m gemv_fp16_amd.timeline" the package is imported
    # already; the library itself loads on first use
    assert gf._lib is None
    gf.LIB_PATH = VARIANT
    print("| split | tile | WGs | span us | entry skew us | prologue us | main loop us median (min-max) "
          "| epilogue us | loop clock GHz median (min-max) | loop cycles per K tile | MFMA share of those cycles "
          "| last store per XCC, us |")
    print("|---|---|---|---|---|---|---|---|---|---|---|---|")
    if a.gemm:
        shape = tuple(int(t) for t in a.gemm.split(","))
        cfg = tuple(int(t) for t in a.cfg.split(",")) if a.cfg else None
        if cfg is not None and len(cfg) == 6:
            cfg = cfg + (0,)
        line, xcd = run_gemm(shape, cfg)
        print(line, flush=True)
        if a.per_xcd:
            print("\n" + xcd, flush=True)
        return
    A0 = torch.from_numpy(inputs.uniform_f16((1024, 16384), 0, inputs.STREAM_A)).cuda()
    B0 = torch.from_numpy(inputs.uniform_f16((1024, 16384), 0, inputs.STREAM_B)).cuda()
    As = [A0] + [A0.clone() for _ in range(3)]
    Bs = [B0] + [B0.clone() for _ in range(3)]
    C32 = torch.empty((1024, 1024), dtype=torch.float32, device="cuda")
    runs = ((a.split, tuple(int(t) for t in a.cfg.split(","))[:6]),) if a.split else CONFIGS
    for split, cfg in runs:
        print(run(split, cfg, As, Bs, C32), flush=True)


if __name__ == "__main__":
    main()

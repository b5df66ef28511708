"""Offline tile-config sweep for gemm_f16_nt and gemv_f16 (one GPU).

    python -m gemv_fp16_amd.sweep gemm --m 8192 --n 8192 --k 8192 --out sweep.json
    python -m gemv_fp16_amd.sweep gemv --n 8192 --k 8192 --out sweep_gemv.json
    python -m gemv_fp16_amd.sweep sparse --m 8192 --n 8192 --k 8192 --out sweep_sparse.json
    python -m gemv_fp16_amd.sweep gemv --n 8192 --k 8192 --out sweep_gemv.json --table 25
        (no GPU: a markdown table of the best 25 records of that shape in the file)
    python -m gemv_fp16_amd.sweep sparse --m 2048 --n 4096 --k 8192 --compare "default;128,256,3,1;256,128,0,1"
        (side by side: the listed configs timed in alternating rounds, operands
        rotated over copies that exceed the MALL; see compare())

A plain host loop in the spirit of the autotune grid on the TileLang FP16
matmul benchmark page (section 2.1: block_M, block_N, block_K, pipeline
stages, threads per block, rasterisation on/off; every candidate is built,
warmed up and timed, the lowest latency wins).  Here the candidates are the
tile configs compiled into the library (the grid minus the ones whose LDS or
wave layout does not fit a CU, reported as "unsupported").

Gate: before timing, each candidate is checked against the CPU oracle's
expected values for the same seeded inputs, read from a file that a
committed script writes with the oracle alone (tests/golden/
make_sweep_expected.py; the default path is that folder's file for the
shape): sampled entries of C for the GEMMs, every output for the GEMV.
Integer inputs in {-2..2} must match bit for bit, uniform inputs within
1 fp16 ulp + 1e-3.  Without an expected file for the shape the sweep refuses
to run.  Legality: like the grid filter of the autotune tutorial page,
configs that do not fit (LDS, wave layout) are "unsupported", and configs
whose compiled kernel spills registers to scratch memory (the build's
resource report, gemv_fp16_amd/resources.py) are marked "spills" and not
timed.  Timing: HIP events around `--reps` back-to-back launches after
`--warmup` launches; the median of `--trials` such batches is recorded.
Results are appended as JSON lines to `--out` as they are measured; a rerun
skips (shape, config) records already present, so an interrupted sweep
resumes.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np


ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
GOLDEN = os.path.join(ROOT, "tests", "golden")


def _u16(t):
    import torch
    return t.cpu().contiguous().view(torch.int16).numpy().view(np.uint16)


def expected_path(op, shape):
    return os.path.join(GOLDEN, "sweep_expected_%s_%s.txt" % (op, "x".join(str(v) for v in shape)))


def load_expected(path, shape):
    """(index columns, uniform fp16 bits, integer fp16 bits) from an expected
    file written by tests/golden/make_sweep_expected.py for `shape`."""
    if not path or not os.path.exists(path):
        raise SystemExit("no oracle expected values for shape %s (%s); write them with "
                         "tests/golden/make_sweep_expected.py" % (shape, path))
    want = "shape " + " ".join(str(v) for v in shape)
    head = [ln[1:].strip() for ln in open(path) if ln.startswith("#")]
    if want not in head:
        raise SystemExit("%s is not for shape %s" % (path, shape))
    a = np.loadtxt(path, comments="#", dtype=np.int64, ndmin=2)
    return a[:, :-2], a[:, -2].astype(np.uint16), a[:, -1].astype(np.uint16)


def _ulp(bits):
    v = np.abs(bits.view(np.float16).astype(np.float64))
    e = np.floor(np.log2(np.where(v > 0, v, 1.0)))
    return np.where(v > 0, 2.0 ** (np.maximum(e, -14) - 10), 2.0 ** -24)


def _close(got, ref):
    g = got.view(np.float16).astype(np.float64)
    r = ref.view(np.float16).astype(np.float64)
    return bool(np.all(np.abs(g - r) <= _ulp(ref) + 1e-3))


def _time_batch(torch, fn, reps, warmup, trials):
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
    return float(np.median(res)), float(np.min(res))


def _done(path):
    seen = set()
    if path and os.path.exists(path):
        for line in open(path):
            try:
                r = json.loads(line)
                seen.add(json.dumps([r["op"], r["shape"], r["config"]], sort_keys=True))
            except (ValueError, KeyError):
                pass
    return seen


def _emit(path, rec):
    line = json.dumps(rec, sort_keys=True)
    print(line, flush=True)
    if path:
        sep = ""
        if os.path.exists(path) and os.path.getsize(path) > 0:
            with open(path, "rb") as f:
                f.seek(-1, os.SEEK_END)
                if f.read(1) != b"\n":
                    sep = "\n"   # a record cut short by an interrupted run keeps its own line
        with open(path, "a") as f:
            f.write(sep + line + "\n")


def _parse_only(only):
    """'bm,bn,bk,stages,threads[,schedule];...' -> set of tuples (empty = all)."""
    out = set()
    for item in only.split(";"):
        if item.strip():
            v = [int(t) for t in item.split(",")]
            out.add(tuple(v + [0] * (6 - len(v))))
    return out


def sweep_gemm(M, N, K, reps, warmup, trials, out, rasters=(0, 1), only="", expected=None):
    import torch
    import gemv_fp16_amd as gf
    import inputs
    from gemv_fp16_amd import resources
    shape = [M, N, K]
    ij, ref_u, ref_i = load_expected(expected or expected_path("gemm", shape), shape)
    ii, jj = ij[:, 0], ij[:, 1]
    A = torch.from_numpy(inputs.uniform_f16((M, K), 0, 0)).cuda()
    B = torch.from_numpy(inputs.uniform_f16((N, K), 0, 1)).cuda()
    Ai = torch.from_numpy(inputs.integer_f16((M, K), 0, 0)).cuda()
    Bi = torch.from_numpy(inputs.integer_f16((N, K), 0, 1)).cuda()
    C = torch.empty((M, N), dtype=torch.float16, device="cuda")
    default = gf.gemm_default_config(M, N, K)
    seen = _done(out)
    flops = 2.0 * M * N * K
    keep = _parse_only(only)
    for cfg, ok in gf.gemm_configs():
        if keep and (cfg["block_m"], cfg["block_n"], cfg["block_k"], cfg["stages"],
                     cfg["threads"], cfg["schedule"]) not in keep:
            continue
        for raster in rasters:
            c = dict(cfg, raster=raster)
            key = json.dumps(["gemm", shape, c], sort_keys=True)
            if key in seen:
                continue
            rec = {"op": "gemm", "shape": shape, "config": c}
            if not ok:
                rec["status"] = "unsupported"
                _emit(out, rec)
                continue
            fig = resources.gemm(c)
            if resources.spills(fig):
                rec.update(status="spills", scratch_bytes=fig["scratch_bytes"], vgpr_spills=fig["vgpr_spills"])
                _emit(out, rec)
                continue
            try:
                ci = _u16(gf.gemm_f16_nt(Ai, Bi, cfg=c))[ii, jj]
                cu = _u16(gf.gemm_f16_nt(A, B, cfg=c))[ii, jj]
            except RuntimeError as e:
                rec["status"] = "error: %s" % e
                _emit(out, rec)
                continue
            if not np.array_equal(ci, ref_i) or not _close(cu, ref_u):
                rec["status"] = "mismatch"
                _emit(out, rec)
                continue
            med, mn = _time_batch(torch, gf.prepare_gemm_f16_nt(A, B, C, cfg=c), reps, warmup, trials)
            rec.update(status="ok", median_ms=round(med * 1e3, 5), min_ms=round(mn * 1e3, 5),
                       tflops=round(flops / med / 1e12, 2), is_default=(c == default))
            _emit(out, rec)


def sweep_sparse(M, N, K, reps, warmup, trials, out, rasters=(0, 1), expected=None):
    """The 2:4 sparse product's tile configs: A uniform (dense, pruned by the
    compression) and 2:4 integer inputs for the bit-exact gate."""
    import torch
    import gemv_fp16_amd as gf
    import inputs
    shape = [M, N, K]
    ij, ref_u, ref_i = load_expected(expected or expected_path("sparse", shape), shape)
    ii, jj = ij[:, 0], ij[:, 1]
    A = torch.from_numpy(inputs.uniform_f16((M, K), 0, 0)).cuda()
    B = torch.from_numpy(inputs.uniform_f16((N, K), 0, 1)).cuda()
    Ai = torch.from_numpy(inputs.sparse24("integer", (M, K), 0, 0)).cuda()
    Bi = torch.from_numpy(inputs.integer_f16((N, K), 0, 1)).cuda()
    Asp, E = gf.sp24_compress_f16(A)
    Aspi, Ei = gf.sp24_compress_f16(Ai)
    del A, Ai
    C = torch.empty((M, N), dtype=torch.float16, device="cuda")
    default = gf.sp_default_config(M, N, K)
    seen = _done(out)
    flops = 2.0 * M * N * K
    for cfg in gf.sp_configs():
        for raster in rasters:
            c = dict(cfg, raster=raster)
            key = json.dumps(["sparse", shape, c], sort_keys=True)
            if key in seen:
                continue
            rec = {"op": "sparse", "shape": shape, "config": c}
            ci = _u16(gf.gemm_sp_f16_nt(Aspi, Ei, Bi, cfg=c))[ii, jj]
            cu = _u16(gf.gemm_sp_f16_nt(Asp, E, B, cfg=c))[ii, jj]
            if not np.array_equal(ci, ref_i) or not _close(cu, ref_u):
                rec["status"] = "mismatch"
                _emit(out, rec)
                continue
            med, mn = _time_batch(torch, gf.prepare_gemm_sp_f16_nt(Asp, E, B, C, cfg=c), reps, warmup, trials)
            rec.update(status="ok", median_ms=round(med * 1e3, 5), min_ms=round(mn * 1e3, 5),
                       tflops_effective=round(flops / med / 1e12, 2), is_default=(c == default))
            _emit(out, rec)


def sweep_gemv(N, K, reps, warmup, trials, out, blocks=(0,), expected=None):
    import torch
    import gemv_fp16_amd as gf
    import inputs
    shape = [N, K]
    nn, ref_u, ref_i = load_expected(expected or expected_path("gemv", shape), shape)
    nn = nn[:, 0]
    wbytes = N * K * 2
    copies = max(1, min(64, -(-(640 << 20) // max(wbytes, 1))))
    Ws = [torch.from_numpy(inputs.uniform_f16((N, K), i, 0)).cuda() for i in range(copies)]
    x = torch.from_numpy(inputs.uniform_f16((K,), 0, 1)).cuda()
    Wi = torch.from_numpy(inputs.integer_f16((N, K), 0, 0)).cuda()
    xi = torch.from_numpy(inputs.integer_f16((K,), 0, 1)).cuda()
    y = torch.empty((N,), dtype=torch.float16, device="cuda")
    default = gf.gemv_default_config(N, K)
    seen = _done(out)
    nbytes = 2.0 * N * K + 2.0 * K + 2.0 * N
    cands = [dict(c0, blocks=nb) for c0 in gf.gemv_configs() for nb in blocks]
    for c in cands:
        key = json.dumps(["gemv", shape, c], sort_keys=True)
        if key in seen:
            continue
        rec = {"op": "gemv", "shape": shape, "config": c}
        yi = _u16(gf.gemv_f16(Wi, xi, cfg=c))[nn]
        yu = _u16(gf.gemv_f16(Ws[0], x, cfg=c))[nn]
        if not np.array_equal(yi, ref_i) or not _close(yu, ref_u):
            rec["status"] = "mismatch"
            _emit(out, rec)
            continue
        calls = [gf.prepare_gemv_f16(w, x, y, cfg=c) for w in Ws]
        state = [0]

        def call(calls=calls, state=state):
            calls[state[0] % copies]()
            state[0] += 1

        med, mn = _time_batch(torch, call, reps, warmup, trials)
        rec.update(status="ok", median_us=round(med * 1e6, 3), min_us=round(mn * 1e6, 3),
                   gbs=round(nbytes / med / 1e9, 1), w_copies=copies, is_default=(c == default))
        _emit(out, rec)


def _cfg_from(op, text, default):
    """'default' or comma-separated values -> config dict.
    gemm: bm,bn,bk,stages,threads,schedule,raster; sparse: bm,bn,stages,raster;
    gemv: rows_per_wave,unroll,waves,blocks."""
    if text.strip() == "default":
        return dict(default)
    v = [int(t) for t in text.split(",")]
    keys = {"gemm": ("block_m", "block_n", "block_k", "stages", "threads", "schedule", "raster"),
            "sparse": ("block_m", "block_n", "stages", "raster"),
            "gemv": ("rows_per_wave", "unroll", "waves", "blocks")}[op]
    if len(v) != len(keys):
        raise SystemExit("config %r: %d values expected (%s)" % (text, len(keys), ",".join(keys)))
    return dict(zip(keys, v))


def compare(op, shape, specs, rounds=8, reps=20):
    """Time the listed configs side by side: each round launches every
    config `reps` times back to back between HIP events, in alternating
    order from round to round, with the operands that stream from memory
    (A and B for the GEMM, A_sparse, E and B for the sparse product, W for
    the GEMV) rotated over enough copies to exceed the MALL three times.
    Prints the median round per config in TFLOP/s (effective for sparse) or
    GB/s.  This is how the library's default choices between close
    candidates are made; a sequential sweep, one config after another on
    warm operands, can rank them differently.  "default" is the default
    tile or launch shape run as one launch with an explicit config, so a
    shape the library would split into two launches (its row-split plan)
    is compared here as one."""
    import torch
    import gemv_fp16_amd as gf
    import inputs
    mall = 256 << 20
    if op == "gemm":
        M, N, K = shape
        copies = max(1, min(8, -(-3 * mall // (2 * (M + N) * K))))
        A = torch.from_numpy(inputs.uniform_f16((M, K), 0, 0)).cuda()
        B = torch.from_numpy(inputs.uniform_f16((N, K), 0, 1)).cuda()
        ops = [(A, B)] + [(A.clone(), B.clone()) for _ in range(copies - 1)]
        C = torch.empty((M, N), dtype=torch.float16, device="cuda")
        default = gf.gemm_default_config(M, N, K)
        make = lambda c: [gf.prepare_gemm_f16_nt(a, b, C, cfg=c) for a, b in ops]
        work, unit = 2.0 * M * N * K / 1e12, "TFLOP/s"
    elif op == "sparse":
        M, N, K = shape
        copies = max(1, min(8, -(-3 * mall // (2 * N * K + M * K + M * K // 8))))
        A = torch.from_numpy(inputs.uniform_f16((M, K), 0, 0)).cuda()
        Asp, E = gf.sp24_compress_f16(A)
        del A
        B = torch.from_numpy(inputs.uniform_f16((N, K), 0, 1)).cuda()
        ops = [(Asp, E, B)] + [(Asp.clone(), E.clone(), B.clone()) for _ in range(copies - 1)]
        C = torch.empty((M, N), dtype=torch.float16, device="cuda")
        default = gf.sp_default_config(M, N, K)
        make = lambda c: [gf.prepare_gemm_sp_f16_nt(a, e, b, C, cfg=c) for a, e, b in ops]
        work, unit = 2.0 * M * N * K / 1e12, "effective TFLOP/s"
    else:
        N, K = shape
        copies = max(1, min(256, -(-3 * mall // (2 * N * K))))
        Ws = [torch.from_numpy(inputs.uniform_f16((N, K), 0, 0)).cuda()]
        Ws += [Ws[0].clone() for _ in range(copies - 1)]
        x = torch.from_numpy(inputs.uniform_f16((K,), 0, 1)).cuda()
        y = torch.empty((N,), dtype=torch.float16, device="cuda")
        default = gf.gemv_default_config(N, K)
        make = lambda c: [gf.prepare_gemv_f16(w, x, y, cfg=c) for w in Ws]
        work, unit = (2.0 * N * K + 2.0 * K + 2.0 * N) / 1e9, "GB/s"
    cfgs, calls, skipped = [], [], []
    for t in specs.split(";"):
        if not t.strip():
            continue
        c = _cfg_from(op, t, default)
        try:
            cl = make(c)
            cl[0]()
            torch.cuda.synchronize()
        except RuntimeError as e:       # a config with no compiled kernel: listed, not timed
            skipped.append((c, str(e)))
            continue
        cfgs.append(c)
        calls.append(cl)
    for cl in calls:
        for i in range(max(reps // 2, 2)):
            cl[i % copies]()
    torch.cuda.synchronize()
    times = [[] for _ in cfgs]
    for r in range(rounds):
        order = list(range(len(cfgs))) if r % 2 == 0 else list(reversed(range(len(cfgs))))
        for j in order:
            s0 = torch.cuda.Event(enable_timing=True)
            s1 = torch.cuda.Event(enable_timing=True)
            s0.record()
            for i in range(reps):
                calls[j][i % copies]()
            s1.record()
            torch.cuda.synchronize()
            times[j].append(s0.elapsed_time(s1) * 1e-3 / reps)
    lines = ["%s %s, %d copies rotated, %d rounds of %d calls; median round" % (
        op, "x".join(map(str, shape)), copies, rounds, reps), "",
        "| config | median us | min us | max us | %s |" % unit, "|---|---|---|---|---|"]
    for c, t in zip(cfgs, times):
        med = float(np.median(t))
        lines.append("| `%s`%s | %.2f | %.2f | %.2f | %.1f |" % (
            json.dumps(c, sort_keys=True), " (default)" if c == default else "", med * 1e6, min(t) * 1e6,
            max(t) * 1e6, work / med))
    for c, e in skipped:
        lines.append("| `%s` | not timed: %s ||||" % (json.dumps(c, sort_keys=True), e.split(": ", 1)[-1]))
    return "\n".join(lines)


def table(op, shape, path, top):
    """Markdown ranking of the timed records of one (op, shape) in a sweep file."""
    recs, other, spilled = [], {}, []
    for line in open(path):
        try:
            r = json.loads(line)
        except ValueError:
            continue
        if r.get("op") != op or r.get("shape") != shape:
            continue
        if r.get("status") == "ok":
            recs.append(r)
        else:
            other[r.get("status")] = other.get(r.get("status"), 0) + 1
            if r.get("status") == "spills":
                spilled.append(r)
    t = "median_us" if op == "gemv" else "median_ms"
    recs.sort(key=lambda r: r[t])
    lines = ["%d timed; %s" % (len(recs), ", ".join("%d %s" % (n, k) for k, n in sorted(other.items())) or
                                 "none untimed"), ""]
    if op == "gemv":
        nb = 2.0 * shape[0] * shape[1] + 2.0 * shape[1] + 2.0 * shape[0]
        lines += ["| rank | rows/wave | unroll | waves | blocks | median us | min us | GB/s | % of 8000 |",
                  "|---|---|---|---|---|---|---|---|---|"]
        for i, r in enumerate(recs[:top]):
            c = r["config"]
            lines.append("| %d | %d | %d | %d | %d | %.3f | %.3f | %.1f | %.1f%s |" % (
                i + 1, c["rows_per_wave"], c["unroll"], c["waves"], c["blocks"], r["median_us"], r["min_us"],
                nb / r["median_us"] / 1e3, nb / r["median_us"] / 8e4, " (default)" if r.get("is_default") else ""))
        d = [i for i, r in enumerate(recs) if r.get("is_default")]
    else:
        key = "tflops" if op == "gemm" else "tflops_effective"
        lines += ["| rank | config | median ms | min ms | TFLOP/s |", "|---|---|---|---|---|"]
        for i, r in enumerate(recs[:top]):
            lines.append("| %d | `%s` | %.4f | %.4f | %.1f%s |" % (
                i + 1, json.dumps(r["config"], sort_keys=True), r["median_ms"], r["min_ms"], r[key],
                " (default)" if r.get("is_default") else ""))
        d = [i for i, r in enumerate(recs) if r.get("is_default")]
    if d:
        lines += ["", "Default: rank %d of %d." % (d[0] + 1, len(recs))]
    if spilled:
        lines += ["", "Not timed because the compiled kernel spills registers (scratch bytes per lane, VGPRs spilled):", ""]
        lines += ["- `%s`: %d B, %d" % (json.dumps(r["config"], sort_keys=True), r.get("scratch_bytes", 0),
                                       r.get("vgpr_spills", 0)) for r in spilled]
    return "\n".join(lines)


def main(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("op", choices=["gemm", "gemv", "sparse"])
    ap.add_argument("--m", type=int, default=8192)
    ap.add_argument("--n", type=int, default=8192)
    ap.add_argument("--k", type=int, default=8192)
    ap.add_argument("--reps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--trials", type=int, default=3)
    ap.add_argument("--raster", type=int, nargs="*", default=[0, 1])
    ap.add_argument("--out", default="")
    ap.add_argument("--only", default="", help="gemm configs 'bm,bn,bk,stages,threads[,schedule];...'")
    ap.add_argument("--blocks", type=int, nargs="*", default=[0], help="gemv grid bounds (0 = none)")
    ap.add_argument("--expected", default="",
                    help="oracle expected-values file (default: tests/golden/sweep_expected_<op>_<shape>.txt)")
    ap.add_argument("--table", type=int, default=0,
                    help="print the best N records of this shape in --out as markdown, and run nothing")
    ap.add_argument("--compare", default="",
                    help="time these configs side by side instead of sweeping ('default' or values, ';'-separated)")
    ap.add_argument("--rounds", type=int, default=8, help="rounds of --compare")
    a = ap.parse_args(argv)
    if a.compare:
        shape = [a.n, a.k] if a.op == "gemv" else [a.m, a.n, a.k]
        print(compare(a.op, shape, a.compare, a.rounds, a.reps), flush=True)
        return
    if a.table:
        shape = [a.n, a.k] if a.op == "gemv" else [a.m, a.n, a.k]
        print(table(a.op, shape, a.out, a.table))
        return
    t = time.time()
    if a.op == "gemm":
        sweep_gemm(a.m, a.n, a.k, a.reps, a.warmup, a.trials, a.out, tuple(a.raster), a.only, a.expected)
    elif a.op == "sparse":
        sweep_sparse(a.m, a.n, a.k, a.reps, a.warmup, a.trials, a.out, tuple(a.raster), a.expected)
    else:
        sweep_gemv(a.n, a.k, a.reps, a.warmup, a.trials, a.out, tuple(a.blocks), a.expected)
    print("sweep done in %.1f s" % (time.time() - t), file=sys.stderr, flush=True)


if __name__ == "__main__":
    main()

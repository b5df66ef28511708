"""Compiler resource figures of the library's kernels.

    python -m gemv_fp16_amd.resources            # markdown table of the default kernels

The build records, for every kernel instantiation, what the compiler reports
for it (its kernel-resource-usage remarks): VGPRs, AGPRs, SGPRs, per-lane
scratch (non-zero means registers spill to memory), statically allocated LDS
and the occupancy in waves per SIMD that the registers allow.  The GEMM
kernels' tile staging uses dynamic LDS, which the launch sets to the tile
config's stage bytes; that figure is listed beside the compiler's.  The
offline sweep uses the scratch figure to mark spilling tile configs.
"""
from __future__ import annotations

import json
import os
import sys

_HERE = os.path.dirname(os.path.abspath(__file__))
RESOURCES = os.path.join(_HERE, "kernel_resources.json")

_cache = None


def load(path: str = RESOURCES) -> dict:
    """{demangled kernel name: figures}; empty if the build left no report."""
    global _cache
    if _cache is None or path != RESOURCES:
        try:
            rep = json.load(open(path))
        except (OSError, ValueError):
            rep = {}
        res = {v["name"]: v for v in rep.values() if "name" in v}
        if path != RESOURCES:
            return res
        _cache = res
    return _cache


def gemm_kernel_name(cfg: dict, epi: int = 0, aligned: bool = True, layout=(0, 0)) -> str:
    """The demangled name of a GEMM instantiation (epilogue 0 = fp16 C)."""
    return ("void gf::gemm_nt_kernel<gf::GemmCfg<%d, %d, %d, %d, %d, %d, %d, %d>, %d, %s>(gf::GemmArgs)" % (
        cfg["block_m"], cfg["block_n"], cfg["block_k"], cfg["stages"], cfg["threads"], cfg.get("schedule", 0),
        layout[0], layout[1], epi, "true" if aligned else "false"))


def gemm(cfg: dict, epi: int = 0, aligned: bool = True, layout=(0, 0), report: dict | None = None):
    """Figures of one GEMM instantiation, or None if unknown."""
    return (report if report is not None else load()).get(gemm_kernel_name(cfg, epi, aligned, layout))


def spills(figures) -> bool:
    return bool(figures) and (figures.get("scratch_bytes", 0) > 0 or figures.get("vgpr_spills", 0) > 0
                              or figures.get("sgpr_spills", 0) > 0)


def gemm_lds_bytes(cfg: dict) -> int:
    """Dynamic LDS of a GEMM launch: the stage ring or the epilogue's
    transpose buffer, whichever is larger (the kernel's LDS_BYTES)."""
    bm, bn, bk, st, nt = cfg["block_m"], cfg["block_n"], cfg["block_k"], cfg["stages"], cfg["threads"]
    nw = nt // 64
    wm = 2 if nw == 4 else (4 if bm > bn else 2)
    wn = nw // wm
    main = st * (bm + bn) * bk * 2
    epi = nw * (bm // wm) * (bn // wn + 8) * 2
    return max(main, epi)


def _row(label, name, fig, lds=None):
    if not fig:
        return "| %s | `%s` | (not in the report) |||||||" % (label, name)
    return "| %s | `%s` | %d | %d | %d | %d | %d | %s | %d |" % (
        label, name.replace("void gf::", "").split("(")[0], fig["vgprs"], fig["agprs"], fig["sgprs"],
        fig["scratch_bytes"], fig["vgpr_spills"], lds if lds is not None else fig["static_lds_bytes"],
        fig["occupancy_waves_per_simd"])


def defaults_table() -> str:
    """Markdown table of the kernels the library runs by default on the
    benchmark workloads."""
    import gemv_fp16_amd as gf
    rep = load()
    lines = ["| workload | kernel | VGPRs | AGPRs | SGPRs | scratch B/lane | VGPR spills | LDS B | waves/SIMD |",
             "|---|---|---|---|---|---|---|---|---|"]
    for (m, n, k) in ((8192, 8192, 8192), (8192, 8192, 1024), (8192, 8192, 256), (2048, 4096, 8192),
                      (1024, 1024, 4096)):
        c = gf.gemm_default_config(m, n, k)
        name = gemm_kernel_name(c)
        lines.append(_row("GEMM %dx%dx%d" % (m, n, k), name, rep.get(name), gemm_lds_bytes(c)))
    big = {"block_m": 256, "block_n": 256, "block_k": 64, "stages": 2, "threads": 256, "schedule": 2}
    for lay, label in (((0, 1), "GEMM NN 8192^3"), ((1, 1), "GEMM TN 8192^3")):
        name = gemm_kernel_name(big, layout=lay)
        lines.append(_row(label, name, rep.get(name), gemm_lds_bytes(big)))
    cands = ({"block_m": 256, "block_n": 256, "block_k": 64, "stages": 2, "threads": 512, "schedule": 0},
             {"block_m": 256, "block_n": 128, "block_k": 64, "stages": 3, "threads": 256, "schedule": 2},
             {"block_m": 128, "block_n": 128, "block_k": 64, "stages": 3, "threads": 256, "schedule": 0},
             {"block_m": 64, "block_n": 64, "block_k": 64, "stages": 3, "threads": 256, "schedule": 0})
    for split in (4, 8, 16):
        # the split-K default tile (the library's rule): the first candidate
        # whose tiles x slices fill the CUs; the 64 x 64 tile for atomics at
        # 16 slices
        for c in cands:
            if (1024 // c["block_m"]) * (1024 // c["block_n"]) * split >= 256:
                break
        for epi, what in ((2, "two-pass store"), (1, "atomic")):
            cc = cands[-1] if epi == 1 and split >= 16 else c
            name = gemm_kernel_name(cc, epi=epi)
            lines.append(_row("split-K 1024^2x16384 s=%d %s" % (split, what), name, rep.get(name),
                              gemm_lds_bytes(cc)))
    for n, k in ((8192, 8192), (1024, 1024)):
        g = gf.gemv_default_config(n, k)
        if g["blocks"] > 0 and k % (8 * g["waves"] * 64 * g["unroll"]) == 0:
            name = "void gf::gemv_split_kernel<%d, %d, %d>(unsigned short const*, unsigned short const*, " \
                   "unsigned short*, int, int)" % (g["rows_per_wave"], g["unroll"], g["waves"])
            lds = 2 * g["waves"] * g["rows_per_wave"] * 4 + 32 + 2 * k
        else:
            name = "void gf::gemv_kernel<%d, %d, %d, true, false>(unsigned short const*, unsigned short " \
                   "const*, unsigned short*, int, int)" % (g["rows_per_wave"], g["unroll"], g["waves"])
            lds = None
        lines.append(_row("GEMV %dx%d" % (n, k), name, rep.get(name), lds))
    return "\n".join(lines)


if __name__ == "__main__":
    sys.path.insert(0, os.path.dirname(_HERE))
    print(defaults_table())

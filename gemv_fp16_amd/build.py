"""Build libgemvfp16.so (HIP for gfx950) in-tree.

    python -m gemv_fp16_amd.build          # or gemv_fp16_amd.build.build()

Objects go to ``_build/`` at the repository root; the library is written
next to this file so that it travels with the source tree.
"""
from __future__ import annotations

import json
import os
import re
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
OBJ = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libgemvfp16.so")
# Per-kernel register, scratch, LDS and occupancy figures from the compiler
# (its kernel-resource-usage remarks), written at every build.
RESOURCES = os.path.join(PKG, "kernel_resources.json")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
N_SHARDS = 8  # must match gf::kGemmShards

FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-munsafe-fp-atomics",
    # packed fp32 VALU ops stay off: only scalar and vector fp32 code paths
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
]


def _units():
    units = [("gemm_shard.hip", "gemm_shard_%d.o" % i, ["-DGF_SHARD=%d" % i]) for i in range(N_SHARDS)]
    units += [("gemv.hip", "gemv.o", []), ("skinny.hip", "skinny.o", []),
              ("sparse.hip", "sparse.o", []), ("api.hip", "api.o", [])]
    return units


_REMARK = re.compile(r"remark:\s+(Function Name|TotalSGPRs|VGPRs|AGPRs|ScratchSize \[bytes/lane\]|"
                     r"Occupancy \[waves/SIMD\]|SGPRs Spill|VGPRs Spill|LDS Size \[bytes/block\]):\s*(\S+)")
_KEYS = {"TotalSGPRs": "sgprs", "VGPRs": "vgprs", "AGPRs": "agprs", "ScratchSize [bytes/lane]": "scratch_bytes",
         "Occupancy [waves/SIMD]": "occupancy_waves_per_simd", "SGPRs Spill": "sgpr_spills",
         "VGPRs Spill": "vgpr_spills", "LDS Size [bytes/block]": "static_lds_bytes"}


def parse_resource_remarks(text: str) -> dict:
    """{mangled kernel name: {vgprs, agprs, sgprs, scratch_bytes, ...}} from
    the compiler's kernel-resource-usage remarks."""
    out, cur = {}, None
    for m in _REMARK.finditer(text):
        key, val = m.group(1), m.group(2)
        if key == "Function Name":
            cur = out.setdefault(val, {})
        elif cur is not None:
            cur[_KEYS[key]] = int(val)
    return out


def _compile(unit):
    src, obj, extra = unit
    out = os.path.join(OBJ, obj)
    cmd = [HIPCC] + FLAGS + extra + ["-Rpass-analysis=kernel-resource-usage", "-c",
                                     os.path.join(CSRC, src), "-o", out]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed for %s:\n%s\n%s" % (src, " ".join(cmd), r.stderr))
    return out, parse_resource_remarks(r.stderr)


def _demangle(names):
    try:
        r = subprocess.run(["c++filt"], input="\n".join(names), capture_output=True, text=True, check=True)
        dem = r.stdout.split("\n")
        if len(dem) >= len(names):
            return dem[:len(names)]
    except (OSError, subprocess.CalledProcessError):
        pass
    return list(names)


# Diagnostic variants: the same library built with one feature switched off,
# into gemv_fp16_amd/variants/<variant>/libgemvfp16.so (load it with
# GEMVFP16_LIB=<path>).  Only for counter comparisons; the product is the
# default build.
VARIANTS = {"noswizzle": ["-DGF_DIAG_NO_LDS_SWIZZLE"], "timeline": ["-DGF_DIAG_TIMELINE"]}


def build_variant(name: str, jobs: int | None = None) -> str:
    out_dir = os.path.join(OBJ, name)
    os.makedirs(out_dir, exist_ok=True)
    units = [(src, os.path.join(name, obj), extra + VARIANTS[name]) for src, obj, extra in _units()]
    jobs = jobs or min(8, os.cpu_count() or 1)
    with ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = [o for o, _ in ex.map(_compile, units)]
    lib_dir = os.path.join(PKG, "variants", name)
    os.makedirs(lib_dir, exist_ok=True)
    lib = os.path.join(lib_dir, "libgemvfp16.so")
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", lib] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n%s\n%s" % (" ".join(cmd), r.stderr))
    return lib


def build(jobs: int | None = None, verbose: bool = False) -> str:
    """Compile every HIP source and link the shared library.  Always rebuilds."""
    os.makedirs(OBJ, exist_ok=True)
    jobs = jobs or min(8, os.cpu_count() or 1)
    with ThreadPoolExecutor(max_workers=jobs) as ex:
        results = list(ex.map(_compile, _units()))
    objs = [o for o, _ in results]
    res = {}
    for _, r in results:
        res.update(r)
    names = sorted(res)
    report = {m: dict(res[m], name=d) for m, d in zip(names, _demangle(names))}
    with open(RESOURCES + ".tmp", "w") as f:
        json.dump(report, f, indent=0, sort_keys=True)
    os.replace(RESOURCES + ".tmp", RESOURCES)
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n%s\n%s" % (" ".join(cmd), r.stderr))
    os.replace(tmp, LIB)
    # Diagnostics (not linked into the library): the HBM streaming-read, the
    # MFMA throughput and the LDS throughput ceiling probes.
    for name in ("readbw", "mfmapeak", "ldsbw"):
        probe = os.path.join(PKG, name)
        cmd = [HIPCC] + [f for f in FLAGS if f != "-fPIC"] + [os.path.join(CSRC, name + ".hip"), "-o",
                                                            probe + ".tmp"]
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError("hipcc failed for %s.hip:\n%s" % (name, r.stderr))
        os.replace(probe + ".tmp", probe)
    if verbose:
        print("built", LIB)
    return LIB


if __name__ == "__main__":
    if len(sys.argv) == 3 and sys.argv[1] == "--variant" and sys.argv[2] in VARIANTS:
        print("built", build_variant(sys.argv[2]))
    else:
        build(verbose=True)
    sys.exit(0)

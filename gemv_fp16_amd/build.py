"""Build libgemvfp16.so (HIP for gfx950) in-tree.

    python -m gemv_fp16_amd.build          # or gemv_fp16_amd.build.build()

Objects go to ``_build/`` at the repository root; the library is written
next to this file so that it travels with the source tree.
"""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
OBJ = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libgemvfp16.so")
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


def _compile(unit):
    src, obj, extra = unit
    out = os.path.join(OBJ, obj)
    cmd = [HIPCC] + FLAGS + extra + ["-c", os.path.join(CSRC, src), "-o", out]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed for %s:\n%s\n%s" % (src, " ".join(cmd), r.stderr))
    return out


def build(jobs: int | None = None, verbose: bool = False) -> str:
    """Compile every HIP source and link the shared library.  Always rebuilds."""
    os.makedirs(OBJ, exist_ok=True)
    jobs = jobs or min(8, os.cpu_count() or 1)
    with ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(_compile, _units()))
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n%s\n%s" % (" ".join(cmd), r.stderr))
    os.replace(tmp, LIB)
    # Diagnostics (not linked into the library): the HBM streaming-read and
    # the MFMA throughput ceiling probes.
    for name in ("readbw", "mfmapeak"):
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
    build(verbose=True)
    sys.exit(0)

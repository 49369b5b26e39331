"""Build libdsrows.so for gfx950 with hipcc, in-tree.

Compiles each translation unit under csrc/ to an object (in parallel) and
links the shared library into scale_invariant_row_amd/_lib/.  Always
recompiles: the caller asked for a build.

    python -m scale_invariant_row_amd.build
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(PKG, "_build")
LIBDIR = os.path.join(PKG, "_lib")
LIB = os.path.join(LIBDIR, "libdsrows.so")
# the benchmark's stream reference (not part of the row library's ABI)
BENCH_LIB = os.path.join(LIBDIR, "libdsbench.so")
BENCH_SOURCES = ["bench_stream.hip"]
SOURCES = ["ds_rows.hip", "inst_l2.hip", "inst_slerp.hip", "inst_rownorm.hip",
           "inst_l2_bwd.hip", "inst_rownorm_bwd.hip", "inst_act.hip", "inst_qk.hip",
           "inst_rescale.hip", "inst_rms.hip", "inst_rms_bwd.hip", "inst_colblock.hip"]
ARCH = "gfx950"

# -ffp-contract=off: only explicit fmaf fuses (the slerp lerp is three
# rounded steps).  Packed fp32 instructions are switched off.  Denormals are
# kept (HIP's default for fp32 on gfx9), and division/sqrt are correctly
# rounded (HIP's default).
CFLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    "-ffp-contract=off",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wextra", "-Wno-unused-parameter", "-Werror",
    f"-I{os.path.join(ROOT, 'include')}", f"-I{CSRC}",
]


def hipcc() -> str:
    path = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(path):
        raise RuntimeError("hipcc not found: cannot build the HIP library")
    return path


def _run(cmd):
    p = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    # the host pass does not know the packed-fp32 feature and says so; harmless
    noise = "'-packed-fp32-ops' is not a recognized feature"
    lines = [l for l in p.stdout.splitlines() if noise not in l]
    return p.returncode, "\n".join(lines)


def build(verbose: bool = False, jobs: int = 4) -> str:
    """Build libdsrows.so and the benchmark's libdsbench.so; returns the former."""
    os.makedirs(BUILD, exist_ok=True)
    os.makedirs(LIBDIR, exist_ok=True)
    cc = hipcc()
    objs, cmds = {}, []
    for src in SOURCES + BENCH_SOURCES:
        obj = os.path.join(BUILD, src.replace(".hip", ".o"))
        objs[src] = obj
        cmds.append([cc, *CFLAGS, "-c", os.path.join(CSRC, src), "-o", obj])
    with cf.ThreadPoolExecutor(max_workers=jobs) as ex:
        results = list(ex.map(_run, cmds))
    for cmd, (rc, out) in zip(cmds, results):
        if verbose and out:
            print(out)
        if rc != 0:
            raise RuntimeError(f"hipcc failed ({rc}): {' '.join(cmd)}\n{out}")
    for lib, srcs in ((LIB, SOURCES), (BENCH_LIB, BENCH_SOURCES)):
        tmp = lib + ".tmp"
        rc, out = _run([cc, f"--offload-arch={ARCH}", "-shared", "-o", tmp,
                        *[objs[s] for s in srcs]])
        if rc != 0:
            raise RuntimeError(f"link failed ({rc}):\n{out}")
        os.replace(tmp, lib)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))

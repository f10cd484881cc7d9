"""Build libequitp.so (HIP, gfx950) in place next to the Python binding.

Steps: compile and run gen_cg.cpp to (re)write cg_table.h, compile every translation unit with
hipcc in parallel, link the shared library.  Always rebuilds (the caller decides when)."""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
PKG = os.path.dirname(HERE)
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libequitp.so")
HIPCC = os.environ.get("HIPCC", shutil.which("hipcc") or "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

# (source, object, extra flags): conv_bwd.hip is built three times (fp32 kernels and the host
# launchers; bf16-operand kernels; per-edge path-subset kernels) and conv_seg.hip twice (plain;
# path subsets), so that the parts compile in parallel
SOURCES = [("equitp.cpp", "equitp.o", []), ("conv_seg.hip", "conv_seg.o", []),
           ("conv_bwd.hip", "conv_bwd.o", []),
           ("conv_bwd.hip", "conv_bwd_bf16.o", ["-DEQUITP_BWD_BF16=1"]),
           ("conv_seg.hip", "conv_seg_mask.o", ["-DEQUITP_MASKED=1"]),
           ("conv_bwd.hip", "conv_bwd_mask.o", ["-DEQUITP_BWD_MASKED=1"]),
           ("linear_graph.hip", "linear_graph.o", []), ("ladder.hip", "ladder.o", []),
           ("full_ladder.hip", "full_ladder.o", []),
           ("mixed.hip", "mixed.o", [])]
FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-fno-gpu-rdc",
    # no packed fp32 math is emitted (v_pk_*_f32)
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
]


def _run(cmd):
    r = subprocess.run(cmd, cwd=HERE, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in r.stdout.splitlines()
                    if "packed-fp32-ops" not in l and "warning generated" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"command failed ({r.returncode}): {' '.join(cmd)}\n{out}")
    return out


def generate_cg_table() -> None:
    os.makedirs(BUILD, exist_ok=True)
    exe = os.path.join(BUILD, "gen_cg")
    cxx = shutil.which("g++") or shutil.which("c++")
    _run([cxx, "-O2", "-std=c++17", "gen_cg.cpp", "-o", exe])
    tmp = os.path.join(BUILD, "cg_table.h")
    _run([exe, tmp])
    dst = os.path.join(HERE, "cg_table.h")
    new = open(tmp).read()
    if not os.path.exists(dst) or open(dst).read() != new:
        with open(dst, "w") as f:
            f.write(new)


def build(jobs: int | None = None, verbose: bool = False) -> str:
    generate_cg_table()
    os.makedirs(BUILD, exist_ok=True)
    objs = []
    cmds = []
    for src, obj_name, extra in SOURCES:
        obj = os.path.join(BUILD, obj_name)
        objs.append(obj)
        cmds.append([HIPCC, *FLAGS, *extra, "-c", src, "-o", obj])
    jobs = jobs or min(len(cmds), max(1, (os.cpu_count() or 2)))
    with cf.ThreadPoolExecutor(max_workers=jobs) as ex:
        for out in ex.map(_run, cmds):
            if verbose and out.strip():
                print(out)
    tmp = LIB + ".tmp"
    _run([HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp])
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))

"""Build libcgtp.so in-tree with hipcc for gfx950.

    python -m clebsch_gordan_tensor_node_amd.build [--incremental] [-j N]

Every translation unit is compiled in parallel; the convolution kernel source is
compiled once per kernel class (-DCGTP_CONV_CLASS=k).  Objects go to ``_build/`` at the
repository root; the shared library is written next to this file.
"""
from __future__ import annotations

import argparse
import os
import re
import shutil
import subprocess
import sys
import time
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libcgtp.so")
N_CONV_CLASSES = 9

ARCH = "gfx950"
FLAGS = [
    "-std=c++17", "-O3", f"--offload-arch={ARCH}", "-fPIC",
    # no packed-FP32 instructions in device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
]


def _hipcc() -> str:
    for cand in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: the HIP toolchain is required to build libcgtp")


def _units():
    units = [("cgtp_api.hip", [], "cgtp_api.o"), ("kernels_graph.hip", [], "kernels_graph.o"),
             ("kernels_bwd.hip", [], "kernels_bwd.o")]
    for c in range(N_CONV_CLASSES):
        units.append(("kernels_conv.hip", [f"-DCGTP_CONV_CLASS={c}"], f"kernels_conv_c{c}.o"))
    return units


_INCLUDE = re.compile(r'^\s*#\s*include\s+"([^"]+)"', re.M)


def _deps(path: str, seen: set) -> set:
    """The file and every local header it includes, transitively."""
    path = os.path.normpath(path)
    if path in seen or not os.path.exists(path):
        return seen
    seen.add(path)
    with open(path) as f:
        for inc in _INCLUDE.findall(f.read()):
            _deps(os.path.join(os.path.dirname(path), inc), seen)
    return seen


def _newest_input(src: str) -> float:
    """Newest modification time among a unit's source and the headers it includes."""
    return max(os.path.getmtime(f) for f in _deps(os.path.join(CSRC, src), set()))


def build(incremental: bool = False, jobs: int | None = None, verbose: bool = True) -> str:
    """Compile and link libcgtp.so; returns its path.  Raises on any compiler error."""
    hipcc = _hipcc()
    os.makedirs(BUILD, exist_ok=True)
    jobs = jobs or min(16, os.cpu_count() or 4)

    def compile_one(unit):
        src, defs, obj = unit
        out = os.path.join(BUILD, obj)
        if incremental and os.path.exists(out) and os.path.getmtime(out) > _newest_input(src):
            return out, 0.0, ""
        t0 = time.time()
        cmd = [hipcc, *FLAGS, *defs, "-c", os.path.join(CSRC, src), "-o", out]
        r = subprocess.run(cmd, capture_output=True, text=True)
        msgs = "\n".join(l for l in (r.stdout + r.stderr).splitlines() if "packed-fp32-ops" not in l)
        if r.returncode != 0:
            raise RuntimeError(f"hipcc failed for {src} {' '.join(defs)}:\n{msgs}")
        return out, time.time() - t0, msgs

    t0 = time.time()
    # the slowest units (the backward's edge pass, the l >= 4 conv classes) start first
    slow = {"kernels_conv_c6.o": 0, "kernels_conv_c7.o": 1, "kernels_conv_c8.o": 2, "kernels_conv_c1.o": 3,
            "kernels_conv_c5.o": 4, "kernels_bwd.o": 5, "kernels_conv_c4.o": 6}
    order = sorted(range(len(_units())), key=lambda k: slow.get(_units()[k][2], 99))
    with ThreadPoolExecutor(max_workers=jobs) as ex:
        done = dict(zip(order, ex.map(compile_one, [_units()[k] for k in order])))
    results = [done[k] for k in range(len(_units()))]
    objs = [r[0] for r in results]
    if verbose:
        for (src, defs, obj), (_, dt, msgs) in zip(_units(), results):
            if dt:
                print(f"  compiled {obj:24s} {dt:6.1f} s", flush=True)
            if msgs.strip():
                print(msgs, flush=True)
    tmp = LIB + ".tmp"
    cmd = [hipcc, "-shared", "-fPIC", f"--offload-arch={ARCH}", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB} in {time.time() - t0:.1f} s", flush=True)
    return LIB


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--incremental", action="store_true", help="reuse objects newer than every source")
    ap.add_argument("-j", type=int, default=None)
    a = ap.parse_args(argv)
    build(incremental=a.incremental, jobs=a.j)


if __name__ == "__main__":
    sys.exit(main())

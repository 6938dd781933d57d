"""Builds the HIP libraries in-tree for gfx950 with hipcc.

* looped_weight_shared_loop_amd/libloop.so : kernels + loop driver + C ABI
* synth/libsynth.so                        : device fills of the seeded inputs

Object files go to _build/ (not committed).  Every call rebuilds.
"""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
ARCH = "gfx950"
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
         # packed fp32 instructions are kept out of the generated code
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-Wno-unused-result"]

LOOP_SOURCES = ["k_rows.hip", "k_gemm.hip", "k_attn.hip", "k_lin.hip", "driver.cpp", "ops.cpp"]


def _run(cmd):
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in r.stdout.splitlines() if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"build failed: {' '.join(cmd)}\n{out}")
    return out


def _compile(src, obj):
    lang = ["-x", "hip"] if src.endswith(".cpp") else []
    _run([HIPCC, *FLAGS, "-I", os.path.join(ROOT, "include"), *lang, "-c", src, "-o", obj])
    return obj


def build_lib(sources, out, objdir):
    os.makedirs(objdir, exist_ok=True)
    jobs = min(8, len(sources), max(1, len(os.sched_getaffinity(0))))
    with ThreadPoolExecutor(jobs) as ex:
        objs = list(ex.map(lambda s: _compile(s, os.path.join(objdir, os.path.basename(s) + ".o")), sources))
    tmp = out + ".tmp"
    _run([HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs])
    os.replace(tmp, out)
    return out


def build(verbose: bool = False):
    objdir = os.path.join(ROOT, "_build")
    loop = build_lib([os.path.join(PKG, "csrc", s) for s in LOOP_SOURCES],
                     os.path.join(PKG, "libloop.so"), os.path.join(objdir, "loop"))
    syn = build_lib([os.path.join(ROOT, "synth", "csrc", "synth_fill.hip")],
                    os.path.join(ROOT, "synth", "libsynth.so"), os.path.join(objdir, "synth"))
    if verbose:
        print("built", loop, syn)
    return loop, syn


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)

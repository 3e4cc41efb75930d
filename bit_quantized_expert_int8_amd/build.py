"""Build libmoeq4.so (the HIP library) and synth/libsynth.so (the device input generator) for gfx950.

Every translation unit is compiled with hipcc for gfx950 only, in parallel, into ``_build/``, then linked
in-tree so the shared objects travel with the source tree.  Usage: ``python -m bit_quantized_expert_int8_amd.build``.
"""
from __future__ import annotations

import concurrent.futures
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
BUILD = os.path.join(ROOT, "_build")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

LIB_SOURCES = ["api.cpp", "quantize.hip", "router.hip", "q4_gemv.hip", "q4_grouped.hip", "q4_mfma.hip", "layer.hip", "cache.hip", "probe.hip"]
LIB_OUT = os.path.join(PKG, "libmoeq4.so")
SYNTH_SOURCES = [os.path.join(ROOT, "synth", "synth_gen.hip")]
SYNTH_OUT = os.path.join(ROOT, "synth", "libsynth.so")
# the generator's host twin (plain C, OpenMP): test and oracle inputs drawn on the CPU
SYNTH_HOST_SOURCE = os.path.join(ROOT, "synth", "synth_host.c")
SYNTH_HOST_OUT = os.path.join(ROOT, "synth", "libsynth_host.so")
# the C part of the CPU oracle (test infrastructure, built here so the checker is ready; never loaded by the
# library): plain -O2, no fast-math, so its arithmetic is IEEE as written
ORACLE_SOURCE = os.path.join(ROOT, "oracle", "ffn_ref.c")
ORACLE_OUT = os.path.join(ROOT, "oracle", "liboracle_ffn.so")
CC = os.environ.get("CC", "gcc")

# -packed-fp32-ops: keep the compiler from emitting packed fp32 arithmetic (plain fp32 code only)
# code object v5: loadable by the HIP runtime torch bundles as well as by /opt/rocm's
HIP_FLAGS = ["-O3", "-std=c++17", "-fPIC", "--offload-arch=gfx950", "-mcode-object-version=5", "-Wall",
             "-Wno-unused-function",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             "-I", os.path.join(ROOT, "include")]


def _compile(src: str, obj: str) -> str:
    cmd = [HIPCC, *HIP_FLAGS]
    if src.endswith(".cpp"):
        cmd += ["-x", "hip"]
    cmd += ["-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return obj


def _link(objs: list[str], out: str) -> None:
    tmp = out + ".tmp"
    cmd = [HIPCC, "-shared", "-fPIC", "--offload-arch=gfx950", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, out)


def _gcc(src: str, out: str, extra: list[str]) -> None:
    tmp = out + ".tmp"
    cmd = [CC, "-O2", "-shared", "-fPIC", "-Wall", *extra, "-o", tmp, src, "-lm"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, out)


def _build_host_c() -> None:
    _gcc(SYNTH_HOST_SOURCE, SYNTH_HOST_OUT, ["-fopenmp"])
    _gcc(ORACLE_SOURCE, ORACLE_OUT, [])


def build(verbose: bool = True) -> list[str]:
    os.makedirs(BUILD, exist_ok=True)
    _build_host_c()
    jobs = []
    for s in LIB_SOURCES:
        jobs.append((os.path.join(PKG, "csrc", s), os.path.join(BUILD, "moeq4_" + os.path.splitext(s)[0] + ".o")))
    for s in SYNTH_SOURCES:
        jobs.append((s, os.path.join(BUILD, "synth_" + os.path.splitext(os.path.basename(s))[0] + ".o")))
    workers = max(1, min(len(jobs), int(os.environ.get("MAX_JOBS", os.cpu_count() or 4))))
    with concurrent.futures.ThreadPoolExecutor(workers) as ex:
        objs = list(ex.map(lambda j: _compile(*j), jobs))
    _link(objs[:len(LIB_SOURCES)], LIB_OUT)
    _link(objs[len(LIB_SOURCES):], SYNTH_OUT)
    if verbose:
        print(f"built {LIB_OUT}\nbuilt {SYNTH_OUT}\nbuilt {SYNTH_HOST_OUT}\nbuilt {ORACLE_OUT}")
    return [LIB_OUT, SYNTH_OUT, SYNTH_HOST_OUT, ORACLE_OUT]


if __name__ == "__main__":
    build()
    sys.exit(0)

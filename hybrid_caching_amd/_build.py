"""Compile the HIP sources of the segment transform into ``libpic.so`` (gfx950).

Run ``python -m hybrid_caching_amd._build`` (or ``__graft_entry__.build()``).
The library is built in-tree next to this file; objects go to ``_build/``.
"""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
OBJ_DIR = os.path.join(HERE, "_build")
LIB_PATH = os.path.join(HERE, "libpic.so")
# diagnostic twin of the library: the dense fp16 build with per-wave barrier
# timers (-DPIC_PHASE_TIMING), every other object shared
TIMING_LIB_PATH = os.path.join(HERE, "libpic_timing.so")
TIMED_SOURCES = ["k_build_dense_h16.hip"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

SOURCES = ["pic_host.cpp", "k_compose.hip", "k_build_dense.hip", "k_build_dense_ws.hip", "k_build_dense_h16.hip", "k_dense_fp16.hip",
           "k_build_scalar_diag.hip", "k_build_sd_pipe.hip", "k_compose_seam.hip",
           "k_build_kda.hip", "k_build_kda_chunk.hip", "k_rerotate.hip", "k_conv_warmup.hip"]

# Packed fp32 VALU forms are disabled for all device code.
COMMON = ["-O3", "-std=c++17", "-fPIC", "--offload-arch=gfx950", "-Xclang", "-target-feature",
          "-Xclang", "-packed-fp32-ops", "-Wall", "-Wno-unused-result",
          "-I" + os.path.join(ROOT, "include"), "-I" + CSRC]


def _compile(src: str, extra=(), suffix: str = "") -> str:
    obj = os.path.join(OBJ_DIR, os.path.splitext(src)[0] + suffix + ".o")
    lang = ["-x", "hip"]  # host-only sources also go through the HIP driver
    cmd = [HIPCC, *COMMON, *lang, *extra, "-c", os.path.join(CSRC, src), "-o", obj]
    res = subprocess.run(cmd, capture_output=True, text=True)
    msgs = "\n".join(l for l in (res.stdout + res.stderr).splitlines()
                     if "packed-fp32-ops" not in l)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{msgs}")
    if msgs.strip():
        print(msgs, file=sys.stderr)
    return obj


def build(verbose: bool = False, extra=()) -> str:
    os.makedirs(OBJ_DIR, exist_ok=True)
    jobs = [(s, tuple(extra), "") for s in SOURCES]
    jobs += [(s, tuple(extra) + ("-DPIC_PHASE_TIMING",), "_timing") for s in TIMED_SOURCES]
    with ThreadPoolExecutor(max_workers=min(4, len(jobs))) as ex:
        objs = list(ex.map(lambda j: _compile(*j), jobs))
    plain = objs[:len(SOURCES)]
    timed = dict(zip(TIMED_SOURCES, objs[len(SOURCES):]))
    timing_objs = [timed.get(s, o) for s, o in zip(SOURCES, plain)]
    for path, objects in ((LIB_PATH, plain), (TIMING_LIB_PATH, timing_objs)):
        tmp = path + ".tmp"
        cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp, *objects]
        res = subprocess.run(cmd, capture_output=True, text=True)
        if res.returncode != 0:
            raise RuntimeError("link failed:\n" + res.stdout + res.stderr)
        os.replace(tmp, path)
        if verbose:
            print("built", path)
    return LIB_PATH


if __name__ == "__main__":
    extra = sys.argv[1:]
    build(verbose=True, extra=extra)

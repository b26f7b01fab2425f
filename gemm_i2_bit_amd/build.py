"""Build the HIP library libbt.so for gfx950 with hipcc (cross-compiles on a
machine without a GPU).  Objects go to _build/ at the repository root; the
library is written next to this file."""
from __future__ import annotations

import glob
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
OBJDIR = os.path.join(ROOT, "_build")
LIB = os.path.join(HERE, "libbt.so")
# timing build: the same library with per-wave timestamps in the streaming
# kernel and the read probe (BT_WAVE_TIMESTAMPS; include/bt_timing.h)
TIMING_LIB = os.path.join(HERE, "libbt_timing.so")
TIMED_SOURCES = ("gemv_stream.hip", "probe.hip")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

ARCH = "gfx950"
DEVICE_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    "-ffp-contract=off",
    # packed fp32 instructions are kept out of every kernel
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # kernel arguments arrive in SGPRs at dispatch (the code object keeps a
    # prologue that loads them where the firmware does not preload)
    "-mllvm", "-amdgpu-kernarg-preload-count=16",
    "-Wall", "-Wno-unused-function",
    "-I", INCLUDE, "-I", CSRC,
]


def sources():
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")))


def build(verbose: bool = False) -> str:
    """Compile every .hip source (in parallel) and link libbt.so, and the
    timing build libbt_timing.so (the timed sources compiled a second time
    with BT_WAVE_TIMESTAMPS, linked with the other objects)."""
    os.makedirs(OBJDIR, exist_ok=True)
    procs = []
    objs = []
    timed_objs = []
    jobs = []
    for src in sources():
        base = os.path.basename(src)[:-4]
        obj = os.path.join(OBJDIR, base + ".o")
        objs.append(obj)
        jobs.append((src, [HIPCC, *DEVICE_FLAGS, "-c", src, "-o", obj]))
        if os.path.basename(src) in TIMED_SOURCES:
            tobj = os.path.join(OBJDIR, "timed_" + base + ".o")
            timed_objs.append(tobj)
            jobs.append((src, [HIPCC, *DEVICE_FLAGS, "-DBT_WAVE_TIMESTAMPS",
                               "-c", src, "-o", tobj]))
        else:
            timed_objs.append(obj)
    for src, cmd in jobs:
        if verbose:
            print(" ".join(cmd), flush=True)
        procs.append((src, subprocess.Popen(cmd, stdout=subprocess.PIPE,
                                            stderr=subprocess.STDOUT)))
    failed = []
    for src, p in procs:
        out, _ = p.communicate()
        text = "\n".join(l for l in out.decode(errors="replace").splitlines()
                         if "packed-fp32-ops" not in l)
        if p.returncode != 0:
            failed.append(src)
            sys.stderr.write(text + "\n")
        elif verbose and text.strip():
            print(text)
    if failed:
        raise RuntimeError(f"hipcc failed for {failed}")
    for lib, lib_objs in ((LIB, objs), (TIMING_LIB, timed_objs)):
        tmp = lib + ".tmp"
        subprocess.check_call([HIPCC, f"--offload-arch={ARCH}", "-shared",
                               "-fPIC", *lib_objs, "-o", tmp])
        os.replace(tmp, lib)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))

"""Build libmk.so (HIP, gfx950) and the seeded-input helper library in-tree.

Run as `python -m decode_persistent_megakernel_02_amd.build`; __graft_entry__.build()
calls `build_all()`.  Always recompiles.
"""
import hashlib
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libmk.so")
ARCH = os.environ.get("MK_OFFLOAD_ARCH", "gfx950")

# Packed-fp32 instructions are kept out of every device build.
HIP_FLAGS = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             "-Wall", "-Wno-unused-function", "-Wno-unused-variable"]


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)


def build_lib(verbose=False, out=LIB, defines=()):
    """Compile the kernels and the host library into `out`; `defines` are extra
    -D options (the MK_SHAPE_* tuning knobs) given to every compile."""
    hipcc = os.path.join(os.environ.get("ROCM_PATH", "/opt/rocm"), "bin", "hipcc")
    # (source, extra defines): the megakernel instances are split over three
    # compiles so that they build in parallel
    srcs = [("kernels.hip", ()), ("mega.hip", ("MK_MEGA_PART=0",)), ("mega.hip", ("MK_MEGA_PART=1",)),
            ("mega.hip", ("MK_MEGA_PART=2",)), ("batched.hip", ()), ("prefill.hip", ()), ("api.hip", ())]
    host = os.path.join(CSRC, "graph.cpp")
    inc = ["-I", CSRC, "-I", os.path.join(ROOT, "include")] + [f"-D{d}" for d in defines]
    bdir = os.path.join(PKG, "_build", hashlib.sha1(" ".join(defines).encode()).hexdigest()[:8]) if defines \
        else os.path.join(PKG, "_build")
    os.makedirs(bdir, exist_ok=True)
    jobs = []
    for name, extra in srcs:
        tag = "_".join(d.replace("=", "") for d in extra)
        obj = os.path.join(bdir, name + (("." + tag) if tag else "") + ".o")
        jobs.append([hipcc] + HIP_FLAGS + inc + [f"-D{d}" for d in extra] + ["-c", "-o", obj, os.path.join(CSRC, name)])
    objs = [j[-2] for j in jobs]
    workers = int(os.environ.get("MAX_JOBS", "0")) or min(len(jobs), os.cpu_count() or 1)
    with ThreadPoolExecutor(max_workers=workers) as ex:
        for f in [ex.submit(_run, j, verbose) for j in jobs]:
            f.result()
    obj = os.path.join(bdir, "graph.o")
    _run(["g++", "-O2", "-std=c++17", "-fPIC", "-Wall"] + inc + ["-c", "-o", obj, host], verbose)
    objs.append(obj)
    tmp = out + ".tmp"
    _run([hipcc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp] + objs + ["-lrocblas"], verbose)
    os.replace(tmp, out)
    return out


def build_synth(verbose=False):
    src = os.path.join(ROOT, "synth", "gen.c")
    out = os.path.join(ROOT, "synth", "libsynth.so")
    _run(["gcc", "-O2", "-fPIC", "-shared", "-ffp-contract=off", "-pthread", "-o", out, src], verbose)
    return out


def build_all(verbose=False):
    build_synth(verbose)
    build_lib(verbose)


if __name__ == "__main__":
    build_all(verbose="-q" not in sys.argv)

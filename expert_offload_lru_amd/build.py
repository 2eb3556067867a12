"""Build the in-tree native libraries.

* ``libmoe_offload.so``: the GPU library (HIP kernels for gfx950, host runtime,
  C ABI of include/moe_offload.h and include/moe_planner.h), built with hipcc.
* ``libmoe_planner.so``: the host slot table alone, built with g++ and no HIP,
  so the LRU planner can be exercised on a machine without a GPU.

Run ``python -m expert_offload_lru_amd.build``.
"""
import concurrent.futures as cf
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

LIB = os.path.join(PKG, "libmoe_offload.so")
PLANNER_LIB = os.path.join(PKG, "libmoe_planner.so")

HIP_SOURCES = ["expert_gemv.hip", "router.hip", "prefill.hip"]
HOST_SOURCES = ["runtime.cpp", "decode.cpp", "uploads.cpp", "file_tier.cpp", "graph.cpp", "prefill_host.cpp",
                "planner.cpp", "planner_capi.cpp", "errors.cpp"]
PLANNER_SOURCES = ["planner.cpp", "planner_capi.cpp", "errors.cpp"]

# device code: no packed fp32 instructions (-packed-fp32-ops); the host pass warns
# that it does not know the feature, which is harmless
HIP_FLAGS = ["--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC", "-I" + INCLUDE, "-I" + CSRC,
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", "-Wno-unused-command-line-argument", "-Wno-unused-value", "-Wno-unused-result"]


def _run(cmd):
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in r.stdout.splitlines() if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError("build failed: " + " ".join(cmd) + "\n" + out)
    return out


def _existing(names):
    return [n for n in names if os.path.exists(os.path.join(CSRC, n))]


def _stale(obj, src):
    """The object is missing or older than its source or any header it may include."""
    if not os.path.exists(obj):
        return True
    deps = [src] + [os.path.join(CSRC, n) for n in os.listdir(CSRC) if n.endswith((".hpp", ".h"))]
    deps += [os.path.join(INCLUDE, n) for n in os.listdir(INCLUDE)]
    return max(os.path.getmtime(d) for d in deps) > os.path.getmtime(obj)


def build(verbose=False, jobs=None, incremental=False):
    """Compile every source (or, with incremental=True, only those whose object is out of
    date) and link both libraries."""
    os.makedirs(BUILD, exist_ok=True)
    jobs = jobs or min(8, len(os.sched_getaffinity(0)))
    cmds, objs = [], []
    for name in _existing(HIP_SOURCES) + HOST_SOURCES:
        obj = os.path.join(BUILD, name + ".o")
        objs.append(obj)
        src = os.path.join(CSRC, name)
        if incremental and not _stale(obj, src):
            continue
        lang = [] if name.endswith(".hip") else ["-x", "hip"]
        cmds.append([HIPCC] + HIP_FLAGS + lang + ["-c", src, "-o", obj])
    with cf.ThreadPoolExecutor(jobs) as ex:
        for out in ex.map(_run, cmds):
            if verbose and out.strip():
                print(out)
    tmp = LIB + ".tmp"
    _run([HIPCC, "--offload-arch=" + ARCH, "-shared", "-fPIC", "-o", tmp] + objs)
    os.replace(tmp, LIB)
    tmp = PLANNER_LIB + ".tmp"
    _run(["g++", "-std=c++17", "-O2", "-fPIC", "-shared", "-Wall", "-I" + INCLUDE, "-I" + CSRC, "-o", tmp]
         + [os.path.join(CSRC, n) for n in PLANNER_SOURCES])
    os.replace(tmp, PLANNER_LIB)
    if verbose:
        print("built", LIB, "and", PLANNER_LIB)
    return LIB


if __name__ == "__main__":
    build(verbose="-v" in sys.argv, incremental="--incremental" in sys.argv)

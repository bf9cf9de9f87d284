"""Build libspec_verify.so and libspec_verify_debug.so (HIP for gfx950) in-tree.

    python -m long_context_tree_amd.build

Every source under csrc/ (HIP kernels in .hip files, host-only code in .cpp files) is compiled
with hipcc for gfx950 only, then linked into long_context_tree_amd/libspec_verify.so next to the
Python binding.  The SPEC_DEBUG library shares every object except the host layer and the
acceptance kernels, which are compiled again with SPEC_DEBUG defined.
"""

from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libspec_verify.so")
ARCH = "gfx950"


def _hipcc() -> str:
    for c in (os.path.join(os.environ.get("ROCM_PATH", "/opt/rocm"), "bin", "hipcc"), shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found (ROCm is required to build libspec_verify)")


FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-function",
    # no packed fp32 instructions anywhere in the device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


# extra flags per source file (none at present)
PER_FILE: dict = {}


# Sources compiled a second time with SPEC_DEBUG for libspec_verify_debug.so (the device-side
# precondition checks and the acceptance witnesses); every other object is shared by both libraries.
DEBUG_SRCS = ("api.hip", "accept.hip")
DEBUG_LIB = os.path.join(HERE, "libspec_verify_debug.so")


def build(verbose: bool = False) -> str:
    hipcc = _hipcc()
    os.makedirs(BUILD, exist_ok=True)
    srcs = sorted(f for f in os.listdir(CSRC) if f.endswith((".hip", ".cpp")))   # .cpp: host code only
    objs = [os.path.join(BUILD, os.path.splitext(s)[0] + ".o") for s in srcs]
    dbg_objs = {s: os.path.join(BUILD, os.path.splitext(s)[0] + ".debug.o") for s in DEBUG_SRCS}
    jobs = [(s, o, []) for s, o in zip(srcs, objs)] + [(s, o, ["-DSPEC_DEBUG=1"]) for s, o in dbg_objs.items()]

    def compile_one(job):
        src, obj, defs = job
        extra = PER_FILE.get(src, []) + defs
        cmd = [hipcc, *FLAGS, *extra, "-c", os.path.join(CSRC, src), "-o", obj]
        r = subprocess.run(cmd, capture_output=True, text=True)
        out = "\n".join(l for l in (r.stdout + r.stderr).splitlines()
                        if "packed-fp32-ops" not in l)
        if r.returncode != 0:
            raise RuntimeError(f"hipcc failed on {src}:\n{out}")
        return out

    # the attention source takes the longest: start it first
    jobs.sort(key=lambda j: j[0] != "tree_attention.hip")
    with cf.ThreadPoolExecutor(max_workers=min(8, len(jobs))) as ex:
        for (src, _, defs), log in zip(jobs, ex.map(compile_one, jobs)):
            if verbose and log.strip():
                print(f"[{src}{' (debug)' if defs else ''}]\n{log}", file=sys.stderr)
    release = objs
    debug = [dbg_objs.get(s, o) for s, o in zip(srcs, objs)]
    for lib_path, lib_objs in ((LIB, release), (DEBUG_LIB, debug)):
        tmp = lib_path + ".tmp"
        cmd = [hipcc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *lib_objs]
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError("link failed:\n" + r.stdout + r.stderr)
        os.replace(tmp, lib_path)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))

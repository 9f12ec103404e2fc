"""Build the HIP library libpa.so in-tree for gfx950.

    python paged_kv_cache_424_amd/build.py             # libpa.so
    python paged_kv_cache_424_amd/build.py --sanitize  # _build/sanitize/libpa.so

(run it as a script: importing the package first would load the old library)

Host-only C++ (allocator, layout) is compiled with g++; the HIP sources with
hipcc --offload-arch=gfx950.  Packed-fp32 instruction selection is turned off
for the device code (-packed-fp32-ops).  Always recompiles.

--sanitize builds a second copy of the library whose host-only C++ (the block
allocator, prefix cache and layout) is instrumented with AddressSanitizer and
UndefinedBehaviorSanitizer (g++; the HIP objects are the regular ones), for
CPU test runs: load it with PA_LIBRARY=<path> and LD_PRELOAD=<g++'s libasan>.
"""

import concurrent.futures
import glob
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libpa.so")
ARCH = "gfx950"

HIPCC_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]
CXX_FLAGS = ["-O2", "-std=c++17", "-fPIC", "-Wall", "-Wextra"]
SAN_FLAGS = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-g"]
SAN_LIB = os.path.join(BUILD, "sanitize", "libpa.so")


def _hipcc():
    for cand in ("/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def _run(cmd):
    res = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in res.stdout.splitlines() if "packed-fp32-ops" not in l)
    if res.returncode != 0:
        raise RuntimeError(f"command failed ({res.returncode}): {' '.join(cmd)}\n{out}")
    return out


def build(verbose=False):
    os.makedirs(BUILD, exist_ok=True)
    hipcc = _hipcc()
    jobs = []
    for src in sorted(glob.glob(os.path.join(CSRC, "*.cpp"))):
        obj = os.path.join(BUILD, os.path.basename(src) + ".o")
        jobs.append(["g++", *CXX_FLAGS, "-c", src, "-o", obj])
    for src in sorted(glob.glob(os.path.join(CSRC, "*.hip"))):
        obj = os.path.join(BUILD, os.path.basename(src) + ".o")
        jobs.append([hipcc, *HIPCC_FLAGS, "-c", src, "-o", obj])
    with concurrent.futures.ThreadPoolExecutor(max_workers=min(8, len(jobs))) as ex:
        for out in ex.map(_run, jobs):
            if verbose and out.strip():
                print(out)
    objs = [j[-1] for j in jobs]
    tmp = LIB + ".tmp"
    _run([hipcc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs])
    os.replace(tmp, LIB)
    return LIB


def build_sanitized():
    """The library with ASan/UBSan-instrumented host C++ (see the module doc).
    Reuses the regular build's HIP objects, building them first if missing."""
    hip_objs = [os.path.join(BUILD, os.path.basename(src) + ".o")
                for src in sorted(glob.glob(os.path.join(CSRC, "*.hip")))]
    if not all(os.path.exists(o) for o in hip_objs):
        build()
    out_dir = os.path.dirname(SAN_LIB)
    os.makedirs(out_dir, exist_ok=True)
    objs = []
    for src in sorted(glob.glob(os.path.join(CSRC, "*.cpp"))):
        obj = os.path.join(out_dir, os.path.basename(src) + ".o")
        _run(["g++", "-O1", "-std=c++17", "-fPIC", *SAN_FLAGS, "-c", src, "-o", obj])
        objs.append(obj)
    tmp = SAN_LIB + ".tmp"
    _run(["g++", "-shared", *SAN_FLAGS, "-o", tmp, *objs, *hip_objs, "-L/opt/rocm/lib", "-lamdhip64"])
    os.replace(tmp, SAN_LIB)
    return SAN_LIB


if __name__ == "__main__":
    if "--sanitize" in sys.argv:
        print(build_sanitized())
    else:
        print(build(verbose="-v" in sys.argv))

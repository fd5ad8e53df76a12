"""Builds libfp8ds.so (the HIP kernels and their C ABI) in-tree for gfx950.

Every source in csrc/ is compiled with hipcc to an object file in parallel,
then linked into delayed_scaling_amd/libfp8ds.so.  Flags: -O3, no fast-math
(IEEE division and fp32 denormals are part of the method's arithmetic), and
packed-fp32 instruction selection switched off.
"""
import concurrent.futures
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libfp8ds.so")
BUILD_DIR = os.path.join(PKG, "_build")
ARCH = "gfx950"


def hipcc():
    path = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(path):
        raise RuntimeError("hipcc not found; the HIP library cannot be built")
    return path


def common_flags():
    return [f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-I", os.path.join(ROOT, "include"), "-I", CSRC]


def _compile(src, obj, extra):
    cmd = [hipcc(), *common_flags(), *extra, "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {os.path.basename(src)}:\n{r.stdout}\n{r.stderr}")
    return obj


def build(verbose=False, extra_flags=()):
    """Compile every csrc/*.hip and link libfp8ds.so.  Returns the library path."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    srcs = sorted(f for f in os.listdir(CSRC) if f.endswith(".hip"))
    jobs = min(len(srcs), int(os.environ.get("MAX_JOBS", "8")))
    with concurrent.futures.ThreadPoolExecutor(max_workers=max(jobs, 1)) as ex:
        futs = [ex.submit(_compile, os.path.join(CSRC, s), os.path.join(BUILD_DIR, s + ".o"), list(extra_flags))
                for s in srcs]
        objs = [f.result() for f in futs]
    tmp = LIB + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


if __name__ == "__main__":
    build(verbose=True, extra_flags=sys.argv[1:])

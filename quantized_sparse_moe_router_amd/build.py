"""Build libmoe_mi355x.so (all HIP kernels + the C entry points) for gfx950 with hipcc."""
import concurrent.futures
import glob
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libmoe_mi355x.so")
PEAKS_SRC = os.path.join(PKG, "peaks", "peaks.hip")
PEAKS_LIB = os.path.join(PKG, "libmoe_peaks.so")   # bench.py's measurement helpers
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

# -packed-fp32-ops: keep the compiler from emitting packed fp32 add/mul/fma.
FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-Wall",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-I" + INCLUDE, "-I" + CSRC]


def _compile(src):
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    cmd = [HIPCC, *FLAGS, "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    msgs = "\n".join(ln for ln in (r.stdout + r.stderr).splitlines()
                     if "unknown target feature" not in ln and "packed-fp32-ops" not in ln
                     and ln.strip() and not ln.startswith("1 warning"))
    if r.returncode != 0:
        raise RuntimeError("hipcc failed for %s:\n%s" % (src, msgs))
    return obj, msgs


def build(verbose=False):
    os.makedirs(BUILD, exist_ok=True)
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    with concurrent.futures.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        results = list(ex.map(_compile, srcs))
    if verbose:
        for _, m in results:
            if m:
                print(m, file=sys.stderr)
    tmp = LIB + ".tmp%d" % os.getpid()
    subprocess.check_call([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp,
                           *[o for o, _ in results]])
    os.replace(tmp, LIB)
    tmp = PEAKS_LIB + ".tmp%d" % os.getpid()
    subprocess.check_call([HIPCC, *FLAGS, "-shared", "-o", tmp, PEAKS_SRC],
                          stderr=subprocess.DEVNULL)
    os.replace(tmp, PEAKS_LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))

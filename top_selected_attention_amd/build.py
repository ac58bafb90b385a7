"""Builds the HIP library (libtsa.so) for gfx950 with hipcc, in-tree, and
beside it the measured-peaks library (peaks/libtsa_peaks.so).

Usage: python top_selected_attention_amd/build.py  (or build() from Python; running it as
a file does not import the package, which needs the library to exist).
Every call recompiles every source.
"""

import concurrent.futures
import glob
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(os.path.dirname(HERE), "include")
BUILD_DIR = os.path.join(HERE, "_build")
LIB_NAME = "libtsa.so"
LIB_PATH = os.path.join(HERE, LIB_NAME)
PEAKS_SRC = os.path.join(HERE, "peaks", "peaks.hip")
PEAKS_LIB = os.path.join(HERE, "peaks", "libtsa_peaks.so")

ARCH = "gfx950"
COMMON = [
    "-O3", "-std=c++17", "-fPIC", "-fvisibility=hidden",
    f"--offload-arch={ARCH}",
    # packed fp32 VALU forms stay off: the compiler's own float code only
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # MFMA accumulators in VGPRs: the kernels touch them with VALU (softmax,
    # scaling), and AGPR-resident accumulators cost a move per element
    "-mllvm", "-amdgpu-mfma-vgpr-form",
    "-I", CSRC, "-I", INCLUDE,
]


def _hipcc():
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    exe = os.path.join(rocm, "bin", "hipcc")
    return exe if os.path.exists(exe) else shutil.which("hipcc")


def _compile(src, obj):
    cmd = [_hipcc(), *COMMON, "-x", "hip", "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{r.stderr}")
    return obj


def build(verbose=True):
    """Compile every source under csrc/ and link libtsa.so next to this file."""
    if _hipcc() is None:
        raise RuntimeError("hipcc not found (set ROCM_PATH)")
    os.makedirs(BUILD_DIR, exist_ok=True)
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")) + glob.glob(os.path.join(CSRC, "*.cpp")))
    jobs = min(len(srcs), int(os.environ.get("MAX_JOBS", os.cpu_count() or 4)), 16)
    objs = []
    with concurrent.futures.ThreadPoolExecutor(max_workers=max(1, jobs)) as ex:
        futs = [ex.submit(_compile, s, os.path.join(BUILD_DIR, os.path.basename(s) + ".o"))
                for s in srcs]
        pfut = ex.submit(_compile, PEAKS_SRC, os.path.join(BUILD_DIR, "peaks.hip.o"))
        for f in futs:
            objs.append(f.result())
        pobj = pfut.result()
    _link(objs, LIB_PATH)
    _link([pobj], PEAKS_LIB)
    if verbose:
        print(f"built {LIB_PATH} from {len(srcs)} sources, and {PEAKS_LIB}")
    return LIB_PATH


def _link(objs, out):
    tmp = out + ".tmp"
    cmd = [_hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link of {os.path.basename(out)} failed:\n{r.stderr}")
    os.replace(tmp, out)


if __name__ == "__main__":
    build()
    sys.exit(0)

"""Build libattn.so (the HIP kernels and the C ABI) for gfx950, in-tree.

Usage: ``python -m attention_pluggable_normalizers_amd.build`` or ``build()``.
Each ``csrc/*.hip`` file is compiled by hipcc to an object, then linked into
``attention_pluggable_normalizers_amd/libattn.so``.
"""

import concurrent.futures
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libattn.so")
ARCH = "gfx950"

# Packed-FP32 VALU forms are disabled for all device code; hipcc -O3 would
# otherwise emit them from ordinary float code.
DEVICE_FLAGS = ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
COMMON = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-I", INCLUDE, "-I", CSRC,
          "-Wall", "-Wno-unused-function"]
# The forward kernels keep matrix-product accumulators in VGPRs: at head dim
# 256 the compiler's AGPR form would move the O accumulators between the two
# register files at every key tile and need more than the 256 registers that
# two waves per SIMD allow.  On finite inputs their device code never makes a
# NaN (the API rejects non-finite scaling and softcap; masked scores are -inf,
# and cache slots past a sequence read as zeros), so it is compiled without
# NaN semantics: a max then needs no canonicalizing instruction per operand
# that is not known to be canonical.  (Inputs holding NaN give undefined
# outputs either way.)  Host code keeps full IEEE semantics.
PER_FILE = {"prefill.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=1", "-Xarch_device", "-fno-honor-nans"]}


def _hipcc():
    h = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(h):
        raise RuntimeError("hipcc not found; the HIP toolchain is required to build libattn")
    return h


def _compile(src, verbose):
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    cmd = [_hipcc(), *COMMON, *DEVICE_FLAGS, *PER_FILE.get(os.path.basename(src), []), "-c", src, "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{r.stdout}\n{r.stderr}")
    return obj


def build(verbose=False, jobs=None):
    """Compile every csrc/*.hip and link libattn.so; returns the library path."""
    os.makedirs(BUILD, exist_ok=True)
    srcs = sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".hip"))
    jobs = jobs or min(len(srcs), 8)
    with concurrent.futures.ThreadPoolExecutor(jobs) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose), srcs))
    tmp = LIB + ".tmp"
    cmd = [_hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs,
           "-Wl,-soname,libattn.so"]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))

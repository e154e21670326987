"""Build the HIP conv2d library (libconv2d_nhwc.so) for gfx950, in-tree.

    python -m convolution_nhwc_implicit_amd.build

Every source under csrc/ is compiled by hipcc for --offload-arch=gfx950 and
linked into one shared library next to this file.  Packed fp32 instructions
are disabled for all device code.
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
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libconv2d_nhwc.so")
ARCH = "gfx950"

SOURCES = ["api.cpp", "igemm.hip", "band.hip", "wino.hip", "wgrad.hip", "wgrad_band.hip", "direct.hip", "repack.hip", "fewchan.hip", "fewchan_wgrad.hip", "fewchan_dgrad.hip", "pointwise.hip", "pointwise_wgrad.hip", "patch.hip"]

COMMON_FLAGS = [
    "-x", "hip", f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    "-Wall", "-Wno-unused-function",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    f"-I{INCLUDE}", f"-I{CSRC}",
]


def hipcc():
    path = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(path):
        raise RuntimeError("hipcc not found: the HIP toolchain is required to build the library")
    return path


def _compile(src, extra):
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [hipcc()] + COMMON_FLAGS + list(extra) + ["-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    msg = "\n".join(l for l in (r.stdout + r.stderr).splitlines() if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{msg}")
    return obj, msg


def build(verbose=False, extra_flags=()):
    """Compile all sources and link libconv2d_nhwc.so.  Always rebuilds."""
    os.makedirs(BUILD, exist_ok=True)
    with concurrent.futures.ThreadPoolExecutor(max_workers=min(8, len(SOURCES))) as ex:
        results = list(ex.map(lambda s: _compile(s, extra_flags), SOURCES))
    for obj, msg in results:
        if verbose and msg.strip():
            print(msg, file=sys.stderr)
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp] + [o for o, _ in results]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n" + r.stdout + r.stderr)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))

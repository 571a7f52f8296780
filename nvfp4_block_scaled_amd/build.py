"""Build libnvfp4.so (the HIP kernels and the C ABI) for gfx950 with hipcc.

Every HIP source is compiled for gfx950 only.  Packed-float32 VALU
instructions are disabled in device code (-packed-fp32-ops); the encode and
decode steps additionally turn off floating-point contraction in the source.
"""
import concurrent.futures as cf
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
ROOT = os.path.dirname(HERE)
LIB = os.path.join(HERE, "libnvfp4.so")
# the benchmark's measurement kernels, a library of their own
CEILING_LIB = os.path.join(HERE, "libnvfp4_ceiling.so")
CEILING_SOURCES = ["ceiling.hip"]
BUILD_DIR = os.path.join(ROOT, "_build")
SOURCES = ["codec.hip", "qmv.hip", "qmv_packed.hip", "gemm.hip", "smallm.hip", "mx_codec.hip", "mx_gemm.hip", "mx_qmv.hip", "gather_ex.hip", "capi.hip"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

COMMON = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-Wall",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"), "-I", CSRC,
]


def _compile(src, verbose):
    obj = os.path.join(BUILD_DIR, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC] + COMMON + ["-c", os.path.join(CSRC, src), "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stdout}\n{r.stderr}")
    return obj


def _link(objs, lib, verbose):
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", lib + ".tmp"] + objs
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(lib + ".tmp", lib)


def build(verbose=False):
    os.makedirs(BUILD_DIR, exist_ok=True)
    srcs = SOURCES + CEILING_SOURCES
    with cf.ThreadPoolExecutor(max_workers=min(4, len(srcs))) as ex:
        objs = dict(zip(srcs, ex.map(lambda s: _compile(s, verbose), srcs)))
    _link([objs[s] for s in SOURCES], LIB, verbose)
    _link([objs[s] for s in CEILING_SOURCES], CEILING_LIB, verbose)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))

"""Build the DFlash head's native libraries in-tree.

* ``libdflash.so``      - the HIP library for gfx950 (all kernels + C ABI);
* ``libdflash_host.so`` - the HIP-free host core alone (g++), for CPU tests.

Run ``python -m block_diffusion_draft_03_amd.build`` (or call ``build()``).
Every call recompiles; objects go to ``_build/`` next to the sources.
"""
import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libdflash.so")
HOST_LIB = os.path.join(PKG, "libdflash_host.so")

HIP_SOURCES = ["k_gemm.hip", "k_bgemm.hip", "k_attn.hip", "k_misc.hip", "dflash.cpp", "host_core.cpp"]
HIPCC_FLAGS = ["--offload-arch=gfx950", "-O3", "-fPIC", "-std=c++17",
               # packed fp32 ops are kept out of generated code
               "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
               "-Wno-unused-result"]
# Per-file flags. The tiled GEMM keeps its MFMA accumulators in ordinary VGPRs:
# with accumulation registers the allocator rotates them every K stage.
EXTRA_FLAGS = {"k_bgemm.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=1"]}


def _hipcc():
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found")


def _run(cmd):
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    if r.returncode != 0:
        raise RuntimeError("command failed:\n" + " ".join(cmd) + "\n" + r.stdout)
    return r.stdout


def build_host_lib():
    os.makedirs(BUILD, exist_ok=True)
    tmp = HOST_LIB + ".tmp"
    _run(["g++", "-O2", "-fPIC", "-shared", "-std=c++17", "-Wall",
          os.path.join(CSRC, "host_core.cpp"), os.path.join(CSRC, "host_capi.cpp"), "-o", tmp])
    os.replace(tmp, HOST_LIB)
    return HOST_LIB


def build_hip_lib(jobs=None):
    os.makedirs(BUILD, exist_ok=True)
    hipcc = _hipcc()
    jobs = jobs or min(8, len(HIP_SOURCES))

    def compile_one(src):
        obj = os.path.join(BUILD, src + ".o")
        _run([hipcc, *HIPCC_FLAGS, *EXTRA_FLAGS.get(src, []), "-x", "hip", "-c", os.path.join(CSRC, src), "-o", obj])
        return obj

    with ThreadPoolExecutor(jobs) as ex:
        objs = list(ex.map(compile_one, HIP_SOURCES))
    tmp = LIB + ".tmp"
    _run([hipcc, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp])
    os.replace(tmp, LIB)
    return LIB


def build():
    build_host_lib()
    build_hip_lib()


if __name__ == "__main__":
    build()
    print("built", LIB, HOST_LIB, file=sys.stderr)

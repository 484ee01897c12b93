"""Build libmtla.so (HIP kernels + C ABI) for gfx950, in-tree.

    python temporally_compressed_latent_amd/build.py

Each source compiles to its own object (in parallel), then hipcc links the
shared library next to this file.  Packed-fp32 instruction forms are disabled
for every HIP translation unit.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
OUT = os.path.join(PKG, "libmtla.so")
BUILD_DIR = os.path.join(ROOT, "_build")
ARCH = "gfx950"

SOURCES = ["capi.hip", "merge.hip", "decode.hip", "prefill.hip", "layer.hip", "backward.hip", "calib.hip"]

HIPCC_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
    "-I", os.path.join(ROOT, "include"),
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libmtla.so)")


# Per-file additions.  prefill.hip: the attention's softmax takes maxima of
# raw MFMA results; without NaN semantics (no input here is NaN) fmaxf needs
# no canonicalising move per value and pairs into v_max3_f32.
FILE_FLAGS = {"prefill.hip": ["-fno-honor-nans"],
              # the decode-step kernels' leading scalar arguments go straight
              # into scalar registers at launch
              "decode.hip": ["-mllvm", "-amdgpu-kernarg-preload-count=8"],
              "layer.hip": ["-mllvm", "-amdgpu-kernarg-preload-count=7"]}


def _compile(src: str, verbose: bool) -> str:
    obj = os.path.join(BUILD_DIR, os.path.splitext(src)[0] + ".o")
    cmd = [hipcc(), *HIPCC_FLAGS, *FILE_FLAGS.get(src, []), "-c", os.path.join(CSRC, src), "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{r.stdout}\n{r.stderr}")
    if verbose and r.stderr.strip():
        print(r.stderr, file=sys.stderr)
    return obj


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD_DIR, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=min(len(SOURCES), os.cpu_count() or 1)) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose), SOURCES))
    tmp = OUT + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, OUT)
    return OUT


# Host-side AddressSanitizer build of the same sources: the C-ABI shim's
# argument checks, workspace sizing and dispatch run instrumented (device code
# is built as usual).  Used by tests/test_capi_asan.py with the ASan runtime
# preloaded.
ASAN_DIR = os.path.join(BUILD_DIR, "asan")
ASAN_OUT = os.path.join(ASAN_DIR, "libmtla_asan.so")
ASAN_FLAGS = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fno-omit-frame-pointer", "-g"]


def asan_runtime() -> str:
    """The clang ASan runtime matching hipcc's compiler."""
    import glob
    root = os.path.dirname(os.path.dirname(os.path.realpath(hipcc())))
    for cand in sorted(glob.glob(os.path.join(root, "lib", "llvm", "lib", "clang", "*", "lib", "linux",
                                              "libclang_rt.asan-x86_64.so"))
                       + sorted(glob.glob("/opt/rocm/lib/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))):
        return cand
    raise RuntimeError("libclang_rt.asan-x86_64.so not found next to hipcc")


def build_host_asan(verbose: bool = False) -> str:
    os.makedirs(ASAN_DIR, exist_ok=True)

    def comp(src):
        obj = os.path.join(ASAN_DIR, os.path.splitext(src)[0] + ".o")
        cmd = [hipcc(), *HIPCC_FLAGS, *FILE_FLAGS.get(src, []), *ASAN_FLAGS, "-c", os.path.join(CSRC, src), "-o", obj]
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"hipcc (host ASan) failed on {src}:\n{r.stdout}\n{r.stderr}")
        return obj
    with cf.ThreadPoolExecutor(max_workers=min(len(SOURCES), os.cpu_count() or 1)) as ex:
        objs = list(ex.map(comp, SOURCES))
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-Xarch_host", "-fsanitize=address",
           "-shared-libsan", "-o", ASAN_OUT, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link (host ASan) failed:\n{r.stdout}\n{r.stderr}")
    return ASAN_OUT


if __name__ == "__main__":
    if "asan" in sys.argv:
        print(build_host_asan(verbose="-v" in sys.argv))
    else:
        print(build(verbose="-v" in sys.argv))

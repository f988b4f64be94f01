"""Builds liboctopus.so (the C-ABI library and its gfx950 kernels) in-tree.

    python -m quantized_decode_attention_octo_amd.build

Every source under csrc/ is compiled with hipcc for gfx950 into _build/ and
linked into quantized_decode_attention_octo_amd/liboctopus.so.  The device
code is compiled without packed-FP32 instructions.

    python -m quantized_decode_attention_octo_amd.build --sanitize

builds liboctopus_san.so (objects in _build_san/) whose host code carries
AddressSanitizer and UndefinedBehaviorSanitizer checks (the device code is
built as usual).  It is loaded with the sanitizer runtime preloaded
(sanitizer_runtime()) and OCTO_LIB naming it, which is how
tests/test_sanitized_abi.py runs the ABI checks.
"""
import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "liboctopus.so")
BUILD_SAN = os.path.join(ROOT, "_build_san")
LIB_SAN = os.path.join(PKG, "liboctopus_san.so")
SOURCES = ["api.cpp", "encode.hip", "decode.hip", "chunk.hip", "reconstruct.hip"]
ARCH = "gfx950"


def hipcc():
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: the OCTOPUS library needs ROCm's hipcc")


def common_flags():
    return [f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall",
            "-Wno-unused-result", f"-I{INCLUDE}", f"-I{CSRC}"]


def device_flags():
    # Keep the device compiler from forming packed FP32 instructions.
    return ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


# The chunk kernels never produce or test a NaN (masked scores are -inf), so
# their maxima need not canonicalize NaN inputs.
FILE_FLAGS = {"chunk.hip": ["-fno-honor-nans"]}


def sanitizer_flags():
    # host compilation only (each flag behind -Xarch_host)
    flags = []
    for f in ("-fsanitize=address", "-fsanitize=undefined", "-fno-sanitize-recover=undefined",
              "-fno-omit-frame-pointer"):
        flags += ["-Xarch_host", f]
    return flags


def sanitizer_runtime():
    """The ASan runtime (with UBSan's handlers) of the hipcc toolchain, to be
    preloaded into a process that loads the sanitized library."""
    r = subprocess.run([hipcc(), "-print-file-name=libclang_rt.asan-x86_64.so"],
                       capture_output=True, text=True)
    path = r.stdout.strip()
    if r.returncode == 0 and os.path.isabs(path) and os.path.exists(path):
        return path
    raise RuntimeError("the ASan runtime of the hipcc toolchain was not found")


def compile_one(src, verbose=False, sanitize=False):
    obj = os.path.join(BUILD_SAN if sanitize else BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [hipcc()] + common_flags() + ["-c", os.path.join(CSRC, src), "-o", obj]
    if src.endswith(".hip"):
        cmd += device_flags()
    cmd += FILE_FLAGS.get(src, [])
    if sanitize:
        cmd += sanitizer_flags()
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{r.stdout}\n{r.stderr}")
    return obj


def build(verbose=False, jobs=None, sanitize=False):
    """Compiles every source and links the shared library; returns its path."""
    os.makedirs(BUILD_SAN if sanitize else BUILD, exist_ok=True)
    jobs = jobs or min(len(SOURCES), os.cpu_count() or 1, 8)
    with ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(lambda s: compile_one(s, verbose, sanitize), SOURCES))
    lib = LIB_SAN if sanitize else LIB
    tmp = lib + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp] + objs
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, lib)
    return lib


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv, sanitize="--sanitize" in sys.argv))

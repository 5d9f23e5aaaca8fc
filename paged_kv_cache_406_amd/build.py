"""Builds libpagedkv.so (host block tables + gfx950 HIP kernels) in-tree.

    python paged_kv_cache_406_amd/build.py                    # the library
    python paged_kv_cache_406_amd/build.py --host-sanitized   # host part under ASan + UBSan

The host part is compiled with g++, the kernels with hipcc for gfx950, and
both are linked by hipcc into ``paged_kv_cache_406_amd/libpagedkv.so``.
Packed fp32 VALU instructions are disabled for all device code.
"""
import os
import shutil
import subprocess
import sys
import tempfile

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libpagedkv.so")
ARCH = "gfx950"

HIP_FLAGS = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
HOST_FLAGS = ["-O2", "-std=c++17", "-fPIC", "-Wall", "-Wextra"]


def _hipcc():
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (set HIPCC)")


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"command failed ({res.returncode}): {' '.join(cmd)}\n{res.stdout}\n{res.stderr}")
    return res


def build(verbose: bool = False) -> str:
    hipcc = _hipcc()
    with tempfile.TemporaryDirectory(prefix="pkv_build_") as tmp:
        host_objs = []
        for src in ("pool.cpp", "prefix_cache.cpp"):
            obj = os.path.join(tmp, src.replace(".cpp", ".o"))
            _run(["g++", *HOST_FLAGS, "-I", INCLUDE, "-c", os.path.join(CSRC, src), "-o", obj], verbose)
            host_objs.append(obj)
        dev_o = os.path.join(tmp, "kernels.o")
        _run([hipcc, *HIP_FLAGS, "-I", INCLUDE, "-c", os.path.join(CSRC, "kernels.hip"),
              "-o", dev_o], verbose)
        tmp_lib = os.path.join(tmp, "libpagedkv.so")
        _run([hipcc, *HIP_FLAGS, "-shared", *host_objs, dev_o, "-o", tmp_lib], verbose)
        shutil.copyfile(tmp_lib, LIB + ".tmp")
        os.replace(LIB + ".tmp", LIB)
    return LIB


SANITIZED_LIB = os.path.join(ROOT, "_build", "libpagedkv_host_asan.so")
SANITIZE_FLAGS = ["-O1", "-g", "-fno-omit-frame-pointer", "-std=c++17", "-fPIC", "-Wall", "-Wextra",
                  "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined"]


def build_host_sanitized(verbose: bool = False) -> str:
    """The host part alone (block tables, prefix cache) built with g++ under
    AddressSanitizer and UndefinedBehaviorSanitizer, for CPU tests: load it
    with PKV_LIBRARY=<path> and the sanitizer runtime preloaded
    (LD_PRELOAD=$(g++ -print-file-name=libasan.so)).  It has no device code."""
    os.makedirs(os.path.dirname(SANITIZED_LIB), exist_ok=True)
    tmp_lib = SANITIZED_LIB + ".tmp"
    _run(["g++", *SANITIZE_FLAGS, "-I", INCLUDE, "-shared", os.path.join(CSRC, "pool.cpp"),
          os.path.join(CSRC, "prefix_cache.cpp"), "-o", tmp_lib], verbose)
    os.replace(tmp_lib, SANITIZED_LIB)
    return SANITIZED_LIB


if __name__ == "__main__":
    if "--host-sanitized" in sys.argv:
        print(build_host_sanitized(verbose="-v" in sys.argv))
    else:
        print(build(verbose="-v" in sys.argv))

"""Build libssm.so (the C ABI of include/ssm.h) from csrc/*.hip for gfx950 with hipcc."""
from __future__ import annotations

import glob
import os
import subprocess
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libssm.so")
BUILD_DIR = os.path.join(ROOT, "_build")
ARCH = "gfx950"

# -packed-fp32-ops: keep the compiler from forming packed FP32 (v_pk_*_f32) instructions.
HIP_FLAGS = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-Wall",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             "-I", os.path.join(ROOT, "include")]


# hipBLASLt runs the projection GEMMs (csrc/ssm_proj.hip).
LINK_LIBS = ["-L/opt/rocm/lib", "-lhipblaslt", "-Wl,-rpath,/opt/rocm/lib"]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    return "hipcc"


def sources():
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")))


# The sanitizer variant (libssm_san.so, loaded when SSM_SANITIZE=1): host code instrumented with
# AddressSanitizer and UndefinedBehaviorSanitizer, device code unchanged; linked with clang++
# against the shared clang sanitizer runtime, which the process preloads (the oracle's sanitizer
# build uses the same runtime).  For CPU-only test runs of the host-side validation.
SAN_LIB = os.path.join(PKG, "libssm_san.so")
SAN_BUILD_DIR = os.path.join(ROOT, "_build", "san")
SAN_HOST_FLAGS = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                  "-Xarch_host", "-fno-omit-frame-pointer", "-Xarch_host", "-g"]
CLANGXX = "/opt/rocm/llvm/bin/clang++"


def build(verbose: bool = False, jobs: int = 8, sanitize: bool = False) -> str:
    build_dir = SAN_BUILD_DIR if sanitize else BUILD_DIR
    os.makedirs(build_dir, exist_ok=True)
    cc = hipcc()
    extra = SAN_HOST_FLAGS if sanitize else []

    def compile_one(src):
        obj = os.path.join(build_dir, os.path.basename(src) + ".o")
        cmd = [cc, *HIP_FLAGS, *extra, "-c", src, "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        r = subprocess.run(cmd, capture_output=True, text=True)
        # the host pass does not know the packed-fp32 target feature; that warning is harmless
        noise = "is not a recognized feature for this target"
        err = "\n".join(l for l in r.stderr.splitlines() if noise not in l)
        if r.returncode != 0:
            raise RuntimeError(f"hipcc failed on {src}:\n{err}")
        if err.strip() and verbose:
            print(err)
        return obj

    with ThreadPoolExecutor(max_workers=max(1, jobs)) as ex:
        objs = list(ex.map(compile_one, sources()))
    out = SAN_LIB if sanitize else LIB
    tmp = out + ".tmp"
    if sanitize:
        san = "-fsanitize=address,undefined"
        cmd = [CLANGXX, "-shared", "-fPIC", san, "-shared-libsan", "-o", tmp, *objs, "-L/opt/rocm/lib",
               "-lamdhip64", *LINK_LIBS]
    else:
        cmd = [cc, "-shared", "-fPIC", f"--offload-arch={ARCH}", "-o", tmp, *objs, *LINK_LIBS]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True, capture_output=not verbose)
    os.replace(tmp, out)
    return out


def sanitizer_runtime() -> str:
    """The clang AddressSanitizer runtime a sanitized test run preloads."""
    found = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    if not found:
        raise FileNotFoundError("clang's libclang_rt.asan-x86_64.so not found under /opt/rocm/llvm")
    return found[-1]


if __name__ == "__main__":
    import sys

    san = "--sanitize" in sys.argv
    print(build(verbose=True, sanitize=san))
    if san:
        print(f"run the CPU tests with: SSM_SANITIZE=1 ASAN_OPTIONS=detect_leaks=0 LD_PRELOAD={sanitizer_runtime()} "
              "python -m pytest tests -m 'not gpu'")

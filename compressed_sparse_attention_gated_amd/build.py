"""Build libcsa2.so (HIP kernels for gfx950 + the C-ABI host layer) in the package directory.

    python -m compressed_sparse_attention_gated_amd.build [-v] [--sanitize]

Every HIP translation unit is compiled with hipcc for gfx950 only; packed-fp32 VALU
instructions are disabled at the code-generation level.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libcsa2.so")
BUILD_DIR = os.path.join(os.path.dirname(PKG), "_build")

SOURCES = ["api.cpp", "compress.hip", "index.hip", "topk.hip", "attn.hip", "proj.hip"]
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libcsa2)")


COMMON_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-function",
    "-Wno-unused-variable", "-Wno-unused-lambda-capture", "-fvisibility=hidden",
    # no packed fp32 VALU instructions in device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


# Per-source code-generation options.  The indexer scan reads its MFMA accumulators with
# ordinary VALU instructions in the epilogue; the VGPR form of the MFMA writes them where
# those instructions read, instead of to accumulation registers that need a copy each.
SOURCE_FLAGS = {
    "index.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
}


def _compile(src: str, verbose: bool) -> str:
    obj = os.path.join(BUILD_DIR, os.path.basename(src) + ".o")
    cmd = [hipcc(), *COMMON_FLAGS, *SOURCE_FLAGS.get(src, []), "-c", os.path.join(CSRC, src), "-o", obj]
    if src.endswith(".cpp"):
        cmd.insert(1, "-x")
        cmd.insert(2, "hip")
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    err = "\n".join(l for l in r.stderr.splitlines() if "packed-fp32-ops" not in l and "unknown target feature" not in l
                    and l.strip())
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {src}\n{r.stderr}")
    if verbose and err:
        print(err)
    return obj


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD_DIR, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=min(len(SOURCES), os.cpu_count() or 4)) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose), SOURCES))
    tmp = LIB + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed\n{r.stderr}")
    os.replace(tmp, LIB)
    return LIB


# AddressSanitizer + UndefinedBehaviorSanitizer build of the host layer (api.cpp) for the
# CPU checks of the C ABI: only host code is instrumented (every sanitizer flag goes to the
# host pass alone); the kernels are the ordinary objects.  The library needs the ASan runtime
# preloaded into the process that loads it (sanitizer_runtime()).
SANITIZE_DIR = os.path.join(BUILD_DIR, "sanitize")
SANITIZE_LIB = os.path.join(SANITIZE_DIR, "libcsa2.so")
SANITIZE_HOST = "-Xarch_host -fsanitize=address -Xarch_host -fsanitize=undefined".split()
SANITIZE_FLAGS = SANITIZE_HOST + ["-fno-omit-frame-pointer", "-g"]


def sanitizer_runtime() -> str | None:
    """The clang ASan runtime of this toolchain (it also carries the UBSan handlers)."""
    import glob

    hits = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    return hits[-1] if hits else None


def build_sanitized(verbose: bool = False) -> str:
    objs = [os.path.join(BUILD_DIR, s + ".o") for s in SOURCES if s != "api.cpp"]
    if not all(os.path.exists(o) for o in objs):
        build(verbose)
    os.makedirs(SANITIZE_DIR, exist_ok=True)
    api_obj = os.path.join(SANITIZE_DIR, "api.cpp.o")
    cmd = [hipcc(), "-x", "hip", *COMMON_FLAGS, *SANITIZE_FLAGS, "-c", os.path.join(CSRC, "api.cpp"), "-o", api_obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: api.cpp (sanitized)\n{r.stderr}")
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *SANITIZE_HOST, "-shared-libsan", "-o", SANITIZE_LIB,
           api_obj, *objs]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed (sanitized)\n{r.stderr}")
    return SANITIZE_LIB


if __name__ == "__main__":
    if "--sanitize" in sys.argv:
        print(build_sanitized(verbose="-v" in sys.argv))
    else:
        print(build(verbose="-v" in sys.argv))

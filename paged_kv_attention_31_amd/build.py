"""Build libpagedattn.so in-tree with hipcc for gfx950.

    python -m paged_kv_attention_31_amd.build        # or: python paged_kv_attention_31_amd/build.py

Every HIP source is compiled with packed fp32 instructions disabled
(``-Xclang -target-feature -Xclang -packed-fp32-ops``); hipcc's host pass warns that it
does not know that feature, which is harmless.
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
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB_NAME = "libpagedattn.so"
LIB_PATH = os.path.join(PKG, LIB_NAME)
SOURCES = ["abi.cpp", "sched.cpp", "append.hip", "decode.hip", "prefill.hip", "norm.hip"]
ARCH = "gfx950"


def _hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libpagedattn)")


def _flags() -> list[str]:
    return [
        f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        "-Wno-unused-command-line-argument",
        "-I", INCLUDE, "-I", CSRC,
    ]


def build(verbose: bool = False) -> str:
    """Compile every source and link the shared library; returns its path."""
    hipcc = _hipcc()
    os.makedirs(BUILD, exist_ok=True)

    def compile_one(src: str) -> str:
        obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
        lang = ["-x", "hip"] if src.endswith(".hip") else []
        cmd = [hipcc, *_flags(), *lang, "-c", os.path.join(CSRC, src), "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"hipcc failed on {src}:\n{r.stdout}\n{r.stderr}")
        noise = [ln for ln in r.stderr.splitlines() if "packed-fp32-ops" not in ln and ln.strip()]
        if verbose and noise:
            print("\n".join(noise), file=sys.stderr)
        return obj

    with cf.ThreadPoolExecutor(min(4, len(SOURCES))) as ex:
        objs = list(ex.map(compile_one, SOURCES))
    tmp = LIB_PATH + ".tmp"
    cmd = [hipcc, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


# Host-side sanitizer build: the host bookkeeping (C ABI validation, page pool, scheduler)
# under AddressSanitizer and UndefinedBehaviorSanitizer.  Only the two host sources are
# instrumented (the flags go to the host pass alone); the kernels' objects are the regular
# ones.  The result loads only into a process that preloads the ASan runtime.
ASAN_BUILD = os.path.join(BUILD, "asan")
ASAN_LIB_PATH = os.path.join(ASAN_BUILD, "libpagedattn_asan.so")
ASAN_SOURCES = ["abi.cpp", "sched.cpp"]
_HOST_SANITIZE = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                  "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host",
                  "-fno-omit-frame-pointer", "-g"]


def asan_runtime() -> str:
    """Path of the ASan runtime matching hipcc's compiler (to preload)."""
    r = subprocess.run([_hipcc(), "-print-file-name=libclang_rt.asan-x86_64.so"],
                       capture_output=True, text=True)
    path = r.stdout.strip()
    if r.returncode != 0 or not os.path.isabs(path) or not os.path.exists(path):
        raise RuntimeError("ASan runtime of the ROCm compiler not found")
    return path


def build_asan(verbose: bool = False) -> str:
    """Build the host-sanitized test library (after ``build()``, whose kernel objects it
    links); returns its path."""
    hipcc = _hipcc()
    os.makedirs(ASAN_BUILD, exist_ok=True)
    objs = []
    for src in ASAN_SOURCES:
        obj = os.path.join(ASAN_BUILD, os.path.splitext(src)[0] + ".o")
        cmd = [hipcc, *_flags(), *_HOST_SANITIZE, "-c", os.path.join(CSRC, src), "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"hipcc failed on {src} (sanitized):\n{r.stdout}\n{r.stderr}")
        objs.append(obj)
    kernels = [os.path.join(BUILD, os.path.splitext(s)[0] + ".o") for s in SOURCES
               if s not in ASAN_SOURCES]
    missing = [k for k in kernels if not os.path.exists(k)]
    if missing:
        raise RuntimeError(f"kernel objects missing (run build() first): {missing}")
    tmp = ASAN_LIB_PATH + ".tmp"
    cmd = [hipcc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-Xarch_host",
           "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined", "-shared-libsan",
           *objs, *kernels, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"sanitized link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, ASAN_LIB_PATH)
    return ASAN_LIB_PATH


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
    if "--asan" in sys.argv:
        print(build_asan(verbose="-v" in sys.argv))

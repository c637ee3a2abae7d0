"""Build libsafe.so (HIP for gfx950) in-tree with hipcc.

Usage: python sparse_query_sdpa_amd/build.py [-v]   (run by path: importing the package
loads the library, which may be missing or older than the sources)
       python sparse_query_sdpa_amd/build.py --host-sanitize   (ASan + UBSan on the host code,
       into _build/hostsan/; load it with SAFE_LIB_PATH and the runtime in LD_PRELOAD)
"""
from __future__ import annotations

import concurrent.futures
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
OBJ = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libsafe.so")

SOURCES = ["api.hip", "attn_fwd.hip", "attn_masked.hip", "attn_short.hip", "kv_assemble.hip", "mask_classify.hip", "pcsp.hip", "sw_cfg.hip", "linear.hip", "probe.hip"]

# Packed fp32 VALU ops are disabled: the compiler still vectorises ordinary code,
# but no v_pk_{add,mul,fma}_f32 is emitted.  (The host pass ignores the feature.)
HIPCC_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"),
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: the HIP toolchain is required to build libsafe")


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in r.stdout.splitlines() if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"command failed ({r.returncode}): {' '.join(cmd)}\n{out}")
    if verbose and out.strip():
        print(out, flush=True)


def build(verbose: bool = False, jobs: int = 0) -> str:
    """Compile every HIP source for gfx950 and link libsafe.so; return its path."""
    cc = hipcc()
    os.makedirs(OBJ, exist_ok=True)
    jobs = jobs or min(8, len(SOURCES))
    objs = []
    cmds = []
    for src in SOURCES:
        obj = os.path.join(OBJ, src.replace(".hip", ".o"))
        objs.append(obj)
        cmds.append([cc, *HIPCC_FLAGS, "-c", os.path.join(CSRC, src), "-o", obj])
    with concurrent.futures.ThreadPoolExecutor(max_workers=jobs) as ex:
        list(ex.map(lambda c: _run(c, verbose), cmds))
    tmp = LIB + ".tmp"
    _run([cc, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp], verbose)
    _check_loads(tmp)
    os.replace(tmp, LIB)
    return LIB


def _check_loads(path: str) -> None:
    """Resolve every symbol of the linked library now: a kernel whose host-side launch stub
    was not emitted links fine but leaves an undefined symbol that only loading reveals."""
    import ctypes
    try:
        ctypes.CDLL(os.path.abspath(path), mode=os.RTLD_NOW | os.RTLD_LOCAL)
    except OSError as e:
        raise RuntimeError(f"the linked library does not load: {e}") from e


# Host-sanitized build: AddressSanitizer and UndefinedBehaviorSanitizer on the host code only
# (argument checks, planners, the C ABI); the device code is the ordinary gfx950 build.  The
# library links the shared sanitizer runtime, which the loading process must preload.
SANITIZE_FLAGS = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                  "-Xarch_host", "-fno-omit-frame-pointer", "-g"]


def sanitizer_runtime() -> str:
    """Path of the shared AddressSanitizer runtime of the HIP toolchain's clang."""
    clang = os.path.join(os.path.dirname(os.path.realpath(hipcc())), "..", "lib", "llvm", "bin", "clang")
    for cand in (clang, "/opt/rocm/llvm/bin/clang", shutil.which("clang")):
        if cand and os.path.exists(cand):
            r = subprocess.run([cand, "-print-file-name=libclang_rt.asan-x86_64.so"], stdout=subprocess.PIPE,
                               text=True)
            path = r.stdout.strip()
            if r.returncode == 0 and os.path.isabs(path) and os.path.exists(path):
                return path
    raise RuntimeError("the clang AddressSanitizer runtime was not found")


def build_host_sanitized(out_dir: str, verbose: bool = False, jobs: int = 0) -> str:
    """Compile the library with the host sanitizers into out_dir; return the library's path."""
    cc = hipcc()
    os.makedirs(out_dir, exist_ok=True)
    jobs = jobs or min(8, len(SOURCES))
    flags = [f for f in HIPCC_FLAGS if f != "-O3"] + ["-O1"] + SANITIZE_FLAGS
    objs = [os.path.join(out_dir, src.replace(".hip", ".o")) for src in SOURCES]
    cmds = [[cc, *flags, "-c", os.path.join(CSRC, src), "-o", obj] for src, obj in zip(SOURCES, objs)]
    with concurrent.futures.ThreadPoolExecutor(max_workers=jobs) as ex:
        list(ex.map(lambda c: _run(c, verbose), cmds))
    lib = os.path.join(out_dir, "libsafe_hostsan.so")
    _run([cc, "--offload-arch=gfx950", "-shared", "-fPIC", *SANITIZE_FLAGS[:4], "-shared-libsan", *objs, "-o", lib],
         verbose)
    return lib


if __name__ == "__main__":
    if "--host-sanitize" in sys.argv:
        print(build_host_sanitized(os.path.join(OBJ, "hostsan"), verbose="-v" in sys.argv))
    else:
        print(build(verbose="-v" in sys.argv))

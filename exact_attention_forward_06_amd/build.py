"""Builds libattn.so (HIP kernels + C-ABI layer) in-tree for gfx950.

    python -m exact_attention_forward_06_amd.build [--verbose] [--sanitized]

Each source is compiled to an object under <repo>/_build in parallel, then
linked into exact_attention_forward_06_amd/libattn.so (written atomically).

--poison also builds exact_attention_forward_06_amd/libattn_poison.so: a
debug build (ATTN_LDS_POISON) whose K/V tile copies first fill their LDS
destination with NaN, so a stage read before its copy has landed shows up as
NaN in the output; run the parity tests against it with ATTN_LIBRARY.

--sanitized also builds <repo>/_build/san/libattn.so: the same device code
with the host side of the C-ABI layer (api.cpp: validation, dispatch,
errors) instrumented by AddressSanitizer and UndefinedBehaviorSanitizer
(host code only; GPU code is never built with a sanitizer).  Load it with
the ASan runtime preloaded (asan_runtime()) and ATTN_LIBRARY pointing at it.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG_DIR)
CSRC = os.path.join(PKG_DIR, "csrc")
BUILD_DIR = os.path.join(ROOT, "_build")
LIB_PATH = os.path.join(PKG_DIR, "libattn.so")
ARCH = "gfx950"

# -packed-fp32-ops: no v_pk_{add,mul,fma}_f32 in the device code.
HIP_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"),
]


def sources():
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC)
                  if f.endswith((".hip", ".cpp")))


def _hipcc():
    exe = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(exe):
        raise RuntimeError("hipcc not found (ROCm is required to build libattn.so)")
    return exe


def _compile(src: str, verbose: bool) -> str:
    obj = os.path.join(BUILD_DIR, os.path.basename(src) + ".o")
    cmd = [_hipcc(), *HIP_FLAGS, "-c", src, "-o", obj]
    if src.endswith(".cpp"):
        cmd[1:1] = ["-x", "hip"]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    msgs = "\n".join(l for l in (r.stdout + r.stderr).splitlines()
                     if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"compiling {os.path.basename(src)} failed:\n{msgs}")
    if verbose and msgs.strip():
        print(msgs, flush=True)
    return obj


def build(verbose: bool = False) -> str:
    """Compile every source and link libattn.so; returns its path."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    srcs = sources()
    with cf.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose), srcs))
    tmp = LIB_PATH + ".tmp"
    cmd = [_hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"linking libattn.so failed:\n{r.stdout}{r.stderr}")
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


SAN_DIR = os.path.join(BUILD_DIR, "san")
SAN_LIB_PATH = os.path.join(SAN_DIR, "libattn.so")
# host-only sanitizer flags: every -fsanitize sits behind -Xarch_host
SAN_FLAGS = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
             "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer"]


def asan_runtime() -> str:
    """Path of clang's shared ASan runtime (to preload into python)."""
    llvm = os.path.join(os.path.dirname(os.path.dirname(_hipcc())), "lib", "llvm", "lib", "clang")
    for ver in sorted(os.listdir(llvm), reverse=True):
        cand = os.path.join(llvm, ver, "lib", "linux", "libclang_rt.asan-x86_64.so")
        if os.path.exists(cand):
            return cand
    raise RuntimeError("libclang_rt.asan-x86_64.so not found")


def build_sanitized(verbose: bool = False) -> str:
    """The host-sanitised variant of libattn.so (see the module docstring);
    the kernel objects are those of build(), compiled here where missing or
    older than the sources and headers.  Returns its path."""
    os.makedirs(SAN_DIR, exist_ok=True)
    newest_header = max(os.path.getmtime(os.path.join(d, f)) for d in (CSRC, os.path.join(ROOT, "include"))
                        for f in os.listdir(d) if f.endswith(".h"))
    stale = [src for src in sources() if not src.endswith("api.cpp")
             and (not os.path.exists(os.path.join(BUILD_DIR, os.path.basename(src) + ".o"))
                  or os.path.getmtime(os.path.join(BUILD_DIR, os.path.basename(src) + ".o"))
                  < max(os.path.getmtime(src), newest_header))]
    if stale:
        os.makedirs(BUILD_DIR, exist_ok=True)
        with cf.ThreadPoolExecutor(max_workers=min(8, len(stale))) as ex:
            list(ex.map(lambda src: _compile(src, verbose), stale))
    api = os.path.join(CSRC, "api.cpp")
    obj = os.path.join(SAN_DIR, "api.cpp.o")
    cmd = [_hipcc(), "-x", "hip", *HIP_FLAGS, "-g", *SAN_FLAGS, "-c", api, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compiling sanitised api.cpp failed:\n{r.stdout}{r.stderr}")
    objs = [obj] + [os.path.join(BUILD_DIR, os.path.basename(s) + ".o") for s in sources() if not s.endswith("api.cpp")]
    cmd = [_hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-shared-libasan", *SAN_FLAGS, *objs,
           "-o", SAN_LIB_PATH]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"linking the sanitised libattn.so failed:\n{r.stdout}{r.stderr}")
    return SAN_LIB_PATH


POISON_LIB_PATH = os.path.join(PKG_DIR, "libattn_poison.so")


def build_poison(verbose: bool = False) -> str:
    """The LDS-poison debug build (see the module docstring).  Returns its path."""
    odir = os.path.join(BUILD_DIR, "poison")
    os.makedirs(odir, exist_ok=True)

    def comp(src):
        obj = os.path.join(odir, os.path.basename(src) + ".o")
        cmd = [_hipcc(), *HIP_FLAGS, "-DATTN_LDS_POISON=1", "-c", src, "-o", obj]
        if src.endswith(".cpp"):
            cmd[1:1] = ["-x", "hip"]
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"compiling {os.path.basename(src)} (poison) failed:\n{r.stdout}{r.stderr}")
        return obj

    srcs = sources()
    with cf.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(comp, srcs))
    tmp = POISON_LIB_PATH + ".tmp"
    r = subprocess.run([_hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp],
                       capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"linking libattn_poison.so failed:\n{r.stdout}{r.stderr}")
    os.replace(tmp, POISON_LIB_PATH)
    return POISON_LIB_PATH


if __name__ == "__main__":
    if "--poison" in sys.argv:
        print(build_poison(verbose="--verbose" in sys.argv))
    elif "--sanitized" in sys.argv:
        print(build_sanitized(verbose="--verbose" in sys.argv))
    else:
        print(build(verbose="--verbose" in sys.argv))

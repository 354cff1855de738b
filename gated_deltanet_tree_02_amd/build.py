"""Compile libgdntree.so for gfx950 with hipcc (in-tree, next to this file).

    python -m gated_deltanet_tree_02_amd.build
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
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build", "gdntree")
LIB = os.path.join(PKG, "libgdntree.so")

SOURCES = ["gdn_tree_api.cpp", "tree_build.hip", "wy_verify.hip", "wy_commit.hip", "fork.hip",
           "tree_attn_api.cpp", "tree_attn.hip", "accept.hip", "round_api.cpp"]
ARCH = "gfx950"


def hipcc() -> str:
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    path = os.path.join(rocm, "bin", "hipcc")
    return path if os.path.exists(path) else (shutil.which("hipcc") or "hipcc")


def _flags():
    return [
        "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-I", INCLUDE, "-I", CSRC,
        "-Wall", "-Wno-unused-function",
        # keep hipcc from emitting packed fp32 arithmetic (v_pk_*_f32)
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    ]


# per-source extra flags: the attention kernels take only finite inputs and
# compare scores with fmaxf, which then needs no NaN canonicalisation
EXTRA_FLAGS = {"tree_attn.hip": ["-fno-honor-nans"]}


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, src + ".o")
    cmd = [hipcc()] + _flags() + EXTRA_FLAGS.get(src, []) + ["-c", os.path.join(CSRC, src), "-o", obj]
    if src.endswith(".hip"):
        cmd[1:1] = ["-x", "hip"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{r.stdout}\n{r.stderr}")
    return obj


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    jobs = min(len(SOURCES), max(1, min(os.cpu_count() or 1, 8)))
    with concurrent.futures.ThreadPoolExecutor(jobs) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [hipcc(), "-shared", "-fPIC", f"--offload-arch={ARCH}", "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print("built", LIB)
    return LIB


# Host-side C ABI sources (no device code): the code a sanitized build checks.
HOST_SOURCES = ["gdn_tree_api.cpp", "tree_attn_api.cpp", "round_api.cpp"]
SAN_BUILD = os.path.join(ROOT, "_build", "gdntree_san")
SAN_LIB = os.path.join(SAN_BUILD, "libgdntree_san.so")
# AddressSanitizer and UndefinedBehaviorSanitizer on the host code only (each
# option behind -Xarch_host; the device code is not instrumented)
SAN_FLAGS = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
             "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host",
             "-fno-omit-frame-pointer", "-g"]


def build_host_sanitized() -> str:
    """A copy of the library whose host-side C ABI code is built with ASan and
    UBSan, linked with the kernel objects of the last regular build (made if
    missing), at _build/gdntree_san/libgdntree_san.so. The sanitizer runtime
    is not linked: load it first (LD_PRELOAD of clang's libclang_rt.asan)."""
    os.makedirs(SAN_BUILD, exist_ok=True)
    dev_objs = [os.path.join(BUILD, f + ".o") for f in SOURCES if f.endswith(".hip")]
    if not all(os.path.exists(o) for o in dev_objs):
        build()
    objs = []
    for f in HOST_SOURCES:
        obj = os.path.join(SAN_BUILD, f + ".o")
        cmd = [hipcc()] + _flags() + SAN_FLAGS + ["-c", os.path.join(CSRC, f), "-o", obj]
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"hipcc failed on {f}:\n{r.stdout}\n{r.stderr}")
        objs.append(obj)
    cmd = [hipcc(), "-shared", "-fPIC", f"--offload-arch={ARCH}", "-o", SAN_LIB] + objs + dev_objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    return SAN_LIB


def asan_runtime() -> str:
    """clang's shared AddressSanitizer runtime (it carries UBSan's too)."""
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    clang = os.path.join(rocm, "llvm", "bin", "clang")
    r = subprocess.run([clang, "-print-file-name=libclang_rt.asan-x86_64.so"], capture_output=True,
                       text=True)
    return r.stdout.strip()


def is_stale() -> bool:
    if not os.path.exists(LIB):
        return True
    t = os.path.getmtime(LIB)
    deps = [os.path.join(CSRC, f) for f in os.listdir(CSRC)] + [
        os.path.join(INCLUDE, f) for f in os.listdir(INCLUDE) if f.endswith(".h")]
    return any(os.path.getmtime(p) > t for p in deps)


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)

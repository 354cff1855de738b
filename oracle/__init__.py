"""CPU oracle for tree-verified Gated DeltaNet (fp64, slow, obviously correct).

TEST INFRASTRUCTURE ONLY: tests, the smoke check and the benchmark's CPU
baseline use it to check and time the GPU library; the library itself never
imports, links or calls anything here, and this package imports nothing from
the library.

The arithmetic lives in gdn_oracle.c (plain C, double precision, optional
OpenMP over (sequence, head)) and, for the full-attention layers of a hybrid
model (tree-masked attention and the accepted-path KV commit), in
attn_oracle.c; this module compiles both with gcc and marshals numpy arrays.
wy.py holds a second, independent formulation (the tree-shaped WY form, dense
linear algebra in numpy) used to check intermediate results.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRCS = [os.path.join(_HERE, "gdn_oracle.c"), os.path.join(_HERE, "attn_oracle.c")]
_DEFAULT_PATH = os.path.join(_HERE, "liboracle.so")
_LIB_PATH = _DEFAULT_PATH
_lock = threading.Lock()
_lib = None

STATUS_OK, STATUS_BAD_ROOT, STATUS_BAD_PARENT, STATUS_BAD_SIZE, STATUS_BAD_ACCEPTED = 0, 1, 2, 3, 4
STATUS_CACHE_FULL = 6


def build(force: bool = True) -> str:
    """Compile liboracle.so with gcc -O2 (no fast-math) and OpenMP."""
    if force or not os.path.exists(_DEFAULT_PATH):
        tmp = _DEFAULT_PATH + ".tmp%d" % os.getpid()
        cmd = ["gcc", "-O2", "-fno-fast-math", "-fopenmp", "-shared", "-fPIC", "-std=c11",
               "-Wall", "-o", tmp] + _SRCS + ["-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _DEFAULT_PATH)
    return _DEFAULT_PATH


_SAN_PATH = os.path.join(os.path.dirname(_HERE), "_build", "oracle_san", "liboracle_san.so")


def build_sanitized() -> str:
    """The oracle built by clang with AddressSanitizer and UBSan (no OpenMP),
    for checking the oracle's own memory accesses; load the sanitizer runtime
    first (LD_PRELOAD of clang's libclang_rt.asan) and select it with
    use_library()."""
    os.makedirs(os.path.dirname(_SAN_PATH), exist_ok=True)
    clang = os.path.join(os.environ.get("ROCM_PATH", "/opt/rocm"), "llvm", "bin", "clang")
    cmd = [clang, "-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
           "-fno-sanitize-recover=undefined", "-shared", "-fPIC", "-std=c11", "-Wall",
           "-Wno-unknown-pragmas", "-o", _SAN_PATH] + _SRCS + ["-lm"]
    subprocess.run(cmd, check=True)
    return _SAN_PATH


def use_library(path: str) -> None:
    """Load the oracle from `path` (a build of the same sources) from now on."""
    global _LIB_PATH, _lib
    with _lock:
        _LIB_PATH, _lib = path, None


def _load():
    global _lib
    with _lock:
        if _lib is None:
            stale = not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < max(
                os.path.getmtime(f) for f in _SRCS)
            if stale and _LIB_PATH == _DEFAULT_PATH:
                build(force=True)
            lib = ctypes.CDLL(_LIB_PATH)
            P = ctypes.c_void_p
            I = ctypes.c_int
            lib.oracle_threads.restype = I
            lib.oracle_set_threads.argtypes = [I]
            lib.oracle_tree.argtypes = [I, I, I, P, P, P, P, P]
            lib.oracle_verify.argtypes = [I, I, I, I, I, I, P, P, P, P, P, P, P, P, P, P]
            lib.oracle_commit.argtypes = [I, I, I, I, I, I, P, P, P, P, P, P, P, P, P, P]
            lib.oracle_fork_replay.argtypes = [I, I, I, I, I, I, P, P, P, P, P, P, P, P, P, P, P]
            lib.oracle_chain.argtypes = [I, I, I, P, P, P, P, P, P, P, P]
            D = ctypes.c_double
            lib.oracle_selective_fork.argtypes = [I, I, I, I, I, I, P, P, P, D, P, P, P, P, P, P,
                                                  P, P, P, P]
            lib.oracle_selective_commit.argtypes = [I, I, I, I, I, I, P, P, P, P, P, P, P, P, P,
                                                    P, P, P]
            lib.oracle_tree_attn.argtypes = [I, I, I, I, I, I, I, P, P, P, P, P, P, P, P,
                                             ctypes.c_double, P, P]
            lib.oracle_tree_attn_commit.argtypes = [I, I, I, I, I, I, P, P, P, P, P, P, P, P, P]
            _lib = lib
    return _lib


def _f64(x) -> np.ndarray:
    return np.ascontiguousarray(x, dtype=np.float64)


def _i32(x) -> np.ndarray:
    return np.ascontiguousarray(x, dtype=np.int32)


def _p(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


def threads() -> int:
    return _load().oracle_threads()


def set_threads(n: int) -> None:
    _load().oracle_set_threads(int(n))


def tree(offsets, parents, max_nodes: int = 64):
    """(depth[T] int32, anc[T] uint64, status[B] int32)."""
    lib = _load()
    offsets, parents = _i32(offsets), _i32(parents)
    B, T = len(offsets) - 1, len(parents)
    depth = np.full(T, -1, np.int32)
    anc = np.zeros(T, np.uint64)
    status = np.zeros(max(B, 1), np.int32)
    lib.oracle_tree(B, T, max_nodes, _p(offsets), _p(parents), _p(depth), _p(anc), _p(status))
    return depth, anc, status[:B]


def verify(offsets, parents, q, k, v, alpha, beta, S0, max_nodes: int = 64):
    """Per-node outputs o[T,H,dv] (float64) and per-sequence status[B]."""
    lib = _load()
    offsets, parents = _i32(offsets), _i32(parents)
    q, k, v, alpha, beta, S0 = map(_f64, (q, k, v, alpha, beta, S0))
    B = len(offsets) - 1
    T, H, dk = q.shape
    dv = v.shape[2]
    assert S0.shape == (B, H, dv, dk)
    o = np.zeros((T, H, dv), np.float64)
    status = np.zeros(max(B, 1), np.int32)
    lib.oracle_verify(B, H, dk, dv, T, max_nodes, _p(offsets), _p(parents), _p(q), _p(k), _p(v),
                      _p(alpha), _p(beta), _p(S0), _p(o), _p(status))
    return o, status[:B]


def commit(offsets, parents, accepted, k, v, alpha, beta, S0, S_out=None, max_nodes: int = 64):
    """Committed states S_out[B,H,dv,dk] (float64) and status[B]. Entries of
    sequences with a nonzero status keep the values of the S_out passed in
    (zeros by default)."""
    lib = _load()
    offsets, parents, accepted = _i32(offsets), _i32(parents), _i32(accepted)
    k, v, alpha, beta, S0 = map(_f64, (k, v, alpha, beta, S0))
    B = len(offsets) - 1
    T, H, dk = k.shape
    dv = v.shape[2]
    out = np.zeros((B, H, dv, dk), np.float64) if S_out is None else _f64(S_out).copy()
    status = np.zeros(max(B, 1), np.int32)
    lib.oracle_commit(B, H, dk, dv, T, max_nodes, _p(offsets), _p(parents), _p(accepted), _p(k),
                      _p(v), _p(alpha), _p(beta), _p(S0), _p(out), _p(status))
    return out, status[:B]


def fork_replay(offsets, parents, q, k, v, alpha, beta, S0, max_nodes: int = 64):
    """Depth-by-depth fork/checkpoint replay: (o[T,H,dv], ckpt[T,H,dv,dk], status)."""
    lib = _load()
    offsets, parents = _i32(offsets), _i32(parents)
    q, k, v, alpha, beta, S0 = map(_f64, (q, k, v, alpha, beta, S0))
    B = len(offsets) - 1
    T, H, dk = q.shape
    dv = v.shape[2]
    o = np.zeros((T, H, dv), np.float64)
    ck = np.zeros((T, H, dv, dk), np.float64)
    status = np.zeros(max(B, 1), np.int32)
    lib.oracle_fork_replay(B, H, dk, dv, T, max_nodes, _p(offsets), _p(parents), _p(q), _p(k),
                           _p(v), _p(alpha), _p(beta), _p(S0), _p(o), _p(ck), _p(status))
    return o, ck, status[:B]


def selective_fork(offsets, parents, conf, threshold, q, k, v, alpha, beta, S0,
                   max_nodes: int = 64):
    """Depth-by-depth fork that saves a checkpoint only for nodes with
    conf <= threshold: (o[T,H,dv], ckpt[T,H,dv,dk] (saved entries only, others
    zero), kept[T] int32, status[B])."""
    lib = _load()
    offsets, parents = _i32(offsets), _i32(parents)
    conf, q, k, v, alpha, beta, S0 = map(_f64, (conf, q, k, v, alpha, beta, S0))
    B = len(offsets) - 1
    T, H, dk = q.shape
    dv = v.shape[2]
    o = np.zeros((T, H, dv), np.float64)
    ck = np.zeros((T, H, dv, dk), np.float64)
    kept = np.zeros(max(T, 1), np.int32)
    status = np.zeros(max(B, 1), np.int32)
    lib.oracle_selective_fork(B, H, dk, dv, T, max_nodes, _p(offsets), _p(parents), _p(conf),
                              float(threshold), _p(q), _p(k), _p(v), _p(alpha), _p(beta), _p(S0),
                              _p(o), _p(ck), _p(kept), _p(status))
    return o, ck, kept[:T], status[:B]


def selective_commit(offsets, parents, kept, accepted, ckpt, k, v, alpha, beta, S0,
                     max_nodes: int = 64):
    """The accepted node's state after a selective-fork verify (its saved
    checkpoint, or rebuilt from the nearest saved ancestor): (S_out, status)."""
    lib = _load()
    offsets, parents, kept, accepted = _i32(offsets), _i32(parents), _i32(kept), _i32(accepted)
    ckpt, k, v, alpha, beta, S0 = map(_f64, (ckpt, k, v, alpha, beta, S0))
    B = len(offsets) - 1
    T, H, dk = k.shape
    dv = v.shape[2]
    out = np.zeros((B, H, dv, dk), np.float64)
    status = np.zeros(max(B, 1), np.int32)
    lib.oracle_selective_commit(B, H, dk, dv, T, max_nodes, _p(offsets), _p(parents), _p(kept),
                                _p(accepted), _p(ckpt), _p(k), _p(v), _p(alpha), _p(beta),
                                _p(S0), _p(out), _p(status))
    return out, status[:B]


def chain(q, k, v, alpha, beta, S0):
    """Plain sequential recurrence of one head over n tokens:
    q,k [n,dk], v [n,dv], alpha,beta [n], S0 [dv,dk] -> (o [n,dv], S_final)."""
    lib = _load()
    q, k, v, alpha, beta, S0 = map(_f64, (q, k, v, alpha, beta, S0))
    n, dk = q.shape
    dv = v.shape[1]
    o = np.zeros((n, dv), np.float64)
    S = np.zeros((dv, dk), np.float64)
    lib.oracle_chain(n, dk, dv, _p(q), _p(k), _p(v), _p(alpha), _p(beta), _p(S0), _p(o), _p(S))
    return o, S


# --------------------------------------------------------------- attention


def tree_attn(offsets, parents, q, k, v, k_cache, v_cache, cache_len, scale=None,
              max_nodes: int = 64):
    """Tree-masked attention o[T,Hq,d] (float64) and status[B].

    q [T,Hq,d]; k, v [T,Hkv,d]; k_cache, v_cache [B,Hkv,cap,d]; cache_len [B].
    scale defaults to 1/sqrt(d)."""
    lib = _load()
    offsets, parents, cache_len = _i32(offsets), _i32(parents), _i32(cache_len)
    q, k, v, kc, vc = (_f64(x) for x in (q, k, v, k_cache, v_cache))
    B, T = len(offsets) - 1, len(parents)
    Hq, d = q.shape[1], q.shape[2]
    Hkv, cap = k.shape[1], kc.shape[2]
    if scale is None:
        scale = 1.0 / np.sqrt(d)
    o = np.zeros((T, Hq, d), np.float64)
    status = np.zeros(max(B, 1), np.int32)
    lib.oracle_tree_attn(B, Hq, Hkv, d, T, max_nodes, cap, _p(offsets), _p(parents), _p(q), _p(k),
                         _p(v), _p(kc), _p(vc), _p(cache_len), float(scale), _p(o), _p(status))
    return o, status[:B]


def tree_attn_commit(offsets, parents, accepted, k, v, k_cache, v_cache, cache_len,
                     max_nodes: int = 64):
    """Caches after appending each accepted path: (k_cache, v_cache, cache_len, status)."""
    lib = _load()
    offsets, parents, accepted = _i32(offsets), _i32(parents), _i32(accepted)
    k, v = _f64(k), _f64(v)
    kc, vc = np.array(k_cache, np.float64), np.array(v_cache, np.float64)
    lens = np.array(cache_len, np.int32)
    B, T = len(offsets) - 1, len(parents)
    Hkv, cap, d = kc.shape[1], kc.shape[2], kc.shape[3]
    status = np.zeros(max(B, 1), np.int32)
    lib.oracle_tree_attn_commit(B, Hkv, d, T, max_nodes, cap, _p(offsets), _p(parents),
                                _p(accepted), _p(k), _p(v), _p(kc), _p(vc), _p(lens), _p(status))
    return kc, vc, lens, status[:B]

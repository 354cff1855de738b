"""Python binding of libgdntree (MI355X / gfx950): tree verification of Gated
DeltaNet layers and of the full-attention layers beside them.

The functions here carry the names of the C entry points declared in
include/gdn_tree.h, include/gdn_tree_attn.h and include/gdn_round.h and only
marshal arguments:
they check torch tensors (device, dtype, shape, contiguity), pass their device
pointers and the current HIP stream to the library, and raise GdnError for a nonzero gdn_status. Every
step of the computation runs in the library's HIP kernels; there is no
fallback. Loading fails loudly when libgdntree.so has not been built.
"""
from __future__ import annotations

import ctypes
import os
import threading
from typing import Optional

__all__ = [
    "GdnError", "GdnTreeDesc", "load_library", "make_desc", "gdn_tree_workspace_bytes",
    "gdn_tree_build", "gdn_tree_verify", "gdn_tree_commit", "gdn_tree_status_string",
    "DTYPE_F32", "DTYPE_BF16", "MODE_WY", "MODE_FORK", "MODE_FORK_DELTA", "MAX_NODES",
    "TREE_STATUS",
    "PreparedCall", "prepare_verify", "prepare_commit",
    "GdnAttnDesc", "make_attn_desc", "gdn_tree_attn_workspace_bytes", "gdn_tree_attn_verify",
    "gdn_tree_attn_commit", "prepare_attn_verify", "prepare_attn_commit",
    "GdnLayerIO", "make_layer_io", "gdn_tree_verify_layers", "gdn_tree_commit_layers",
    "prepare_verify_layers", "prepare_commit_layers",
    "gdn_tree_commit_verify", "gdn_tree_commit_verify_layers", "prepare_commit_verify_layers",
    "gdn_tree_replay_verify", "gdn_tree_replay_verify_layers", "prepare_replay_verify_layers",
    "gdn_tree_replay_commit", "gdn_tree_replay_commit_layers", "prepare_replay_commit_layers",
    "PREV_SHIFT", "prev_code",
    "gdn_tree_fork_selective_workspace_bytes", "gdn_tree_fork_selective_verify",
    "gdn_tree_fork_selective_commit", "prepare_fork_selective_verify",
    "gdn_tree_attn_verify_noalloc",
    "prepare_fork_selective_commit",
    "GdnAttnLayerIO", "make_attn_layer_io", "gdn_tree_attn_commit_layers",
    "prepare_attn_commit_layers",
    "gdn_tree_accept_greedy", "gdn_tree_accept_sampling",
    "gdn_tree_accept_sampling_split_workspace_bytes", "gdn_tree_accept_sampling_splits",
    "gdn_tree_accept_sampling_split", "prepare_accept_sampling_split", "GdnRoundDesc", "GdnRoundLayout", "make_round_desc",
    "gdn_round_plan", "gdn_round_tree_for_budget", "RoundGraph", "GdnRoundPrev",
]

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libgdntree.so")

DTYPE_F32, DTYPE_BF16 = 0, 1
MODE_WY, MODE_FORK, MODE_FORK_DELTA = 0, 1, 2
MAX_NODES = 64
TREE_STATUS = {0: "ok", 1: "bad root", 2: "bad parent", 3: "bad size", 4: "bad accepted",
               5: "too deep", 6: "cache full", 7: "bad token", 8: "too many kept"}
# fused round-boundary calls: the previous round's commit code sits above this shift
PREV_SHIFT = 4


def prev_code(code: int) -> int:
    """A previous-round code in the position the fused calls report it."""
    return code << PREV_SHIFT


class GdnError(RuntimeError):
    def __init__(self, code: int, where: str):
        super().__init__(f"{where}: {gdn_tree_status_string(code)} (gdn_status {code})")
        self.code = code


class GdnTreeDesc(ctypes.Structure):
    _fields_ = [
        ("num_seqs", ctypes.c_int32), ("num_heads", ctypes.c_int32),
        ("dk", ctypes.c_int32), ("dv", ctypes.c_int32),
        ("total_nodes", ctypes.c_int32), ("max_nodes", ctypes.c_int32),
        ("max_depth", ctypes.c_int32), ("io_dtype", ctypes.c_int32), ("mode", ctypes.c_int32),
    ]


class GdnAttnDesc(ctypes.Structure):
    _fields_ = [
        ("num_seqs", ctypes.c_int32), ("num_q_heads", ctypes.c_int32),
        ("num_kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
        ("total_nodes", ctypes.c_int32), ("max_nodes", ctypes.c_int32),
        ("cache_capacity", ctypes.c_int32), ("max_cache_len", ctypes.c_int32),
    ]


class GdnLayerIO(ctypes.Structure):
    _fields_ = [(name, ctypes.c_void_p) for name in
                ("q", "k", "v", "alpha", "beta", "S0", "o", "S_out", "workspace")]


class GdnAttnLayerIO(ctypes.Structure):
    _fields_ = [(name, ctypes.c_void_p) for name in ("q", "k", "v", "k_cache", "v_cache", "o")]


class GdnRoundDesc(ctypes.Structure):
    _fields_ = [("gdn", GdnTreeDesc), ("n_gdn_layers", ctypes.c_int32),
                ("attn", GdnAttnDesc), ("n_attn_layers", ctypes.c_int32)]


class GdnRoundLayout(ctypes.Structure):
    _fields_ = [(name, ctypes.c_size_t) for name in
                ("total_bytes", "gdn_ws_bytes", "gdn_ws_stride", "attn_ws_bytes",
                 "attn_ws_offset", "attn_ws_stride")]


class GdnRoundIO(ctypes.Structure):
    _fields_ = [
        ("offsets", ctypes.c_void_p), ("parents", ctypes.c_void_p),
        ("gdn_layers", ctypes.POINTER(GdnLayerIO)), ("attn_layers", ctypes.POINTER(GdnAttnLayerIO)),
        ("layer_kinds", ctypes.POINTER(ctypes.c_int32)), ("cache_len", ctypes.c_void_p),
        ("attn_scale", ctypes.c_float), ("arena", ctypes.c_void_p), ("arena_bytes", ctypes.c_size_t),
        ("draft_tokens", ctypes.c_void_p), ("target_tokens", ctypes.c_void_p),
        ("accepted", ctypes.c_void_p), ("accept_len", ctypes.c_void_p),
        ("next_token", ctypes.c_void_p), ("tree_status", ctypes.c_void_p),
    ]


class GdnRoundPrev(ctypes.Structure):
    _fields_ = [
        ("gdn", GdnTreeDesc), ("offsets", ctypes.c_void_p), ("parents", ctypes.c_void_p),
        ("accepted", ctypes.c_void_p), ("gdn_layers", ctypes.POINTER(GdnLayerIO)),
    ]


_lock = threading.Lock()
_lib = None


def load_library() -> ctypes.CDLL:
    """Load libgdntree.so from this package directory (no build, no fallback)."""
    global _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(LIB_PATH):
                raise ImportError(
                    f"{LIB_PATH} is missing: build it with `python -m gated_deltanet_tree_02_amd.build` "
                    "(or __graft_entry__.build()); there is no CPU fallback")
            lib = ctypes.CDLL(LIB_PATH)
            P, S, I = ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int
            D = ctypes.POINTER(GdnTreeDesc)
            lib.gdn_tree_workspace_bytes.argtypes = [D]
            lib.gdn_tree_workspace_bytes.restype = S
            lib.gdn_tree_build.argtypes = [D, P, P, P, P, P, P]
            lib.gdn_tree_build.restype = I
            lib.gdn_tree_verify.argtypes = [D, P, P, P, P, P, P, P, P, P, P, S, P, P]
            lib.gdn_tree_verify.restype = I
            lib.gdn_tree_commit.argtypes = [D, P, P, P, P, P, P, P, S, P, P]
            lib.gdn_tree_commit.restype = I
            A = ctypes.POINTER(GdnAttnDesc)
            lib.gdn_tree_attn_workspace_bytes.argtypes = [A]
            lib.gdn_tree_attn_workspace_bytes.restype = S
            lib.gdn_tree_attn_verify.argtypes = [A, P, P, P, P, P, P, P, P, ctypes.c_float, P, P,
                                                 S, P, P]
            lib.gdn_tree_attn_verify.restype = I
            lib.gdn_tree_attn_verify_noalloc.argtypes = [A, P, P, P, P, P, P, P, P,
                                                         ctypes.c_float, P, P, P]
            lib.gdn_tree_attn_verify_noalloc.restype = I
            lib.gdn_tree_attn_commit.argtypes = [A, P, P, P, P, P, P, P, P, P, P]
            lib.gdn_tree_attn_commit.restype = I
            LY = ctypes.POINTER(GdnLayerIO)
            lib.gdn_tree_verify_layers.argtypes = [D, ctypes.c_int32, P, P, LY, S, P, P]
            lib.gdn_tree_verify_layers.restype = I
            lib.gdn_tree_commit_layers.argtypes = [D, ctypes.c_int32, P, P, P, LY, S, P, P]
            lib.gdn_tree_commit_layers.restype = I
            lib.gdn_tree_commit_verify.argtypes = [D, P, P, P, P, P, S, D, P, P, P, P, P, P, P,
                                                   P, P, P, P, S, P, P]
            lib.gdn_tree_commit_verify.restype = I
            lib.gdn_tree_commit_verify_layers.argtypes = [D, D, ctypes.c_int32, P, P, P, P, P,
                                                          LY, S, LY, S, P, P]
            lib.gdn_tree_commit_verify_layers.restype = I
            lib.gdn_tree_replay_verify.argtypes = [D, P, P, P, P, P, P, P, D, P, P, P, P, P, P,
                                                   P, P, P, P, P, P]
            lib.gdn_tree_replay_verify.restype = I
            lib.gdn_tree_replay_verify_layers.argtypes = [D, D, ctypes.c_int32, P, P, P, P, P,
                                                          LY, LY, P, P]
            lib.gdn_tree_replay_verify_layers.restype = I
            lib.gdn_tree_replay_commit.argtypes = [D, P, P, P, P, P, P, P, P, P, P, P]
            lib.gdn_tree_replay_commit.restype = I
            lib.gdn_tree_replay_commit_layers.argtypes = [D, ctypes.c_int32, P, P, P, LY, P, P]
            lib.gdn_tree_replay_commit_layers.restype = I
            F = ctypes.c_float
            lib.gdn_tree_fork_selective_workspace_bytes.argtypes = [D, ctypes.c_int32]
            lib.gdn_tree_fork_selective_workspace_bytes.restype = S
            lib.gdn_tree_fork_selective_verify.argtypes = [D, P, P, P, F, ctypes.c_int32, P, P,
                                                           P, P, P, P, P, P, S, P, P]
            lib.gdn_tree_fork_selective_verify.restype = I
            lib.gdn_tree_fork_selective_commit.argtypes = [D, P, P, P, F, ctypes.c_int32, P, P,
                                                           P, P, P, P, P, P, S, P, P]
            lib.gdn_tree_fork_selective_commit.restype = I
            AL = ctypes.POINTER(GdnAttnLayerIO)
            lib.gdn_tree_attn_commit_layers.argtypes = [A, ctypes.c_int32, P, P, P, AL, P, P, P]
            lib.gdn_tree_attn_commit_layers.restype = I
            lib.gdn_tree_accept_greedy.argtypes = [D, P, P, P, P, P, P, P, P, P]
            lib.gdn_tree_accept_greedy.restype = I
            lib.gdn_tree_accept_sampling.argtypes = [D, P, P, P, P, P, ctypes.c_int32, P, P, P,
                                                     P, P, P]
            lib.gdn_tree_accept_sampling.restype = I
            lib.gdn_tree_accept_sampling_split_workspace_bytes.argtypes = [D, ctypes.c_int32]
            lib.gdn_tree_accept_sampling_split_workspace_bytes.restype = S
            lib.gdn_tree_accept_sampling_splits.argtypes = [D]
            lib.gdn_tree_accept_sampling_splits.restype = ctypes.c_int32
            lib.gdn_tree_accept_sampling_split.argtypes = [D, P, P, P, P, P, ctypes.c_int32, P,
                                                           ctypes.c_int32, P, S, P, P, P, P, P]
            lib.gdn_tree_accept_sampling_split.restype = I
            R = ctypes.POINTER(GdnRoundDesc)
            lib.gdn_round_plan.argtypes = [R, ctypes.POINTER(GdnRoundLayout)]
            lib.gdn_round_plan.restype = I
            i32p = ctypes.POINTER(ctypes.c_int32)
            lib.gdn_round_tree_for_budget.argtypes = [R, S, ctypes.c_int32, i32p, i32p, i32p,
                                                      ctypes.POINTER(ctypes.c_size_t)]
            lib.gdn_round_tree_for_budget.restype = I
            lib.gdn_round_capture.argtypes = [R, ctypes.POINTER(GdnRoundIO), P,
                                              ctypes.POINTER(ctypes.c_void_p)]
            lib.gdn_round_capture.restype = I
            lib.gdn_round_capture_replay.argtypes = [R, ctypes.POINTER(GdnRoundIO),
                                                     ctypes.POINTER(GdnRoundPrev), P,
                                                     ctypes.POINTER(ctypes.c_void_p)]
            lib.gdn_round_capture_replay.restype = I
            lib.gdn_round_launch.argtypes = [P, P]
            lib.gdn_round_launch.restype = I
            lib.gdn_round_destroy.argtypes = [P]
            lib.gdn_round_destroy.restype = None
            lib.gdn_tree_status_string.argtypes = [I]
            lib.gdn_tree_status_string.restype = ctypes.c_char_p
            _lib = lib
    return _lib


def gdn_tree_status_string(code: int) -> str:
    return load_library().gdn_tree_status_string(int(code)).decode()


def make_desc(num_seqs: int, num_heads: int, dk: int, dv: int, total_nodes: int,
              max_nodes: int, io_dtype: int = DTYPE_BF16, mode: int = MODE_WY,
              max_depth: int = 0) -> GdnTreeDesc:
    return GdnTreeDesc(int(num_seqs), int(num_heads), int(dk), int(dv), int(total_nodes),
                       int(max_nodes), int(max_depth), int(io_dtype), int(mode))


def gdn_tree_workspace_bytes(desc: GdnTreeDesc) -> int:
    return int(load_library().gdn_tree_workspace_bytes(ctypes.byref(desc)))


def make_attn_desc(num_seqs: int, num_q_heads: int, num_kv_heads: int, head_dim: int,
                   total_nodes: int, max_nodes: int, cache_capacity: int,
                   max_cache_len: Optional[int] = None) -> GdnAttnDesc:
    mcl = cache_capacity if max_cache_len is None else max_cache_len
    return GdnAttnDesc(int(num_seqs), int(num_q_heads), int(num_kv_heads), int(head_dim),
                       int(total_nodes), int(max_nodes), int(cache_capacity), int(mcl))


def gdn_tree_attn_workspace_bytes(desc: GdnAttnDesc) -> int:
    return int(load_library().gdn_tree_attn_workspace_bytes(ctypes.byref(desc)))


# ------------------------------------------------------------------ marshalling


def _torch():
    import torch
    return torch


def _io_dtype(desc):
    torch = _torch()
    return torch.bfloat16 if desc.io_dtype == DTYPE_BF16 else torch.float32


def _ptr(t, name, dtype=None, shape=None, device=None, allow_none=False):
    if t is None:
        if allow_none:
            return None
        raise ValueError(f"{name} is required")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name}: dtype {t.dtype}, expected {dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name}: shape {tuple(t.shape)}, expected {tuple(shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    return t.data_ptr() if t.numel() > 0 else None


def _stream(stream, device):
    torch = _torch()
    s = torch.cuda.current_stream(device) if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _check(code: int, where: str):
    if code != 0:
        raise GdnError(code, where)


def gdn_tree_build(desc, offsets, parents, depth, anc_mask, tree_status, stream=None):
    """Ancestor masks (int64 tensor holding the uint64 bit patterns) and depths."""
    torch = _torch()
    B, T = desc.num_seqs, desc.total_nodes
    dev = offsets.device
    args = [
        _ptr(offsets, "offsets", torch.int32, (B + 1,), dev),
        _ptr(parents, "parents", torch.int32, (T,), dev),
        _ptr(depth, "depth", torch.int32, (T,), dev),
        _ptr(anc_mask, "anc_mask", torch.int64, (T,), dev),
        _ptr(tree_status, "tree_status", torch.int32, (B,), dev),
    ]
    with torch.cuda.device(dev):
        _check(load_library().gdn_tree_build(ctypes.byref(desc), *args, _stream(stream, dev)),
               "gdn_tree_build")


def _verify_args(desc, offsets, parents, q, k, v, alpha, beta, S0, o, workspace, tree_status):
    torch = _torch()
    B, H, T, dk, dv = desc.num_seqs, desc.num_heads, desc.total_nodes, desc.dk, desc.dv
    dev = offsets.device
    io = _io_dtype(desc)
    return dev, [
        _ptr(offsets, "offsets", torch.int32, (B + 1,), dev),
        _ptr(parents, "parents", torch.int32, (T,), dev),
        _ptr(q, "q", io, (T, H, dk), dev),
        _ptr(k, "k", io, (T, H, dk), dev),
        _ptr(v, "v", io, (T, H, dv), dev),
        _ptr(alpha, "alpha", torch.float32, (T, H), dev),
        _ptr(beta, "beta", torch.float32, (T, H), dev),
        _ptr(S0, "S0", torch.float32, (B, H, dv, dk), dev),
        _ptr(o, "o", io, (T, H, dv), dev),
        _ptr(workspace, "workspace", torch.uint8, None, dev),
        ctypes.c_size_t(workspace.numel()),
        _ptr(tree_status, "tree_status", torch.int32, (B,), dev),
    ]


def _commit_args(desc, offsets, parents, accepted, k, S0, S_out, workspace, tree_status):
    torch = _torch()
    B, H, T, dk, dv = desc.num_seqs, desc.num_heads, desc.total_nodes, desc.dk, desc.dv
    dev = offsets.device
    io = _io_dtype(desc)
    return dev, [
        _ptr(offsets, "offsets", torch.int32, (B + 1,), dev),
        _ptr(parents, "parents", torch.int32, (T,), dev),
        _ptr(accepted, "accepted", torch.int32, (B,), dev),
        _ptr(k, "k", io, (T, H, dk), dev, allow_none=desc.mode == MODE_FORK),
        _ptr(S0, "S0", torch.float32, (B, H, dv, dk), dev),
        _ptr(S_out, "S_out", torch.float32, (B, H, dv, dk), dev),
        _ptr(workspace, "workspace", torch.uint8, None, dev),
        ctypes.c_size_t(workspace.numel()),
        _ptr(tree_status, "tree_status", torch.int32, (B,), dev),
    ]


def gdn_tree_verify(desc, offsets, parents, q, k, v, alpha, beta, S0, o, workspace,
                    tree_status, stream=None):
    torch = _torch()
    dev, args = _verify_args(desc, offsets, parents, q, k, v, alpha, beta, S0, o, workspace,
                             tree_status)
    with torch.cuda.device(dev):
        _check(load_library().gdn_tree_verify(ctypes.byref(desc), *args, _stream(stream, dev)),
               "gdn_tree_verify")


def gdn_tree_commit(desc, offsets, parents, accepted, k, S0, S_out, workspace, tree_status,
                    stream=None):
    torch = _torch()
    dev, args = _commit_args(desc, offsets, parents, accepted, k, S0, S_out, workspace,
                             tree_status)
    with torch.cuda.device(dev):
        _check(load_library().gdn_tree_commit(ctypes.byref(desc), *args, _stream(stream, dev)),
               "gdn_tree_commit")


class PreparedCall:
    """One entry point with its arguments checked and marshalled once; calling
    it enqueues the same work again on the stream captured at preparation.
    The tensors must stay alive and unmoved while the object is used."""

    def __init__(self, name, desc, args, stream, keep):
        self._fn = getattr(load_library(), name)
        self._name = name
        self._desc = type(desc).from_buffer_copy(desc)
        self._args = (ctypes.byref(self._desc),) + tuple(args) + (stream,)
        self._keep = keep

    def __call__(self):
        code = self._fn(*self._args)
        if code != 0:
            raise GdnError(code, self._name)


def prepare_verify(desc, offsets, parents, q, k, v, alpha, beta, S0, o, workspace, tree_status,
                   stream=None) -> PreparedCall:
    tensors = (offsets, parents, q, k, v, alpha, beta, S0, o, workspace, tree_status)
    dev, args = _verify_args(desc, *tensors)
    return PreparedCall("gdn_tree_verify", desc, args, _stream(stream, dev), tensors)


def prepare_commit(desc, offsets, parents, accepted, k, S0, S_out, workspace, tree_status,
                   stream=None) -> PreparedCall:
    tensors = (offsets, parents, accepted, k, S0, S_out, workspace, tree_status)
    dev, args = _commit_args(desc, *tensors)
    return PreparedCall("gdn_tree_commit", desc, args, _stream(stream, dev), tensors)


# ------------------------------------------------------------------ attention layers


def _attn_verify_args(desc, offsets, parents, q, k, v, k_cache, v_cache, cache_len, scale, o,
                      workspace, tree_status):
    torch = _torch()
    B, Hq, Hkv, T, d = (desc.num_seqs, desc.num_q_heads, desc.num_kv_heads, desc.total_nodes,
                        desc.head_dim)
    cap = desc.cache_capacity
    dev = offsets.device
    bf = torch.bfloat16
    if scale is None:
        scale = d ** -0.5
    ws = None if workspace is None else _ptr(workspace, "workspace", torch.uint8, None, dev)
    return dev, [
        _ptr(offsets, "offsets", torch.int32, (B + 1,), dev),
        _ptr(parents, "parents", torch.int32, (T,), dev),
        _ptr(q, "q", bf, (T, Hq, d), dev),
        _ptr(k, "k", bf, (T, Hkv, d), dev),
        _ptr(v, "v", bf, (T, Hkv, d), dev),
        _ptr(k_cache, "k_cache", bf, (B, Hkv, cap, d), dev),
        _ptr(v_cache, "v_cache", bf, (B, Hkv, cap, d), dev),
        _ptr(cache_len, "cache_len", torch.int32, (B,), dev),
        ctypes.c_float(float(scale)),
        _ptr(o, "o", bf, (T, Hq, d), dev),
        ws,
        ctypes.c_size_t(0 if workspace is None else workspace.numel()),
        _ptr(tree_status, "tree_status", torch.int32, (B,), dev),
    ]


def _attn_commit_args(desc, offsets, parents, accepted, k, v, k_cache, v_cache, cache_len,
                      tree_status):
    torch = _torch()
    B, Hkv, T, d = desc.num_seqs, desc.num_kv_heads, desc.total_nodes, desc.head_dim
    cap = desc.cache_capacity
    dev = offsets.device
    bf = torch.bfloat16
    return dev, [
        _ptr(offsets, "offsets", torch.int32, (B + 1,), dev),
        _ptr(parents, "parents", torch.int32, (T,), dev),
        _ptr(accepted, "accepted", torch.int32, (B,), dev),
        _ptr(k, "k", bf, (T, Hkv, d), dev),
        _ptr(v, "v", bf, (T, Hkv, d), dev),
        _ptr(k_cache, "k_cache", bf, (B, Hkv, cap, d), dev),
        _ptr(v_cache, "v_cache", bf, (B, Hkv, cap, d), dev),
        _ptr(cache_len, "cache_len", torch.int32, (B,), dev),
        _ptr(tree_status, "tree_status", torch.int32, (B,), dev),
    ]


def gdn_tree_attn_verify(desc, offsets, parents, q, k, v, k_cache, v_cache, cache_len, o,
                         workspace, tree_status, scale=None, stream=None):
    """Tree-masked attention of every node over its cached prefix and its root
    path (bf16 tensors; scale defaults to 1/sqrt(head_dim))."""
    torch = _torch()
    dev, args = _attn_verify_args(desc, offsets, parents, q, k, v, k_cache, v_cache, cache_len,
                                  scale, o, workspace, tree_status)
    with torch.cuda.device(dev):
        _check(load_library().gdn_tree_attn_verify(ctypes.byref(desc), *args,
                                                   _stream(stream, dev)),
               "gdn_tree_attn_verify")


def gdn_tree_attn_verify_noalloc(desc, offsets, parents, q, k, v, k_cache, v_cache, cache_len,
                                 o, tree_status, scale=None, stream=None):
    """gdn_tree_attn_verify with the library's fixed per-GPU scratch instead of
    a workspace (no device allocation by the library)."""
    torch = _torch()
    dev, args = _attn_verify_args(desc, offsets, parents, q, k, v, k_cache, v_cache, cache_len,
                                  scale, o, None, tree_status)
    args = args[:-3] + args[-1:]            # no workspace pointer and size
    with torch.cuda.device(dev):
        _check(load_library().gdn_tree_attn_verify_noalloc(ctypes.byref(desc), *args,
                                                           _stream(stream, dev)),
               "gdn_tree_attn_verify_noalloc")


def gdn_tree_attn_commit(desc, offsets, parents, accepted, k, v, k_cache, v_cache, cache_len,
                         tree_status, stream=None):
    """Append the accepted path's K/V rows to the caches and advance cache_len."""
    torch = _torch()
    dev, args = _attn_commit_args(desc, offsets, parents, accepted, k, v, k_cache, v_cache,
                                  cache_len, tree_status)
    with torch.cuda.device(dev):
        _check(load_library().gdn_tree_attn_commit(ctypes.byref(desc), *args,
                                                   _stream(stream, dev)),
               "gdn_tree_attn_commit")


def prepare_attn_verify(desc, offsets, parents, q, k, v, k_cache, v_cache, cache_len, o,
                        workspace, tree_status, scale=None, stream=None) -> PreparedCall:
    tensors = (offsets, parents, q, k, v, k_cache, v_cache, cache_len, o, workspace, tree_status)
    dev, args = _attn_verify_args(desc, offsets, parents, q, k, v, k_cache, v_cache, cache_len,
                                  scale, o, workspace, tree_status)
    return PreparedCall("gdn_tree_attn_verify", desc, args, _stream(stream, dev), tensors)


def prepare_attn_commit(desc, offsets, parents, accepted, k, v, k_cache, v_cache, cache_len,
                        tree_status, stream=None) -> PreparedCall:
    tensors = (offsets, parents, accepted, k, v, k_cache, v_cache, cache_len, tree_status)
    dev, args = _attn_commit_args(desc, *tensors)
    return PreparedCall("gdn_tree_attn_commit", desc, args, _stream(stream, dev), tensors)


# ------------------------------------------------------------------ layer-batched calls


def make_layer_io(desc, q=None, k=None, v=None, alpha=None, beta=None, S0=None, o=None,
                  S_out=None, workspace=None) -> GdnLayerIO:
    """One layer's buffers for the layer-batched calls (shapes checked against
    the descriptor; a field a call does not use may be None)."""
    torch = _torch()
    B, H, T, dk, dv = desc.num_seqs, desc.num_heads, desc.total_nodes, desc.dk, desc.dv
    io = _io_dtype(desc)
    f = lambda t, name, dt, shape: _ptr(t, name, dt, shape, allow_none=True)
    return GdnLayerIO(
        f(q, "q", io, (T, H, dk)), f(k, "k", io, (T, H, dk)), f(v, "v", io, (T, H, dv)),
        f(alpha, "alpha", torch.float32, (T, H)), f(beta, "beta", torch.float32, (T, H)),
        f(S0, "S0", torch.float32, (B, H, dv, dk)), f(o, "o", io, (T, H, dv)),
        f(S_out, "S_out", torch.float32, (B, H, dv, dk)),
        f(workspace, "workspace", torch.uint8, None))


def _layers_array(layers):
    arr = (GdnLayerIO * max(1, len(layers)))()
    for i, ly in enumerate(layers):
        arr[i] = ly
    return arr


def gdn_tree_verify_layers(desc, offsets, parents, layers, workspace_bytes, tree_status,
                           stream=None):
    """Verify every layer in `layers` (GdnLayerIO list) on the shared tree."""
    torch = _torch()
    B, T = desc.num_seqs, desc.total_nodes
    dev = offsets.device
    arr = _layers_array(layers)
    with torch.cuda.device(dev):
        _check(load_library().gdn_tree_verify_layers(
            ctypes.byref(desc), len(layers), _ptr(offsets, "offsets", torch.int32, (B + 1,), dev),
            _ptr(parents, "parents", torch.int32, (T,), dev), arr, ctypes.c_size_t(workspace_bytes),
            _ptr(tree_status, "tree_status", torch.int32, (B,), dev), _stream(stream, dev)),
            "gdn_tree_verify_layers")


def gdn_tree_commit_layers(desc, offsets, parents, accepted, layers, workspace_bytes,
                           tree_status, stream=None):
    """Commit every layer in `layers` (GdnLayerIO list) on the shared tree."""
    torch = _torch()
    B, T = desc.num_seqs, desc.total_nodes
    dev = offsets.device
    arr = _layers_array(layers)
    with torch.cuda.device(dev):
        _check(load_library().gdn_tree_commit_layers(
            ctypes.byref(desc), len(layers), _ptr(offsets, "offsets", torch.int32, (B + 1,), dev),
            _ptr(parents, "parents", torch.int32, (T,), dev),
            _ptr(accepted, "accepted", torch.int32, (B,), dev), arr,
            ctypes.c_size_t(workspace_bytes),
            _ptr(tree_status, "tree_status", torch.int32, (B,), dev), _stream(stream, dev)),
            "gdn_tree_commit_layers")


def prepare_verify_layers(desc, offsets, parents, layers, workspace_bytes, tree_status,
                          keep=(), stream=None) -> PreparedCall:
    """Marshalled gdn_tree_verify_layers; `keep` holds the tensors behind `layers`."""
    torch = _torch()
    B, T = desc.num_seqs, desc.total_nodes
    dev = offsets.device
    arr = _layers_array(layers)
    args = [ctypes.c_int32(len(layers)), _ptr(offsets, "offsets", torch.int32, (B + 1,), dev),
            _ptr(parents, "parents", torch.int32, (T,), dev), arr,
            ctypes.c_size_t(workspace_bytes),
            _ptr(tree_status, "tree_status", torch.int32, (B,), dev)]
    return PreparedCall("gdn_tree_verify_layers", desc, args, _stream(stream, dev),
                        (offsets, parents, tree_status, arr, tuple(keep)))


def prepare_commit_layers(desc, offsets, parents, accepted, layers, workspace_bytes, tree_status,
                          keep=(), stream=None) -> PreparedCall:
    """Marshalled gdn_tree_commit_layers; `keep` holds the tensors behind `layers`."""
    torch = _torch()
    B, T = desc.num_seqs, desc.total_nodes
    dev = offsets.device
    arr = _layers_array(layers)
    args = [ctypes.c_int32(len(layers)), _ptr(offsets, "offsets", torch.int32, (B + 1,), dev),
            _ptr(parents, "parents", torch.int32, (T,), dev),
            _ptr(accepted, "accepted", torch.int32, (B,), dev), arr,
            ctypes.c_size_t(workspace_bytes),
            _ptr(tree_status, "tree_status", torch.int32, (B,), dev)]
    return PreparedCall("gdn_tree_commit_layers", desc, args, _stream(stream, dev),
                        (offsets, parents, accepted, tree_status, arr, tuple(keep)))


# ------------------------------------------------- previous commit fused into verify


def _prev_args(prev_desc, desc, prev_offsets, prev_parents, accepted, dev):
    torch = _torch()
    if prev_desc.num_seqs != desc.num_seqs:
        raise ValueError("prev_desc and desc must have the same num_seqs")
    B, pT = desc.num_seqs, prev_desc.total_nodes
    return [_ptr(prev_offsets, "prev_offsets", torch.int32, (B + 1,), dev),
            _ptr(prev_parents, "prev_parents", torch.int32, (pT,), dev),
            _ptr(accepted, "accepted", torch.int32, (B,), dev)]


def gdn_tree_commit_verify(prev_desc, prev_offsets, prev_parents, accepted, prev_k,
                           prev_workspace, desc, offsets, parents, q, k, v, alpha, beta, S0,
                           S_out, o, workspace, tree_status, stream=None):
    """The previous round's commit (accepted path of the previous tree into
    S_out, from S0) and this round's verify against S_out, in one pass over
    the state."""
    torch = _torch()
    dev, va = _verify_args(desc, offsets, parents, q, k, v, alpha, beta, S0, o, workspace,
                           tree_status)
    B, H, dk, dv = desc.num_seqs, desc.num_heads, desc.dk, desc.dv
    pa = _prev_args(prev_desc, desc, prev_offsets, prev_parents, accepted, dev)
    pa += [_ptr(prev_k, "prev_k", _io_dtype(prev_desc), (prev_desc.total_nodes, H, dk), dev),
           _ptr(prev_workspace, "prev_workspace", torch.uint8, None, dev),
           ctypes.c_size_t(prev_workspace.numel())]
    s_out = _ptr(S_out, "S_out", torch.float32, (B, H, dv, dk), dev)
    # va: offsets, parents, q, k, v, alpha, beta, S0, o, workspace, bytes, tree_status
    args = pa + [ctypes.byref(desc)] + va[:8] + [s_out] + va[8:]
    with torch.cuda.device(dev):
        _check(load_library().gdn_tree_commit_verify(ctypes.byref(prev_desc), *args,
                                                     _stream(stream, dev)),
               "gdn_tree_commit_verify")


def _commit_verify_layers_args(prev_desc, desc, prev_offsets, prev_parents, accepted, offsets,
                               parents, prev_layers, prev_workspace_bytes, layers,
                               workspace_bytes, tree_status):
    torch = _torch()
    if len(prev_layers) != len(layers):
        raise ValueError("prev_layers and layers must have the same length")
    B, T = desc.num_seqs, desc.total_nodes
    dev = offsets.device
    desc_copy = type(desc).from_buffer_copy(desc)
    pa = _prev_args(prev_desc, desc, prev_offsets, prev_parents, accepted, dev)
    parr, arr = _layers_array(prev_layers), _layers_array(layers)
    args = [ctypes.byref(desc_copy), ctypes.c_int32(len(layers))] + pa + [
        _ptr(offsets, "offsets", torch.int32, (B + 1,), dev),
        _ptr(parents, "parents", torch.int32, (T,), dev), parr,
        ctypes.c_size_t(prev_workspace_bytes), arr, ctypes.c_size_t(workspace_bytes),
        _ptr(tree_status, "tree_status", torch.int32, (B,), dev)]
    return dev, args, (desc_copy, parr, arr)


def gdn_tree_commit_verify_layers(prev_desc, desc, prev_offsets, prev_parents, accepted,
                                  offsets, parents, prev_layers, prev_workspace_bytes, layers,
                                  workspace_bytes, tree_status, stream=None):
    """gdn_tree_commit_verify for every layer: `prev_layers` (GdnLayerIO made
    with prev_desc: k and workspace) and `layers` (GdnLayerIO made with desc:
    q, k, v, alpha, beta, S0, o, S_out, workspace)."""
    torch = _torch()
    dev, args, _ = _commit_verify_layers_args(prev_desc, desc, prev_offsets, prev_parents,
                                              accepted, offsets, parents, prev_layers,
                                              prev_workspace_bytes, layers, workspace_bytes,
                                              tree_status)
    with torch.cuda.device(dev):
        _check(load_library().gdn_tree_commit_verify_layers(ctypes.byref(prev_desc), *args,
                                                            _stream(stream, dev)),
               "gdn_tree_commit_verify_layers")


def prepare_commit_verify_layers(prev_desc, desc, prev_offsets, prev_parents, accepted, offsets,
                                 parents, prev_layers, prev_workspace_bytes, layers,
                                 workspace_bytes, tree_status, keep=(),
                                 stream=None) -> PreparedCall:
    """Marshalled gdn_tree_commit_verify_layers; `keep` holds the tensors
    behind `prev_layers` and `layers`."""
    dev, args, held = _commit_verify_layers_args(prev_desc, desc, prev_offsets, prev_parents,
                                                 accepted, offsets, parents, prev_layers,
                                                 prev_workspace_bytes, layers, workspace_bytes,
                                                 tree_status)
    return PreparedCall("gdn_tree_commit_verify_layers", prev_desc, args, _stream(stream, dev),
                        (prev_offsets, prev_parents, accepted, offsets, parents, tree_status,
                         held, tuple(keep)))


def gdn_tree_replay_verify(prev_desc, prev_offsets, prev_parents, accepted, prev_k, prev_v,
                           prev_alpha, prev_beta, desc, offsets, parents, q, k, v, alpha, beta,
                           S0, S_out, o, tree_status, stream=None):
    """The previous round's accepted path replayed on the state (S0 -> S_out)
    and this round's verify against S_out, in one pass over the state and
    with no workspace."""
    torch = _torch()
    B, H, T, dk, dv = desc.num_seqs, desc.num_heads, desc.total_nodes, desc.dk, desc.dv
    pT = prev_desc.total_nodes
    dev = offsets.device
    io, pio = _io_dtype(desc), _io_dtype(prev_desc)
    pa = _prev_args(prev_desc, desc, prev_offsets, prev_parents, accepted, dev)
    pa += [_ptr(prev_k, "prev_k", pio, (pT, H, dk), dev), _ptr(prev_v, "prev_v", pio, (pT, H, dv), dev),
           _ptr(prev_alpha, "prev_alpha", torch.float32, (pT, H), dev),
           _ptr(prev_beta, "prev_beta", torch.float32, (pT, H), dev)]
    ca = [ctypes.byref(desc), _ptr(offsets, "offsets", torch.int32, (B + 1,), dev),
          _ptr(parents, "parents", torch.int32, (T,), dev), _ptr(q, "q", io, (T, H, dk), dev),
          _ptr(k, "k", io, (T, H, dk), dev), _ptr(v, "v", io, (T, H, dv), dev),
          _ptr(alpha, "alpha", torch.float32, (T, H), dev),
          _ptr(beta, "beta", torch.float32, (T, H), dev),
          _ptr(S0, "S0", torch.float32, (B, H, dv, dk), dev),
          _ptr(S_out, "S_out", torch.float32, (B, H, dv, dk), dev), _ptr(o, "o", io, (T, H, dv), dev),
          _ptr(tree_status, "tree_status", torch.int32, (B,), dev)]
    with torch.cuda.device(dev):
        _check(load_library().gdn_tree_replay_verify(ctypes.byref(prev_desc), *pa, *ca,
                                                     _stream(stream, dev)),
               "gdn_tree_replay_verify")


def _replay_verify_layers_args(prev_desc, desc, prev_offsets, prev_parents, accepted, offsets,
                               parents, prev_layers, layers, tree_status):
    torch = _torch()
    if len(prev_layers) != len(layers):
        raise ValueError("prev_layers and layers must have the same length")
    B, T = desc.num_seqs, desc.total_nodes
    dev = offsets.device
    desc_copy = type(desc).from_buffer_copy(desc)
    pa = _prev_args(prev_desc, desc, prev_offsets, prev_parents, accepted, dev)
    parr, arr = _layers_array(prev_layers), _layers_array(layers)
    args = [ctypes.byref(desc_copy), ctypes.c_int32(len(layers))] + pa + [
        _ptr(offsets, "offsets", torch.int32, (B + 1,), dev),
        _ptr(parents, "parents", torch.int32, (T,), dev), parr, arr,
        _ptr(tree_status, "tree_status", torch.int32, (B,), dev)]
    return dev, args, (desc_copy, parr, arr)


def gdn_tree_replay_verify_layers(prev_desc, desc, prev_offsets, prev_parents, accepted,
                                  offsets, parents, prev_layers, layers, tree_status,
                                  stream=None):
    """gdn_tree_replay_verify for every layer: `prev_layers` (GdnLayerIO made
    with prev_desc: k, v, alpha, beta) and `layers` (GdnLayerIO made with desc:
    q, k, v, alpha, beta, S0, o, S_out)."""
    torch = _torch()
    dev, args, _ = _replay_verify_layers_args(prev_desc, desc, prev_offsets, prev_parents,
                                              accepted, offsets, parents, prev_layers, layers,
                                              tree_status)
    with torch.cuda.device(dev):
        _check(load_library().gdn_tree_replay_verify_layers(ctypes.byref(prev_desc), *args,
                                                            _stream(stream, dev)),
               "gdn_tree_replay_verify_layers")


def prepare_replay_verify_layers(prev_desc, desc, prev_offsets, prev_parents, accepted, offsets,
                                 parents, prev_layers, layers, tree_status, keep=(),
                                 stream=None) -> PreparedCall:
    """Marshalled gdn_tree_replay_verify_layers; `keep` holds the tensors
    behind `prev_layers` and `layers`."""
    dev, args, held = _replay_verify_layers_args(prev_desc, desc, prev_offsets, prev_parents,
                                                 accepted, offsets, parents, prev_layers, layers,
                                                 tree_status)
    return PreparedCall("gdn_tree_replay_verify_layers", prev_desc, args, _stream(stream, dev),
                        (prev_offsets, prev_parents, accepted, offsets, parents, tree_status,
                         held, tuple(keep)))


def gdn_tree_replay_commit(desc, offsets, parents, accepted, k, v, alpha, beta, S0, S_out,
                           tree_status, stream=None):
    """Commit by replaying the accepted path from its own k, v, alpha, beta
    (no workspace): S_out = the accepted node's state, or S0 for -1."""
    torch = _torch()
    B, H, T, dk, dv = desc.num_seqs, desc.num_heads, desc.total_nodes, desc.dk, desc.dv
    dev = offsets.device
    io = _io_dtype(desc)
    args = [_ptr(offsets, "offsets", torch.int32, (B + 1,), dev),
            _ptr(parents, "parents", torch.int32, (T,), dev),
            _ptr(accepted, "accepted", torch.int32, (B,), dev),
            _ptr(k, "k", io, (T, H, dk), dev), _ptr(v, "v", io, (T, H, dv), dev),
            _ptr(alpha, "alpha", torch.float32, (T, H), dev),
            _ptr(beta, "beta", torch.float32, (T, H), dev),
            _ptr(S0, "S0", torch.float32, (B, H, dv, dk), dev),
            _ptr(S_out, "S_out", torch.float32, (B, H, dv, dk), dev),
            _ptr(tree_status, "tree_status", torch.int32, (B,), dev)]
    with torch.cuda.device(dev):
        _check(load_library().gdn_tree_replay_commit(ctypes.byref(desc), *args,
                                                     _stream(stream, dev)),
               "gdn_tree_replay_commit")


def _replay_commit_layers_args(desc, offsets, parents, accepted, layers, tree_status):
    torch = _torch()
    B, T = desc.num_seqs, desc.total_nodes
    dev = offsets.device
    arr = _layers_array(layers)
    args = [ctypes.c_int32(len(layers)), _ptr(offsets, "offsets", torch.int32, (B + 1,), dev),
            _ptr(parents, "parents", torch.int32, (T,), dev),
            _ptr(accepted, "accepted", torch.int32, (B,), dev), arr,
            _ptr(tree_status, "tree_status", torch.int32, (B,), dev)]
    return dev, args, arr


def gdn_tree_replay_commit_layers(desc, offsets, parents, accepted, layers, tree_status,
                                  stream=None):
    """gdn_tree_replay_commit for every layer in `layers` (GdnLayerIO: k, v,
    alpha, beta, S0, S_out) on the shared tree."""
    torch = _torch()
    dev, args, _ = _replay_commit_layers_args(desc, offsets, parents, accepted, layers,
                                              tree_status)
    with torch.cuda.device(dev):
        _check(load_library().gdn_tree_replay_commit_layers(ctypes.byref(desc), *args,
                                                            _stream(stream, dev)),
               "gdn_tree_replay_commit_layers")


def prepare_replay_commit_layers(desc, offsets, parents, accepted, layers, tree_status, keep=(),
                                 stream=None) -> PreparedCall:
    """Marshalled gdn_tree_replay_commit_layers; `keep` holds the tensors behind `layers`."""
    dev, args, arr = _replay_commit_layers_args(desc, offsets, parents, accepted, layers,
                                                tree_status)
    return PreparedCall("gdn_tree_replay_commit_layers", desc, args, _stream(stream, dev),
                        (offsets, parents, accepted, tree_status, arr, tuple(keep)))


# ------------------------------------------------------------------ selective fork


def gdn_tree_fork_selective_workspace_bytes(desc, max_kept: int) -> int:
    return int(load_library().gdn_tree_fork_selective_workspace_bytes(ctypes.byref(desc),
                                                                      int(max_kept)))


def _selective_args(desc, offsets, parents, confidence, threshold, max_kept):
    torch = _torch()
    B, T = desc.num_seqs, desc.total_nodes
    dev = offsets.device
    return dev, [_ptr(offsets, "offsets", torch.int32, (B + 1,), dev),
                 _ptr(parents, "parents", torch.int32, (T,), dev),
                 _ptr(confidence, "confidence", torch.float32, (T,), dev),
                 ctypes.c_float(threshold), ctypes.c_int32(max_kept)]


def _ws_args(workspace, dev):
    torch = _torch()
    if workspace is None:
        return [None, ctypes.c_size_t(0)]
    return [_ptr(workspace, "workspace", torch.uint8, None, dev),
            ctypes.c_size_t(workspace.numel())]


def _selective_verify_args(desc, offsets, parents, confidence, threshold, max_kept, q, k, v,
                           alpha, beta, S0, o, workspace, tree_status):
    torch = _torch()
    B, H, T, dk, dv = desc.num_seqs, desc.num_heads, desc.total_nodes, desc.dk, desc.dv
    io = _io_dtype(desc)
    dev, args = _selective_args(desc, offsets, parents, confidence, threshold, max_kept)
    args += [_ptr(q, "q", io, (T, H, dk), dev), _ptr(k, "k", io, (T, H, dk), dev),
             _ptr(v, "v", io, (T, H, dv), dev), _ptr(alpha, "alpha", torch.float32, (T, H), dev),
             _ptr(beta, "beta", torch.float32, (T, H), dev),
             _ptr(S0, "S0", torch.float32, (B, H, dv, dk), dev), _ptr(o, "o", io, (T, H, dv), dev)]
    args += _ws_args(workspace, dev)
    args.append(_ptr(tree_status, "tree_status", torch.int32, (B,), dev))
    return dev, args


def _selective_commit_args(desc, offsets, parents, confidence, threshold, max_kept, accepted, k,
                           v, alpha, beta, S0, S_out, workspace, tree_status):
    torch = _torch()
    B, H, T, dk, dv = desc.num_seqs, desc.num_heads, desc.total_nodes, desc.dk, desc.dv
    io = _io_dtype(desc)
    dev, args = _selective_args(desc, offsets, parents, confidence, threshold, max_kept)
    args += [_ptr(accepted, "accepted", torch.int32, (B,), dev),
             _ptr(k, "k", io, (T, H, dk), dev), _ptr(v, "v", io, (T, H, dv), dev),
             _ptr(alpha, "alpha", torch.float32, (T, H), dev),
             _ptr(beta, "beta", torch.float32, (T, H), dev),
             _ptr(S0, "S0", torch.float32, (B, H, dv, dk), dev),
             _ptr(S_out, "S_out", torch.float32, (B, H, dv, dk), dev)]
    args += _ws_args(workspace, dev)
    args.append(_ptr(tree_status, "tree_status", torch.int32, (B,), dev))
    return dev, args


def gdn_tree_fork_selective_verify(desc, offsets, parents, confidence, threshold, max_kept, q, k,
                                   v, alpha, beta, S0, o, workspace, tree_status, stream=None):
    """Depth-by-depth fork keeping checkpoints only for nodes with
    confidence <= threshold (at most max_kept per sequence)."""
    torch = _torch()
    dev, args = _selective_verify_args(desc, offsets, parents, confidence, threshold, max_kept, q,
                                       k, v, alpha, beta, S0, o, workspace, tree_status)
    with torch.cuda.device(dev):
        _check(load_library().gdn_tree_fork_selective_verify(ctypes.byref(desc), *args,
                                                             _stream(stream, dev)),
               "gdn_tree_fork_selective_verify")


def gdn_tree_fork_selective_commit(desc, offsets, parents, confidence, threshold, max_kept,
                                   accepted, k, v, alpha, beta, S0, S_out, workspace, tree_status,
                                   stream=None):
    """The accepted node's state after a selective-fork verify."""
    torch = _torch()
    dev, args = _selective_commit_args(desc, offsets, parents, confidence, threshold, max_kept,
                                       accepted, k, v, alpha, beta, S0, S_out, workspace,
                                       tree_status)
    with torch.cuda.device(dev):
        _check(load_library().gdn_tree_fork_selective_commit(ctypes.byref(desc), *args,
                                                             _stream(stream, dev)),
               "gdn_tree_fork_selective_commit")


def prepare_fork_selective_verify(desc, offsets, parents, confidence, threshold, max_kept, q, k,
                                  v, alpha, beta, S0, o, workspace, tree_status,
                                  stream=None) -> PreparedCall:
    tensors = (offsets, parents, confidence, q, k, v, alpha, beta, S0, o, workspace, tree_status)
    dev, args = _selective_verify_args(desc, offsets, parents, confidence, threshold, max_kept, q,
                                       k, v, alpha, beta, S0, o, workspace, tree_status)
    return PreparedCall("gdn_tree_fork_selective_verify", desc, args, _stream(stream, dev),
                        tensors)


def prepare_fork_selective_commit(desc, offsets, parents, confidence, threshold, max_kept,
                                  accepted, k, v, alpha, beta, S0, S_out, workspace, tree_status,
                                  stream=None) -> PreparedCall:
    tensors = (offsets, parents, confidence, accepted, k, v, alpha, beta, S0, S_out, workspace,
               tree_status)
    dev, args = _selective_commit_args(desc, offsets, parents, confidence, threshold, max_kept,
                                       accepted, k, v, alpha, beta, S0, S_out, workspace,
                                       tree_status)
    return PreparedCall("gdn_tree_fork_selective_commit", desc, args, _stream(stream, dev),
                        tensors)


# ------------------------------------------------------------------ attention layers, batched


def make_attn_layer_io(desc, q=None, k=None, v=None, k_cache=None, v_cache=None,
                       o=None) -> GdnAttnLayerIO:
    """One attention layer's buffers for gdn_tree_attn_commit_layers and a
    captured round (shapes checked against the descriptor)."""
    torch = _torch()
    B, Hq, Hkv, T, d = (desc.num_seqs, desc.num_q_heads, desc.num_kv_heads, desc.total_nodes,
                        desc.head_dim)
    cap = desc.cache_capacity
    bf = torch.bfloat16
    f = lambda t, name, shape: _ptr(t, name, bf, shape, allow_none=True)
    return GdnAttnLayerIO(f(q, "q", (T, Hq, d)), f(k, "k", (T, Hkv, d)), f(v, "v", (T, Hkv, d)),
                          f(k_cache, "k_cache", (B, Hkv, cap, d)),
                          f(v_cache, "v_cache", (B, Hkv, cap, d)), f(o, "o", (T, Hq, d)))


def _attn_layers_array(layers):
    arr = (GdnAttnLayerIO * max(1, len(layers)))()
    for i, ly in enumerate(layers):
        arr[i] = ly
    return arr


def gdn_tree_attn_commit_layers(desc, offsets, parents, accepted, layers, cache_len, tree_status,
                                stream=None):
    """Append the accepted path's K/V rows to every layer's caches (layers:
    GdnAttnLayerIO list sharing cache_len), then advance cache_len once."""
    torch = _torch()
    B, T = desc.num_seqs, desc.total_nodes
    dev = offsets.device
    arr = _attn_layers_array(layers)
    with torch.cuda.device(dev):
        _check(load_library().gdn_tree_attn_commit_layers(
            ctypes.byref(desc), len(layers), _ptr(offsets, "offsets", torch.int32, (B + 1,), dev),
            _ptr(parents, "parents", torch.int32, (T,), dev),
            _ptr(accepted, "accepted", torch.int32, (B,), dev), arr,
            _ptr(cache_len, "cache_len", torch.int32, (B,), dev),
            _ptr(tree_status, "tree_status", torch.int32, (B,), dev), _stream(stream, dev)),
            "gdn_tree_attn_commit_layers")


def prepare_attn_commit_layers(desc, offsets, parents, accepted, layers, cache_len, tree_status,
                               keep=(), stream=None) -> PreparedCall:
    """Marshalled gdn_tree_attn_commit_layers; `keep` holds the tensors behind `layers`."""
    torch = _torch()
    B, T = desc.num_seqs, desc.total_nodes
    dev = offsets.device
    arr = _attn_layers_array(layers)
    args = [ctypes.c_int32(len(layers)), _ptr(offsets, "offsets", torch.int32, (B + 1,), dev),
            _ptr(parents, "parents", torch.int32, (T,), dev),
            _ptr(accepted, "accepted", torch.int32, (B,), dev), arr,
            _ptr(cache_len, "cache_len", torch.int32, (B,), dev),
            _ptr(tree_status, "tree_status", torch.int32, (B,), dev)]
    return PreparedCall("gdn_tree_attn_commit_layers", desc, args, _stream(stream, dev),
                        (offsets, parents, accepted, cache_len, tree_status, arr, tuple(keep)))


# ------------------------------------------------------------------ acceptance and rounds


def gdn_tree_accept_greedy(desc, offsets, parents, draft_tokens, target_tokens, accepted,
                           accept_len, next_token, tree_status, stream=None):
    """Greedy acceptance of every tree: accepted node, path length and the
    target's next token per sequence (int32 tensors)."""
    torch = _torch()
    B, T = desc.num_seqs, desc.total_nodes
    dev = offsets.device
    i32 = torch.int32
    args = [_ptr(offsets, "offsets", i32, (B + 1,), dev), _ptr(parents, "parents", i32, (T,), dev),
            _ptr(draft_tokens, "draft_tokens", i32, (T,), dev),
            _ptr(target_tokens, "target_tokens", i32, (T,), dev),
            _ptr(accepted, "accepted", i32, (B,), dev), _ptr(accept_len, "accept_len", i32, (B,), dev),
            _ptr(next_token, "next_token", i32, (B,), dev),
            _ptr(tree_status, "tree_status", i32, (B,), dev)]
    with torch.cuda.device(dev):
        _check(load_library().gdn_tree_accept_greedy(ctypes.byref(desc), *args,
                                                     _stream(stream, dev)),
               "gdn_tree_accept_greedy")


def gdn_tree_accept_sampling(desc, offsets, parents, draft_tokens, target_probs, draft_probs,
                             uniforms, accepted, accept_len, next_token, tree_status,
                             stream=None):
    """Rejection-sampling acceptance of every tree: target_probs and
    draft_probs [T, V] fp32, uniforms [T, 2] fp32; int32 outputs per sequence."""
    torch = _torch()
    B, T = desc.num_seqs, desc.total_nodes
    dev = offsets.device
    i32, f32 = torch.int32, torch.float32
    V = int(target_probs.shape[-1])
    args = [_ptr(offsets, "offsets", i32, (B + 1,), dev), _ptr(parents, "parents", i32, (T,), dev),
            _ptr(draft_tokens, "draft_tokens", i32, (T,), dev),
            _ptr(target_probs, "target_probs", f32, (T, V), dev),
            _ptr(draft_probs, "draft_probs", f32, (T, V), dev), ctypes.c_int32(V),
            _ptr(uniforms, "uniforms", f32, (T, 2), dev),
            _ptr(accepted, "accepted", i32, (B,), dev), _ptr(accept_len, "accept_len", i32, (B,), dev),
            _ptr(next_token, "next_token", i32, (B,), dev),
            _ptr(tree_status, "tree_status", i32, (B,), dev)]
    with torch.cuda.device(dev):
        _check(load_library().gdn_tree_accept_sampling(ctypes.byref(desc), *args,
                                                       _stream(stream, dev)),
               "gdn_tree_accept_sampling")


def gdn_tree_accept_sampling_split_workspace_bytes(desc, vocab: int) -> int:
    return int(load_library().gdn_tree_accept_sampling_split_workspace_bytes(ctypes.byref(desc),
                                                                            int(vocab)))


def gdn_tree_accept_sampling_splits(desc) -> int:
    """Workgroups per sequence that splits = 0 picks on the current device."""
    return int(load_library().gdn_tree_accept_sampling_splits(ctypes.byref(desc)))


def _sampling_split_args(desc, offsets, parents, draft_tokens, target_probs, draft_probs,
                         uniforms, splits, workspace, accepted, accept_len, next_token,
                         tree_status):
    torch = _torch()
    B, T = desc.num_seqs, desc.total_nodes
    dev = offsets.device
    i32, f32 = torch.int32, torch.float32
    V = int(target_probs.shape[-1])
    return [_ptr(offsets, "offsets", i32, (B + 1,), dev), _ptr(parents, "parents", i32, (T,), dev),
            _ptr(draft_tokens, "draft_tokens", i32, (T,), dev),
            _ptr(target_probs, "target_probs", f32, (T, V), dev),
            _ptr(draft_probs, "draft_probs", f32, (T, V), dev), ctypes.c_int32(V),
            _ptr(uniforms, "uniforms", f32, (T, 2), dev), ctypes.c_int32(int(splits))] + \
        _ws_args(workspace, dev) + \
        [_ptr(accepted, "accepted", i32, (B,), dev), _ptr(accept_len, "accept_len", i32, (B,), dev),
         _ptr(next_token, "next_token", i32, (B,), dev),
         _ptr(tree_status, "tree_status", i32, (B,), dev)]


def gdn_tree_accept_sampling_split(desc, offsets, parents, draft_tokens, target_probs,
                                   draft_probs, uniforms, splits, workspace, accepted, accept_len,
                                   next_token, tree_status, stream=None):
    """gdn_tree_accept_sampling with every row pass spread over `splits`
    workgroups per sequence (0: the device's pick; else 1, 2, 4, 8 or 16);
    workspace: uint8 of gdn_tree_accept_sampling_split_workspace_bytes(desc, V)
    bytes, all zero before its first use (every call leaves it zero), or
    None with splits = 1."""
    torch = _torch()
    dev = offsets.device
    args = _sampling_split_args(desc, offsets, parents, draft_tokens, target_probs, draft_probs,
                                uniforms, splits, workspace, accepted, accept_len, next_token,
                                tree_status)
    with torch.cuda.device(dev):
        _check(load_library().gdn_tree_accept_sampling_split(ctypes.byref(desc), *args,
                                                             _stream(stream, dev)),
               "gdn_tree_accept_sampling_split")


def prepare_accept_sampling_split(desc, offsets, parents, draft_tokens, target_probs,
                                  draft_probs, uniforms, splits, workspace, accepted, accept_len,
                                  next_token, tree_status, stream=None, keep=()):
    """Marshalled gdn_tree_accept_sampling_split."""
    dev = offsets.device
    args = _sampling_split_args(desc, offsets, parents, draft_tokens, target_probs, draft_probs,
                                uniforms, splits, workspace, accepted, accept_len, next_token,
                                tree_status)
    return PreparedCall("gdn_tree_accept_sampling_split", desc, args, _stream(stream, dev),
                        (offsets, parents, draft_tokens, target_probs, draft_probs, uniforms,
                         workspace, accepted, accept_len, next_token, tree_status, tuple(keep)))


def make_round_desc(gdn_desc=None, n_gdn_layers=0, attn_desc=None, n_attn_layers=0) -> GdnRoundDesc:
    return GdnRoundDesc(gdn_desc if gdn_desc is not None else GdnTreeDesc(), int(n_gdn_layers),
                        attn_desc if attn_desc is not None else GdnAttnDesc(), int(n_attn_layers))


def gdn_round_plan(rdesc) -> GdnRoundLayout:
    out = GdnRoundLayout()
    _check(load_library().gdn_round_plan(ctypes.byref(rdesc), ctypes.byref(out)), "gdn_round_plan")
    return out


def gdn_round_tree_for_budget(rdesc, budget_bytes: int, max_depth: int):
    """(branching, depth, nodes, state_bytes) of the largest complete tree
    whose speculative state fits the budget."""
    k, d, n = ctypes.c_int32(), ctypes.c_int32(), ctypes.c_int32()
    nb = ctypes.c_size_t()
    _check(load_library().gdn_round_tree_for_budget(
        ctypes.byref(rdesc), ctypes.c_size_t(int(budget_bytes)), int(max_depth), ctypes.byref(k),
        ctypes.byref(d), ctypes.byref(n), ctypes.byref(nb)), "gdn_round_tree_for_budget")
    return k.value, d.value, n.value, nb.value


class RoundGraph:
    """One speculative round (every layer's verify in model order, greedy
    acceptance, every layer's commit) recorded once with gdn_round_capture on
    `stream` (a torch.cuda.Stream, not the null stream) and replayed with
    launch(). The tensors passed here are checked and kept alive by the
    object; the layer descriptions (GdnLayerIO, GdnAttnLayerIO) hold raw
    pointers only, so the tensors behind them must be passed in `keep` (or
    otherwise outlive the object). The graph reads every buffer's contents
    at each launch."""

    def __init__(self, rdesc, offsets, parents, gdn_layers, attn_layers, arena, draft_tokens,
                 target_tokens, accepted, accept_len, next_token, tree_status, cache_len=None,
                 layer_kinds=None, attn_scale=None, stream=None, keep=(), prev=None):
        """prev: None, or a dict for gdn_round_capture_replay (the previous
        round committed by replay inside this round's GDN verifies): "desc"
        (its GdnTreeDesc), "offsets", "parents", "accepted" (tensors) and
        "gdn_layers" (GdnLayerIO list with k, v, alpha, beta)."""
        torch = _torch()
        g, a = rdesc.gdn, rdesc.attn
        B = g.num_seqs if rdesc.n_gdn_layers > 0 else a.num_seqs
        T = g.total_nodes if rdesc.n_gdn_layers > 0 else a.total_nodes
        if len(gdn_layers) != rdesc.n_gdn_layers or len(attn_layers) != rdesc.n_attn_layers:
            raise ValueError("layer lists do not match the round descriptor")
        dev = offsets.device
        i32 = torch.int32
        self._rdesc = GdnRoundDesc.from_buffer_copy(rdesc)
        self._gdn = _layers_array(gdn_layers)
        self._attn = _attn_layers_array(attn_layers)
        kinds = None
        if layer_kinds is not None:
            kinds = (ctypes.c_int32 * max(1, len(layer_kinds)))(*[int(x) for x in layer_kinds])
        self._kinds = kinds
        scale = (a.head_dim ** -0.5 if a.head_dim > 0 else 1.0) if attn_scale is None else attn_scale
        io = GdnRoundIO()
        io.offsets = _ptr(offsets, "offsets", i32, (B + 1,), dev)
        io.parents = _ptr(parents, "parents", i32, (T,), dev)
        io.gdn_layers = ctypes.cast(self._gdn, ctypes.POINTER(GdnLayerIO))
        io.attn_layers = ctypes.cast(self._attn, ctypes.POINTER(GdnAttnLayerIO))
        io.layer_kinds = ctypes.cast(kinds, ctypes.POINTER(ctypes.c_int32)) if kinds else None
        io.cache_len = _ptr(cache_len, "cache_len", i32, (B,), dev, allow_none=True)
        io.attn_scale = float(scale)
        io.arena = _ptr(arena, "arena", torch.uint8, None, dev, allow_none=True)
        io.arena_bytes = 0 if arena is None else arena.numel()
        io.draft_tokens = _ptr(draft_tokens, "draft_tokens", i32, (T,), dev)
        io.target_tokens = _ptr(target_tokens, "target_tokens", i32, (T,), dev)
        io.accepted = _ptr(accepted, "accepted", i32, (B,), dev)
        io.accept_len = _ptr(accept_len, "accept_len", i32, (B,), dev)
        io.next_token = _ptr(next_token, "next_token", i32, (B,), dev)
        io.tree_status = _ptr(tree_status, "tree_status", i32, (B,), dev)
        self._io = io
        self._keep = (offsets, parents, arena, draft_tokens, target_tokens, accepted, accept_len,
                      next_token, tree_status, cache_len, tuple(keep))
        self._lib = load_library()
        self._handle = ctypes.c_void_p()
        s = torch.cuda.current_stream(dev) if stream is None else stream
        self._prev = None
        if prev is not None:
            pd = prev["desc"]
            if len(prev["gdn_layers"]) != rdesc.n_gdn_layers:
                raise ValueError("prev gdn_layers do not match the round descriptor")
            pr = GdnRoundPrev()
            pr.gdn = type(pd).from_buffer_copy(pd)
            pr.offsets = _ptr(prev["offsets"], "prev offsets", i32, (pd.num_seqs + 1,), dev)
            pr.parents = _ptr(prev["parents"], "prev parents", i32, (pd.total_nodes,), dev)
            pr.accepted = _ptr(prev["accepted"], "prev accepted", i32, (pd.num_seqs,), dev)
            self._prev_layers = _layers_array(prev["gdn_layers"])
            pr.gdn_layers = ctypes.cast(self._prev_layers, ctypes.POINTER(GdnLayerIO))
            self._prev = pr
            self._keep = self._keep + ((prev["offsets"], prev["parents"], prev["accepted"]),)
        with torch.cuda.device(dev):
            if self._prev is None:
                _check(self._lib.gdn_round_capture(ctypes.byref(self._rdesc), ctypes.byref(io),
                                                   ctypes.c_void_p(s.cuda_stream),
                                                   ctypes.byref(self._handle)),
                       "gdn_round_capture")
            else:
                _check(self._lib.gdn_round_capture_replay(
                    ctypes.byref(self._rdesc), ctypes.byref(io), ctypes.byref(self._prev),
                    ctypes.c_void_p(s.cuda_stream), ctypes.byref(self._handle)),
                    "gdn_round_capture_replay")
        self._dev = dev

    def launch(self, stream=None):
        if not self._handle:
            raise RuntimeError("round graph already destroyed")
        _check(self._lib.gdn_round_launch(self._handle, _stream(stream, self._dev)),
               "gdn_round_launch")

    def close(self):
        if self._handle:
            self._lib.gdn_round_destroy(self._handle)
            self._handle = ctypes.c_void_p()

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

"""Helpers for the GPU parity tests: move a seeded workload to the device, run
the library through its C ABI binding, bring results back, and compare with
the oracle using the normwise relative error the tolerances are stated in."""
from __future__ import annotations

import numpy as np
import torch

import gated_deltanet_tree_02_amd as gt
import gdn_inputs as gi
import oracle

TOL = {"f32": 1e-4, "bf16": 2e-2}


def dev():
    return torch.device("cuda:0")


def to_dev_io(x: np.ndarray, io: str) -> torch.Tensor:
    if io == "bf16":
        bits = gi.bf16_bits(x)
        return torch.from_numpy(bits.view(np.int16)).to(dev()).view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(x, np.float32)).to(dev())


def from_dev_io(t: torch.Tensor) -> np.ndarray:
    if t.dtype == torch.bfloat16:
        bits = t.view(torch.int16).cpu().numpy().view(np.uint16)
        return gi.bf16_bits_to_f32(bits)
    return t.cpu().numpy()


def f32(x) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(x, np.float32)).to(dev())


def i32(x) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(x, np.int32)).to(dev())


def nan_bytes(nbytes: int) -> torch.Tensor:
    """A workspace of nbytes (at least 4) filled with fp32 NaN patterns, so
    that any part a kernel reads without having written it shows up in the
    results."""
    n = max(4, (nbytes + 3) // 4 * 4)
    return torch.full((n // 4,), float("nan"), device=dev()).view(torch.uint8)[:max(nbytes, 1)]


class DeviceLayer:
    """One layer of a workload resident on the GPU, plus outputs/workspace."""

    def __init__(self, w: gi.Workload, layer: int = 0, mode: int = gt.MODE_WY,
                 max_nodes: int | None = None, max_depth: int = 0):
        self.w, self.layer = w, layer
        self.desc = gt.make_desc(w.B, w.H, w.dk, w.dv, w.T,
                                 max_nodes if max_nodes is not None else max(1, min(64, w.max_nodes)),
                                 gt.DTYPE_BF16 if w.io == "bf16" else gt.DTYPE_F32, mode, max_depth)
        self.offsets = i32(w.offsets)
        self.parents = i32(w.parents)
        self.accepted = i32(w.accepted)
        self.q = to_dev_io(w.q[layer], w.io)
        self.k = to_dev_io(w.k[layer], w.io)
        self.v = to_dev_io(w.v[layer], w.io)
        self.alpha = f32(w.alpha[layer])
        self.beta = f32(w.beta[layer])
        self.S0 = f32(w.S0[layer])
        self.o = torch.full_like(self.v, float("nan"))
        nbytes = gt.gdn_tree_workspace_bytes(self.desc)
        self.ws = nan_bytes(nbytes)
        self.status = torch.full((w.B,), -7, dtype=torch.int32, device=dev())
        self.S_out = torch.full_like(self.S0, float("nan"))

    def verify(self):
        gt.gdn_tree_verify(self.desc, self.offsets, self.parents, self.q, self.k, self.v,
                           self.alpha, self.beta, self.S0, self.o, self.ws, self.status)

    def commit(self, S_out=None):
        gt.gdn_tree_commit(self.desc, self.offsets, self.parents, self.accepted, self.k, self.S0,
                           self.S_out if S_out is None else S_out, self.ws, self.status)

    def o_np(self):
        return from_dev_io(self.o).astype(np.float64)

    def wy_parts(self):
        """(U [T,H,dv], g2 [T,H]) from the WY workspace."""
        T, H, dv = self.w.T, self.w.H, self.w.dv
        ub = (T * H * dv * 4 + 255) // 256 * 256
        raw = self.ws.cpu().numpy()
        U = raw[:T * H * dv * 4].view(np.float32).reshape(T, H, dv)
        g2 = raw[ub:ub + T * H * 4].view(np.float32).reshape(T, H)
        return U, g2


def oracle_layer(w: gi.Workload, layer: int = 0, max_nodes: int = 64):
    o, st = oracle.verify(w.offsets, w.parents, w.q[layer], w.k[layer], w.v[layer],
                          w.alpha[layer], w.beta[layer], w.S0[layer], max_nodes=max_nodes)
    S, stc = oracle.commit(w.offsets, w.parents, w.accepted, w.k[layer], w.v[layer],
                           w.alpha[layer], w.beta[layer], w.S0[layer], max_nodes=max_nodes)
    return o, st, S, stc


def rel_err_rows(got: np.ndarray, ref: np.ndarray) -> float:
    """max over vectors (last axis) of ||got - ref|| / ||ref||; all-zero
    reference vectors must be matched exactly."""
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    g = got.reshape(-1, got.shape[-1])
    r = ref.reshape(-1, ref.shape[-1])
    num = np.linalg.norm(g - r, axis=1)
    den = np.linalg.norm(r, axis=1)
    zero = den == 0
    if np.any(num[zero] != 0):
        return float("inf")
    if np.all(zero):
        return 0.0
    return float(np.max(num[~zero] / den[~zero]))


def rel_err_states(got: np.ndarray, ref: np.ndarray) -> float:
    """max over (b,h) of Frobenius-norm relative error."""
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    g = got.reshape(got.shape[0] * got.shape[1], -1)
    r = ref.reshape(ref.shape[0] * ref.shape[1], -1)
    return rel_err_rows(g, r)


def sub_workload(w: gi.Workload, seqs, layers=None, heads=None) -> gi.Workload:
    """The listed sequences (and layers/heads) of a workload, renumbered."""
    seqs = list(seqs)
    layers = list(range(w.layers)) if layers is None else list(layers)
    heads = list(range(w.H)) if heads is None else list(heads)
    rows = np.concatenate([np.arange(w.offsets[b], w.offsets[b + 1]) for b in seqs])
    sizes = [int(w.offsets[b + 1] - w.offsets[b]) for b in seqs]
    offsets = np.zeros(len(seqs) + 1, np.int32)
    offsets[1:] = np.cumsum(sizes)
    L = np.array(layers)[:, None]
    return gi.Workload(
        B=len(seqs), H=len(heads), dk=w.dk, dv=w.dv, io=w.io, layers=len(layers),
        parents_list=[w.parents_list[b] for b in seqs], offsets=offsets,
        parents=w.parents[rows].copy(), accepted=w.accepted[seqs].copy(),
        q=w.q[L, rows][:, :, heads].copy(), k=w.k[L, rows][:, :, heads].copy(),
        v=w.v[L, rows][:, :, heads].copy(), alpha=w.alpha[L, rows][:, :, heads].copy(),
        beta=w.beta[L, rows][:, :, heads].copy(),
        S0=w.S0[L, np.array(seqs)][:, :, heads].copy())


# ------------------------------------------------------------------ attention layers


def bits_to_dev(bits: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(dev()).view(torch.bfloat16)


def dev_to_bits(t: torch.Tensor) -> np.ndarray:
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


class DeviceAttn:
    """One attention layer's inputs on the GPU, outputs and workspace."""

    def __init__(self, w: gi.AttnWorkload, max_nodes: int | None = None,
                 max_cache_len: int | None = None):
        self.w = w
        lens = w.cache_len
        mcl = max_cache_len if max_cache_len is not None else (
            int(min(max(lens.max(initial=0), 0), w.cap)))
        self.desc = gt.make_attn_desc(w.B, w.Hq, w.Hkv, w.d, w.T,
                                      max_nodes if max_nodes is not None else min(64, w.max_nodes),
                                      w.cap, mcl)
        self.offsets = i32(w.offsets)
        self.parents = i32(w.parents)
        self.accepted = i32(w.accepted)
        self.cache_len = i32(w.cache_len)
        self.q = to_dev_io(w.q, "bf16")
        self.k = to_dev_io(w.k, "bf16")
        self.v = to_dev_io(w.v, "bf16")
        self.kc = bits_to_dev(w.kc_bits)
        self.vc = bits_to_dev(w.vc_bits)
        self.o = torch.full_like(self.q, float("nan"))
        nbytes = gt.gdn_tree_attn_workspace_bytes(self.desc)
        self.ws = nan_bytes(nbytes) if nbytes else None
        self.status = torch.full((w.B,), -7, dtype=torch.int32, device=dev())

    def verify(self, scale=None):
        gt.gdn_tree_attn_verify(self.desc, self.offsets, self.parents, self.q, self.k, self.v,
                                self.kc, self.vc, self.cache_len, self.o, self.ws, self.status,
                                scale=scale)

    def commit(self):
        gt.gdn_tree_attn_commit(self.desc, self.offsets, self.parents, self.accepted, self.k,
                                self.v, self.kc, self.vc, self.cache_len, self.status)

    def o_np(self):
        return from_dev_io(self.o).astype(np.float64)


def attn_sub(w: gi.AttnWorkload, seqs) -> gi.AttnWorkload:
    """The listed sequences of an attention workload, renumbered."""
    seqs = list(seqs)
    rows = np.concatenate([np.arange(w.offsets[b], w.offsets[b + 1]) for b in seqs])
    sizes = [int(w.offsets[b + 1] - w.offsets[b]) for b in seqs]
    offsets = np.zeros(len(seqs) + 1, np.int32)
    offsets[1:] = np.cumsum(sizes)
    idx = np.array(seqs)
    return gi.AttnWorkload(
        B=len(seqs), Hq=w.Hq, Hkv=w.Hkv, d=w.d, cap=w.cap,
        parents_list=[w.parents_list[b] for b in seqs], offsets=offsets,
        parents=w.parents[rows].copy(), accepted=w.accepted[idx].copy(),
        cache_len=w.cache_len[idx].copy(), q=w.q[rows].copy(), k=w.k[rows].copy(),
        v=w.v[rows].copy(), kc_bits=w.kc_bits[idx].copy(), vc_bits=w.vc_bits[idx].copy())


def oracle_attn(w: gi.AttnWorkload, max_nodes: int = 64, scale=None):
    kc, vc = w.cache_values()
    return oracle.tree_attn(w.offsets, w.parents, w.q, w.k, w.v, kc, vc, w.cache_len,
                            scale=scale, max_nodes=max_nodes)


def oracle_attn_commit(w: gi.AttnWorkload, max_nodes: int = 64):
    kc, vc = w.cache_values()
    return oracle.tree_attn_commit(w.offsets, w.parents, w.accepted, w.k, w.v, kc, vc,
                                   w.cache_len, max_nodes=max_nodes)

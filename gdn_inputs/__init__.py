"""Seeded synthetic inputs for tree-verified Gated DeltaNet layers.

This module is shared by the oracle-side tests and the GPU path. It holds no
arithmetic of the method itself: it only draws trees, per-node vectors, gates,
states and accepted nodes, and rounds the drawn values to the storage dtype.

Workload shapes follow the pages:
  * the Qwen3.5-9B GDN layer shape, 24 GDN layers x 16 key heads x a 128x128
    state (rainlin-top "Qwen3.5 tree spec", section 6 "overhead analysis",
    memory part);
  * the k=2/d=2 tree with nodes root,A,B,C,D,E,F and the accepted path
    root->A->C (same page, section 4 "Fork/Checkpoint" and section 5
    "dual use of checkpoints");
  * k-ary trees of 7/15/40 nodes (same page, section 6 table and section 8);
  * per-level branching lists such as [2,2,1,1] (anrans handbook
    "speculative" chapter, "implementation" section and exercise 1).

Value distributions (q,k ~ N(0,1) then L2-normalised, v ~ N(0,1),
alpha ~ U(0.9,1), beta = sigmoid(N(0,1)), S0 ~ N(0, 0.1^2)) are the synthetic
recipe of the five workload configurations this library is measured on.

The full-attention layers of the same hybrid stack (rainlin-top "Qwen3.5 tree
spec", section 3: one attention layer after every three GDN layers) get their
own workloads (ATTN_CONFIGS): q, k, v and the committed K/V cache ~ N(0,1)
per element, bf16, so scaled scores are O(1) as after the per-head norms of
the handbook's reference model; cache rows past a sequence's committed length
hold values too, which verification must never read into a result.
"""
from __future__ import annotations

import concurrent.futures
import dataclasses
import os
from typing import List, Optional, Sequence

import numpy as np

__all__ = [
    "CONFIGS", "Workload", "kary_parents", "chain_parents", "branching_parents",
    "random_tree_parents", "make_workload", "make_config", "round_to_bf16",
    "bf16_bits", "bf16_bits_to_f32", "path_to_root", "pick_accepted",
    "ATTN_CONFIGS", "AttnWorkload", "make_attn_workload", "make_attn_config",
]

# ---------------------------------------------------------------------------
# bf16 rounding (storage format only): round-to-nearest-even of an fp32 value
# to its upper 16 bits, as the bf16 format defines it.
# ---------------------------------------------------------------------------


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """fp32 array -> uint16 bf16 bit patterns, round to nearest even."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    lsb = (u >> 16) & 1
    r = (u + 0x7FFF + lsb) >> 16
    out = r.astype(np.uint16)
    nan = np.isnan(x)
    if nan.any():
        out[nan] = 0x7FC0
    return out


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def round_to_bf16(x: np.ndarray) -> np.ndarray:
    """fp32 values rounded to bf16 and widened back to fp32 (exact)."""
    return bf16_bits_to_f32(bf16_bits(x))


# ---------------------------------------------------------------------------
# Tree shapes. Every tree is a parents list in topological order: node 0 is
# the root with parent -1, and every other node's parent has a smaller index.
# ---------------------------------------------------------------------------


def kary_parents(k: int, d: int) -> List[int]:
    """Complete k-ary tree of depth d (root = depth 0) in BFS order."""
    n = sum(k ** i for i in range(d + 1))
    return [-1] + [(i - 1) // k for i in range(1, n)]


def chain_parents(n: int) -> List[int]:
    return [-1] + list(range(n - 1))


def branching_parents(branching: Sequence[int]) -> List[int]:
    """Level-by-level expansion: every frontier node gets branching[l] children."""
    parents, frontier = [-1], [0]
    for width in branching:
        nxt = []
        for node in frontier:
            for _ in range(width):
                parents.append(node)
                nxt.append(len(parents) - 1)
        frontier = nxt
    return parents


def random_tree_parents(rng: np.random.Generator, nmin: int = 16, nmax: int = 64,
                        max_depth: int = 6, max_children: int = 4) -> List[int]:
    """Dynamic (EAGLE-2-like) draft tree: size ~ U{nmin..nmax}; each new node
    hangs under a uniformly chosen earlier node that is shallower than
    max_depth and has fewer than max_children children."""
    n = int(rng.integers(nmin, nmax + 1))
    parents, level, nchild = [-1], [0], [0]
    for _ in range(1, n):
        open_nodes = [j for j in range(len(parents))
                      if level[j] < max_depth and nchild[j] < max_children]
        p = int(open_nodes[int(rng.integers(len(open_nodes)))])
        parents.append(p)
        level.append(level[p] + 1)
        nchild.append(0)
        nchild[p] += 1
    return parents


def path_to_root(parents: Sequence[int], node: int) -> List[int]:
    """Nodes from the root down to `node` (inclusive)."""
    out = []
    while node != -1:
        out.append(node)
        node = parents[node]
    return out[::-1]


def pick_accepted(rng: np.random.Generator, parents: Sequence[int]) -> int:
    """Uniform leaf, then a uniform accepted prefix length along its path."""
    n = len(parents)
    has_child = [False] * n
    for p in parents[1:]:
        has_child[p] = True
    leaves = [i for i in range(n) if not has_child[i]]
    leaf = leaves[int(rng.integers(len(leaves)))]
    path = path_to_root(parents, leaf)
    length = int(rng.integers(1, len(path) + 1))
    return path[length - 1]


# ---------------------------------------------------------------------------
# Workloads
# ---------------------------------------------------------------------------

CONFIGS = {
    "c1": dict(desc="tiny: 1 seq, 1 head, dk=dv=32, fp32, tree k=2 d=2 (7 nodes)",
               B=1, H=1, dk=32, dv=32, io="f32", layers=1, tree="fixed",
               parents=[-1, 0, 0, 1, 1, 2, 2], accepted="fixed", accepted_node=3, seed=0),
    "c2": dict(desc="chain gamma=5 (6 nodes incl. root), B=1, 16 heads, 128x128, bf16 io",
               B=1, H=16, dk=128, dv=128, io="bf16", layers=1, tree="chain", n=6,
               accepted="leafprefix", seed=1),
    "c3": dict(desc="tree k=2 d=3 (15 nodes), B=32, 16 heads, 128x128, bf16 io",
               B=32, H=16, dk=128, dv=128, io="bf16", layers=1, tree="kary", k=2, d=3,
               accepted="leafprefix", seed=2),
    "c4": dict(desc="tree k=3 d=3 (40 nodes), 24 GDN layers, B=64, 16 heads, 128x128, bf16 io",
               B=64, H=16, dk=128, dv=128, io="bf16", layers=24, tree="kary", k=3, d=3,
               accepted="leafprefix", seed=3),
    "c5": dict(desc="ragged random trees 16-64 nodes, depth<=6, 1-4 children, B=128, 16 heads, bf16 io",
               B=128, H=16, dk=128, dv=128, io="bf16", layers=1, tree="random",
               nmin=16, nmax=64, max_depth=6, max_children=4,
               accepted="leafprefix", seed=4),
}


@dataclasses.dataclass
class Workload:
    """All inputs of one batch. Float tensors hold the exact stored values
    (bf16-representable when io == 'bf16'); *_bits hold the bf16 bit patterns."""
    B: int
    H: int
    dk: int
    dv: int
    io: str
    layers: int
    parents_list: List[List[int]]
    offsets: np.ndarray          # [B+1] int32
    parents: np.ndarray          # [T] int32, local indices, root -1
    accepted: np.ndarray         # [B] int32, local index of the last accepted node
    q: np.ndarray                # [L,T,H,dk] float32
    k: np.ndarray                # [L,T,H,dk] float32
    v: np.ndarray                # [L,T,H,dv] float32
    alpha: np.ndarray            # [L,T,H] float32
    beta: np.ndarray             # [L,T,H] float32
    S0: np.ndarray               # [L,B,H,dv,dk] float32, S[r][c] multiplies k[c]

    @property
    def T(self) -> int:
        return int(self.offsets[-1])

    @property
    def max_nodes(self) -> int:
        return max(len(p) for p in self.parents_list) if self.parents_list else 1

    def max_depth(self) -> int:
        best = 0
        for p in self.parents_list:
            lvl = [0] * len(p)
            for i in range(1, len(p)):
                lvl[i] = lvl[p[i]] + 1
            best = max(best, max(lvl))
        return best

    def io_bits(self, name: str, layer: int = 0) -> np.ndarray:
        return bf16_bits(getattr(self, name)[layer])


def _unit_rows(rng: np.random.Generator, shape) -> np.ndarray:
    x = rng.standard_normal(shape, dtype=np.float32)
    n = np.sqrt(np.sum(x * x, axis=-1, keepdims=True, dtype=np.float32))
    return (x / n).astype(np.float32)


def _draw_layer(seed_seq: np.random.SeedSequence, T: int, B: int, H: int, dk: int, dv: int,
                io: str, s0_std: float):
    """One layer's q, k, v, alpha, beta, S0; each tensor from its own child
    stream, so layers can be drawn in any order or in parallel."""
    sq, sk, sv, sa, sb, ss = (np.random.Generator(np.random.PCG64(c)) for c in seed_seq.spawn(6))
    q = _unit_rows(sq, (T, H, dk))
    k = _unit_rows(sk, (T, H, dk))
    v = sv.standard_normal((T, H, dv), dtype=np.float32)
    if io == "bf16":
        q, k, v = round_to_bf16(q), round_to_bf16(k), round_to_bf16(v)
    alpha = sa.uniform(0.9, 1.0, size=(T, H)).astype(np.float32)
    logits = sb.standard_normal((T, H))
    beta = (1.0 / (1.0 + np.exp(-logits))).astype(np.float32)
    S0 = ss.standard_normal((B, H, dv, dk), dtype=np.float32)
    S0 *= np.float32(s0_std)
    return q, k, v, alpha, beta, S0


def make_workload(parents_list: Sequence[Sequence[int]], H: int, dk: int, dv: int,
                  io: str = "bf16", layers: int = 1, seed=0,
                  accepted: Optional[Sequence[int]] = None,
                  s0_std: float = 0.1, threads: int = 0) -> Workload:
    """Draw every per-layer input for the given trees.

    Seeding: SeedSequence(seed) (or the SeedSequence passed as seed) spawns a
    layer parent and an accepted-node child; the layer parent spawns one child
    per layer, which spawns q, k, v, alpha, beta logits and S0 in that order.
    Layer i's values therefore do not depend on how many layers are drawn."""
    parents_list = [list(map(int, p)) for p in parents_list]
    B = len(parents_list)
    sizes = [len(p) for p in parents_list]
    offsets = np.zeros(B + 1, dtype=np.int32)
    offsets[1:] = np.cumsum(sizes)
    T = int(offsets[-1])
    parents = np.array([x for p in parents_list for x in p], dtype=np.int32)
    L = layers
    root = seed if isinstance(seed, np.random.SeedSequence) else np.random.SeedSequence(seed)
    layer_parent, acc_seed = root.spawn(2)
    children = layer_parent.spawn(L)
    q = np.empty((L, T, H, dk), np.float32)
    k = np.empty((L, T, H, dk), np.float32)
    v = np.empty((L, T, H, dv), np.float32)
    alpha = np.empty((L, T, H), np.float32)
    beta = np.empty((L, T, H), np.float32)
    S0 = np.empty((L, B, H, dv, dk), np.float32)

    def one(layer):
        q[layer], k[layer], v[layer], alpha[layer], beta[layer], S0[layer] = _draw_layer(
            children[layer], T, B, H, dk, dv, io, s0_std)

    nthreads = threads or min(L, os.cpu_count() or 1, 16)
    if nthreads > 1:
        with concurrent.futures.ThreadPoolExecutor(nthreads) as ex:
            list(ex.map(one, range(L)))
    else:
        for layer in range(L):
            one(layer)
    if accepted is None:
        arng = np.random.Generator(np.random.PCG64(acc_seed))
        acc = np.array([pick_accepted(arng, p) for p in parents_list], dtype=np.int32)
    else:
        acc = np.asarray(accepted, dtype=np.int32)
    return Workload(B=B, H=H, dk=dk, dv=dv, io=io, layers=L, parents_list=parents_list,
                    offsets=offsets, parents=parents, accepted=acc, q=q, k=k, v=v,
                    alpha=alpha, beta=beta, S0=S0)


def config_trees(name: str, rng: np.random.Generator) -> List[List[int]]:
    c = CONFIGS[name]
    if c["tree"] == "fixed":
        return [list(c["parents"]) for _ in range(c["B"])]
    if c["tree"] == "chain":
        return [chain_parents(c["n"]) for _ in range(c["B"])]
    if c["tree"] == "kary":
        return [kary_parents(c["k"], c["d"]) for _ in range(c["B"])]
    if c["tree"] == "random":
        return [random_tree_parents(rng, c["nmin"], c["nmax"], c["max_depth"], c["max_children"])
                for _ in range(c["B"])]
    raise ValueError(c["tree"])


def make_config(name: str, layers: Optional[int] = None, seed: Optional[int] = None) -> Workload:
    """One of the five workload configurations. `layers` keeps only the first
    layers (the values drawn for them do not change)."""
    c = CONFIGS[name]
    tree_seed, data_seed = np.random.SeedSequence(c["seed"] if seed is None else seed).spawn(2)
    trees = config_trees(name, np.random.Generator(np.random.PCG64(tree_seed)))
    acc = [c["accepted_node"]] * len(trees) if c["accepted"] == "fixed" else None
    return make_workload(trees, H=c["H"], dk=c["dk"], dv=c["dv"], io=c["io"],
                         layers=c["layers"] if layers is None else layers, seed=data_seed,
                         accepted=acc)


# ---------------------------------------------------------------------------
# Full-attention layer workloads (tree-masked attention verify and the KV
# commit). The pages give no attention head shape; these use 16 query heads
# sharing 4 K/V heads of size 128 beside the 16-head GDN layers.
# ---------------------------------------------------------------------------

ATTN_CONFIGS = {
    "fa_small": dict(desc="8 seqs, tree k=2 d=3 (15 nodes), Hq=16, Hkv=4, d=128, "
                          "ragged cached prefixes 0..600 (cap 640)",
                     B=8, Hq=16, Hkv=4, d=128, tree="kary", k=2, depth=3, cap=640,
                     lens=("uniform", 0, 600), seed=11),
    "fa_c4": dict(desc="64 seqs, tree k=3 d=3 (40 nodes), Hq=16, Hkv=4, d=128, "
                       "cached prefix 4096 per sequence (cap 4160)",
                  B=64, Hq=16, Hkv=4, d=128, tree="kary", k=3, depth=3, cap=4160,
                  lens=("fixed", 4096), seed=12),
}


@dataclasses.dataclass
class AttnWorkload:
    """Inputs of one full-attention layer under a draft tree. q, k, v hold the
    exact stored values (bf16-representable fp32); the caches are kept as bf16
    bit patterns [B, Hkv, cap, d] (cache_values widens one sequence)."""
    B: int
    Hq: int
    Hkv: int
    d: int
    cap: int
    parents_list: List[List[int]]
    offsets: np.ndarray          # [B+1] int32
    parents: np.ndarray          # [T] int32
    accepted: np.ndarray         # [B] int32
    cache_len: np.ndarray        # [B] int32
    q: np.ndarray                # [T, Hq, d] float32
    k: np.ndarray                # [T, Hkv, d] float32
    v: np.ndarray                # [T, Hkv, d] float32
    kc_bits: np.ndarray          # [B, Hkv, cap, d] uint16
    vc_bits: np.ndarray          # [B, Hkv, cap, d] uint16

    @property
    def T(self) -> int:
        return int(self.offsets[-1])

    @property
    def max_nodes(self) -> int:
        return max(len(p) for p in self.parents_list) if self.parents_list else 1

    def cache_values(self, seqs=None):
        """(k_cache, v_cache) as float32 for the listed sequences (all by default)."""
        idx = slice(None) if seqs is None else np.asarray(list(seqs))
        return bf16_bits_to_f32(self.kc_bits[idx]), bf16_bits_to_f32(self.vc_bits[idx])


def make_attn_workload(parents_list: Sequence[Sequence[int]], Hq: int, Hkv: int, d: int,
                       cap: int, cache_len: Sequence[int], seed=0,
                       accepted: Optional[Sequence[int]] = None,
                       threads: int = 0) -> AttnWorkload:
    """Draw q, k, v and both caches for the given trees and committed lengths.

    Seeding: SeedSequence(seed) spawns (q, k, v, accepted, caches); the cache
    child spawns one child per sequence, which draws that sequence's K then V
    cache rows, so a sequence's cache does not depend on the batch size."""
    parents_list = [list(map(int, p)) for p in parents_list]
    B = len(parents_list)
    offsets = np.zeros(B + 1, dtype=np.int32)
    offsets[1:] = np.cumsum([len(p) for p in parents_list])
    T = int(offsets[-1])
    parents = np.array([x for p in parents_list for x in p], dtype=np.int32)
    root = seed if isinstance(seed, np.random.SeedSequence) else np.random.SeedSequence(seed)
    sq, sk, sv, sa, sc = root.spawn(5)
    draw = lambda ss, shape: round_to_bf16(
        np.random.Generator(np.random.PCG64(ss)).standard_normal(shape, dtype=np.float32))
    q = draw(sq, (T, Hq, d))
    k = draw(sk, (T, Hkv, d))
    v = draw(sv, (T, Hkv, d))
    kc = np.empty((B, Hkv, cap, d), np.uint16)
    vc = np.empty((B, Hkv, cap, d), np.uint16)
    children = sc.spawn(B)

    def one(b):
        g = np.random.Generator(np.random.PCG64(children[b]))
        kc[b] = bf16_bits(g.standard_normal((Hkv, cap, d), dtype=np.float32))
        vc[b] = bf16_bits(g.standard_normal((Hkv, cap, d), dtype=np.float32))

    nthreads = threads or min(B, os.cpu_count() or 1, 16)
    if nthreads > 1:
        with concurrent.futures.ThreadPoolExecutor(nthreads) as ex:
            list(ex.map(one, range(B)))
    else:
        for b in range(B):
            one(b)
    if accepted is None:
        arng = np.random.Generator(np.random.PCG64(sa))
        acc = np.array([pick_accepted(arng, p) for p in parents_list], dtype=np.int32)
    else:
        acc = np.asarray(accepted, dtype=np.int32)
    return AttnWorkload(B=B, Hq=Hq, Hkv=Hkv, d=d, cap=cap, parents_list=parents_list,
                        offsets=offsets, parents=parents, accepted=acc,
                        cache_len=np.asarray(cache_len, np.int32), q=q, k=k, v=v,
                        kc_bits=kc, vc_bits=vc)


def make_attn_config(name: str, seed: Optional[int] = None) -> AttnWorkload:
    c = ATTN_CONFIGS[name]
    tree_seed, data_seed = np.random.SeedSequence(c["seed"] if seed is None else seed).spawn(2)
    rng = np.random.Generator(np.random.PCG64(tree_seed))
    trees = [kary_parents(c["k"], c["depth"]) for _ in range(c["B"])]
    kind = c["lens"][0]
    if kind == "fixed":
        lens = [c["lens"][1]] * c["B"]
    else:
        lens = rng.integers(c["lens"][1], c["lens"][2] + 1, size=c["B"]).tolist()
    return make_attn_workload(trees, c["Hq"], c["Hkv"], c["d"], c["cap"], lens, seed=data_seed)


# ---------------------------------------------------------------------------
# Draft and target tokens for acceptance
# ---------------------------------------------------------------------------


def draft_confidences(rng: np.random.Generator, parents_list: Sequence[Sequence[int]],
                      p_dominant: float = 0.5) -> np.ndarray:
    """The draft model's confidence in every node's token, as float32 [T]
    (the input of a selective fork). Siblings are alternatives drawn from one
    distribution, so their confidences share a unit of mass: with probability
    p_dominant a node's first child takes U(0.95, 1] of it (a dominant token)
    and the others split the rest (Dirichlet(1, ...)); otherwise the children
    and the undrafted remainder split the unit uniformly (Dirichlet over
    children + 1 parts). The root, the token the target itself emitted, has
    confidence 1."""
    out = []
    for parents in parents_list:
        n = len(parents)
        conf = np.zeros(n, np.float64)
        conf[0] = 1.0
        children = [[] for _ in range(n)]
        for c in range(1, n):
            children[parents[c]].append(c)
        for kids in children:
            if not kids:
                continue
            if rng.random() < p_dominant:
                top = 0.95 + 0.05 * (1.0 - rng.random())
                conf[kids[0]] = top
                if len(kids) > 1:
                    conf[kids[1:]] = (1.0 - top) * rng.dirichlet(np.ones(len(kids)))[:-1]
            else:
                conf[kids] = rng.dirichlet(np.ones(len(kids) + 1))[:-1]
        out.append(conf)
    return np.concatenate(out).astype(np.float32)


def draft_target_tokens(rng: np.random.Generator, parents_list: Sequence[Sequence[int]],
                        accepted: Sequence[int], vocab: int = 32000):
    """Token ids for a batch of trees: draft tokens distinct among the
    children of every node (a top-k expansion proposes distinct tokens), and
    the target model's predicted next token at every node, drawn so that the
    prediction names the next node of the given accepted path along it, and
    names none of a node's children elsewhere (a prediction outside the tree).
    Returns (draft [T], target [T]) int32; accepted[b] = -1 draws predictions
    that match no child anywhere."""
    drafts, targets = [], []
    for parents, a in zip(parents_list, accepted):
        n = len(parents)
        children = [[] for _ in range(n)]
        for c in range(1, n):
            children[parents[c]].append(c)
        draft = np.zeros(n, np.int64)
        draft[0] = int(rng.integers(vocab))
        for p in range(n):
            if children[p]:
                draft[children[p]] = rng.choice(vocab, size=len(children[p]), replace=False)
        nxt = {}
        if a >= 0:
            path = path_to_root(parents, int(a))
            nxt = {path[i]: path[i + 1] for i in range(len(path) - 1)}
        target = np.zeros(n, np.int64)
        for p in range(n):
            if p in nxt:
                target[p] = draft[nxt[p]]
            else:
                taken = {int(draft[c]) for c in children[p]}
                t = int(rng.integers(vocab))
                while t in taken:
                    t = int(rng.integers(vocab))
                target[p] = t
        drafts.append(draft)
        targets.append(target)
    return (np.concatenate(drafts).astype(np.int32), np.concatenate(targets).astype(np.int32))

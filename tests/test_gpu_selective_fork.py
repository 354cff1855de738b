"""GPU parity of the selective fork (fork page "Qwen3.5 tree spec", section 8:
a node whose draft confidence is above 0.95 saves no checkpoint):
gdn_tree_fork_selective_verify / _commit against the oracle's selective fork.

Bar: outputs and committed states within 1e-4 (fp32 io) or 2e-2 (bf16 io)
normwise relative error, saved checkpoints against the oracle's to the same
bar, status codes and the set of saved nodes exact. With every node saved the
selective kernels must reproduce the plain fork bit for bit."""
import numpy as np
import pytest
import torch

import gated_deltanet_tree_02_amd as gt
import gdn_inputs as gi
import oracle

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():  # the -m gpu suite only runs on a GPU machine
    pytest.skip("no GPU", allow_module_level=True)

from gpu_util import (TOL, DeviceLayer, f32, rel_err_rows, rel_err_states,  # noqa: E402
                      sub_workload)

THETA = 0.95


def _say(*a):
    print("[gpu-selective-fork]", *a, flush=True)


def _saved_counts(w, conf):
    return [int((conf[w.offsets[b]:w.offsets[b + 1]] <= THETA).sum()) for b in range(w.B)]


class Selective:
    """A layer's selective-fork verify and commit on the GPU."""

    def __init__(self, L: DeviceLayer, conf, max_kept, threshold=THETA):
        self.L, self.threshold, self.max_kept = L, threshold, max_kept
        self.conf = f32(conf)
        nbytes = gt.gdn_tree_fork_selective_workspace_bytes(L.desc, max_kept)
        self.ws = torch.full((max(nbytes, 1) // 4,), float("nan"), device="cuda").view(torch.uint8)
        self.ws = self.ws[:nbytes] if nbytes else None

    def verify(self):
        L = self.L
        gt.gdn_tree_fork_selective_verify(L.desc, L.offsets, L.parents, self.conf, self.threshold,
                                          self.max_kept, L.q, L.k, L.v, L.alpha, L.beta, L.S0,
                                          L.o, self.ws, L.status)

    def commit(self, S_out):
        L = self.L
        gt.gdn_tree_fork_selective_commit(L.desc, L.offsets, L.parents, self.conf,
                                          self.threshold, self.max_kept, L.accepted, L.k, L.v,
                                          L.alpha, L.beta, L.S0, S_out, self.ws, L.status)

    def slots(self):
        w = self.L.w
        return self.ws.view(torch.float32).view(w.B * self.max_kept, w.H, w.dv, w.dk)


def _check_against_oracle(w, conf, L, sel, S_out, seqs, tol):
    """The sampled sequences' outputs, saved checkpoints and commits."""
    sw = sub_workload(w, seqs, layers=[0])
    rows = np.concatenate([np.arange(w.offsets[b], w.offsets[b + 1]) for b in seqs])
    sconf = np.asarray(conf, np.float64)[rows]
    x = [np.asarray(a[0], np.float64) for a in (sw.q, sw.k, sw.v, sw.alpha, sw.beta, sw.S0)]
    o_ref, ck_ref, kept, st = oracle.selective_fork(sw.offsets, sw.parents, sconf, THETA, *x)
    assert np.all(st == 0)
    e_o = rel_err_rows(L.o_np()[rows], o_ref)
    # the GPU's saved states: sequence b's saved nodes in node order from slot b*max_kept
    slots = sel.slots().cpu().numpy()
    e_ck = 0.0
    for i, b in enumerate(seqs):
        lo, n = int(w.offsets[b]), int(w.offsets[b + 1] - w.offsets[b])
        rank = 0
        for t in range(n):
            if kept[sw.offsets[i] + t]:
                got = slots[b * sel.max_kept + rank]
                e_ck = max(e_ck, rel_err_states(got[None], ck_ref[sw.offsets[i] + t][None]))
                rank += 1
    S_ref, stc = oracle.selective_commit(sw.offsets, sw.parents, kept, sw.accepted, ck_ref,
                                         x[1], x[2], x[3], x[4], x[5])
    assert np.all(stc == 0)
    e_s = rel_err_states(S_out.cpu().numpy()[seqs], S_ref)
    return e_o, e_ck, e_s


@pytest.mark.parametrize("name,nseq,p_dom", [("c1", None, 0.5), ("c3", 8, 0.5), ("c5", 4, 0.5),
                                             ("c3", 8, 1.0), ("c5", 4, 0.0)])
def test_selective_fork_matches_oracle(name, nseq, p_dom):
    w = gi.make_config(name, layers=1)
    conf = gi.draft_confidences(np.random.default_rng(7), w.parents_list, p_dominant=p_dom)
    counts = _saved_counts(w, conf)
    max_kept = max(counts)
    # (the descriptor's mode is not read by the selective calls; WY keeps the
    # helper's own workspace small)
    L = DeviceLayer(w, 0, max_nodes=64, max_depth=w.max_depth())
    sel = Selective(L, conf, max_kept)
    sel.verify()
    S_out = torch.full_like(L.S0, float("nan"))
    sel.commit(S_out)
    torch.cuda.synchronize()
    assert np.all(L.status.cpu().numpy() == 0)
    seqs = list(range(w.B)) if nseq is None else sorted(
        np.random.default_rng(8).choice(w.B, min(nseq, w.B), replace=False).tolist())
    e_o, e_ck, e_s = _check_against_oracle(w, conf, L, sel, S_out, seqs, TOL[w.io])
    _say(f"{name} p_dominant={p_dom}: saved {sum(counts)} of {w.T} nodes (max {max_kept} per "
         f"sequence); o {e_o:.3e}, checkpoints {e_ck:.3e}, commit {e_s:.3e}")
    assert e_o <= TOL[w.io] and e_ck <= TOL[w.io] and e_s <= TOL[w.io]


def test_selective_fork_with_every_node_saved_is_the_plain_fork():
    """Threshold above every confidence: the same outputs, checkpoints and
    commits as GDN_MODE_FORK, bit for bit (uniform trees, so the slots are the
    plain fork's node-indexed checkpoints)."""
    w = gi.make_config("c3", layers=1)
    conf = gi.draft_confidences(np.random.default_rng(9), w.parents_list)
    L = DeviceLayer(w, 0, max_nodes=64, max_depth=w.max_depth())
    F = DeviceLayer(w, 0, mode=gt.MODE_FORK, max_nodes=64, max_depth=w.max_depth())
    sel = Selective(L, conf, 15, threshold=2.0)
    sel.verify()
    S_sel = torch.full_like(L.S0, float("nan"))
    sel.commit(S_sel)
    F.verify()
    F.commit()
    torch.cuda.synchronize()
    assert np.all(L.status.cpu().numpy() == 0) and np.all(F.status.cpu().numpy() == 0)
    assert torch.equal(L.o, F.o)
    assert torch.equal(sel.ws[:F.ws.numel()], F.ws)
    assert torch.equal(S_sel, F.S_out)


def test_selective_fork_with_no_node_saved():
    """Threshold below every confidence: no workspace at all; every node
    rebuilt from S0 along its path; commit in place."""
    w = gi.make_workload([gi.kary_parents(2, 3), gi.chain_parents(9), [-1]], 4, 64, 64,
                         io="bf16", seed=13)
    w.accepted[:] = [12, 8, 0]
    conf = gi.draft_confidences(np.random.default_rng(14), w.parents_list)
    L = DeviceLayer(w, 0, max_nodes=64, max_depth=w.max_depth())
    sel = Selective(L, conf, 0, threshold=-1.0)
    assert sel.ws is None
    sel.verify()
    S0 = L.S0.clone()
    sel.commit(L.S0)                                   # in place
    torch.cuda.synchronize()
    assert np.all(L.status.cpu().numpy() == 0)
    x = [np.asarray(a[0], np.float64) for a in (w.q, w.k, w.v, w.alpha, w.beta, w.S0)]
    o_ref, _ = oracle.verify(w.offsets, w.parents, *x)
    S_ref, _ = oracle.commit(w.offsets, w.parents, w.accepted, *x[1:])
    e_o = rel_err_rows(L.o_np(), o_ref)
    e_s = rel_err_states(L.S0.cpu().numpy(), S_ref)
    _say(f"nothing saved: o {e_o:.3e}, commit {e_s:.3e}")
    assert e_o <= TOL["bf16"] and e_s <= TOL["bf16"]
    assert not torch.equal(L.S0[0], S0[0])


def test_selective_fork_status_codes():
    """Too many saved nodes for max_kept, a bad root, a tree deeper than
    max_depth, and an accepted index out of range: the sequence gets its code,
    zero output rows (verify) and no commit; the others are unaffected."""
    trees = [gi.kary_parents(2, 2)] * 3 + [gi.chain_parents(6), gi.kary_parents(2, 2)]
    w = gi.make_workload(trees, 2, 64, 64, io="bf16", seed=15)
    w.accepted[:] = [3, 4, 5, 2, 7]
    conf = np.full(w.T, 0.99, np.float32)
    conf[w.offsets[1]:w.offsets[1] + 4] = 0.5          # 4 saved nodes > max_kept = 3
    conf[w.offsets[0] + 1] = 0.5                       # one saved node
    L = DeviceLayer(w, 0, max_nodes=64, max_depth=3)
    par = L.parents.cpu().numpy()
    par[w.offsets[2]] = 0                              # bad root
    L.parents.copy_(torch.from_numpy(par))
    sel = Selective(L, conf, 3)
    sel.verify()
    torch.cuda.synchronize()
    st = L.status.cpu().numpy().tolist()
    # seq 3: a chain of depth 5 > max_depth 3
    assert st == [0, 8, 1, 5, 0], st
    o = L.o_np()
    for b in (1, 2, 3):
        assert np.all(o[w.offsets[b]:w.offsets[b + 1]] == 0), b
    S_out = torch.full_like(L.S0, float("nan"))
    sel.commit(S_out)
    torch.cuda.synchronize()
    # seq 4: accepted 7 is outside its 7 nodes
    assert L.status.cpu().numpy().tolist() == [0, 8, 1, 5, 4]
    for b in (1, 2, 3, 4):
        assert torch.isnan(S_out[b]).all(), b
    keep = [0]
    sw = sub_workload(w, keep)
    x = [np.asarray(a[0], np.float64) for a in (sw.q, sw.k, sw.v, sw.alpha, sw.beta, sw.S0)]
    S_ref, _ = oracle.commit(sw.offsets, sw.parents, sw.accepted, *x[1:])
    assert rel_err_states(S_out.cpu().numpy()[keep], S_ref) <= TOL["bf16"]


@pytest.mark.parametrize("d,io", [(32, "f32"), (64, "bf16"), (64, "f32"), (128, "f32")])
def test_selective_fork_head_sizes_and_dtypes(d, io):
    """The other head sizes and io dtypes, on ragged random trees and a deep
    chain (depth 9), with a third of the confidences at or below the threshold:
    outputs, saved checkpoints and commits against the oracle."""
    rng = np.random.default_rng(200 + d + (1 if io == "f32" else 0))
    trees = [gi.random_tree_parents(rng, 3, 40, max_depth=6) for _ in range(5)]
    trees += [gi.chain_parents(10), [-1]]
    w = gi.make_workload(trees, 3, d, d, io=io, seed=201 + d)
    w.accepted[:] = [gi.pick_accepted(rng, t) for t in trees]
    w.accepted[-1] = 0
    conf = np.where(rng.random(w.T) < 1 / 3, rng.uniform(0.2, 0.95, w.T),
                    rng.uniform(0.9501, 1.0, w.T)).astype(np.float32)
    conf[w.offsets[:-1]] = 1.0
    counts = _saved_counts(w, conf)
    max_kept = max(max(counts), 1)
    L = DeviceLayer(w, 0, max_nodes=64, max_depth=w.max_depth())
    sel = Selective(L, conf, max_kept)
    sel.verify()
    S_out = torch.full_like(L.S0, float("nan"))
    sel.commit(S_out)
    torch.cuda.synchronize()
    assert np.all(L.status.cpu().numpy() == 0)
    e_o, e_ck, e_s = _check_against_oracle(w, conf, L, sel, S_out, list(range(w.B)), TOL[io])
    _say(f"d={d} {io}: saved {sum(counts)} of {w.T}; o {e_o:.3e}, checkpoints {e_ck:.3e}, "
         f"commit {e_s:.3e}")
    assert e_o <= TOL[io] and e_ck <= TOL[io] and e_s <= TOL[io]

"""Pins of the oracle's selective fork (fork page "Qwen3.5 tree spec",
section 8, "selective fork": a node whose draft confidence is above 0.95 is
processed without saving a checkpoint, the others fork and save one as in
section 4). Its unsaved states are rebuilt from the nearest saved ancestor
where needed, so outputs and commits must equal the per-path replay that
defines them; with every node saved it must be the plain depth-by-depth fork
of section 4, and with none saved the plain recurrence from S0. CPU only."""
import numpy as np
import pytest

import gdn_inputs as gi
import oracle

THETA = 0.95


def _rel(a, b):
    a, b = np.asarray(a, np.float64), np.asarray(b, np.float64)
    return float(np.max(np.abs(a - b)) / max(np.max(np.abs(b)), 1e-300))


def _inputs(w, layer=0):
    return [np.asarray(x[layer], np.float64) for x in (w.q, w.k, w.v, w.alpha, w.beta, w.S0)]


def _workload(trees, seed, H=2, d=8):
    return gi.make_workload(trees, H=H, dk=d, dv=d, io="f32", seed=seed)


TREES = [gi.kary_parents(2, 2), gi.chain_parents(7), gi.kary_parents(3, 2),
         gi.branching_parents([3, 2, 1]), [-1]]


def _random_trees(seed, count=6):
    rng = np.random.default_rng(seed)
    return [gi.random_tree_parents(rng, 2, 24, max_depth=5) for _ in range(count)]


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_outputs_and_every_commit_equal_per_path_replay(seed):
    """Random trees, random confidences on both sides of the threshold: every
    node's output, and the committed state for every possible accepted node
    (also -1), equal the oracle's per-path replay from S0."""
    trees = TREES + _random_trees(10 + seed)
    w = _workload(trees, seed)
    q, k, v, a, b, S0 = _inputs(w)
    rng = np.random.default_rng(100 + seed)
    conf = rng.uniform(0.9, 1.0, w.T)           # about half above 0.95
    o, ck, kept, st = oracle.selective_fork(w.offsets, w.parents, conf, THETA, q, k, v, a, b, S0)
    o_ref, st_ref = oracle.verify(w.offsets, w.parents, q, k, v, a, b, S0)
    assert np.all(st == 0) and np.all(st_ref == 0)
    assert 0 < kept.sum() < w.T
    assert _rel(o, o_ref) < 1e-12
    n = np.diff(w.offsets)
    for j in range(-1, int(n.max())):
        acc = np.minimum(j, n - 1).astype(np.int32)
        S, s1 = oracle.selective_commit(w.offsets, w.parents, kept, acc, ck, k, v, a, b, S0)
        S_ref, s2 = oracle.commit(w.offsets, w.parents, acc, k, v, a, b, S0)
        assert np.all(s1 == 0) and np.all(s2 == 0)
        assert _rel(S, S_ref) < 1e-12, j


def test_every_node_saved_is_the_plain_fork():
    """Confidences at or below the threshold everywhere: a checkpoint for
    every node, bit-identical to the depth-by-depth fork of section 4."""
    w = _workload(TREES, 3)
    q, k, v, a, b, S0 = _inputs(w)
    conf = np.random.default_rng(4).uniform(0.0, THETA, w.T)
    o, ck, kept, st = oracle.selective_fork(w.offsets, w.parents, conf, THETA, q, k, v, a, b, S0)
    o_f, ck_f, st_f = oracle.fork_replay(w.offsets, w.parents, q, k, v, a, b, S0)
    assert np.all(kept == 1)
    np.testing.assert_array_equal(o, o_f)
    np.testing.assert_array_equal(ck, ck_f)


def test_no_node_saved_is_the_plain_recurrence():
    """Confidences above the threshold everywhere: no checkpoint at all; the
    outputs are the per-path replay's bit for bit, and committing a chain's
    prefix of L tokens gives the sequential recurrence over those L tokens."""
    w = _workload([gi.chain_parents(7), gi.kary_parents(2, 3)], 5, H=1)
    q, k, v, a, b, S0 = _inputs(w)
    conf = np.full(w.T, 0.99)
    o, ck, kept, st = oracle.selective_fork(w.offsets, w.parents, conf, THETA, q, k, v, a, b, S0)
    o_ref, _ = oracle.verify(w.offsets, w.parents, q, k, v, a, b, S0)
    assert kept.sum() == 0 and not ck.any()
    np.testing.assert_array_equal(o, o_ref)
    for L in range(1, 8):
        acc = np.array([L - 1, 0], np.int32)
        S, st = oracle.selective_commit(w.offsets, w.parents, kept, acc, ck, k, v, a, b, S0)
        _, S_chain = oracle.chain(q[:L, 0], k[:L, 0], v[:L, 0], a[:L, 0], b[:L, 0], S0[0, 0])
        np.testing.assert_array_equal(S[0, 0], S_chain)


def test_threshold_boundary():
    """0.95 itself keeps its checkpoint (only a confidence above it skips);
    the next float above 0.95 does not."""
    w = _workload([gi.chain_parents(4)], 6, H=1)
    q, k, v, a, b, S0 = _inputs(w)
    up = np.nextafter(THETA, 1.0)
    conf = np.array([THETA, up, THETA, up])
    _, ck, kept, _ = oracle.selective_fork(w.offsets, w.parents, conf, THETA, q, k, v, a, b, S0)
    assert kept.tolist() == [1, 0, 1, 0]
    assert ck[0].any() and not ck[1].any() and ck[2].any() and not ck[3].any()


def test_saved_checkpoint_is_the_node_state_and_commit_starts_there():
    """A saved checkpoint is the node's own state (the per-path replay), and
    the commit of a node below it starts from that checkpoint: replacing the
    saved checkpoint of the accepted node's nearest saved ancestor by another
    state moves the commit to the recurrence from that other state."""
    w = _workload([gi.chain_parents(6)], 7, H=1, d=6)
    q, k, v, a, b, S0 = _inputs(w)
    conf = np.array([0.99, 0.5, 0.99, 0.99, 0.5, 0.99])     # saved: nodes 1 and 4
    o, ck, kept, _ = oracle.selective_fork(w.offsets, w.parents, conf, THETA, q, k, v, a, b, S0)
    assert kept.tolist() == [0, 1, 0, 0, 1, 0]
    for node in (1, 4):
        S_ref, _ = oracle.commit(w.offsets, w.parents, [node], k, v, a, b, S0)
        assert _rel(ck[node, 0], S_ref[0, 0]) < 1e-13
    other = np.random.default_rng(8).standard_normal(ck[1, 0].shape)
    ck2 = ck.copy()
    ck2[1, 0] = other
    S, _ = oracle.selective_commit(w.offsets, w.parents, kept, [3], ck2, k, v, a, b, S0)
    _, S_from_other = oracle.chain(q[2:4, 0], k[2:4, 0], v[2:4, 0], a[2:4, 0], b[2:4, 0], other)
    np.testing.assert_array_equal(S[0, 0], S_from_other)


def test_sibling_perturbation_leaves_other_branches_bit_identical():
    """Isolation of branches (fork page sections 2 and 4) holds with any
    pattern of saved checkpoints: changing one node's inputs changes only its
    own subtree's outputs."""
    parents = gi.kary_parents(2, 3)
    w = _workload([parents], 9, H=2)
    q, k, v, a, b, S0 = _inputs(w)
    conf = np.random.default_rng(9).uniform(0.9, 1.0, w.T)
    o1, *_ = oracle.selective_fork(w.offsets, w.parents, conf, THETA, q, k, v, a, b, S0)
    node = 2
    k2, v2 = k.copy(), v.copy()
    k2[node] = -k2[node]
    v2[node] += 1.0
    o2, *_ = oracle.selective_fork(w.offsets, w.parents, conf, THETA, q, k2, v2, a, b, S0)
    _, anc, _ = oracle.tree(w.offsets, w.parents)
    for t in range(len(parents)):
        in_subtree = (int(anc[t]) >> node) & 1
        if in_subtree:
            assert not np.array_equal(o1[t], o2[t]), t
        else:
            np.testing.assert_array_equal(o1[t], o2[t])


def test_checkpoint_count_and_bad_trees():
    """One checkpoint per node at or below the threshold; malformed trees
    report the same codes as the other oracle functions and keep nothing."""
    trees = [gi.kary_parents(3, 3), [0, 0], [-1, 1]]
    w = _workload([gi.kary_parents(3, 3), gi.chain_parents(2), gi.chain_parents(2)], 11, H=1)
    par = w.parents.copy()
    par[40] = 0                    # bad root
    par[43] = 1                    # bad parent (not below its index)
    q, k, v, a, b, S0 = _inputs(w)
    conf = gi.draft_confidences(np.random.default_rng(12), [gi.kary_parents(3, 3)] + trees[1:],
                                p_dominant=0.7)
    o, ck, kept, st = oracle.selective_fork(w.offsets, par, conf, THETA, q, k, v, a, b, S0)
    assert st.tolist() == [0, 1, 2]
    assert kept[:40].tolist() == (conf[:40] <= THETA).astype(int).tolist()
    assert kept[40:].sum() == 0
    assert conf[0] == 1.0 and kept[0] == 0               # the root's own token is certain
    assert kept[:40].sum() < 40

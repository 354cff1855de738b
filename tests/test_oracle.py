"""Pins of the CPU oracle against facts that do not come from the oracle itself:
values the pages print, closed forms of the gated delta rule, invariants, and
an independent formulation (dense tree-WY in numpy). CPU only."""
import itertools

import numpy as np
import pytest

import gdn_inputs as gi
import oracle
from oracle import wy
from conftest import read_golden


def _tree_inputs(parents, H=1, dk=8, dv=6, seed=0, io="f32", **kw):
    return gi.make_workload([parents], H=H, dk=dk, dv=dv, io=io, seed=seed, **kw)


def _oracle_o(w, layer=0):
    return oracle.verify(w.offsets, w.parents, w.q[layer], w.k[layer], w.v[layer],
                         w.alpha[layer], w.beta[layer], w.S0[layer])


# ---------------------------------------------------------------- tree / mask


def test_handbook_mask_golden():
    rows = read_golden("handbook_tree_mask.txt")
    parents = [int(x) for x in rows[0][1:]]
    mask = np.array([[int(x) for x in r] for r in rows[1:]], dtype=bool)
    depth, anc, st = oracle.tree([0, len(parents)], parents)
    assert st.tolist() == [0]
    got = np.array([[(int(anc[i]) >> j) & 1 for j in range(len(parents))] for i in range(len(parents))],
                   dtype=bool)
    np.testing.assert_array_equal(got, mask)
    # depth = number of visible nodes minus one
    np.testing.assert_array_equal(depth, mask.sum(1) - 1)


def test_fork_levels_golden():
    rows = read_golden("fork_levels_k2d2.txt")
    labels = rows[0][1:]
    parents = [int(x) for x in rows[1][1:]]
    depth, anc, st = oracle.tree([0, len(parents)], parents)
    assert st.tolist() == [0]
    for r in rows[2:5]:
        lvl = int(r[1])
        assert sorted(labels.index(x) for x in r[2:]) == [i for i in range(len(parents)) if depth[i] == lvl]
    path = [labels.index(x) for x in rows[5][1:]]
    acc = path[-1]
    assert [j for j in range(len(parents)) if (int(anc[acc]) >> j) & 1] == path
    assert parents == gi.CONFIGS["c1"]["parents"]


def test_node_counts():
    # k-ary trees of 7/15/40 nodes including the root; branching lists 14 and 30 draft nodes
    assert [len(gi.kary_parents(2, 2)), len(gi.kary_parents(2, 3)), len(gi.kary_parents(3, 3))] == [7, 15, 40]
    assert len(gi.branching_parents([2, 2, 1, 1])) - 1 == 14
    assert len(gi.branching_parents([3, 3, 2])) - 1 == 30


def _all_topological_trees(n):
    for choice in itertools.product(*[range(i) for i in range(1, n)]):
        yield [-1] + list(choice)


def test_tree_bruteforce_small():
    """Every tree in topological order with up to 8 nodes (5,914 trees, one
    batch per size): ancestor sets from boolean reachability (matrix
    products) equal the oracle's walk, and depth is the ancestor count."""
    for n in range(1, 9):
        trees = list(_all_topological_trees(n))
        offsets = np.arange(len(trees) + 1, dtype=np.int32) * n
        depth, anc, st = oracle.tree(offsets, np.concatenate(trees).astype(np.int32))
        assert np.all(st == 0)
        bits = (anc.astype(np.uint64)[:, None] >> np.arange(n, dtype=np.uint64)) & np.uint64(1)
        for b, parents in enumerate(trees):
            M = wy.ancestor_matrix(parents).astype(np.uint64)
            np.testing.assert_array_equal(bits[b * n:(b + 1) * n], M)
            np.testing.assert_array_equal(depth[b * n:(b + 1) * n], M.sum(1) - 1)


def test_tree_status_codes():
    T = 4
    cases = [
        ([0, 4], [-1, 0, 0, 1], 0),
        ([0, 4], [0, 0, 0, 1], 1),       # root not at index 0
        ([0, 4], [-1, 0, 2, 1], 2),      # parent not smaller than child
        ([0, 4], [-1, 0, -1, 1], 2),     # second root
        ([0, 4], [-1, 0, 7, 1], 2),      # out of range
        ([0, 0], [-1, 0, 0, 1], 3),      # empty tree
        ([0, 5], [-1, 0, 0, 1], 3),      # range beyond T
    ]
    for offsets, parents, code in cases:
        _, _, st = oracle.tree(offsets, parents[:T])
        assert st.tolist() == [code], (offsets, parents)
    _, _, st = oracle.tree([0, 4], [-1, 0, 0, 1], max_nodes=3)
    assert st.tolist() == [3]
    par = [-1] + list(range(64))
    _, _, st = oracle.tree([0, 65], par)
    assert st.tolist() == [3]
    _, _, st = oracle.tree([0, 64], par[:64])
    assert st.tolist() == [0]


# ---------------------------------------------------------------- closed forms


def _gamma(parents, alpha):
    M = wy.ancestor_matrix(parents)
    return np.array([np.prod(alpha[M[t]].astype(np.float64)) for t in range(len(parents))])


@pytest.mark.parametrize("parents", [gi.kary_parents(2, 2), gi.chain_parents(5), gi.kary_parents(3, 2)])
def test_no_write_is_pure_decay(parents):
    """beta = 0: S_t = Gamma_t S0 with Gamma_t the product of alpha over the
    node and its ancestors, so o_t = Gamma_t S0 q_t."""
    w = _tree_inputs(parents, H=2, dk=8, dv=5, seed=3)
    w.beta[:] = 0.0
    o, st = _oracle_o(w)
    for h in range(2):
        G = _gamma(parents, w.alpha[0][:, h])
        exp = G[:, None] * (w.q[0][:, h].astype(np.float64) @ w.S0[0][0, h].astype(np.float64).T)
        np.testing.assert_allclose(o[:, h], exp, rtol=1e-12, atol=1e-14)
    w.alpha[:] = 1.0
    o, _ = _oracle_o(w)
    exp = np.einsum("thc,hrc->thr", w.q[0].astype(np.float64), w.S0[0][0].astype(np.float64))
    np.testing.assert_allclose(o, exp, rtol=1e-12, atol=1e-14)
    acc = len(parents) - 1
    S, st = oracle.commit(w.offsets, w.parents, [acc], w.k[0], w.v[0], w.alpha[0], w.beta[0], w.S0[0])
    np.testing.assert_allclose(S[0], w.S0[0][0], rtol=0, atol=0)


@pytest.mark.parametrize("parents", [gi.kary_parents(2, 2), gi.chain_parents(6)])
def test_delta_write_property(parents):
    """beta = 1 and unit k_t: S_t k_t = v_t exactly (the delta rule overwrites
    the value stored under key k_t), whatever alpha and S0 are; so q_t = k_t
    reads v_t back."""
    w = _tree_inputs(parents, H=2, dk=8, dv=5, seed=4)
    k64 = w.k[0].astype(np.float64)
    k64 /= np.linalg.norm(k64, axis=-1, keepdims=True)     # unit norm in fp64
    o, _ = oracle.verify(w.offsets, w.parents, k64, k64, w.v[0], w.alpha[0],
                         np.ones_like(w.beta[0]), w.S0[0])
    np.testing.assert_allclose(o, w.v[0].astype(np.float64), rtol=1e-12, atol=1e-12)


def test_orthonormal_recall_and_isolation():
    """Orthonormal keys across the whole tree, beta = 1. Then, for the state of
    node t, S_t k_j = (Gamma_t / Gamma_j) v_j for every j on t's path, and
    S_t k_s = Gamma_t S0 k_s for every node s off the path (siblings leave
    no trace). With every q_t set to the root key, o_t = (Gamma_t/alpha_root) v_root."""
    parents = gi.kary_parents(2, 2) + [3, 3, 4]           # 10 nodes, depth 3
    n, dk, dv = len(parents), 12, 4
    rng = np.random.default_rng(7)
    Qm, _ = np.linalg.qr(rng.standard_normal((dk, dk)))
    k = Qm[:n, None, :]                                   # [n,1,dk], exactly orthonormal in fp64
    q = np.repeat(k[:1], n, axis=0)
    v = rng.standard_normal((n, 1, dv))
    alpha = rng.uniform(0.5, 1.0, (n, 1))
    beta = np.ones((n, 1))
    S0 = rng.standard_normal((1, 1, dv, dk))
    offsets = [0, n]
    G = _gamma(parents, alpha[:, 0])
    o, _ = oracle.verify(offsets, parents, q, k, v, alpha, beta, S0)
    np.testing.assert_allclose(o[:, 0], (G / G[0])[:, None] * v[0, 0][None, :], rtol=1e-12, atol=1e-12)
    M = wy.ancestor_matrix(parents)
    for a in range(n):
        S, st = oracle.commit(offsets, parents, [a], k, v, alpha, beta, S0)
        for j in range(n):
            got = S[0, 0] @ k[j, 0]
            exp = (G[a] / G[j]) * v[j, 0] if M[a, j] else G[a] * (S0[0, 0] @ k[j, 0])
            np.testing.assert_allclose(got, exp, rtol=1e-12, atol=1e-12)


def test_single_node_from_zero_state():
    """S0 = 0, one node: o = beta v (k.q)."""
    w = _tree_inputs([-1], H=3, dk=8, dv=5, seed=6)
    w.S0[:] = 0.0
    o, _ = _oracle_o(w)
    kq = np.sum(w.k[0].astype(np.float64) * w.q[0], axis=-1)
    np.testing.assert_allclose(o, (w.beta[0] * kq)[..., None] * w.v[0], rtol=1e-12, atol=1e-14)


def test_linear_in_values_and_state():
    parents = gi.kary_parents(2, 2)
    w1 = _tree_inputs(parents, H=2, dk=8, dv=5, seed=8)
    w2 = _tree_inputs(parents, H=2, dk=8, dv=5, seed=9)
    w2.q[:], w2.k[:], w2.alpha[:], w2.beta[:] = w1.q, w1.k, w1.alpha, w1.beta
    o1, _ = _oracle_o(w1)
    o2, _ = _oracle_o(w2)
    ws = _tree_inputs(parents, H=2, dk=8, dv=5, seed=8)
    ws.v[:] = w1.v.astype(np.float64) + w2.v
    ws.S0[:] = w1.S0.astype(np.float64) + w2.S0
    o12 = oracle.verify(ws.offsets, ws.parents, ws.q[0], ws.k[0],
                        w1.v[0].astype(np.float64) + w2.v[0], ws.alpha[0], ws.beta[0],
                        w1.S0[0].astype(np.float64) + w2.S0[0])[0]
    np.testing.assert_allclose(o12, o1 + o2, rtol=1e-12, atol=1e-12)


# --------------------------------------------- independent formulation + self-checks


@pytest.mark.parametrize("parents", [
    gi.CONFIGS["c1"]["parents"], gi.chain_parents(6), gi.kary_parents(3, 2),
    gi.branching_parents([2, 2, 1, 1])])
def test_wy_dense_matches_path_replay(parents):
    w = _tree_inputs(parents, H=2, dk=16, dv=12, seed=11)
    o, _ = _oracle_o(w)
    O, U, g = wy.wy_batch(w.offsets, w.parents, w.q[0], w.k[0], w.v[0], w.alpha[0], w.beta[0], w.S0[0])
    np.testing.assert_allclose(O, o, rtol=1e-11, atol=1e-12)
    for a in range(len(parents)):
        S, _ = oracle.commit(w.offsets, w.parents, [a], w.k[0], w.v[0], w.alpha[0], w.beta[0], w.S0[0])
        for h in range(2):
            Sw = wy.wy_commit(parents, a, w.k[0][:, h], U[:, h], g[:, h], w.S0[0][0, h])
            np.testing.assert_allclose(Sw, S[0, h], rtol=1e-11, atol=1e-12)


def test_random_trees_wy_vs_replay():
    rng = np.random.default_rng(12)
    trees = [gi.random_tree_parents(rng, 5, 20, 6, 4) for _ in range(4)]
    w = gi.make_workload(trees, H=2, dk=16, dv=8, io="bf16", seed=13)
    o, st = _oracle_o(w)
    assert st.tolist() == [0] * 4
    O, _, _ = wy.wy_batch(w.offsets, w.parents, w.q[0], w.k[0], w.v[0], w.alpha[0], w.beta[0], w.S0[0])
    np.testing.assert_allclose(O, o, rtol=1e-10, atol=1e-12)


def test_chain_equals_sequential_recurrence():
    """Self-check 1: a chain-shaped tree gives the plain sequential recurrence."""
    n = 6
    w = _tree_inputs(gi.chain_parents(n), H=3, dk=8, dv=5, seed=14)
    o, _ = _oracle_o(w)
    for h in range(3):
        oc, Sf = oracle.chain(w.q[0][:, h], w.k[0][:, h], w.v[0][:, h], w.alpha[0][:, h],
                              w.beta[0][:, h], w.S0[0][0, h])
        np.testing.assert_array_equal(o[:, h], oc)
        for L in range(1, n + 1):
            S, _ = oracle.commit(w.offsets, w.parents, [L - 1], w.k[0], w.v[0], w.alpha[0], w.beta[0], w.S0[0])
            _, SL = oracle.chain(w.q[0][:L, h], w.k[0][:L, h], w.v[0][:L, h], w.alpha[0][:L, h],
                                 w.beta[0][:L, h], w.S0[0][0, h])
            np.testing.assert_array_equal(S[0, h], SL)


@pytest.mark.parametrize("parents", [gi.CONFIGS["c1"]["parents"], gi.kary_parents(3, 3)])
def test_fork_replay_equals_path_replay(parents):
    """Self-check 2: depth-by-depth fork/checkpoint replay equals per-path
    replay, and every checkpoint equals that node's committed state."""
    w = _tree_inputs(parents, H=2, dk=8, dv=6, seed=15)
    o, _ = _oracle_o(w)
    of, ck, st = oracle.fork_replay(w.offsets, w.parents, w.q[0], w.k[0], w.v[0], w.alpha[0], w.beta[0], w.S0[0])
    np.testing.assert_array_equal(of, o)
    for a in range(len(parents)):
        S, _ = oracle.commit(w.offsets, w.parents, [a], w.k[0], w.v[0], w.alpha[0], w.beta[0], w.S0[0])
        np.testing.assert_array_equal(ck[a], S[0])


def test_rollback_example_root_A_C():
    """The page's rollback example: accept root->A->C; the kept state is the
    state after the tokens root, A, C run in sequence."""
    rows = read_golden("fork_levels_k2d2.txt")
    labels = rows[0][1:]
    parents = [int(x) for x in rows[1][1:]]
    path = [labels.index(x) for x in rows[5][1:]]
    w = _tree_inputs(parents, H=1, dk=8, dv=6, seed=16)
    S, st = oracle.commit(w.offsets, w.parents, [path[-1]], w.k[0], w.v[0], w.alpha[0], w.beta[0], w.S0[0])
    _, Sc = oracle.chain(w.q[0][path, 0], w.k[0][path, 0], w.v[0][path, 0], w.alpha[0][path, 0],
                         w.beta[0][path, 0], w.S0[0][0, 0])
    np.testing.assert_array_equal(S[0, 0], Sc)


def test_sibling_perturbation_leaves_other_branches_bit_identical():
    """Self-check 3: changing one node's inputs changes only the outputs of
    that node and its descendants; every other output is bit-identical."""
    parents = gi.kary_parents(3, 2)
    M = wy.ancestor_matrix(parents)
    base = _tree_inputs(parents, H=2, dk=8, dv=6, seed=17)
    o0, _ = _oracle_o(base)
    rng = np.random.default_rng(18)
    for j in range(1, len(parents)):
        w = _tree_inputs(parents, H=2, dk=8, dv=6, seed=17)
        w.q[0][j] += rng.standard_normal(w.q[0][j].shape).astype(np.float32)
        w.k[0][j] += rng.standard_normal(w.k[0][j].shape).astype(np.float32)
        w.v[0][j] += rng.standard_normal(w.v[0][j].shape).astype(np.float32)
        w.alpha[0][j] *= np.float32(0.5)
        w.beta[0][j] = np.float32(0.25)
        o1, _ = _oracle_o(w)
        sub = M[:, j]                 # nodes that have j on their path
        np.testing.assert_array_equal(o1[~sub], o0[~sub])
        assert np.all(np.abs(o1[sub] - o0[sub]).max(axis=-1) > 0)


def test_commit_edge_cases():
    parents = gi.kary_parents(2, 2)
    w = _tree_inputs(parents, H=2, dk=8, dv=6, seed=19)
    S, st = oracle.commit(w.offsets, w.parents, [-1], w.k[0], w.v[0], w.alpha[0], w.beta[0], w.S0[0])
    assert st.tolist() == [0]
    np.testing.assert_array_equal(S, w.S0[0].astype(np.float64))
    marker = np.full(w.S0[0].shape, 7.0)
    for bad in (7, -2, 100):
        S, st = oracle.commit(w.offsets, w.parents, [bad], w.k[0], w.v[0], w.alpha[0], w.beta[0],
                              w.S0[0], S_out=marker)
        assert st.tolist() == [4]
        np.testing.assert_array_equal(S, marker)
    # committed state reads back the verified output of the accepted node
    o, _ = _oracle_o(w)
    for a in range(len(parents)):
        S, _ = oracle.commit(w.offsets, w.parents, [a], w.k[0], w.v[0], w.alpha[0], w.beta[0], w.S0[0])
        for h in range(2):
            np.testing.assert_allclose(S[0, h] @ w.q[0][a, h].astype(np.float64), o[a, h], rtol=1e-12, atol=1e-13)


def test_invalid_tree_rows_zero():
    w = gi.make_workload([[-1, 0, 0], [-1, 0, 0, 1]], H=1, dk=8, dv=4, io="f32", seed=20)
    w.parents[4] = 2          # second tree: node 1 points at itself+1 -> bad parent
    o, st = _oracle_o(w)
    assert st.tolist() == [0, 2]
    assert np.all(o[3:] == 0) and np.any(o[:3] != 0)

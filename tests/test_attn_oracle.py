"""Pins for the tree-masked attention oracle (oracle/attn_oracle.c).

The oracle loops node by node over the visible keys. These tests check it
against things that do not share its code: dense matrix-form attention with
an explicit mask written here in numpy (for a chain the mask is the causal
one), closed forms (one visible key; all scores equal), the head grouping
written as an explicit repetition of the K/V heads, branch isolation, and the
commit's gather of the accepted path (anrans handbook "speculative",
implementation section: tree tokens see the cached prefix and their own
ancestors; only the accepted path's K/V is appended, in path order).
"""
import numpy as np
import pytest

import gdn_inputs as gi
import oracle


def _dense_masked_attention(q, K, V, mask, scale):
    """softmax(scale q K^T + log mask) V for one head: q [n,d], K/V [m,d], mask [n,m] bool."""
    s = scale * q @ K.T
    s = np.where(mask, s, -np.inf)
    s = s - s.max(axis=1, keepdims=True)
    w = np.exp(s)
    w /= w.sum(axis=1, keepdims=True)
    return w @ V


def _ancestor_mask(parents):
    """Row i marks i and its ancestors: row parents[i] (built first, since a
    parent precedes its children) plus i itself."""
    vis = np.eye(len(parents), dtype=bool)
    for i in range(1, len(parents)):
        vis[i] |= vis[parents[i]]
    return vis


def _random_case(rng, parents_list, Hq, Hkv, d, cap, lens):
    T = sum(len(p) for p in parents_list)
    B = len(parents_list)
    offsets = np.concatenate([[0], np.cumsum([len(p) for p in parents_list])]).astype(np.int32)
    parents = np.concatenate([np.asarray(p, np.int32) for p in parents_list])
    q = rng.standard_normal((T, Hq, d))
    k = rng.standard_normal((T, Hkv, d))
    v = rng.standard_normal((T, Hkv, d))
    kc = rng.standard_normal((B, Hkv, cap, d))
    vc = rng.standard_normal((B, Hkv, cap, d))
    return offsets, parents, q, k, v, kc, vc, np.asarray(lens, np.int32)


def _dense_reference(offsets, parents, q, k, v, kc, vc, lens, scale):
    """Dense masked attention per sequence and head, K/V heads repeated per group."""
    T, Hq, d = q.shape
    Hkv = k.shape[1]
    G = Hq // Hkv
    o = np.zeros_like(q)
    for b in range(len(offsets) - 1):
        lo, hi = offsets[b], offsets[b + 1]
        L = lens[b]
        mask = np.concatenate([np.ones((hi - lo, L), bool), _ancestor_mask(parents[lo:hi])], 1)
        krep = np.repeat(k[lo:hi], G, axis=1)               # [n, Hq, d]
        vrep = np.repeat(v[lo:hi], G, axis=1)
        kcrep = np.repeat(kc[b, :, :L], G, axis=0)           # [Hq, L, d]
        vcrep = np.repeat(vc[b, :, :L], G, axis=0)
        for h in range(Hq):
            K = np.concatenate([kcrep[h], krep[:, h]], 0)
            V = np.concatenate([vcrep[h], vrep[:, h]], 0)
            o[lo:hi, h] = _dense_masked_attention(q[lo:hi, h], K, V, mask, scale)
    return o


def test_single_node_empty_cache_returns_its_value():
    rng = np.random.default_rng(1)
    off, par, q, k, v, kc, vc, lens = _random_case(rng, [[-1]], 4, 2, 16, 4, [0])
    o, st = oracle.tree_attn(off, par, q, k, v, kc, vc, lens)
    assert st.tolist() == [0]
    for h in range(4):
        np.testing.assert_allclose(o[0, h], v[0, h // 2], rtol=0, atol=1e-15)


def test_chain_equals_dense_causal_attention():
    rng = np.random.default_rng(2)
    n, L, d = 9, 13, 32
    off, par, q, k, v, kc, vc, lens = _random_case(rng, [gi.chain_parents(n)], 2, 2, d, 32, [L])
    o, st = oracle.tree_attn(off, par, q, k, v, kc, vc, lens)
    assert st.tolist() == [0]
    causal = np.concatenate([np.ones((n, L), bool), np.tril(np.ones((n, n), bool))], 1)
    for h in range(2):
        K = np.concatenate([kc[0, h, :L], k[:, h]], 0)
        V = np.concatenate([vc[0, h, :L], v[:, h]], 0)
        ref = _dense_masked_attention(q[:, h], K, V, causal, 1 / np.sqrt(d))
        np.testing.assert_allclose(o[:, h], ref, rtol=1e-12, atol=1e-13)


@pytest.mark.parametrize("Hq,Hkv", [(4, 4), (4, 2), (8, 1)])
def test_trees_equal_dense_masked_attention_with_head_groups(Hq, Hkv):
    rng = np.random.default_rng(3 + Hq + Hkv)
    trees = [gi.kary_parents(2, 2), gi.branching_parents([3, 2]), [-1],
             gi.random_tree_parents(rng, 5, 20)]
    lens = [7, 0, 3, 11]
    off, par, q, k, v, kc, vc, lens = _random_case(rng, trees, Hq, Hkv, 16, 12, lens)
    o, st = oracle.tree_attn(off, par, q, k, v, kc, vc, lens, scale=0.3)
    assert st.tolist() == [0] * 4
    ref = _dense_reference(off, par, q, k, v, kc, vc, lens, 0.3)
    np.testing.assert_allclose(o, ref, rtol=1e-12, atol=1e-13)


def test_equal_scores_give_the_mean_of_visible_values():
    rng = np.random.default_rng(4)
    parents = gi.kary_parents(3, 2)
    off, par, q, k, v, kc, vc, lens = _random_case(rng, [parents], 2, 1, 8, 6, [5])
    q[:] = 0.0
    o, st = oracle.tree_attn(off, par, q, k, v, kc, vc, lens)
    anc = _ancestor_mask(parents)
    for t in range(len(parents)):
        vis = np.concatenate([vc[0, 0, :5], v[anc[t], 0]], 0)
        for h in range(2):
            np.testing.assert_allclose(o[t, h], vis.mean(0), rtol=1e-13, atol=1e-14)


def test_sibling_perturbation_leaves_other_branches_bit_identical():
    rng = np.random.default_rng(5)
    parents = gi.kary_parents(2, 3)          # 15 nodes
    off, par, q, k, v, kc, vc, lens = _random_case(rng, [parents], 4, 2, 16, 8, [8])
    o1, _ = oracle.tree_attn(off, par, q, k, v, kc, vc, lens)
    node = 2                                  # root's second child: subtree 2, 5, 6, 11..14
    k2, v2 = k.copy(), v.copy()
    k2[node] += 1.0
    v2[node] -= 2.0
    o2, _ = oracle.tree_attn(off, par, q, k2, v2, kc, vc, lens)
    anc = _ancestor_mask(parents)
    in_subtree = anc[:, node]
    assert in_subtree.sum() == 7
    assert np.array_equal(o1[~in_subtree], o2[~in_subtree])
    assert np.all(np.abs(o1[in_subtree] - o2[in_subtree]).max(axis=(1, 2)) > 0)


def test_commit_appends_the_accepted_path_root_first():
    rng = np.random.default_rng(6)
    trees = [gi.kary_parents(2, 2), gi.chain_parents(4), [-1]]
    off, par, q, k, v, kc, vc, lens = _random_case(rng, trees, 2, 2, 8, 10, [3, 0, 10])
    accepted = [5, 3, -1]                    # path 0 -> 2 -> 5; whole chain; nothing
    kc2, vc2, lens2, st = oracle.tree_attn_commit(off, par, accepted, k, v, kc, vc, lens)
    assert st.tolist() == [0, 0, 0]
    assert lens2.tolist() == [6, 4, 10]
    for r, node in enumerate([0, 2, 5]):
        assert np.array_equal(kc2[0, :, 3 + r], k[off[0] + node])
        assert np.array_equal(vc2[0, :, 3 + r], v[off[0] + node])
    for r in range(4):
        assert np.array_equal(kc2[1, :, r], k[off[1] + r])
    assert np.array_equal(kc2[0, :, :3], kc[0, :, :3]) and np.array_equal(kc2[0, :, 6:], kc[0, :, 6:])
    assert np.array_equal(kc2[2], kc[2]) and np.array_equal(vc2[2], vc[2])


def test_commit_status_codes_leave_caches_untouched():
    rng = np.random.default_rng(7)
    trees = [gi.chain_parents(5), gi.chain_parents(3), [-1, 0], [-1, 0]]
    off, par, q, k, v, kc, vc, lens = _random_case(rng, trees, 2, 1, 8, 6, [3, 0, 0, 0])
    bad = par.copy()
    bad[off[3] + 1] = 1                       # a node that is its own parent
    kc2, vc2, lens2, st = oracle.tree_attn_commit(off, bad, [4, 7, -2, 1], k, v, kc, vc, lens)
    # 5-node path onto 3 cached rows overflows 6 slots; 7 and -2 are out of range
    assert st.tolist() == [oracle.STATUS_CACHE_FULL, oracle.STATUS_BAD_ACCEPTED,
                           oracle.STATUS_BAD_ACCEPTED, oracle.STATUS_BAD_PARENT]
    assert lens2.tolist() == [3, 0, 0, 0]
    assert np.array_equal(kc2, kc) and np.array_equal(vc2, vc)


def test_commit_then_next_token_equals_causal_attention_over_the_grown_prefix():
    """After committing a path, a one-node tree at the next position sees
    exactly the old prefix, the path and itself."""
    rng = np.random.default_rng(8)
    parents = gi.kary_parents(3, 2)
    off, par, q, k, v, kc, vc, lens = _random_case(rng, [parents], 2, 2, 16, 20, [6])
    kc2, vc2, lens2, st = oracle.tree_attn_commit(off, par, [7], k, v, kc, vc, lens)  # 0 -> 2 -> 7
    assert st.tolist() == [0] and lens2.tolist() == [9]
    q1 = rng.standard_normal((1, 2, 16))
    k1 = rng.standard_normal((1, 2, 16))
    v1 = rng.standard_normal((1, 2, 16))
    o, st = oracle.tree_attn([0, 1], [-1], q1, k1, v1, kc2, vc2, lens2)
    for h in range(2):
        K = np.concatenate([kc[0, h, :6], k[[0, 2, 7], h], k1[:, h]], 0)
        V = np.concatenate([vc[0, h, :6], v[[0, 2, 7], h], v1[:, h]], 0)
        ref = _dense_masked_attention(q1[:, h], K, V, np.ones((1, 10), bool), 1 / 4.0)
        np.testing.assert_allclose(o[0, h], ref[0], rtol=1e-12, atol=1e-13)


def test_invalid_trees_and_cache_lengths_give_zero_rows():
    rng = np.random.default_rng(9)
    trees = [[-1, 0], [0, 0], [-1, 0]]
    off, par, q, k, v, kc, vc, lens = _random_case(rng, trees, 2, 1, 8, 4, [0, 0, 5])
    o, st = oracle.tree_attn(off, par, q, k, v, kc, vc, lens)
    assert st.tolist() == [0, oracle.STATUS_BAD_ROOT, oracle.STATUS_BAD_SIZE]
    assert np.all(o[2:] == 0) and np.any(o[:2] != 0)

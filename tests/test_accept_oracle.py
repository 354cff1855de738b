"""Pins for the greedy-acceptance oracle (oracle/accept.py).

The oracle follows the handbook's walk (anrans.github.io ai-infra-handbooks
"speculative", implementation section): from the root, descend into the first
child whose draft token equals the target's prediction at the current node.
These tests check it against things that do not share its code: a brute-force
characterisation (with distinct sibling tokens, the accepted node is the
deepest node whose every edge from the root matches), closed cases (a chain
that matches throughout, a root whose prediction matches no child, a lone
root), the first-in-node-order rule where two siblings match, and the status
codes of malformed trees.

Sampling mode (the chapter's exercise on sampling with a tree: candidates
accepted with probability min(1, p/q), the target replaced by the normalised
positive part of p - q after each rejection, a final draw from the last
residual) is pinned by the property the handbook states for it, exactly: over
every ordered draw of the candidates from the draft without replacement, the
emitted token has the target's distribution. Closed cases and a hand-worked
walk pin the decisions and the inverse-CDF draw.
"""
import numpy as np
import pytest

import gdn_inputs as gi
from oracle import accept as acc


def _edges_match(parents, draft, target, t):
    """Every node c != root on t's root path has draft[c] == target[parent(c)]."""
    c = t
    while parents[c] != -1:
        p = parents[c]
        if draft[c] != target[p]:
            return False
        c = p
    return True


def _depth(parents, t):
    d = 0
    while parents[t] != -1:
        t = parents[t]
        d += 1
    return d


def _distinct_sibling_tokens(rng, parents, vocab):
    """Draft tokens with no two children of one node equal."""
    n = len(parents)
    draft = np.zeros(n, np.int32)
    for p in range(n):
        kids = [c for c in range(n) if parents[c] == p]
        if kids:
            draft[kids] = rng.choice(vocab, size=len(kids), replace=False)
    return draft


@pytest.mark.parametrize("seed", range(12))
def test_brute_force_deepest_matching_node(seed):
    rng = np.random.default_rng(seed)
    n = int(rng.integers(1, 65))
    parents = np.asarray(gi.random_tree_parents(rng, n, n), np.int32)
    vocab = 6
    draft = _distinct_sibling_tokens(rng, parents, vocab)
    # make matches likely: the target at a node usually names one of its children
    target = rng.integers(0, vocab, n).astype(np.int32)
    for p in range(n):
        kids = [c for c in range(n) if parents[c] == p]
        if kids and rng.random() < 0.8:
            target[p] = draft[rng.choice(kids)]
    matching = [t for t in range(n) if _edges_match(parents, draft, target, t)]
    deepest = max(matching, key=lambda t: _depth(parents, t))
    # the matching nodes form one root path: depths are distinct
    assert len({_depth(parents, t) for t in matching}) == len(matching)
    offsets = np.array([0, n], np.int32)
    a, length, nxt, st = acc.accept_greedy(offsets, parents, draft, target)
    assert st[0] == acc.STATUS_OK
    assert a[0] == deepest
    assert length[0] == _depth(parents, deepest) + 1
    assert nxt[0] == target[deepest]


def test_chain_matching_throughout_accepts_everything():
    n = 9
    parents = np.asarray(gi.chain_parents(n), np.int32)
    target = np.arange(100, 100 + n, dtype=np.int32)
    draft = np.concatenate([[0], target[:-1]]).astype(np.int32)   # node i drafts target[i-1]
    a, length, nxt, st = acc.accept_greedy(np.array([0, n], np.int32), parents, draft, target)
    assert (a[0], length[0], nxt[0], st[0]) == (n - 1, n, 100 + n - 1, 0)


def test_no_match_keeps_the_root_and_lone_root():
    parents = np.asarray(gi.kary_parents(3, 2), np.int32)
    n = len(parents)
    draft = np.full(n, 7, np.int32)
    target = np.full(n, 8, np.int32)
    one = np.array([-1], np.int32)
    offsets = np.array([0, n, n + 1], np.int32)
    a, length, nxt, st = acc.accept_greedy(offsets, np.concatenate([parents, one]),
                                           np.concatenate([draft, [3]]).astype(np.int32),
                                           np.concatenate([target, [4]]).astype(np.int32))
    assert a.tolist() == [0, 0] and length.tolist() == [1, 1] and nxt.tolist() == [8, 4]
    assert st.tolist() == [0, 0]


def test_first_matching_sibling_wins_even_when_a_later_one_goes_deeper():
    # root's children 1 and 2 both carry token 5 = the root's prediction; only 2 has a
    # matching child (3). The walk takes node 1 (first in node order) and stops there.
    parents = np.array([-1, 0, 0, 2], np.int32)
    draft = np.array([0, 5, 5, 7], np.int32)
    target = np.array([5, 9, 7, 1], np.int32)
    a, length, nxt, st = acc.accept_greedy(np.array([0, 4], np.int32), parents, draft, target)
    assert (a[0], length[0], nxt[0], st[0]) == (1, 2, 9, 0)
    # with node 1 relabelled to a non-matching token the deeper branch is taken
    draft[1] = 6
    a, length, nxt, _ = acc.accept_greedy(np.array([0, 4], np.int32), parents, draft, target)
    assert (a[0], length[0], nxt[0]) == (3, 3, 1)


def test_root_token_is_not_read():
    parents = np.array([-1, 0], np.int32)
    target = np.array([4, 2], np.int32)
    for root_tok in (4, -5, 123):
        draft = np.array([root_tok, 4], np.int32)
        a, length, _, _ = acc.accept_greedy(np.array([0, 2], np.int32), parents, draft, target)
        assert (a[0], length[0]) == (1, 2)


def test_status_codes_of_malformed_trees():
    trees = [[0, 0, 1], [-1, 1, 0], [-1, 0, 2], [-1, 0, 0]]
    offsets = np.concatenate([[0], np.cumsum([len(t) for t in trees])]).astype(np.int32)
    parents = np.concatenate([np.asarray(t, np.int32) for t in trees])
    T = len(parents)
    draft = np.zeros(T, np.int32)
    target = np.zeros(T, np.int32)
    a, length, nxt, st = acc.accept_greedy(offsets, parents, draft, target)
    assert st.tolist() == [1, 2, 2, 0]
    assert a.tolist()[:3] == [-1, -1, -1] and length.tolist()[:3] == [0, 0, 0]
    assert nxt.tolist()[:3] == [-1, -1, -1]
    assert (a[3], length[3]) == (1, 2)                    # first child matches token 0
    # empty and oversize ranges
    a, length, nxt, st = acc.accept_greedy(np.array([0, 0, 65], np.int32),
                                           np.array([-1] + list(range(64)), np.int32),
                                           np.zeros(65, np.int32), np.zeros(65, np.int32))
    assert st.tolist() == [3, 3] and a.tolist() == [-1, -1]


# ------------------------------------------------------------------ sampling mode


def _perm_prob(q, cands):
    """Probability that sampling without replacement from q yields `cands` in order."""
    q = np.asarray(q, np.float64).copy()
    pr = 1.0
    for x in cands:
        pr *= q[x] / q.sum()
        q[x] = 0.0
    return pr


@pytest.mark.parametrize("m", [1, 2, 3, 4])
@pytest.mark.parametrize("seed", [0, 1, 2])
def test_sampling_step_preserves_the_target_distribution(m, seed):
    """Handbook, exercises (sampling with a tree): the emitted token has the
    target's distribution. Exact: every ordered draw of m distinct candidates
    from q (without replacement), weighted by its probability, times the
    step's acceptance and residual probabilities, sums to p."""
    import itertools
    rng = np.random.default_rng(seed)
    V = 6
    p = rng.dirichlet(np.ones(V) * 0.7)
    q = rng.dirichlet(np.ones(V) * 0.7)
    out = np.zeros(V)
    for cands in itertools.permutations(range(V), m):
        w = _perm_prob(q, cands)
        probs, resid = acc.node_plan(p, q, list(cands))
        reach = 1.0
        for x, a in zip(cands, probs):
            out[x] += w * reach * a
            reach *= 1.0 - a
        out += w * reach * resid
    np.testing.assert_allclose(out, p, rtol=0, atol=1e-12)


def test_sampling_step_closed_cases():
    p = np.array([0.5, 0.3, 0.2, 0.0])
    # the draft equal to the target: every candidate is accepted
    a, _ = acc.node_plan(p, p, [0, 2])
    assert a[0] == 1.0
    # a candidate the target never emits is always rejected; the residual of
    # a one-hot draft on it is the target itself
    onehot = np.array([0.0, 0.0, 0.0, 1.0])
    a, r = acc.node_plan(p, onehot, [3])
    assert a == [0.0]
    np.testing.assert_allclose(r, p, atol=1e-15)
    # no candidates: the final draw is from p
    a, r = acc.node_plan(p, onehot, [])
    assert a == [] and np.allclose(r, p)


def test_sampling_walk_decisions_and_inverse_cdf():
    # one root with two children; node 1 has one child
    parents = np.array([-1, 0, 0, 1], np.int32)
    V = 4
    P = np.array([[0.1, 0.6, 0.2, 0.1], [0.25, 0.25, 0.25, 0.25], [0.7, 0.1, 0.1, 0.1],
                  [0.4, 0.3, 0.2, 0.1]])
    Q = np.array([[0.1, 0.2, 0.6, 0.1], [0.05, 0.05, 0.1, 0.8], [0.25] * 4, [0.25] * 4])
    draft = np.array([0, 2, 1, 3], np.int32)        # candidates: node 1 -> token 2, node 2 -> 1
    # node 1 (token 2): accept prob min(1, 0.2/0.6) = 1/3
    U = np.array([[0.0, 0.0], [0.2, 0.0], [0.0, 0.0], [0.0, 0.0]])
    path, tok = acc.accept_sampling_one(parents, draft, P, Q, U)
    # accepted node 1; at node 1 its child (token 3) has p 0.25 < q 0.8 -> u=0 accepts
    assert path == [0, 1, 3]
    # at leaf 3 the final draw with u = 0: the first token of P[3]
    assert tok == 0
    U[3, 1] = 0.45                                   # cdf of P[3]: .4 .7 .9 1.0
    assert acc.accept_sampling_one(parents, draft, P, Q, U)[1] == 1
    U[1, 0] = 0.5                                    # reject node 1 (0.5 >= 1/3)
    # second candidate (token 1): against the residual norm(max(0, p - q)) and q
    # without token 2, renormalised
    a, _ = acc.node_plan(P[0], Q[0], [2, 1])
    res = np.maximum(P[0] - Q[0], 0)
    res /= res.sum()
    q2 = Q[0].copy()
    q2[2] = 0
    q2 /= q2.sum()
    assert a == [pytest.approx(1 / 3), pytest.approx(min(1.0, res[1] / q2[1]))]
    path, _ = acc.accept_sampling_one(parents, draft, P, Q, U)
    assert path == [0, 2]                            # residual puts all mass on token 1
    # node 2 drafting token 3 instead: no residual mass there, always rejected;
    # the final draw comes from the residual after both rejections
    draft[2] = 3
    a, r = acc.node_plan(P[0], Q[0], [2, 3])
    assert a[1] == 0.0 and r[1] == pytest.approx(1.0)
    for u in (0.0, 0.5, 0.999):
        U[2, 0] = u
        U[0, 1] = u
        path, tok = acc.accept_sampling_one(parents, draft, P, Q, U)
        assert path == [0] and tok == 1

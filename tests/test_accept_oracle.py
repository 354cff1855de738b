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

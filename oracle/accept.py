"""Greedy acceptance of a verified draft tree, the plain way (test
infrastructure only, like the rest of this package: nothing in the GPU library
imports it, and it imports nothing from the library).

Follows the generation loop of the handbook (anrans.github.io
ai-infra-handbooks "speculative", implementation section): the accepted path
starts at the root; at the current node the target's predicted next token is
compared with the draft token of every child, scanning nodes in index order;
the first match is appended to the path and becomes the current node; when no
child matches the walk ends. The target's prediction at the last accepted node
is the token the target contributes itself (the next round's root).

Tree checks and status codes are those of the library's header (size, then
root, then parents), re-derived here from the definitions.
"""
from __future__ import annotations

import numpy as np

STATUS_OK, STATUS_BAD_ROOT, STATUS_BAD_PARENT, STATUS_BAD_SIZE = 0, 1, 2, 3
STATUS_BAD_TOKEN = 7


def tree_check(offsets, parents, b, max_nodes=64):
    """Status of sequence b's node range and parent array."""
    lo, hi = int(offsets[b]), int(offsets[b + 1])
    n = hi - lo
    if lo < 0 or hi > len(parents) or n < 1 or n > max_nodes:
        return STATUS_BAD_SIZE
    if int(parents[lo]) != -1:
        return STATUS_BAD_ROOT
    for i in range(1, n):
        p = int(parents[lo + i])
        if p < 0 or p >= i:
            return STATUS_BAD_PARENT
    return STATUS_OK


def accept_one(parents, draft_tokens, target_tokens):
    """The greedy walk on one tree (local arrays): the accepted path (node
    indices, root first). Children are listed per node in index order, so the
    first listed child whose draft token equals the target's prediction at the
    current node is the one taken."""
    kids = [[] for _ in range(len(parents))]
    for c in range(1, len(parents)):
        kids[int(parents[c])].append(c)
    walk = [0]
    while True:
        want = int(target_tokens[walk[-1]])
        hits = [c for c in kids[walk[-1]] if int(draft_tokens[c]) == want]
        if not hits:
            return walk
        walk.append(hits[0])


def accept_greedy(offsets, parents, draft_tokens, target_tokens, max_nodes=64):
    """Per sequence: (accepted last node, path length, next token, status);
    a rejected sequence gets (-1, 0, -1, code)."""
    offsets = np.asarray(offsets)
    B = len(offsets) - 1
    accepted = np.full(B, -1, np.int32)
    length = np.zeros(B, np.int32)
    nxt = np.full(B, -1, np.int32)
    status = np.zeros(B, np.int32)
    for b in range(B):
        st = tree_check(offsets, parents, b, max_nodes)
        status[b] = st
        if st != STATUS_OK:
            continue
        lo, hi = int(offsets[b]), int(offsets[b + 1])
        path = accept_one(parents[lo:hi], draft_tokens[lo:hi], target_tokens[lo:hi])
        accepted[b] = path[-1]
        length[b] = len(path)
        nxt[b] = int(target_tokens[lo + path[-1]])
    return accepted, length, nxt, status


# ---------------------------------------------------------------------------
# Sampling mode: multi-candidate rejection sampling down the tree
# ---------------------------------------------------------------------------
#
# The handbook's second exercise (same chapter, exercises: sampling with a
# tree) describes it level by level: at a node, the children -- the draft's
# candidates -- are considered in turn, each accepted with probability
# min(1, p(x)/q(x)); after a rejection the target distribution becomes
# norm(max(0, p - q)) and the next candidate is considered, with q adjusted
# to the way the candidates were drawn; when every candidate is rejected, one
# token is drawn from the last residual and the walk ends. Readings taken
# here: a node's children were drawn from the draft's distribution at that
# node without replacement (a tree's siblings carry distinct tokens), so after
# rejecting x the proposal becomes q with x removed, renormalised; an
# accepted child starts afresh with its own p and q; a node without children
# draws the target's own next token from its p. A residual of zero mass (p no
# larger than q anywhere) leaves p unchanged.


def node_plan(p, q, cands):
    """The step at one node with candidates `cands` (draft tokens of its
    children, in node order): the probability that each candidate is
    accepted once every earlier one was rejected (candidate x is accepted iff
    u * q(x) < p(x) for a uniform u in [0, 1): min(1, p(x)/q(x)), or 1 when
    q(x) = 0 < p(x)), and the distribution the final token is drawn from when
    all are rejected. fp64."""
    p = np.asarray(p, np.float64).copy()
    q = np.asarray(q, np.float64).copy()
    acc_prob = []
    for x in cands:
        px, qx = p[x], q[x]
        if qx > 0:
            acc_prob.append(min(1.0, px / qx))
        else:
            acc_prob.append(1.0 if px > 0 else 0.0)
        res = np.maximum(p - q, 0.0)
        z = res.sum()
        if z > 0:
            p = res / z
        q[x] = 0.0
        s = q.sum()
        if s > 0:
            q = q / s
    return acc_prob, p


def accept_sampling_one(parents, draft_tokens, target_probs, draft_probs, uniforms,
                        margins=None):
    """One tree (local arrays): (accepted path, next token). uniforms[t, 0]
    decides node t as a candidate (accepted iff it is below the acceptance
    probability), uniforms[t, 1] draws the final token at t by inverse CDF
    (the first token whose cumulative mass exceeds u times the total).
    `margins`, when a list, receives the distance of every decision from its
    threshold (relative to the total mass for the draw)."""
    n = len(parents)
    path, node = [0], 0
    while True:
        kids = [c for c in range(n) if int(parents[c]) == node]
        acc, resid = node_plan(target_probs[node], draft_probs[node],
                               [int(draft_tokens[c]) for c in kids])
        nxt = None
        for c, a in zip(kids, acc):
            u = float(uniforms[c, 0])
            if margins is not None:
                margins.append(abs(u - a))
            if u < a:
                nxt = c
                break
        if nxt is None:
            cdf = np.cumsum(resid)
            target = float(uniforms[node, 1]) * cdf[-1]
            tok = min(int(np.searchsorted(cdf, target, side="right")), len(resid) - 1)
            if margins is not None:
                lo_edge = cdf[tok - 1] if tok > 0 else 0.0
                gap = min(abs(target - lo_edge), abs(cdf[tok] - target))
                margins.append(gap / max(cdf[-1], 1e-300))
            return path, tok
        path.append(nxt)
        node = nxt


def accept_sampling(offsets, parents, draft_tokens, target_probs, draft_probs, uniforms,
                    max_nodes=64, margins=None):
    """Per sequence: (accepted last node, path length, next token, status);
    a rejected sequence gets (-1, 0, -1, code), code 7 for a draft token
    outside [0, V) (the tokens index the probability rows). target_probs,
    draft_probs: [T, V]; uniforms [T, 2]."""
    offsets = np.asarray(offsets)
    B = len(offsets) - 1
    accepted = np.full(B, -1, np.int32)
    length = np.zeros(B, np.int32)
    nxt = np.full(B, -1, np.int32)
    status = np.zeros(B, np.int32)
    for b in range(B):
        st = tree_check(offsets, parents, b, max_nodes)
        status[b] = st
        if st != STATUS_OK:
            continue
        lo, hi = int(offsets[b]), int(offsets[b + 1])
        V = np.asarray(target_probs).shape[-1]
        if any(not 0 <= int(x) < V for x in draft_tokens[lo + 1:hi]):
            status[b] = STATUS_BAD_TOKEN
            continue
        path, tok = accept_sampling_one(parents[lo:hi], draft_tokens[lo:hi], target_probs[lo:hi],
                                        draft_probs[lo:hi], uniforms[lo:hi], margins)
        accepted[b] = path[-1]
        length[b] = len(path)
        nxt[b] = tok
    return accepted, length, nxt, status

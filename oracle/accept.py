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
    """The handbook's walk on one tree (local arrays): the accepted path (node
    indices, root first)."""
    n = len(parents)
    path, node = [0], 0
    while True:
        pred = int(target_tokens[node])
        child = None
        for c in range(n):
            if int(parents[c]) == node and int(draft_tokens[c]) == pred:
                child = c
                break
        if child is None:
            return path
        path.append(child)
        node = child


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

"""Tree-shaped WY form of the gated delta rule, dense fp64 numpy.

TEST INFRASTRUCTURE ONLY (see the package docstring). This is a second,
independent route to the same numbers as the per-path replay in
gdn_oracle.c. It is used to pin the replay oracle (two different
computations of one definition must agree to rounding) and to check the GPU
library's stored intermediates (pseudo-values and gate prefixes) stage by
stage.

The TreeWY abstract (arxivdaily 2608.20961, English abstract) states the
idea: one triangular solve per draft tree gives every node's output, a small
pseudo-value matrix replaces per-node states, and only the accepted state is
rebuilt at commit. The equations below are the plainest derivation that
reaches that from the gated delta rule S_t = a_t S_p (I - b_t k_t k_t^T)
+ b_t v_t k_t^T, with A(t) = ancestors of t including t and
G_t = prod_{j in A(t)} a_j = exp(g_t):

  S_t = G_t S0 + sum_{i in A(t)} (G_t / G_i) u_i k_i^T        (induction on depth)
  u_t = b_t (v_t - G_t S0 k_t - sum_{i in A(t), i != t} (G_t/G_i)(k_i.k_t) u_i)
  i.e. (I + A_kk) U = diag(b) (V - diag(G) K S0^T),
       A_kk[t,i] = b_t (G_t/G_i) (k_t.k_i) for i a proper ancestor of t,
  O = diag(G) Q S0^T + A_qk U,  A_qk[t,i] = (G_t/G_i)(q_t.k_i) for i in A(t),
  S_a = G_a S0 + sum_{i in A(a)} (G_a/G_i) u_i k_i^T             (commit).

I + A_kk is unit lower triangular in topological order, so one triangular
solve per (tree, head) gives U.
"""
from __future__ import annotations

import numpy as np
import scipy.linalg


def ancestor_matrix(parents) -> np.ndarray:
    """M[t, i] = True iff i is t or an ancestor of t (boolean reachability
    through the parent relation, built by repeated boolean products)."""
    n = len(parents)
    P = np.zeros((n, n), dtype=bool)
    for t, p in enumerate(parents):
        if p >= 0:
            P[t, p] = True
    M = np.eye(n, dtype=bool)
    reach = np.eye(n, dtype=bool)
    for _ in range(n):
        reach = (reach.astype(np.int64) @ P.astype(np.int64)) > 0
        if not reach.any():
            break
        M |= reach
    return M


def wy_tree(parents, q, k, v, alpha, beta, S0):
    """One tree, one head. q,k [n,dk]; v [n,dv]; alpha,beta [n]; S0 [dv,dk].
    Returns dict with g (natural-log gate prefix), U [n,dv], O [n,dv]."""
    q, k, v, alpha, beta, S0 = (np.asarray(x, dtype=np.float64) for x in (q, k, v, alpha, beta, S0))
    M = ancestor_matrix(parents)
    g = M.astype(np.float64) @ np.log(alpha)
    G = np.exp(g)
    ratio = np.where(M, np.exp(g[:, None] - g[None, :]), 0.0)
    strict = M & ~np.eye(len(parents), dtype=bool)
    Akk = np.where(strict, beta[:, None] * ratio * (k @ k.T), 0.0)
    Aqk = np.where(M, ratio * (q @ k.T), 0.0)
    R = beta[:, None] * (v - G[:, None] * (k @ S0.T))
    U = scipy.linalg.solve_triangular(np.eye(len(parents)) + Akk, R, lower=True, unit_diagonal=True)
    O = G[:, None] * (q @ S0.T) + Aqk @ U
    return {"g": g, "U": U, "O": O, "M": M}


def wy_commit(parents, node, k, U, g, S0):
    """State of `node` rebuilt from pseudo-values: G_a S0 + sum (G_a/G_i) u_i k_i^T."""
    if node < 0:
        return np.array(S0, dtype=np.float64, copy=True)
    M = ancestor_matrix(parents)
    path = np.nonzero(M[node])[0]
    w = np.exp(g[node] - g[path])
    return np.exp(g[node]) * np.asarray(S0, np.float64) + (U[path] * w[:, None]).T @ np.asarray(k, np.float64)[path]


def wy_batch(offsets, parents, q, k, v, alpha, beta, S0):
    """Whole batch: returns (O [T,H,dv], U [T,H,dv], g [T,H])."""
    T, H, dk = q.shape
    dv = v.shape[2]
    O = np.zeros((T, H, dv))
    U = np.zeros((T, H, dv))
    g = np.zeros((T, H))
    for b in range(len(offsets) - 1):
        lo, hi = int(offsets[b]), int(offsets[b + 1])
        par = [int(x) for x in parents[lo:hi]]
        for h in range(H):
            r = wy_tree(par, q[lo:hi, h], k[lo:hi, h], v[lo:hi, h], alpha[lo:hi, h],
                        beta[lo:hi, h], S0[b, h])
            O[lo:hi, h], U[lo:hi, h], g[lo:hi, h] = r["O"], r["U"], r["g"]
    return O, U, g

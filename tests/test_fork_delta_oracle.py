"""Pin of the identity behind the delta-compressed fork checkpoints
(fork page "Qwen3.5 tree spec", section 8, checkpoint compression: keep only
what a child's state adds to its parent's).

Under the gated delta rule a child's checkpoint minus its decayed parent's is
exactly rank one: C_t - alpha_t C_p = u_t k_t^T with u_t = beta_t (v_t -
alpha_t C_p k_t). The GPU library's delta-fork mode keeps u_t and rebuilds the
accepted state from the deltas of its path with the WY commit, which is right
only if these u_t are the WY pseudo-values. Checked here in fp64 between the
oracle's two independent routes: the depth-by-depth fork replay
(oracle/gdn_oracle.c) and the dense tree-WY solve (oracle/wy.py)."""
import numpy as np
import pytest

import gdn_inputs as gi
import oracle
from oracle import wy


@pytest.mark.parametrize("name", ["c1", "c2"])
def test_fork_deltas_are_rank_one_wy_pseudo_values(name):
    w = gi.make_config(name)
    if name == "c2":
        w = gi.make_workload([gi.kary_parents(3, 2), gi.chain_parents(6)], H=3, dk=32, dv=32,
                             io="f32", seed=17)
    q, k, v, a, b, S0 = (np.asarray(x[0], np.float64) for x in (w.q, w.k, w.v, w.alpha, w.beta,
                                                                 w.S0))
    _, ck, st = oracle.fork_replay(w.offsets, w.parents, q, k, v, a, b, S0)
    assert (st == 0).all()
    _, U, g = wy.wy_batch(w.offsets, w.parents, q, k, v, a, b, S0)
    worst = 0.0
    for s in range(w.B):
        lo, hi = int(w.offsets[s]), int(w.offsets[s + 1])
        for t in range(hi - lo):
            p = int(w.parents[lo + t])
            for h in range(w.H):
                Cp = S0[s, h] if p < 0 else ck[lo + p, h]
                D = ck[lo + t, h] - a[lo + t, h] * Cp
                R = np.outer(U[lo + t, h], k[lo + t, h])
                worst = max(worst, np.linalg.norm(D - R) / np.linalg.norm(D))
                sv = np.linalg.svd(D, compute_uv=False)
                assert sv[1] <= 1e-12 * sv[0]
    assert worst <= 1e-12


def test_commit_from_deltas_equals_checkpoint():
    """Rebuilding the accepted state from S0 and its path's deltas (the WY
    commit) gives the fork checkpoint of that node."""
    w = gi.make_workload([gi.kary_parents(2, 3)] * 2, H=2, dk=32, dv=32, io="f32", seed=23)
    q, k, v, a, b, S0 = (np.asarray(x[0], np.float64) for x in (w.q, w.k, w.v, w.alpha, w.beta,
                                                                 w.S0))
    _, ck, _ = oracle.fork_replay(w.offsets, w.parents, q, k, v, a, b, S0)
    _, U, g = wy.wy_batch(w.offsets, w.parents, q, k, v, a, b, S0)
    for s in range(w.B):
        lo, hi = int(w.offsets[s]), int(w.offsets[s + 1])
        par = [int(x) for x in w.parents[lo:hi]]
        for node in range(hi - lo):
            for h in range(w.H):
                S = wy.wy_commit(par, node, k[lo:hi, h], U[lo:hi, h], g[lo:hi, h], S0[s, h])
                ref = ck[lo + node, h]
                assert np.linalg.norm(S - ref) <= 1e-12 * np.linalg.norm(ref)

"""GPU parity of the fused round boundary, gdn_tree_commit_verify[_layers] and
gdn_tree_replay_verify[_layers]: the previous round's commit (from its
pseudo-values, or by replaying its accepted path) and this round's verify in
one pass over the state.

Reference: the oracle's commit of the previous tree's accepted path (fp64 path
replay from S0), then the oracle's verify of this round's tree from that
committed state. Agreement bar as for the separate calls: 1e-4 (fp32 io) or
2e-2 (bf16 io) normwise relative error per output vector and per (sequence,
head) state; status codes bit-exact. The fused results are also compared with
the library's own separate commit + verify, and the layer-batched, in-place
and out-of-place forms with each other (bit-identical)."""
import numpy as np
import pytest
import torch

import gated_deltanet_tree_02_amd as gt
import gdn_inputs as gi
import oracle

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():  # the -m gpu suite only runs on a GPU machine
    pytest.skip("no GPU", allow_module_level=True)

from gpu_util import (TOL, DeviceLayer, rel_err_rows, rel_err_states,  # noqa: E402
                      sub_workload)


def _say(*a):
    print("[gpu-commit-verify]", *a, flush=True)


MODES = ["wy", "replay"]


def _fused(P, C, S0, S_out, mode="wy"):
    """One fused call: commit P's accepted paths (S0 -> S_out), verify C on S_out."""
    if mode == "wy":
        gt.gdn_tree_commit_verify(P.desc, P.offsets, P.parents, P.accepted, P.k, P.ws, C.desc,
                                  C.offsets, C.parents, C.q, C.k, C.v, C.alpha, C.beta, S0,
                                  S_out, C.o, C.ws, C.status)
    else:
        gt.gdn_tree_replay_verify(P.desc, P.offsets, P.parents, P.accepted, P.k, P.v, P.alpha,
                                  P.beta, C.desc, C.offsets, C.parents, C.q, C.k, C.v, C.alpha,
                                  C.beta, S0, S_out, C.o, C.status)


def _fused_layers(Ps, Cs, S0s, S_outs, status, mode="wy"):
    """The layer-batched form over the layers (DeviceLayer lists)."""
    P0, C0 = Ps[0], Cs[0]
    if mode == "wy":
        pio = [gt.make_layer_io(P.desc, k=P.k, workspace=P.ws) for P in Ps]
        cio = [gt.make_layer_io(C.desc, q=C.q, k=C.k, v=C.v, alpha=C.alpha, beta=C.beta, S0=S,
                                o=C.o, S_out=So, workspace=C.ws)
               for C, S, So in zip(Cs, S0s, S_outs)]
        gt.gdn_tree_commit_verify_layers(P0.desc, C0.desc, P0.offsets, P0.parents, P0.accepted,
                                         C0.offsets, C0.parents, pio, P0.ws.numel(), cio,
                                         C0.ws.numel(), status)
    else:
        pio = [gt.make_layer_io(P.desc, k=P.k, v=P.v, alpha=P.alpha, beta=P.beta) for P in Ps]
        cio = [gt.make_layer_io(C.desc, q=C.q, k=C.k, v=C.v, alpha=C.alpha, beta=C.beta, S0=S,
                                o=C.o, S_out=So) for C, S, So in zip(Cs, S0s, S_outs)]
        gt.gdn_tree_replay_verify_layers(P0.desc, C0.desc, P0.offsets, P0.parents, P0.accepted,
                                         C0.offsets, C0.parents, pio, cio, status)


def _oracle_rounds(wp, wc, layer=0):
    S_ref, stc = oracle.commit(wp.offsets, wp.parents, wp.accepted, wp.k[layer], wp.v[layer],
                               wp.alpha[layer], wp.beta[layer], wp.S0[layer])
    o_ref, st = oracle.verify(wc.offsets, wc.parents, wc.q[layer], wc.k[layer], wc.v[layer],
                              wc.alpha[layer], wc.beta[layer], S_ref)
    return S_ref, stc, o_ref, st


def _case(prev_trees, cur_trees, H, d, io, seed, force_acc=None):
    wp = gi.make_workload(prev_trees, H, d, d, io=io, seed=seed)
    wc = gi.make_workload(cur_trees, H, d, d, io=io, seed=seed + 1000)
    for b, a in (force_acc or {}).items():   # -1: the state is kept as it is
        wp.accepted[b] = a
    return wp, wc


CASES = {
    # previous k=3 d=3 trees (three 16-node tiles), this round ragged up to 64 nodes
    "kary_then_ragged": lambda: _case(
        [gi.kary_parents(3, 3)] * 8,
        [gi.random_tree_parents(np.random.default_rng(7 + i)) for i in range(8)],
        4, 128, "bf16", 11, force_acc={2: -1}),
    # a deep previous chain: accepted paths longer than one staging round
    "deep_chain_then_kary": lambda: _case(
        [gi.chain_parents(n) for n in (12, 9, 5, 1, 30)], [gi.kary_parents(2, 2)] * 5,
        4, 64, "bf16", 12, force_acc={0: 11, 1: 6, 4: 29}),
    # bf16 rows of 128 with this round's trees in three node tiles: the path
    # rows stay in registers; deep chains need several rounds of them
    "deep_chain_then_kary3_d128": lambda: _case(
        [gi.chain_parents(n) for n in (12, 30, 3, 7, 1, 5)], [gi.kary_parents(3, 3)] * 6,
        4, 128, "bf16", 15, force_acc={0: 11, 1: 29, 2: 2, 3: 4, 4: 0, 5: -1}),
    "tiny_fp32": lambda: _case([[-1, 0, 0, 1, 1, 2, 2]] * 2, [gi.kary_parents(2, 3)] * 2,
                               2, 32, "f32", 13, force_acc={0: 3, 1: -1}),
    "ragged_fp32_d128": lambda: _case(
        [gi.random_tree_parents(np.random.default_rng(30 + i), 16, 40) for i in range(4)],
        [gi.random_tree_parents(np.random.default_rng(40 + i), 2, 20) for i in range(4)],
        2, 128, "f32", 14),
}


@pytest.mark.parametrize("mode", MODES)
@pytest.mark.parametrize("name", list(CASES))
def test_commit_verify_matches_oracle(name, mode):
    wp, wc = CASES[name]()
    deep = max(len(gi.path_to_root(p, a)) if a >= 0 else 0
               for p, a in zip(wp.parents_list, wp.accepted))
    _say(f"{name}: B={wp.B} H={wp.H} d={wp.dk} io={wp.io} prev T={wp.T} cur T={wc.T} "
         f"longest accepted path {deep}")
    P, C = DeviceLayer(wp, 0), DeviceLayer(wc, 0)
    P.verify()
    S0 = P.S0.clone()
    S_out = torch.full_like(S0, float("nan"))
    _fused(P, C, S0, S_out, mode)
    torch.cuda.synchronize()
    S_ref, stc, o_ref, st = _oracle_rounds(wp, wc)
    assert np.all(stc == 0) and np.all(st == 0)
    assert np.all(C.status.cpu().numpy() == 0)
    tol = TOL[wp.io]
    e_s = rel_err_states(S_out.cpu().numpy(), S_ref)
    e_o = rel_err_rows(C.o_np(), o_ref)
    _say(f"{name} ({mode}): S err {e_s:.3e}, o err {e_o:.3e} (tol {tol})")
    assert e_s <= tol and e_o <= tol
    # accepted = -1 keeps the state bit for bit
    for b in np.nonzero(wp.accepted < 0)[0]:
        assert torch.equal(S_out[b], S0[b])
    # the library's separate commit, then verify on the committed state
    S_sep = torch.full_like(S0, float("nan"))
    P.commit(S_out=S_sep)
    C2 = DeviceLayer(wc, 0)
    C2.S0 = S_sep
    C2.verify()
    torch.cuda.synchronize()
    e_ss = rel_err_states(S_out.cpu().numpy(), S_sep.cpu().numpy())
    e_oo = rel_err_rows(C.o_np(), C2.o_np())
    _say(f"{name} ({mode}): fused vs separate calls: S {e_ss:.3e}, o {e_oo:.3e}")
    # (the replay applies the path as a recurrence: another fp32 rounding order)
    assert e_ss <= (1e-6 if mode == "wy" else 2e-5)
    # (fp32 io: the pseudo-value path matches the separate calls' rounding
    # order; the replay applies the path as a recurrence)
    assert e_oo <= ((1e-6 if mode == "wy" else 1e-5) if wp.io == "f32" else 8e-3)
    if mode == "wy":
        U, g2 = C.wy_parts()
        U2, g22 = C2.wy_parts()
        assert rel_err_rows(U, U2) <= 1e-5 and np.array_equal(g2, g22)


@pytest.mark.parametrize("mode", MODES)
def test_commit_verify_in_place_equals_out_of_place(mode):
    wp, wc = CASES["kary_then_ragged"]()
    P, C1, C2 = DeviceLayer(wp, 0), DeviceLayer(wc, 0), DeviceLayer(wc, 0)
    P.verify()
    S_keep = P.S0.clone()
    S_out = torch.full_like(S_keep, float("nan"))
    _fused(P, C1, P.S0, S_out, mode)
    S_in = S_keep.clone()
    _fused(P, C2, S_in, S_in, mode)
    torch.cuda.synchronize()
    assert torch.equal(P.S0, S_keep)            # out of place leaves S0 alone
    assert torch.equal(S_in, S_out)
    assert torch.equal(C1.o, C2.o)
    if mode == "wy":
        for x, y in zip(C1.wy_parts(), C2.wy_parts()):
            assert np.array_equal(x, y)


@pytest.mark.parametrize("mode", MODES)
def test_commit_verify_layers_bit_identical_to_single_calls(mode):
    L = 3
    rng = np.random.default_rng(5)
    prev_trees = [gi.random_tree_parents(rng, 8, 48) for _ in range(6)]
    cur_trees = [gi.random_tree_parents(rng, 8, 48) for _ in range(6)]
    wp = gi.make_workload(prev_trees, 4, 128, 128, io="bf16", layers=L, seed=21)
    wc = gi.make_workload(cur_trees, 4, 128, 128, io="bf16", layers=L, seed=22)
    Ps = [DeviceLayer(wp, l) for l in range(L)]
    Cs = [DeviceLayer(wc, l) for l in range(L)]
    Cb = [DeviceLayer(wc, l) for l in range(L)]
    for P in Ps:
        P.verify()
    S_single = [P.S0.clone() for P in Ps]
    S_batch = [P.S0.clone() for P in Ps]
    for P, C, S in zip(Ps, Cs, S_single):
        _fused(P, C, S, S, mode)
    status = torch.full((wp.B,), -7, dtype=torch.int32, device="cuda")
    _fused_layers(Ps, Cb, S_batch, S_batch, status, mode)
    torch.cuda.synchronize()
    assert np.all(status.cpu().numpy() == 0)
    for l in range(L):
        assert torch.equal(S_single[l], S_batch[l]), l
        assert torch.equal(Cs[l].o, Cb[l].o), l
        if mode == "wy":
            for x, y in zip(Cs[l].wy_parts(), Cb[l].wy_parts()):
                assert np.array_equal(x, y), l


@pytest.mark.parametrize("mode", MODES)
def test_commit_verify_status_codes(mode):
    """Two outcomes per sequence: this round's tree in the low bits, the
    previous round's commit above gt.PREV_SHIFT. A rejected previous commit
    (bad previous tree, accepted index out of range) leaves S_out unwritten
    and zeroes the o rows; a rejected current tree zeroes its o rows but the
    previous commit is still applied (nothing of the accepted tokens is lost);
    accepted = -1 checks nothing of the previous tree. Other sequences are
    unaffected."""
    prev_trees = [gi.kary_parents(2, 2)] * 8
    cur_trees = [gi.kary_parents(2, 2)] * 6 + [gi.kary_parents(2, 3), gi.kary_parents(2, 2)]
    wp = gi.make_workload(prev_trees, 2, 64, 64, io="bf16", seed=31)
    wc = gi.make_workload(cur_trees, 2, 64, 64, io="bf16", seed=32)
    wp.accepted[:] = [3, 9, 4, 5, -1, -1, 6, 8]
    P = DeviceLayer(wp, 0)
    C = DeviceLayer(wc, 0, max_nodes=7)     # seq 6 (15 nodes) is too large this round
    P.verify()
    torch.cuda.synchronize()
    assert np.all(P.status.cpu().numpy() == 0)
    # seqs 2 and 5: the previous tree is rewritten with a bad parent after its verify
    par = P.parents.cpu().numpy()
    for b in (2, 5):
        par[wp.offsets[b] + 3] = 5
    P.parents.copy_(torch.from_numpy(par))
    # seqs 3 and 7: this round's tree has a bad root
    cpar = C.parents.cpu().numpy()
    for b in (3, 7):
        cpar[wc.offsets[b]] = 0
    C.parents.copy_(torch.from_numpy(cpar))
    S0 = P.S0.clone()
    S_out = torch.full_like(S0, float("nan"))
    _fused(P, C, S0, S_out, mode)
    torch.cuda.synchronize()
    st = C.status.cpu().numpy()
    prev = gt.prev_code
    # 0 ok; 1 accepted out of range; 2 bad previous parent; 3 bad root now;
    # 4, 5 accepted -1 (5's previous tree is bad but unchecked); 6 too large
    # now; 7 bad root now and accepted out of range
    assert st.tolist() == [0, prev(4), prev(2), 1, 0, 0, 3, 1 | prev(4)]
    o = C.o_np()
    U, g2 = C.wy_parts()
    for b in (1, 2, 3, 7):
        rows = slice(wc.offsets[b], wc.offsets[b + 1])
        assert np.all(o[rows] == 0), b
        if mode == "wy":
            assert np.all(U[rows] == 0) and np.all(g2[rows] == 0)
    for b in (1, 2, 7):                      # previous commit rejected: not written
        assert torch.isnan(S_out[b]).all(), b
    for b in (4, 5):                         # accepted -1: S0 copied
        assert torch.equal(S_out[b], S0[b]), b
    # the previous commit applied to 0, 3 (this round rejected) and 6 (too large now)
    done = [0, 3, 6]
    sp = sub_workload(wp, done)
    S_ref, stc = oracle.commit(sp.offsets, sp.parents, sp.accepted, sp.k[0], sp.v[0],
                               sp.alpha[0], sp.beta[0], sp.S0[0])
    assert np.all(stc == 0)
    e_s = rel_err_states(S_out.cpu().numpy()[done], S_ref)
    _say(f"status codes ({mode}): committed state err {e_s:.3e} on sequences {done}")
    assert e_s <= TOL["bf16"]
    # this round's outputs of 0 (against its committed state), 4 and 5 (against S0)
    keep = [0, 4, 5]
    sc = sub_workload(wc, keep)
    S_keep = np.stack([S_ref[0], wp.S0[0][4], wp.S0[0][5]])
    o_ref, st_ref = oracle.verify(sc.offsets, sc.parents, sc.q[0], sc.k[0], sc.v[0], sc.alpha[0],
                                  sc.beta[0], S_keep)
    assert np.all(st_ref == 0)
    rows = np.concatenate([np.arange(wc.offsets[b], wc.offsets[b + 1]) for b in keep])
    assert rel_err_rows(o[rows], o_ref) <= TOL["bf16"]


@pytest.mark.parametrize("mode", MODES)
def test_commit_verify_bad_previous_node_range(mode):
    """A previous round whose node range is malformed: too many nodes for its
    descriptor, a range shifted onto another sequence's nodes (its first node
    is no root), or a range past the node count. Each rejects that sequence's
    previous commit (S_out unwritten, o rows zero) with the code above
    gt.PREV_SHIFT; accepted = -1 checks nothing; the other sequences commit
    and verify as the oracle does."""
    prev_trees = [gi.kary_parents(2, 2)] * 6
    cur_trees = [gi.kary_parents(2, 2)] * 6
    wp = gi.make_workload(prev_trees, 2, 64, 64, io="bf16", seed=33)
    wc = gi.make_workload(cur_trees, 2, 64, 64, io="bf16", seed=34)
    wp.accepted[:] = [3, 5, 3, 4, 6, -1]
    P, C = DeviceLayer(wp, 0), DeviceLayer(wc, 0)
    P.verify()
    torch.cuda.synchronize()
    assert np.all(P.status.cpu().numpy() == 0)
    offs = wp.offsets.copy()
    offs[3] += 1          # seq 2: 8 nodes (> 7); seq 3: starts on its own second node
    offs[5] = wp.T + 5    # seq 4 ends past the node count; seq 5 is empty (unchecked)
    P.offsets.copy_(torch.from_numpy(offs.astype(np.int32)))
    S0 = P.S0.clone()
    S_out = torch.full_like(S0, float("nan"))
    _fused(P, C, S0, S_out, mode)
    torch.cuda.synchronize()
    prev = gt.prev_code
    assert C.status.cpu().numpy().tolist() == [0, 0, prev(3), prev(1), prev(3), 0]
    o = C.o_np()
    for b in (2, 3, 4):
        assert torch.isnan(S_out[b]).all(), b
        assert np.all(o[wc.offsets[b]:wc.offsets[b + 1]] == 0), b
    assert torch.equal(S_out[5], S0[5])
    done = [0, 1]
    sp = sub_workload(wp, done)
    S_ref, stc = oracle.commit(sp.offsets, sp.parents, sp.accepted, sp.k[0], sp.v[0],
                               sp.alpha[0], sp.beta[0], sp.S0[0])
    assert np.all(stc == 0)
    e_s = rel_err_states(S_out.cpu().numpy()[done], S_ref)
    keep = [0, 1, 5]
    sc = sub_workload(wc, keep)
    S_keep = np.stack([S_ref[0], S_ref[1], wp.S0[0][5]])
    o_ref, st_ref = oracle.verify(sc.offsets, sc.parents, sc.q[0], sc.k[0], sc.v[0], sc.alpha[0],
                                  sc.beta[0], S_keep)
    assert np.all(st_ref == 0)
    rows = np.concatenate([np.arange(wc.offsets[b], wc.offsets[b + 1]) for b in keep])
    e_o = rel_err_rows(o[rows], o_ref)
    _say(f"bad previous node range ({mode}): committed state err {e_s:.3e}, o err {e_o:.3e}")
    assert e_s <= TOL["bf16"] and e_o <= TOL["bf16"]


@pytest.mark.parametrize("mode", MODES)
def test_commit_verify_c4_full_size_sampled(mode):
    """Two consecutive rounds of the k=3 d=3, B=64, 16-head, 128x128 workload
    over all 24 GDN layers in one layer-batched launch (the benchmark's
    configuration); the oracle recomputes sampled (layer, sequence) units."""
    wp = gi.make_config("c4")
    wc = gi.make_config("c4", seed=104)
    L = wp.layers
    Ps = [DeviceLayer(wp, l) for l in range(L)]
    for P in Ps:
        P.verify()
    Cs = [DeviceLayer(wc, l) for l in range(L)]
    status = torch.full((wp.B,), -7, dtype=torch.int32, device="cuda")
    S = [P.S0 for P in Ps]
    _fused_layers(Ps, Cs, S, S, status, mode)
    torch.cuda.synchronize()
    assert np.all(status.cpu().numpy() == 0)
    rng = np.random.default_rng(41)
    layers = sorted(rng.choice(L, 2, replace=False).tolist())
    seqs = sorted(rng.choice(wp.B, 5, replace=False).tolist())
    rows = np.concatenate([np.arange(wc.offsets[b], wc.offsets[b + 1]) for b in seqs])
    for layer in layers:
        sp = sub_workload(wp, seqs, layers=[layer])
        sc = sub_workload(wc, seqs, layers=[layer])
        S_ref, _, o_ref, _ = _oracle_rounds(sp, sc)
        e_s = rel_err_states(Ps[layer].S0.cpu().numpy()[seqs], S_ref)
        e_o = rel_err_rows(Cs[layer].o_np()[rows], o_ref)
        _say(f"c4 ({mode}) layer {layer} seqs {seqs}: S err {e_s:.3e}, o err {e_o:.3e}")
        assert e_s <= TOL["bf16"] and e_o <= TOL["bf16"]


@pytest.mark.parametrize("mode", MODES)
@pytest.mark.parametrize("name,nseq", [("c3", 32), ("c5", 12)])
def test_commit_verify_full_size_one_layer(name, nseq, mode):
    """The k=2 d=3 (B=32) and ragged (B=128, 16-64 nodes) workloads at full
    size, two consecutive rounds with their own trees (ragged: the next
    round's trees differ from the previous round's), in the benchmark's
    launch; the oracle recomputes every sequence (c3) or a sample including
    the largest and smallest trees (c5)."""
    wp = gi.make_config(name)
    wc = gi.make_config(name, seed=gi.CONFIGS[name]["seed"] + 100)
    P, C = DeviceLayer(wp, 0, max_nodes=64), DeviceLayer(wc, 0, max_nodes=64)
    P.verify()
    status = torch.full((wp.B,), -7, dtype=torch.int32, device="cuda")
    _fused_layers([P], [C], [P.S0], [P.S0], status, mode)
    torch.cuda.synchronize()
    assert np.all(status.cpu().numpy() == 0)
    if nseq >= wp.B:
        seqs = list(range(wp.B))
    else:
        rng = np.random.default_rng(43)
        sp, sc = np.diff(wp.offsets), np.diff(wc.offsets)
        seqs = sorted(set([int(np.argmax(sp)), int(np.argmin(sp)), int(np.argmax(sc)),
                           int(np.argmin(sc))] + rng.choice(wp.B, nseq, replace=False).tolist()))
    rows = np.concatenate([np.arange(wc.offsets[b], wc.offsets[b + 1]) for b in seqs])
    S_ref, _, o_ref, _ = _oracle_rounds(sub_workload(wp, seqs), sub_workload(wc, seqs))
    e_s = rel_err_states(P.S0.cpu().numpy()[seqs], S_ref)
    e_o = rel_err_rows(C.o_np()[rows], o_ref)
    _say(f"{name} ({mode}) full size, {len(seqs)} sequences: S err {e_s:.3e}, o err {e_o:.3e}")
    assert e_s <= TOL["bf16"] and e_o <= TOL["bf16"]


@pytest.mark.parametrize("mode", MODES)
def test_multi_round_pipeline_against_the_oracle(mode):
    """Six rounds, each with its own random trees, inputs and accepted paths:
    round r's fused call commits round r-1 and verifies round r (in place on
    the state); every round's outputs, and the state after the last round's
    separate commit, follow the oracle's sequence of commits and verifies."""
    rng = np.random.default_rng(99)
    B, H, d, R = 4, 2, 128, 6
    rounds = []
    for r in range(R):
        trees = [gi.random_tree_parents(rng, 2, 48, max_depth=5) for _ in range(B)]
        w = gi.make_workload(trees, H, d, d, io="bf16", seed=500 + r)
        if r == 1:
            w.accepted[0] = -1                     # one sequence keeps its state once
        rounds.append(w)
    layers = [DeviceLayer(w, 0, max_nodes=64) for w in rounds]
    S = layers[0].S0                               # the state, updated in place
    S_ref = np.asarray(rounds[0].S0[0], np.float64)
    for r, (w, C) in enumerate(zip(rounds, layers)):
        if r == 0:
            C.S0 = S
            C.verify()
        else:
            _fused(layers[r - 1], C, S, S, mode)
            P = rounds[r - 1]
            S_ref, _ = oracle.commit(P.offsets, P.parents, P.accepted, P.k[0], P.v[0],
                                     P.alpha[0], P.beta[0], S_ref)
        torch.cuda.synchronize()
        assert np.all(C.status.cpu().numpy() == 0), r
        o_ref, _ = oracle.verify(w.offsets, w.parents, w.q[0], w.k[0], w.v[0], w.alpha[0],
                                 w.beta[0], S_ref)
        e_o = rel_err_rows(C.o_np(), o_ref)
        e_s = rel_err_states(S.cpu().numpy(), S_ref)
        _say(f"multi-round ({mode}) round {r}: o err {e_o:.3e}, state err {e_s:.3e}")
        assert e_o <= TOL["bf16"] and e_s <= TOL["bf16"], r
    # the last round committed with the separate call (from its workspace)
    last, L = rounds[-1], layers[-1]
    L.S0 = S.clone()                                # the state the last round verified against
    if mode == "replay":                            # replay verifies write no workspace
        L.verify()
    L.commit(S_out=S)
    torch.cuda.synchronize()
    S_ref, _ = oracle.commit(last.offsets, last.parents, last.accepted, last.k[0], last.v[0],
                             last.alpha[0], last.beta[0], S_ref)
    e_s = rel_err_states(S.cpu().numpy(), S_ref)
    _say(f"multi-round ({mode}) final commit: state err {e_s:.3e}")
    assert e_s <= TOL["bf16"]

"""Layer-batched verify/commit (gdn_tree_verify_layers / gdn_tree_commit_layers)
against the per-layer calls, through the C ABI: the same kernels per
workgroup, so outputs, workspaces, committed states and status codes must be
bit-identical; and the per-layer results stay within the oracle tolerance."""
import numpy as np
import pytest
import torch

import gated_deltanet_tree_02_amd as gt
import gdn_inputs as gi

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():  # the -m gpu suite only runs on a GPU machine
    pytest.skip("no GPU", allow_module_level=True)

from gpu_util import TOL, DeviceLayer, oracle_layer, rel_err_rows, rel_err_states  # noqa: E402


def _say(*a):
    print("[gpu-layers]", *a, flush=True)


def _run_both(w, mode=gt.MODE_WY, max_depth=0):
    """Per-layer calls and layer-batched calls on copies of the same inputs."""
    single = [DeviceLayer(w, layer=l, mode=mode, max_depth=max_depth) for l in range(w.layers)]
    batched = [DeviceLayer(w, layer=l, mode=mode, max_depth=max_depth) for l in range(w.layers)]
    for d in single:
        d.verify()
    for d in single:
        d.commit()
    d0 = batched[0]
    nb = gt.gdn_tree_workspace_bytes(d0.desc)
    ios = [gt.make_layer_io(d.desc, q=d.q, k=d.k, v=d.v, alpha=d.alpha, beta=d.beta, S0=d.S0,
                            o=d.o, S_out=d.S_out, workspace=d.ws) for d in batched]
    status = torch.full((w.B,), -7, dtype=torch.int32, device="cuda")
    gt.gdn_tree_verify_layers(d0.desc, d0.offsets, d0.parents, ios, nb, status)
    gt.gdn_tree_commit_layers(d0.desc, d0.offsets, d0.parents, d0.accepted, ios, nb, status)
    torch.cuda.synchronize()
    return single, batched, status


def _assert_identical(single, batched, status):
    for l, (a, b) in enumerate(zip(single, batched)):
        assert torch.equal(a.o.view(torch.int16) if a.o.dtype == torch.bfloat16 else a.o,
                           b.o.view(torch.int16) if b.o.dtype == torch.bfloat16 else b.o), l
        if a.desc.mode == gt.MODE_WY:          # U and g2 (the alignment padding is never written)
            (ua, ga), (ub, gb) = a.wy_parts(), b.wy_parts()
            assert np.array_equal(ua, ub) and np.array_equal(ga, gb), l
        assert torch.equal(a.S_out.view(torch.int32), b.S_out.view(torch.int32)), l
    assert torch.equal(single[-1].status, status)


@pytest.mark.parametrize("name,layers", [("c3", 3), ("c5", 2), ("c1", 4)])
def test_layers_bit_identical_to_per_layer_calls(name, layers):
    _say(name, layers)
    w = gi.make_config(name, layers=layers) if name != "c1" else gi.make_workload(
        [[-1, 0, 0, 1, 1, 2, 2]] * 3, H=2, dk=32, dv=32, io="f32", layers=layers, seed=5)
    single, batched, status = _run_both(w)
    _assert_identical(single, batched, status)
    # and the per-layer results meet the oracle bar (first and last layer)
    for l in (0, layers - 1):
        o, st, S, _ = oracle_layer(w, layer=l)
        assert rel_err_rows(batched[l].o_np(), o) <= TOL[w.io]
        assert rel_err_states(batched[l].S_out.cpu().numpy(), S) <= TOL[w.io]


def test_more_layers_than_one_launch_holds():
    """40 layers: two launches of up to 32 layers each."""
    _say("40 layers")
    rng = np.random.default_rng(3)
    trees = [gi.random_tree_parents(rng, 5, 20) for _ in range(3)]
    w = gi.make_workload(trees, H=2, dk=64, dv=64, io="bf16", layers=40, seed=9)
    single, batched, status = _run_both(w)
    _assert_identical(single, batched, status)


def test_fork_mode_layers_match():
    _say("fork layers")
    w = gi.make_config("c3", layers=2)
    single, batched, status = _run_both(w, mode=gt.MODE_FORK, max_depth=3)
    for a, b in zip(single, batched):
        assert torch.equal(a.o.view(torch.int16), b.o.view(torch.int16))
        assert torch.equal(a.S_out, b.S_out)


def test_fork_delta_layers_match():
    """FORK_DELTA: per-layer verify launches, then the layer-batched WY commit
    over the kept deltas: identical to the per-layer calls."""
    _say("fork-delta layers")
    w = gi.make_config("c3", layers=2)
    single, batched, status = _run_both(w, mode=gt.MODE_FORK_DELTA, max_depth=3)
    for a, b in zip(single, batched):
        assert torch.equal(a.o, b.o)
        assert torch.equal(a.S_out, b.S_out)
    o, _, S, _ = oracle_layer(w, layer=1)
    assert rel_err_rows(batched[1].o_np(), o) <= TOL[w.io]
    assert rel_err_states(batched[1].S_out.cpu().numpy(), S) <= TOL[w.io]


def test_layers_status_codes():
    _say("status")
    trees = [gi.chain_parents(5), [0, 0, 1], [-1, 1, 0], [-1, 0]]
    w = gi.make_workload(trees, H=2, dk=32, dv=32, io="bf16", layers=3, seed=4,
                         accepted=[4, 1, 1, 2])
    single, batched, status = _run_both(w)
    assert status.cpu().tolist() == single[-1].status.cpu().tolist() == [0, 1, 2, 4]
    for a, b in zip(single, batched):          # bitwise: rejected sequences keep their NaN fill
        assert torch.equal(a.S_out.view(torch.int32), b.S_out.view(torch.int32))

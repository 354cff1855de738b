"""The no-allocation attention verify, gdn_tree_attn_verify_noalloc: the
split-cache partials in the library's fixed per-GPU scratch instead of a
caller workspace. Against gdn_tree_attn_verify with a NaN-filled workspace on
the same inputs: outputs and status bit-identical, on two calls in a row on
one GPU, the second with a smaller input (the scratch keeps the first call's
contents), a call with no split (no scratch at all), and a descriptor whose
partials exceed the scratch, rejected before anything is enqueued. The first
call's outputs are also checked against the oracle."""
import ctypes

import numpy as np
import pytest
import torch

import gated_deltanet_tree_02_amd as gt
import gdn_inputs as gi

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():  # the -m gpu suite only runs on a GPU machine
    pytest.skip("no GPU", allow_module_level=True)

from gpu_util import TOL, DeviceAttn, oracle_attn, rel_err_rows  # noqa: E402

SCRATCH = 32 << 20


def _say(*a):
    print("[gpu-no-alloc]", *a, flush=True)


def _case(trees, Hq, Hkv, lens, cap, seed):
    w = gi.make_attn_workload(trees, Hq, Hkv, 128, cap, lens, seed=seed)
    A = DeviceAttn(w)
    nbytes = gt.gdn_tree_attn_workspace_bytes(A.desc)
    return w, A, nbytes


def _both(A, nbytes):
    """(o, status) of the workspace call and of the no-allocation call."""
    ws = (torch.full((nbytes // 4,), float("nan"), device="cuda").view(torch.uint8)
          if nbytes else None)
    o_ws = torch.full_like(A.o, float("nan"))
    st_ws = torch.full_like(A.status, -7)
    gt.gdn_tree_attn_verify(A.desc, A.offsets, A.parents, A.q, A.k, A.v, A.kc, A.vc, A.cache_len,
                            o_ws, ws, st_ws)
    o_na = torch.full_like(A.o, float("nan"))
    st_na = torch.full_like(A.status, -7)
    gt.gdn_tree_attn_verify_noalloc(A.desc, A.offsets, A.parents, A.q, A.k, A.v, A.kc, A.vc,
                                    A.cache_len, o_na, st_na)
    torch.cuda.synchronize()
    return (o_ws, st_ws), (o_na, st_na)


def test_noalloc_verify_equals_workspace_verify_on_two_calls():
    rng = np.random.default_rng(3)
    # a larger split case: 4 sequences x 4 K/V heads (16 pairs: 16 splits)
    trees1 = [gi.kary_parents(3, 3)] * 2 + [gi.random_tree_parents(rng, 20, 64) for _ in range(2)]
    w1, A1, n1 = _case(trees1, 16, 4, [1900, 1000, 0, 1537], 2048, 41)
    # then a smaller one: 2 sequences, fewer rows and splits
    trees2 = [gi.kary_parents(2, 2), gi.chain_parents(5)]
    w2, A2, n2 = _case(trees2, 16, 4, [300, 65], 512, 42)
    _say(f"partials: {n1} then {n2} bytes (scratch {SCRATCH})")
    assert 0 < n2 < n1 <= SCRATCH
    for name, w, A, n in (("first", w1, A1, n1), ("second, smaller", w2, A2, n2)):
        (o_ws, st_ws), (o_na, st_na) = _both(A, n)
        assert np.all(st_na.cpu().numpy() == 0)
        assert torch.equal(st_ws, st_na), name
        assert torch.equal(o_ws.view(torch.int16), o_na.view(torch.int16)), name
        _say(f"{name} call: bit-identical to the workspace call")
    o_ref, _ = oracle_attn(w1)
    (o_ws, _), _ = _both(A1, n1)
    e = rel_err_rows(o_ws.float().cpu().numpy().astype(np.float64), o_ref)
    _say(f"first call against the oracle: {e:.3e}")
    assert e <= TOL["bf16"]


def test_noalloc_verify_without_a_split_and_over_the_limit():
    # 64 sequences x 4 K/V heads = 256 pairs: the cache is not split, no scratch
    trees = [gi.kary_parents(2, 3)] * 64
    w, A, n = _case(trees, 16, 4, [200] * 64, 256, 43)
    assert n == 0
    (o_ws, st_ws), (o_na, st_na) = _both(A, n)
    assert torch.equal(st_ws, st_na) and torch.equal(o_ws.view(torch.int16), o_na.view(torch.int16))
    # 255 sequences of 64 nodes, 4 query heads on one K/V head: two splits of
    # every cache, partials of 65 MB, more than the scratch holds
    big = gt.make_attn_desc(255, 4, 1, 128, 255 * 64, 64, 8192, 8192)
    need = gt.gdn_tree_attn_workspace_bytes(big)
    _say(f"oversize descriptor needs {need} bytes")
    assert need > SCRATCH
    lib = gt.load_library()
    fake = 0x1000
    rc = lib.gdn_tree_attn_verify_noalloc(ctypes.byref(big), fake, fake, fake, fake, fake, fake,
                                          fake, fake, 0.1, fake, fake, None)
    assert rc == 7                          # GDN_ERR_SCRATCH, checked before any launch

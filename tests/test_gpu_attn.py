"""GPU parity of the tree-masked attention verify and the accepted-path KV
commit against the oracle, through the C ABI.

Bar: node outputs within 2e-2 normwise relative error per (node, head) row
(bf16 inputs and outputs, fp32 arithmetic); status codes, committed caches and
lengths bit-exact. Rows of a rejected sequence are zero on both sides."""
import numpy as np
import pytest
import torch

import gated_deltanet_tree_02_amd as gt
import gdn_inputs as gi

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():  # the -m gpu suite only runs on a GPU machine
    pytest.skip("no GPU", allow_module_level=True)

from gpu_util import (TOL, DeviceAttn, attn_sub, dev_to_bits, oracle_attn,  # noqa: E402
                      oracle_attn_commit, rel_err_rows)

BF16_TOL = TOL["bf16"]


def _say(*a):
    print("[gpu-attn]", *a, flush=True)


def _valid_rows(w, status):
    """Node rows of sequences whose node range is well formed."""
    keep = np.zeros(w.T, bool)
    for b in range(w.B):
        lo, hi = w.offsets[b], w.offsets[b + 1]
        if 1 <= hi - lo <= 64:
            keep[lo:hi] = True
    return keep


def _check_verify(w, max_nodes=None, scale=None, expect_split=None):
    da = DeviceAttn(w, max_nodes=max_nodes)
    if expect_split is not None:
        assert (gt.gdn_tree_attn_workspace_bytes(da.desc) > 0) == expect_split
    da.verify(scale=scale)
    torch.cuda.synchronize()
    o_ref, st_ref = oracle_attn(w, max_nodes=da.desc.max_nodes, scale=scale)
    st = da.status.cpu().numpy()
    np.testing.assert_array_equal(st, st_ref)
    keep = _valid_rows(w, st)
    got = da.o_np()
    err = rel_err_rows(got[keep], o_ref[keep])
    _say("verify", w.B, w.Hq, w.Hkv, w.d, "max rel err", err)
    assert err <= BF16_TOL
    assert not np.isnan(got[keep]).any()
    return da


# ------------------------------------------------------------------ verify


def test_fa_small_matches_oracle():
    _say("fa_small")
    w = gi.make_attn_config("fa_small")
    _check_verify(w)


@pytest.mark.parametrize("Hq,Hkv,d", [(4, 4, 64), (8, 2, 128), (8, 1, 64), (16, 4, 128),
                                      (2, 1, 128), (6, 3, 64)])
def test_head_groups_dims_and_ragged_prefixes(Hq, Hkv, d):
    _say("shapes", Hq, Hkv, d)
    rng = np.random.default_rng(100 + Hq * 7 + Hkv + d)
    G = Hq // Hkv
    nmax = min(64, 256 // G)
    trees = [gi.kary_parents(2, 2), gi.branching_parents([3, 2]), [-1],
             gi.random_tree_parents(rng, 5, min(20, nmax)), gi.chain_parents(nmax),
             gi.kary_parents(3, 2)]
    lens = [0, 1, 63, 64, 65, 130]
    w = gi.make_attn_workload(trees, Hq, Hkv, d, 200, lens, seed=int(rng.integers(1 << 30)))
    _check_verify(w)


def test_full_tiles_64_nodes_and_256_rows():
    _say("64 nodes x 4 heads per K/V head")
    rng = np.random.default_rng(7)
    trees = [gi.chain_parents(64), gi.random_tree_parents(rng, 64, 64), gi.kary_parents(2, 5)[:64]]
    w = gi.make_attn_workload(trees, 8, 2, 128, 300, [100, 0, 257], seed=8)
    _check_verify(w)


def test_custom_scale():
    _say("scale 0.3")
    w = gi.make_attn_workload([gi.kary_parents(2, 3)] * 3, 8, 2, 64, 128, [5, 77, 128], seed=9)
    _check_verify(w, scale=0.3)


@pytest.mark.parametrize("lens", [[3000], [2900, 5], [0, 1000, 64]])
def test_split_cache_combine(lens):
    """Few (sequence, K/V head) pairs and long prefixes: the cache is split
    over workgroups and the partial results are merged."""
    _say("split", lens)
    B = len(lens)
    trees = [gi.kary_parents(3, 2)] * B
    w = gi.make_attn_workload(trees, 8, 2, 128, 3072, lens, seed=10 + B)
    _check_verify(w, expect_split=True)


def test_fa_c4_full_size_sampled():
    """The full-size layer in the launch configuration the benchmark times;
    three sequences checked against the oracle, every row finite."""
    _say("fa_c4 full size")
    w = gi.make_attn_config("fa_c4")
    da = DeviceAttn(w)
    da.verify()
    torch.cuda.synchronize()
    st = da.status.cpu().numpy()
    assert (st == 0).all()
    got = da.o_np()
    assert np.isfinite(got).all()
    seqs = [0, 37, 63]
    sub = attn_sub(w, seqs)
    o_ref, st_ref = oracle_attn(sub)
    assert (st_ref == 0).all()
    rows = np.concatenate([np.arange(w.offsets[b], w.offsets[b + 1]) for b in seqs])
    err = rel_err_rows(got[rows], o_ref)
    _say("fa_c4 sampled max rel err", err)
    assert err <= BF16_TOL


# ------------------------------------------------------------------ commit


def test_commit_bit_exact_fa_small():
    _say("commit fa_small")
    w = gi.make_attn_config("fa_small")
    w.accepted[3] = -1                       # one sequence accepts nothing
    da = DeviceAttn(w)
    da.verify()
    da.commit()
    torch.cuda.synchronize()
    kc_ref, vc_ref, lens_ref, st_ref = oracle_attn_commit(w)
    np.testing.assert_array_equal(da.status.cpu().numpy(), st_ref)
    np.testing.assert_array_equal(da.cache_len.cpu().numpy(), lens_ref)
    np.testing.assert_array_equal(dev_to_bits(da.kc), gi.bf16_bits(kc_ref.astype(np.float32)))
    np.testing.assert_array_equal(dev_to_bits(da.vc), gi.bf16_bits(vc_ref.astype(np.float32)))


def test_commit_then_verify_next_tree():
    """Verify, commit, then verify a new tree over the grown prefix: equal to
    the oracle run on the oracle's own committed caches."""
    _say("commit then verify")
    w = gi.make_attn_workload([gi.kary_parents(2, 3)] * 4, 8, 2, 128, 160, [0, 40, 100, 140],
                              seed=21)
    da = DeviceAttn(w, max_cache_len=w.cap)
    da.verify()
    da.commit()
    kc_ref, vc_ref, lens_ref, _ = oracle_attn_commit(w)
    w2 = gi.make_attn_workload([gi.branching_parents([2, 2, 1])] * 4, 8, 2, 128, 160,
                               lens_ref, seed=22)
    w2.kc_bits = gi.bf16_bits(kc_ref.astype(np.float32))
    w2.vc_bits = gi.bf16_bits(vc_ref.astype(np.float32))
    da2 = DeviceAttn(w2, max_cache_len=w.cap)
    da2.kc, da2.vc, da2.cache_len = da.kc, da.vc, da.cache_len     # the caches the GPU grew
    da2.verify()
    torch.cuda.synchronize()
    o_ref, st_ref = oracle_attn(w2)
    np.testing.assert_array_equal(da2.status.cpu().numpy(), st_ref)
    assert rel_err_rows(da2.o_np(), o_ref) <= BF16_TOL


def test_commit_full_size_rows_and_untouched():
    _say("commit fa_c4")
    w = gi.make_attn_config("fa_c4")
    da = DeviceAttn(w)
    da.commit()
    torch.cuda.synchronize()
    assert (da.status.cpu().numpy() == 0).all()
    lens = da.cache_len.cpu().numpy()
    kc = dev_to_bits(da.kc)
    vc = dev_to_bits(da.vc)
    kb, vb = gi.bf16_bits(w.k), gi.bf16_bits(w.v)
    for b in range(w.B):
        path = gi.path_to_root(w.parents_list[b], int(w.accepted[b]))         # root first
        L = int(w.cache_len[b])
        assert lens[b] == L + len(path)
        rows = w.offsets[b] + np.array(path)
        np.testing.assert_array_equal(kc[b, :, L:L + len(path)], kb[rows].transpose(1, 0, 2))
        np.testing.assert_array_equal(vc[b, :, L:L + len(path)], vb[rows].transpose(1, 0, 2))
        np.testing.assert_array_equal(kc[b, :, :L], w.kc_bits[b, :, :L])
        np.testing.assert_array_equal(kc[b, :, L + len(path):], w.kc_bits[b, :, L + len(path):])
        np.testing.assert_array_equal(vc[b, :, :L], w.vc_bits[b, :, :L])


# ------------------------------------------------------------------ status codes


def test_status_codes_zero_rows_and_untouched_caches():
    _say("status codes")
    trees = [gi.chain_parents(5), [0, 0, 1], [-1, 1, 0], [-1, 0], gi.kary_parents(2, 2), [-1]]
    lens = [4, 0, 0, 50, 7, 6]
    # malformed trees have no root path to draw an accepted node from
    w = gi.make_attn_workload(trees, 4, 2, 64, 8, lens, seed=31, accepted=[4, 1, 1, 1, 7, -2])
    da = DeviceAttn(w, max_cache_len=8)
    # sequence 3's committed length 50 exceeds the declared maximum (8)
    da.verify()
    torch.cuda.synchronize()
    st = da.status.cpu().numpy()
    assert st.tolist() == [0, 1, 2, 3, 0, 0]
    o = da.o_np()
    for b in (1, 2, 3):
        assert (o[w.offsets[b]:w.offsets[b + 1]] == 0).all()
    kc0, vc0 = dev_to_bits(da.kc).copy(), dev_to_bits(da.vc).copy()
    da.commit()
    torch.cuda.synchronize()
    # a 5-node path on 4 rows overflows 8 slots; 7 and -2 are outside [-1, N)
    assert da.status.cpu().numpy().tolist() == [6, 1, 2, 3, 4, 4]
    assert da.cache_len.cpu().numpy().tolist() == lens
    np.testing.assert_array_equal(dev_to_bits(da.kc), kc0)
    np.testing.assert_array_equal(dev_to_bits(da.vc), vc0)


def test_empty_batch_is_a_no_op():
    desc = gt.make_attn_desc(0, 4, 2, 64, 0, 8, 16)
    z = torch.zeros(1, dtype=torch.int32, device="cuda")
    st = torch.zeros(0, dtype=torch.int32, device="cuda")
    bf = torch.bfloat16
    e = torch.zeros((0, 4, 64), dtype=bf, device="cuda")
    ek = torch.zeros((0, 2, 64), dtype=bf, device="cuda")
    ec = torch.zeros((0, 2, 16, 64), dtype=bf, device="cuda")
    gt.gdn_tree_attn_verify(desc, z, z[:0], e, ek, ek, ec, ec, st, e.clone(), None, st)
    gt.gdn_tree_attn_commit(desc, z, z[:0], st, ek, ek, ec, ec, st, st)
    torch.cuda.synchronize()

#!/usr/bin/env python3
"""Tree-GDN verify + commit throughput on one MI355X.

One step = one round of the whole hot path over one batch on every GDN layer
of the workload: each layer's state takes the previous round's commit (the
accepted paths) and this round's trees are verified against it. By default
(`--step replay`) a step is one gdn_tree_replay_verify_layers launch, which
commits the previous round by replaying its accepted paths on the states and
verifies in the same pass, keeping no workspace; `--step fused` commits from
the previous round's pseudo-values instead (gdn_tree_commit_verify_layers).
The first round's verify is issued before timing starts, so K timed steps do
K commits and K verifies per layer. `--step separate` times the separate
calls instead: every layer verified and then committed in place, as one
launch per kernel (gdn_tree_verify_layers, gdn_tree_commit_layers), or one
launch per layer with `--launch per-layer`. The JSON line reports every
schedule, and per-launch records of the other workloads (`configs`: the tiny
tree, the chain, the k=2 d=3 batch and the ragged batch), each timed while
rotating through more than 1 GiB of independent copies so that no launch
finds its state in L2 or the Infinity Cache.
Default workload: k=3 d=3 draft trees (40 nodes incl. root), 24 GDN layers
with independent inputs and states, batch 64, 16 heads, 128x128 fp32 state,
bf16 q/k/v (Qwen3.5-9B GDN shape). Inputs are seeded synthetic data resident
in HBM before timing starts; the 24 layers' states (1.5 GiB) are far larger
than the 256 MB Infinity Cache, so layer-to-layer traffic reaches HBM.

Prints ONE JSON line. The metric is verified draft nodes per second per GDN
layer (nodes of all trees, root included, times layers, per second), with the
dominant kernel's roofline fraction, the fork/checkpoint baseline's time and
memory, and the CPU oracle timed on a bounded sample as a reported baseline.

A second leg ("fa_layers") times the 8 full-attention layers of the same
32-layer hybrid stack on the same trees: tree-masked attention verify over a
4096-row committed prefix (16 query heads sharing 4 K/V heads of 128, bf16)
and the accepted-path KV commit, each layer with its own inputs and cache.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "tree-GDN verified draft nodes/s per layer (1 GPU) + % HBM/MFMA peak"
HBM_PEAK_GBS = 8000.0
MFMA_BF16_TFLOPS = 2500.0
CSRC = os.path.join(ROOT, "gated_deltanet_tree_02_amd", "csrc")
TRAFFIC_FILES = [os.path.join(ROOT, "profiles", "gdn_wy_c3_c4_c5_hbm_traffic.md"),
                 os.path.join(ROOT, "profiles", "tree_attn_fa_c4_hbm_traffic.md")]
# sources whose hash ties a recorded counter measurement to the kernels it measured
KERNEL_SOURCES = {"verify": ["wy_verify.hip", "device_common.h", "launch.h"],
                  "commit_verify": ["wy_verify.hip", "device_common.h", "launch.h"],
                  "replay_verify": ["wy_verify.hip", "device_common.h", "launch.h"],
                  "commit": ["wy_commit.hip", "device_common.h", "launch.h"],
                  "replay_commit": ["wy_commit.hip", "device_common.h", "launch.h"],
                  "attn_verify": ["tree_attn.hip", "device_common.h", "launch.h",
                                  "tree_attn_api.cpp"]}


def kernel_source_hash(kind):
    h = hashlib.sha256()
    for f in KERNEL_SOURCES[kind]:
        with open(os.path.join(CSRC, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def recorded_traffic(kind, config):
    """HBM bytes per launch from the committed rocprofv3 FETCH_SIZE/WRITE_SIZE
    summary, if it was taken on this config with the current kernel sources;
    else None. The summary holds lines
      traffic <kind> <config> <source-hash> <bytes>"""
    pat = re.compile(rf"^traffic\s+{kind}\s+{config}\s+(\w+)\s+(\d+)\s*$")
    for path in TRAFFIC_FILES:
        if not os.path.exists(path):
            continue
        with open(path) as fh:
            for line in fh:
                m = pat.match(line.strip().strip("`"))
                if m and m.group(1) == kernel_source_hash(kind):
                    return int(m.group(2))
    return None


def traffic_fields(kind, config, alg_bytes):
    """The recorded HBM bytes of one launch of this kernel on this workload
    (None while unmeasured for the current sources) and their ratio to the
    algorithmic bytes."""
    t = recorded_traffic(kind, config)
    return {"traffic_bytes": t, "traffic_over_alg": round(t / alg_bytes, 3) if t else None}


def cpu_model():
    """The host CPU's model name as lscpu reports it (else /proc/cpuinfo), or None."""
    import subprocess
    try:
        out = subprocess.run(["lscpu"], capture_output=True, text=True, timeout=10).stdout
        for line in out.splitlines():
            if line.strip().startswith("Model name:"):
                return line.split(":", 1)[1].strip()
    except (OSError, subprocess.SubprocessError):
        pass
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def log(*a):
    print("[bench]", *a, file=sys.stderr, flush=True)


def parse():
    p = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    # after an idle period the first ~25 launches of a leg run up to 20% slower
    # (per-launch times fall steadily, then stay flat); 30 untimed steps settle it
    p.add_argument("--warmup", type=int, default=30)
    p.add_argument("--config", default="c4", choices=["c1", "c2", "c3", "c4", "c5"])
    p.add_argument("--mode", default="wy", choices=["wy", "fork"])
    p.add_argument("--fork-steps", type=int, default=3, help="timed steps of the fork baseline (0 = skip)")
    p.add_argument("--cpu-seconds", type=float, default=10.0, help="oracle sample budget (0 = skip)")
    p.add_argument("--launch", default="layers", choices=["layers", "per-layer"],
                   help="WY leg: every layer in one launch per kernel (gdn_tree_*_layers) or one "
                        "launch per layer")
    p.add_argument("--step", default="replay", choices=["replay", "fused", "separate"],
                   help="what a timed step is: one launch that replays the previous round's "
                        "accepted path on the state and verifies (no workspace), one launch "
                        "that commits the previous round from its pseudo-values and verifies, "
                        "or the separate verify and commit launches (WY, layer-batched)")
    p.add_argument("--secondary-steps", type=int, default=20,
                   help="timed steps of the schedule that is not the headline (0 = skip)")
    p.add_argument("--per-layer-steps", type=int, default=10,
                   help="after a layer-batched WY leg, timed steps with one launch per layer "
                        "(0 = skip)")
    p.add_argument("--round-steps", type=int, default=10,
                   help="timed rounds of the hybrid stack as one captured graph (0 = skip)")
    p.add_argument("--attn-steps", type=int, default=10,
                   help="timed steps of the full-attention leg (0 = skip)")
    p.add_argument("--attn-only", action="store_true",
                   help="run only the full-attention leg (profiling)")
    p.add_argument("--config-steps", type=int, default=50,
                   help="timed launches per schedule of the per-configuration records "
                        "(c1, c2, c3, c5; 0 = skip)")
    p.add_argument("--configs", default="c1,c2,c3,c5",
                   help="workloads of the per-configuration records")
    p.add_argument("--configs-only", action="store_true",
                   help="run only the per-configuration records (profiling)")
    p.add_argument("--pmc-calibration", action="store_true",
                   help="after the timed legs, run a plain 256 MiB device copy three times "
                        "(reads and writes 256 MiB each): the known-size kernel that scales "
                        "rocprofv3 FETCH_SIZE / WRITE_SIZE to bytes")
    return p.parse_args()


def algorithmic_bytes(w, io_bytes, gi):
    """Bytes the method itself must move per layer (state once, per-node data once)."""
    B, H, T, dk, dv = w.B, w.H, w.T, w.dk, w.dv
    tree = (B + 1) * 4 + T * 4
    per_node_head_verify = io_bytes * (2 * dk + dv) + 8 + io_bytes * dv + 4 * dv + 4
    verify = B * H * 4 * dv * dk + T * H * per_node_head_verify + tree
    path = sum(len(gi.path_to_root(p, int(a))) if a >= 0 else 0
               for p, a in zip(w.parents_list, w.accepted))
    commit = B * H * 8 * dv * dk + path * H * (4 * dv + io_bytes * dk + 4) + tree + B * 4
    fork_verify = T * H * (8 * dv * dk + io_bytes * (2 * dk + dv) + 8 + io_bytes * dv) + tree
    fork_commit = B * H * 8 * dv * dk + tree + B * 4
    return verify, commit, fork_verify, fork_commit


def pmc_calibration(dev):
    """A plain copy of known size for scaling FETCH_SIZE / WRITE_SIZE counters:
    torch.mul over 256 MiB of fp32, three times (reads and writes 256 MiB)."""
    import torch
    x = torch.ones(64 << 20, device=dev)
    y = torch.empty_like(x)
    for _ in range(3):
        torch.mul(x, 1.0, out=y)
    torch.cuda.synchronize()
    del x, y
    log("pmc calibration: 3 x copy of 256 MiB done")


def attn_algorithmic_bytes(offsets, Hq, Hkv, d, cache_len, path_nodes):
    """Bytes one full-attention layer must move: every node's query and
    output, the tree's own K/V rows and each sequence's committed K/V rows
    read once (verify); the accepted rows read and written once (commit)."""
    B = len(offsets) - 1
    T = int(offsets[-1])
    meta = (B + 1) * 4 + T * 4 + B * 4 + B * 4
    verify = (T * Hq * d * 2 * 2 + T * Hkv * d * 2 * 2
              + int(sum(int(x) for x in cache_len)) * Hkv * d * 2 * 2 + meta)
    commit = path_nodes * Hkv * d * 2 * 2 * 2 + meta + B * 4
    return verify, commit


def attention_leg(args, gt, gi, w_trees, dev):
    """The full-attention layers of the hybrid stack on the GDN workload's
    trees: per step every layer verified, then every layer committed; the
    committed lengths are reset after each step (outside the kernel timings)."""
    import numpy as np
    import torch
    c = gi.ATTN_CONFIGS["fa_c4"]
    n_layers = 8
    Hq, Hkv, d, cap, L0 = c["Hq"], c["Hkv"], c["d"], c["cap"], c["lens"][1]
    B, T = w_trees.B, w_trees.T
    t0 = time.time()
    g = torch.Generator(device=dev)
    g.manual_seed(1234)
    wl = gi.make_attn_workload(w_trees.parents_list, Hq, Hkv, d, 0, [L0] * B, seed=4321,
                               accepted=w_trees.accepted)
    offsets = torch.from_numpy(wl.offsets).to(dev)
    parents = torch.from_numpy(wl.parents).to(dev)
    accepted = torch.from_numpy(wl.accepted).to(dev)
    lens0 = torch.full((n_layers, B), L0, dtype=torch.int32, device=dev)
    lens = lens0.clone()
    status = torch.zeros(B, dtype=torch.int32, device=dev)
    desc = gt.make_attn_desc(B, Hq, Hkv, d, T, wl.max_nodes, cap, cap)
    nbytes = gt.gdn_tree_attn_workspace_bytes(desc)
    ver, com, keep = [], [], []
    for layer in range(n_layers):
        randn = lambda *shape: torch.randn(*shape, generator=g, device=dev).to(torch.bfloat16)
        q, k, v = randn(T, Hq, d), randn(T, Hkv, d), randn(T, Hkv, d)
        kc, vc = randn(B, Hkv, cap, d), randn(B, Hkv, cap, d)
        o = torch.empty_like(q)
        ws = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=dev)
        cl = lens[layer]
        ver.append(gt.prepare_attn_verify(desc, offsets, parents, q, k, v, kc, vc, cl, o, ws,
                                          status))
        com.append(gt.prepare_attn_commit(desc, offsets, parents, accepted, k, v, kc, vc, cl,
                                          status))
        keep.append((q, k, v, kc, vc, o, ws))
    torch.cuda.synchronize()
    log(f"attention leg: {n_layers} layers, cap {cap}, prefix {L0}, split workspace "
        f"{nbytes / 2**20:.1f} MiB, gen {time.time() - t0:.1f}s")

    def one_step():
        for f in ver:
            f()
        for f in com:
            f()
        lens.copy_(lens0)

    for _ in range(args.warmup):
        one_step()
    torch.cuda.synchronize()
    steps = args.attn_steps
    stream = torch.cuda.current_stream(dev)
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(steps)]
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    for s in range(steps):
        ev[s][0].record(stream)
        for f in ver:
            f()
        ev[s][1].record(stream)
        for f in com:
            f()
        ev[s][2].record(stream)
        lens.copy_(lens0)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t_start
    st = status.cpu().numpy()
    if np.any(st != 0):
        raise RuntimeError(f"nonzero attention tree status {np.unique(st)}")
    v_us = 1e3 * sum(e[0].elapsed_time(e[1]) for e in ev) / steps / n_layers
    c_us = 1e3 * sum(e[1].elapsed_time(e[2]) for e in ev) / steps / n_layers
    # the KV append of all layers as one launch (one committed length shared
    # by the layers, as in a model); not in --attn-only runs, which profile
    # the per-layer kernels
    # (several launches back to back between the events, each appending after
    # the previous one, so the GPU does not wait for the host; the cache has
    # room for reps appends of the longest path)
    cb_us = None
    if not args.attn_only:
        ios = [gt.make_attn_layer_io(desc, k=x[1], v=x[2], k_cache=x[3], v_cache=x[4]) for x in keep]
        shared = lens0[0].clone()
        batched = gt.prepare_attn_commit_layers(desc, offsets, parents, accepted, ios, shared, status,
                                                keep=keep)
        longest = max(len(gi.path_to_root(p, int(a))) for p, a in
                      zip(wl.parents_list, wl.accepted) if a >= 0)
        reps = max(1, min(8, (cap - L0) // longest))
        evb = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(steps)]
        for s in range(steps):
            evb[s][0].record(stream)
            for _ in range(reps):
                batched()
            evb[s][1].record(stream)
            shared.copy_(lens0[0])
        torch.cuda.synchronize()
        if np.any(status.cpu().numpy() != 0):
            raise RuntimeError("nonzero status in the layer-batched KV append")
        cb_us = 1e3 * sum(e[0].elapsed_time(e[1]) for e in evb) / steps / reps
    path = sum(len(gi.path_to_root(p, int(a))) if a >= 0 else 0
               for p, a in zip(wl.parents_list, wl.accepted))
    vb, cb = attn_algorithmic_bytes(wl.offsets, Hq, Hkv, d, [L0] * B, path)
    flops = 0
    for b in range(B):
        n = int(wl.offsets[b + 1] - wl.offsets[b])
        depth_sum = sum(len(gi.path_to_root(wl.parents_list[b], t)) for t in range(n))
        flops += 4 * d * Hq * (n * L0 + depth_sum)          # QK^T and PV over the visible keys
    kern = {
        "verify": {"avg_us": round(v_us, 3), "alg_bytes": int(vb),
                   "achieved_GBs": round(vb / v_us / 1e3, 1),
                   "frac_hbm": round(vb / v_us / 1e3 / HBM_PEAK_GBS, 4),
                   "flops": int(flops), "achieved_TFLOPs": round(flops / v_us / 1e6, 1),
                   "frac_mfma_bf16": round(flops / v_us / 1e6 / MFMA_BF16_TFLOPS, 4)},
        "commit": {"avg_us": round(c_us, 3), "alg_bytes": int(cb),
                   "achieved_GBs": round(cb / c_us / 1e3, 1),
                   "frac_hbm": round(cb / c_us / 1e3 / HBM_PEAK_GBS, 4),
                   "all_layers_one_launch_us": round(cb_us, 3) if cb_us else None},
    }
    out = {
        "workload": c["desc"].replace("64 seqs, tree k=3 d=3 (40 nodes)",
                                      f"{B} seqs, the GDN workload's trees ({T} nodes)"),
        "layers": n_layers, "steps": steps,
        "ms_per_step": round(1e3 * elapsed / steps, 4),
        "nodes_per_s_per_layer": round(T * n_layers * steps / elapsed, 1),
        "roofline": {"kernel": "tree_attn_verify", "bound": "hbm", "achieved": kern["verify"]["achieved_GBs"],
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": kern["verify"]["frac_hbm"],
                     "traffic": recorded_traffic("attn_verify", "fa_c4")},
        "kernels": kern, "split_workspace_bytes": int(nbytes),
    }
    log(f"attention: {out['ms_per_step']} ms/step, verify {v_us:.2f} us, commit {c_us:.2f} us per layer")
    return out


def fused_leg(args, gt, w, layers, offsets, parents, accepted, status, vb, cb, dev, steps,
              warmup, per_layer=False, replay=False):
    """Consecutive rounds through gdn_tree_commit_verify_layers: each step
    commits the previous round's accepted paths into the state and verifies
    this round's trees against it, in one launch over all layers (one pass
    over the state per round instead of verify's read plus commit's read and
    write). Two workspaces per layer alternate between rounds; the trees and
    inputs of every round are the workload's, the state evolves in place."""
    import numpy as np
    import torch
    L = len(layers)
    desc = gt.make_desc(w.B, w.H, w.dk, w.dv, w.T, w.max_nodes,
                        gt.DTYPE_BF16 if w.io == "bf16" else gt.DTYPE_F32, gt.MODE_WY)
    nbytes = gt.gdn_tree_workspace_bytes(desc)
    ws = [[torch.empty(nbytes, dtype=torch.uint8, device=dev) for _ in range(L)]
          for _ in range(2)]
    outs = [torch.empty_like(ly["v"]) for ly in layers]
    ios = [[gt.make_layer_io(desc, q=ly["q"], k=ly["k"], v=ly["v"], alpha=ly["alpha"],
                             beta=ly["beta"], S0=ly["S"], o=o, S_out=ly["S"], workspace=wl)
            for ly, o, wl in zip(layers, outs, ws[i])] for i in range(2)]
    first = gt.prepare_verify_layers(desc, offsets, parents, ios[0], nbytes, status,
                                     keep=(layers, ws, outs))
    # step i commits from workspace i % 2 and verifies into the other one; with
    # per_layer, one launch per layer (as a model forward issues them)
    groups = [[l] for l in range(L)] if per_layer else [list(range(L))]
    if replay:
        # the previous round's inputs are this workload's (same trees and
        # inputs every round); no workspace
        pio = [gt.make_layer_io(desc, k=ly["k"], v=ly["v"], alpha=ly["alpha"], beta=ly["beta"])
               for ly in layers]
        cio = [gt.make_layer_io(desc, q=ly["q"], k=ly["k"], v=ly["v"], alpha=ly["alpha"],
                                beta=ly["beta"], S0=ly["S"], o=o, S_out=ly["S"])
               for ly, o in zip(layers, outs)]
        calls = [[gt.prepare_replay_verify_layers(desc, desc, offsets, parents, accepted, offsets,
                                                  parents, [pio[l] for l in grp],
                                                  [cio[l] for l in grp], status,
                                                  keep=(layers, outs)) for grp in groups]] * 2
    else:
        calls = [[gt.prepare_commit_verify_layers(desc, desc, offsets, parents, accepted,
                                                  offsets, parents, [ios[i][l] for l in grp],
                                                  nbytes, [ios[1 - i][l] for l in grp], nbytes,
                                                  status, keep=(layers, ws, outs))
                  for grp in groups] for i in range(2)]

    def step(i):
        for c in calls[i % 2]:
            c()
    first()
    for i in range(warmup):
        step(i)
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(steps)]
    t0 = time.perf_counter()
    for i in range(steps):
        ev[i][0].record()
        step(warmup + i)
        ev[i][1].record()
    torch.cuda.synchronize()
    el = time.perf_counter() - t0
    if np.any(status.cpu().numpy() != 0):
        raise RuntimeError("nonzero status in the fused leg")
    times = sorted(a.elapsed_time(b) * 1e3 for a, b in ev)        # us per launch
    med = times[steps // 2]
    us_layer = sum(times) / steps / L                               # mean launch, per layer
    fb = vb + cb - w.B * w.H * 4 * w.dv * w.dk                       # state read once
    if replay:
        # no pseudo-values or gate prefixes written; the path's k, v, alpha,
        # beta read instead of its U, k, g
        io_b = 2 if w.io == "bf16" else 4
        import gdn_inputs as gi
        path = sum(len(gi.path_to_root(p, int(a))) if a >= 0 else 0
                   for p, a in zip(w.parents_list, w.accepted))
        fb -= w.T * w.H * (4 * w.dv + 4)
        fb += path * w.H * (io_b * w.dv + 8 - 4 * w.dv - 4)
    out = {"steps": steps, "warmup": warmup, "layers_per_launch": 1 if per_layer else L,
           "ms_per_step": round(1e3 * el / steps, 4),
           "launch_us_mean": round(sum(times) / steps, 2),
           "launch_us_median": round(med, 2),
           "launch_us_p10_p90": [round(times[steps // 10], 2), round(times[(9 * steps) // 10], 2)],
           "us_per_layer": round(us_layer, 3),
           "us_per_layer_median": round(med / L, 3),
           "alg_bytes_per_layer": int(fb),
           "achieved_GBs": round(fb / us_layer / 1e3, 1),
           "frac_hbm": round(fb / us_layer / 1e3 / HBM_PEAK_GBS, 4),
           "nodes_per_s_per_layer": round(w.T * L * steps / el, 1)}
    log(f"fused previous {'replay' if replay else 'commit'} + verify"
        f"{' (one launch per layer)' if per_layer else ''}: {out}")
    del ws, outs, ios, calls, first
    torch.cuda.empty_cache()
    return out


def fork_delta_leg(args, gt, gi, w, layers, offsets, parents, accepted, status, max_depth, run,
                   dev):
    """The fork baseline with delta-compressed checkpoints (GDN_MODE_FORK_DELTA):
    verify depth by depth, one layer at a time, keeping per node only the
    rank-one delta (the WY pseudo-value) and the gate; commit of all layers
    in one launch from the deltas. The layers' verify-time states share one
    region of a round arena (gdn_round_plan)."""
    import torch
    L = len(layers)
    desc = gt.make_desc(w.B, w.H, w.dk, w.dv, w.T, w.max_nodes,
                        gt.DTYPE_BF16 if w.io == "bf16" else gt.DTYPE_F32,
                        gt.MODE_FORK_DELTA, max_depth)
    plan = gt.gdn_round_plan(gt.make_round_desc(desc, L))
    arena = torch.empty(plan.total_bytes, dtype=torch.uint8, device=dev)
    ws = [arena[l * plan.gdn_ws_stride:l * plan.gdn_ws_stride + plan.gdn_ws_bytes]
          for l in range(L)]
    outs = [torch.empty_like(ly["v"]) for ly in layers]
    ver = [gt.prepare_verify(desc, offsets, parents, ly["q"], ly["k"], ly["v"], ly["alpha"],
                             ly["beta"], ly["S"], o, wl, status)
           for ly, o, wl in zip(layers, outs, ws)]
    ios = [gt.make_layer_io(desc, k=ly["k"], S0=ly["S"], S_out=ly["S"], workspace=wl)
           for ly, wl in zip(layers, ws)]
    com = [gt.prepare_commit_layers(desc, offsets, parents, accepted, ios, plan.gdn_ws_bytes,
                                    status, keep=(layers, arena))]
    el, v_ms, c_ms = run(ver, com, args.fork_steps, 1)
    import numpy as np
    if np.any(status.cpu().numpy() != 0):
        raise RuntimeError("nonzero status in the delta-fork leg")
    internal = sum(len(set(p[1:])) for p in w.parents_list)      # nodes with children
    out = {"ms_per_step": round(1e3 * el / args.fork_steps, 3),
           "nodes_per_s_per_layer": round(w.T * L * args.fork_steps / el, 1),
           "verify_us_per_layer": round(1e3 * v_ms / L, 2),
           "commit_us_per_layer": round(1e3 * c_ms / L, 2),
           "kept_bytes_per_layer": int(plan.gdn_ws_stride),
           "verify_state_bytes_shared": int(plan.gdn_ws_bytes - plan.gdn_ws_stride),
           "states_written_per_layer_bytes": int(internal * w.H * w.dv * w.dk * 4),
           "arena_bytes": int(plan.total_bytes), "steps": args.fork_steps}
    log(f"fork with delta checkpoints: {out}")
    del arena, ws, outs, ver, com
    torch.cuda.empty_cache()
    return out


def selective_fork_leg(args, gt, gi, w, layers, offsets, parents, accepted, status, max_depth,
                       run, dev, p_dominant=0.5, threshold=0.95):
    """The fork baseline with selective fork (gdn_tree_fork_selective_*): a
    node saves its checkpoint only when the draft's confidence in it is at
    most 0.95. Confidences are drawn per node (gdn_inputs.draft_confidences:
    siblings share one unit of mass, a dominant first child with probability
    p_dominant, the root certain); every sequence gets the largest number of
    saved nodes of the batch as its slot budget. Verify one layer at a time,
    depth by depth; commit one layer at a time."""
    import numpy as np
    import torch
    L = len(layers)
    conf_np = gi.draft_confidences(np.random.default_rng(2026), w.parents_list, p_dominant)
    conf = torch.from_numpy(conf_np).to(dev)
    saved = [int((conf_np[w.offsets[b]:w.offsets[b + 1]] <= threshold).sum()) for b in range(w.B)]
    max_kept = max(saved)
    desc = gt.make_desc(w.B, w.H, w.dk, w.dv, w.T, w.max_nodes,
                        gt.DTYPE_BF16 if w.io == "bf16" else gt.DTYPE_F32, gt.MODE_FORK, max_depth)
    nbytes = gt.gdn_tree_fork_selective_workspace_bytes(desc, max_kept)
    ws = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=dev)[:nbytes] if nbytes else None
    outs = [torch.empty_like(ly["v"]) for ly in layers]
    ver = [gt.prepare_fork_selective_verify(desc, offsets, parents, conf, threshold, max_kept,
                                            ly["q"], ly["k"], ly["v"], ly["alpha"], ly["beta"],
                                            ly["S"], o, ws, status)
           for ly, o in zip(layers, outs)]
    com = [gt.prepare_fork_selective_commit(desc, offsets, parents, conf, threshold, max_kept,
                                            accepted, ly["k"], ly["v"], ly["alpha"], ly["beta"],
                                            ly["S"], ly["S"], ws, status) for ly in layers]
    el, v_ms, c_ms = run(ver, com, args.fork_steps, 1)
    if np.any(status.cpu().numpy() != 0):
        raise RuntimeError("nonzero status in the selective-fork leg")
    node_ckpt = w.H * w.dv * w.dk * 4
    out = {"ms_per_step": round(1e3 * el / args.fork_steps, 3),
           "nodes_per_s_per_layer": round(w.T * L * args.fork_steps / el, 1),
           "verify_us_per_layer": round(1e3 * v_ms / L, 2),
           "commit_us_per_layer": round(1e3 * c_ms / L, 2),
           "threshold": threshold, "p_dominant": p_dominant,
           "saved_nodes": int(sum(saved)), "nodes": int(w.T),
           "saved_fraction": round(sum(saved) / w.T, 4), "max_kept": int(max_kept),
           "workspace_bytes_per_layer": int(nbytes),
           "saved_bytes_per_layer": int(sum(saved) * node_ckpt),
           "steps": args.fork_steps}
    log(f"selective fork: {out}")
    del ws, outs, ver, com, conf
    torch.cuda.empty_cache()
    return out


def sampling_accept_leg(args, gt, gi, w, offsets, parents, dev, V=151936):
    """Sampling-mode acceptance on the GDN workload's trees over a Qwen-sized
    vocabulary, every row pass split over the workgroups the device fits per
    sequence (gdn_tree_accept_sampling_split), and with one workgroup per
    sequence (gdn_tree_accept_sampling) beside it: per node a target and a draft
    distribution from peaked logits (a few favoured tokens over a spread),
    the draft's logits the target's plus noise, children drawn from the
    parent's draft distribution without replacement; seeded, drawn on the GPU."""
    import numpy as np
    import torch
    B, T = w.B, w.T
    g = torch.Generator(device=dev)
    g.manual_seed(2024)

    def peaked(noise_from=None):
        if noise_from is None:
            z = 1.5 * torch.randn(T, V, generator=g, device=dev)
            idx = torch.randint(0, V, (T, 4), generator=g, device=dev)
            boost = 8.0 + 6.0 * torch.rand(T, 4, generator=g, device=dev)
            z.scatter_add_(1, idx, boost)
            return z
        return noise_from + 0.7 * torch.randn(T, V, generator=g, device=dev)

    zt = peaked()
    zd = peaked(zt)
    P = torch.softmax(zt, dim=-1)
    del zt
    Q = torch.softmax(zd, dim=-1)
    del zd
    draft = torch.zeros(T, dtype=torch.int32, device=dev)
    for b, tree in enumerate(w.parents_list):
        lo = int(w.offsets[b])
        kids = {}
        for c in range(1, len(tree)):
            kids.setdefault(tree[c], []).append(c)
        for u, cs in kids.items():
            tok = torch.multinomial(Q[lo + u], len(cs), replacement=False, generator=g)
            draft[lo + torch.tensor(cs, device=dev)] = tok.to(torch.int32)
    U = torch.rand(T, 2, generator=g, device=dev)
    desc = gt.make_desc(B, 1, 128, 128, T, w.max_nodes)
    outs = [[torch.zeros(B, dtype=torch.int32, device=dev) for _ in range(4)] for _ in range(2)]
    one = lambda: gt.gdn_tree_accept_sampling(desc, offsets, parents, draft, P, Q, U, *outs[0])
    splits = gt.gdn_tree_accept_sampling_splits(desc)
    # zero once: every call leaves the workspace zero
    ws = torch.zeros(max(1, gt.gdn_tree_accept_sampling_split_workspace_bytes(desc, V)),
                     dtype=torch.uint8, device=dev)
    split = gt.prepare_accept_sampling_split(desc, offsets, parents, draft, P, Q, U, splits, ws,
                                             *outs[1])
    # the visited rows (about 276 MB) could sit in the 256 MB Infinity Cache
    # from the previous call: a 1 GiB buffer is read between timed calls
    flush = torch.ones(1 << 28, device=dev)
    stream = torch.cuda.current_stream(dev)
    steps = 20

    def timed(call):
        for _ in range(3):
            call()
        torch.cuda.synchronize()
        ev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(steps)]
        for s_ in range(steps):
            flush.sum()
            ev[s_][0].record(stream)
            call()
            ev[s_][1].record(stream)
        torch.cuda.synchronize()
        return sorted(e[0].elapsed_time(e[1]) * 1e3 for e in ev)

    t_one = timed(one)
    t_split = timed(split)
    res = [[o.cpu().numpy() for o in x] for x in outs]
    if np.any(res[0][3] != 0) or np.any(res[1][3] != 0):
        raise RuntimeError("nonzero status in the sampling acceptance")
    if not all(np.array_equal(a, b) for a, b in zip(res[0], res[1])):
        raise RuntimeError("the split sampling acceptance disagrees with the one-workgroup call")
    lens = res[0][1]
    # rows every walk must read: the two rows of each node it visits
    rows_bytes = int(lens.sum()) * 2 * V * 4
    med, med1 = t_split[steps // 2], t_one[steps // 2]
    out = {"vocab": V, "steps": steps, "splits": int(splits),
           "us_per_call_median": round(med, 2),
           "us_per_call_p10_p90": [round(t_split[steps // 10], 2),
                                   round(t_split[(9 * steps) // 10], 2)],
           "mean_accept_len": round(float(lens.mean()), 3),
           "visited_rows_bytes": rows_bytes,
           "visited_rows_GBs": round(rows_bytes / med / 1e3, 1),
           "cache_eviction": "1 GiB read between timed calls",
           "one_workgroup_per_sequence": {"us_per_call_median": round(med1, 2),
                                          "visited_rows_GBs": round(rows_bytes / med1 / 1e3, 1)}}
    log(f"sampling acceptance: {out}")
    del P, Q, flush, ws, split
    torch.cuda.empty_cache()
    return out


def config_legs(args, gt, gi, dev):
    """Per-launch records of the other workloads, one GDN layer each (the
    headline covers the 24-layer k=3 d=3 stack). For every workload, two
    schedules, each timed launch by launch with HIP events on the launching
    stream (median, p10/p90): the fused round boundary by replay
    (gdn_tree_replay_verify_layers, one layer per launch: the previous
    round's accepted paths replayed on the state, this round's tree verified),
    and the separate verify and commit launches. Launches must not find their
    data in the 4 MB L2 or the 256 MB Infinity Cache: the k=2 d=3 and ragged
    batches rotate through independent copies of the layer totalling more
    than 1 GiB (as the layers of a model do); the tiny tree and the chain are
    a few hundred KiB per copy, so a 1 GiB buffer is read between timed
    launches instead (outside the events)."""
    import numpy as np
    import torch
    names = [c for c in args.configs.split(",") if c]
    steps, warm = args.config_steps, 10
    out = {}
    flush = None
    for name in names:
        t0 = time.time()
        w = gi.make_config(name, layers=1)
        io_t = torch.bfloat16 if w.io == "bf16" else torch.float32
        io_bytes = 2 if w.io == "bf16" else 4
        B, H, T, dk, dv = w.B, w.H, w.T, w.dk, w.dv
        desc = gt.make_desc(B, H, dk, dv, T, w.max_nodes,
                            gt.DTYPE_BF16 if w.io == "bf16" else gt.DTYPE_F32, gt.MODE_WY)
        nbytes = gt.gdn_tree_workspace_bytes(desc)
        per_copy = B * H * dv * dk * 4 + T * H * (io_bytes * (2 * dk + 2 * dv) + 8) + nbytes
        rotate = per_copy * 8 >= (1 << 30) // 4          # large enough to rotate
        copies = max(2, -(-(1 << 30) // per_copy)) if rotate else 1
        if not rotate and flush is None:
            flush = torch.ones(1 << 28, device=dev)       # 1 GiB, read between launches

        def put(x, io=False):
            t = torch.from_numpy(np.ascontiguousarray(x)).to(dev)
            return t.to(io_t) if io else t
        offsets, parents, accepted = put(w.offsets), put(w.parents), put(w.accepted)
        status = torch.zeros(B, dtype=torch.int32, device=dev)
        base = dict(q=put(w.q[0], True), k=put(w.k[0], True), v=put(w.v[0], True),
                    alpha=put(w.alpha[0]), beta=put(w.beta[0]), S=put(w.S0[0]))
        cps = [base] + [{k_: x.clone() for k_, x in base.items()} for _ in range(copies - 1)]
        for c in cps:
            c["o"] = torch.empty_like(c["v"])
        replay_calls = []
        for c in cps:
            pio = gt.make_layer_io(desc, k=c["k"], v=c["v"], alpha=c["alpha"], beta=c["beta"])
            cio = gt.make_layer_io(desc, q=c["q"], k=c["k"], v=c["v"], alpha=c["alpha"],
                                   beta=c["beta"], S0=c["S"], o=c["o"], S_out=c["S"])
            replay_calls.append(gt.prepare_replay_verify_layers(
                desc, desc, offsets, parents, accepted, offsets, parents, [pio], [cio], status,
                keep=(c,)))
        torch.cuda.synchronize()
        stream = torch.cuda.current_stream(dev)

        def timed(fns_per_launch, n):
            """n launches (each a list of calls, one event interval per call)."""
            k = len(fns_per_launch(0))
            ev = [[torch.cuda.Event(enable_timing=True) for _ in range(k + 1)] for _ in range(n)]
            for i in range(warm + n):
                if flush is not None and not rotate:
                    flush.sum()
                fns = fns_per_launch(i)
                if i < warm:
                    for f in fns:
                        f()
                    continue
                e = ev[i - warm]
                e[0].record(stream)
                for j, f in enumerate(fns):
                    f()
                    e[j + 1].record(stream)
            torch.cuda.synchronize()
            if np.any(status.cpu().numpy() != 0):
                raise RuntimeError(f"nonzero status in the {name} record")
            return [sorted(e[j].elapsed_time(e[j + 1]) * 1e3 for e in ev) for j in range(k)]

        def stats(times):
            n = len(times)
            return {"launch_us_median": round(times[n // 2], 3),
                    "launch_us_p10_p90": [round(times[n // 10], 3), round(times[(9 * n) // 10], 3)],
                    "launch_us_mean": round(sum(times) / n, 3)}

        # the first round's verify, so that every timed launch commits a round
        for c in cps:
            gt.gdn_tree_verify(desc, offsets, parents, c["q"], c["k"], c["v"], c["alpha"],
                               c["beta"], c["S"], c["o"],
                               torch.empty(nbytes, dtype=torch.uint8, device=dev), status)
        (rt,) = timed(lambda i: [replay_calls[i % copies]], steps)
        vb, cb, _, _ = algorithmic_bytes(w, io_bytes, gi)
        path = sum(len(gi.path_to_root(p, int(a))) if a >= 0 else 0
                   for p, a in zip(w.parents_list, w.accepted))
        rb = vb + cb - B * H * 4 * dv * dk - T * H * (4 * dv + 4) + path * H * (
            io_bytes * dv + 8 - 4 * dv - 4)
        rec = {"workload": gi.CONFIGS[name]["desc"], "batch": B, "total_nodes": T,
               "copies": copies, "rotation_bytes": int(per_copy * copies) if rotate else None,
               "cache_eviction": (f"rotation through {copies} copies" if rotate
                                  else "1 GiB read between timed launches")}
        r = stats(rt)
        r.update({"alg_bytes": int(rb),
                  "achieved_GBs_median": round(rb / r["launch_us_median"] / 1e3, 1),
                  "frac_hbm_median": round(rb / r["launch_us_median"] / 1e3 / HBM_PEAK_GBS, 4),
                  "nodes_per_s_per_layer": round(T / (r["launch_us_median"] * 1e-6), 1)},
                 **traffic_fields("replay_verify", name, rb))
        rec["replay"] = r
        del replay_calls
        # the separate verify and commit launches (workspace per copy)
        sep = []
        for c in cps:
            c["ws"] = torch.empty(nbytes, dtype=torch.uint8, device=dev)
            sep.append([gt.prepare_verify(desc, offsets, parents, c["q"], c["k"], c["v"],
                                          c["alpha"], c["beta"], c["S"], c["o"], c["ws"], status),
                        gt.prepare_commit(desc, offsets, parents, accepted, c["k"], c["S"],
                                          c["S"], c["ws"], status)])
        vt, ct = timed(lambda i: sep[i % copies], steps)
        sv, sc = stats(vt), stats(ct)
        v_med, c_med = sv["launch_us_median"], sc["launch_us_median"]
        rec["separate"] = {
            "verify": dict(sv, alg_bytes=int(vb),
                           frac_hbm_median=round(vb / v_med / 1e3 / HBM_PEAK_GBS, 4),
                           **traffic_fields("verify", name, vb)),
            "commit": dict(sc, alg_bytes=int(cb),
                           frac_hbm_median=round(cb / c_med / 1e3 / HBM_PEAK_GBS, 4),
                           **traffic_fields("commit", name, cb)),
            "nodes_per_s_per_layer": round(T / ((v_med + c_med) * 1e-6), 1)}
        rec["steps"] = steps
        log(f"config {name} ({time.time() - t0:.1f}s): {rec}")
        out[name] = rec
        del sep, cps, base
        torch.cuda.empty_cache()
    del flush
    torch.cuda.empty_cache()
    return out


def round_leg(args, gt, gi, w, layers, offsets, parents, dev):
    """One whole speculative round of the 32-layer hybrid stack, in model
    order (three GDN layers, then one full-attention layer, eight times):
    every layer's verify, greedy acceptance from draft and target tokens
    (drawn so that the workload's accepted paths are the ones accepted),
    the commit of all GDN layers and the KV append of all attention layers.
    Timed as one captured HIP graph per round (gdn_round_capture) and as the
    same calls issued one by one from Python."""
    import numpy as np
    import torch
    c = gi.ATTN_CONFIGS["fa_c4"]
    n_attn = 8
    n_gdn = len(layers)
    Hq, Hkv, d, cap, L0 = c["Hq"], c["Hkv"], c["d"], c["cap"], c["lens"][1]
    B, T = w.B, w.T
    kinds = ([0, 0, 0, 1] * n_attn)[:n_gdn + n_attn] if n_gdn == 3 * n_attn else \
        [0] * n_gdn + [1] * n_attn
    gdesc = gt.make_desc(B, w.H, w.dk, w.dv, T, w.max_nodes, gt.DTYPE_BF16, gt.MODE_WY)
    adesc = gt.make_attn_desc(B, Hq, Hkv, d, T, w.max_nodes, cap, cap)
    rdesc = gt.make_round_desc(gdesc, n_gdn, adesc, n_attn)
    layout = gt.gdn_round_plan(rdesc)
    g = torch.Generator(device=dev)
    g.manual_seed(99)
    randn = lambda *shape: torch.randn(*shape, generator=g, device=dev).to(torch.bfloat16)
    attn = []
    for _ in range(n_attn):
        attn.append(dict(q=randn(T, Hq, d), k=randn(T, Hkv, d), v=randn(T, Hkv, d),
                         kc=randn(B, Hkv, cap, d), vc=randn(B, Hkv, cap, d),
                         o=torch.empty(T, Hq, d, dtype=torch.bfloat16, device=dev)))
    outs = [torch.empty_like(ly["v"]) for ly in layers]
    rng = np.random.default_rng(7)
    d_np, t_np = gi.draft_target_tokens(rng, w.parents_list, w.accepted)
    draft = torch.from_numpy(d_np).to(dev)
    target = torch.from_numpy(t_np).to(dev)
    lens0 = torch.full((B,), L0, dtype=torch.int32, device=dev)
    cache_len = lens0.clone()
    acc, alen, nxt, status = (torch.zeros(B, dtype=torch.int32, device=dev) for _ in range(4))
    arena = torch.empty(max(1, layout.total_bytes), dtype=torch.uint8, device=dev)
    gdn_io = [gt.make_layer_io(gdesc, q=ly["q"], k=ly["k"], v=ly["v"], alpha=ly["alpha"],
                               beta=ly["beta"], S0=ly["S"], o=o, S_out=ly["S"])
              for ly, o in zip(layers, outs)]
    attn_io = [gt.make_attn_layer_io(adesc, q=a["q"], k=a["k"], v=a["v"], k_cache=a["kc"],
                                     v_cache=a["vc"], o=a["o"]) for a in attn]
    stream = torch.cuda.Stream(dev)
    torch.cuda.synchronize()
    graph = gt.RoundGraph(rdesc, offsets, parents, gdn_io, attn_io, arena, draft, target, acc,
                          alen, nxt, status, cache_len=cache_len, layer_kinds=kinds,
                          stream=stream, keep=(layers, attn, outs))
    # the same round as individual calls (per-layer workspaces carved from the arena)
    ws = lambda l: arena[l * layout.gdn_ws_stride:l * layout.gdn_ws_stride + layout.gdn_ws_bytes]
    calls, gi_, ai_ = [], 0, 0
    for kind in kinds:
        if kind == 0:
            ly = layers[gi_]
            calls.append(gt.prepare_verify(gdesc, offsets, parents, ly["q"], ly["k"], ly["v"],
                                           ly["alpha"], ly["beta"], ly["S"], outs[gi_], ws(gi_),
                                           status, stream=stream))
            gi_ += 1
        else:
            a = attn[ai_]
            calls.append(gt.prepare_attn_verify(adesc, offsets, parents, a["q"], a["k"], a["v"],
                                                a["kc"], a["vc"], cache_len, a["o"], None, status,
                                                stream=stream))
            ai_ += 1
    e_gdn = [gt.make_layer_io(gdesc, k=ly["k"], S0=ly["S"], S_out=ly["S"], workspace=ws(l))
             for l, ly in enumerate(layers)]

    def eager():
        for f in calls:
            f()
        gt.gdn_tree_accept_greedy(gdesc, offsets, parents, draft, target, acc, alen, nxt, status,
                                  stream=stream)
        gt.gdn_tree_commit_layers(gdesc, offsets, parents, acc, e_gdn, layout.gdn_ws_bytes,
                                  status, stream=stream)
        gt.gdn_tree_attn_commit_layers(adesc, offsets, parents, acc, attn_io, cache_len, status,
                                       stream=stream)

    def timed(fn, steps):
        ev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(steps)]
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for s in range(steps):
            ev[s][0].record(stream)
            fn()
            ev[s][1].record(stream)
            with torch.cuda.stream(stream):
                cache_len.copy_(lens0)
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        if np.any(status.cpu().numpy() != 0):
            raise RuntimeError(f"nonzero status in the round: {np.unique(status.cpu().numpy())}")
        times = sorted(e[0].elapsed_time(e[1]) for e in ev)
        return wall / steps * 1e3, times[len(times) // 2], times

    launch = lambda: graph.launch(stream)
    for _ in range(2):
        launch()
        eager()
        with torch.cuda.stream(stream):
            cache_len.copy_(lens0)
    steps = args.round_steps
    g_wall, g_med, g_times = timed(launch, steps)
    e_wall, e_med, _ = timed(eager, steps)
    expect = np.array([len(gi.path_to_root(p, int(a))) for p, a in
                       zip(w.parents_list, w.accepted)], np.int32)
    got_len = alen.cpu().numpy()
    if not np.array_equal(got_len, expect):
        raise RuntimeError("round acceptance differs from the drawn accepted paths")
    graph.close()
    # the same round with the previous round's GDN commit replayed inside the
    # GDN verifies (gdn_round_capture_replay): the previous round is the same
    # trees and inputs with the workload's accepted paths (a buffer of its own)
    prev_acc = torch.from_numpy(np.ascontiguousarray(w.accepted, np.int32)).to(dev)
    prev_io = [gt.make_layer_io(gdesc, k=ly["k"], v=ly["v"], alpha=ly["alpha"], beta=ly["beta"])
               for ly in layers]
    rgraph = gt.RoundGraph(rdesc, offsets, parents, gdn_io, attn_io, arena, draft, target, acc,
                           alen, nxt, status, cache_len=cache_len, layer_kinds=kinds,
                           stream=stream, keep=(layers, attn, outs),
                           prev=dict(desc=gdesc, offsets=offsets, parents=parents,
                                     accepted=prev_acc, gdn_layers=prev_io))
    rlaunch = lambda: rgraph.launch(stream)
    for _ in range(2):
        rlaunch()
        with torch.cuda.stream(stream):
            cache_len.copy_(lens0)
    r_wall, r_med, r_times = timed(rlaunch, steps)
    rgraph.close()
    out = {
        "layers": {"gdn": n_gdn, "attention": n_attn,
                   "order": "3 GDN, 1 attention, x8" if kinds[:4] == [0, 0, 0, 1] else "GDN, attention"},
        "steps": steps, "graph_ms_per_round_median": round(g_med, 4),
        "graph_ms_per_round_p10_p90": [round(g_times[steps // 10], 4),
                                       round(g_times[(9 * steps) // 10], 4)],
        "eager_ms_per_round_median": round(e_med, 4),
        "graph_wall_ms_per_round": round(g_wall, 4), "eager_wall_ms_per_round": round(e_wall, 4),
        "kernel_launches_per_round": n_gdn + n_attn + 3,
        "replay_graph_ms_per_round_median": round(r_med, 4),
        "replay_graph_ms_per_round_p10_p90": [round(r_times[steps // 10], 4),
                                              round(r_times[(9 * steps) // 10], 4)],
        "replay_nodes_per_s_all_layers": round(T / (r_med * 1e-3), 1),
        "replay_kernel_launches_per_round": n_gdn + n_attn + 2,
        "nodes_per_s_all_layers": round(T / (g_med * 1e-3), 1),
        "mean_accept_len": round(float(got_len.mean()), 3),
        "arena_bytes": int(layout.total_bytes),
    }
    log(f"round: {out}")
    return out


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only; --gpus {args.gpus} is not supported "
              "(the path has no multi-GPU form in this library)", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import gated_deltanet_tree_02_amd as gt
    import gdn_inputs as gi

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    t0 = time.time()
    w = gi.make_config(args.config)
    log(f"workload {args.config}: B={w.B} T={w.T} layers={w.layers} gen {time.time() - t0:.1f}s")
    L = w.layers
    if args.attn_only:
        fa = attention_leg(args, gt, gi, w, dev)
        if args.pmc_calibration:
            pmc_calibration(dev)
        print(json.dumps({"fa_layers": fa}), flush=True)
        return
    if args.configs_only:
        print(json.dumps({"configs": config_legs(args, gt, gi, dev)}), flush=True)
        return
    io_t = torch.bfloat16 if w.io == "bf16" else torch.float32
    io_bytes = 2 if w.io == "bf16" else 4
    max_depth = w.max_depth()

    def put(x, io=False):
        t = torch.from_numpy(np.ascontiguousarray(x)).to(dev)
        return t.to(io_t) if io else t

    offsets = put(w.offsets)
    parents = put(w.parents)
    accepted = put(w.accepted)
    status = torch.zeros(w.B, dtype=torch.int32, device=dev)
    layers = []
    for layer in range(L):
        layers.append(dict(q=put(w.q[layer], True), k=put(w.k[layer], True), v=put(w.v[layer], True),
                           alpha=put(w.alpha[layer]), beta=put(w.beta[layer]), S=put(w.S0[layer])))
    torch.cuda.synchronize()

    def make_calls(mode, batched=False):
        desc = gt.make_desc(w.B, w.H, w.dk, w.dv, w.T, w.max_nodes,
                            gt.DTYPE_BF16 if w.io == "bf16" else gt.DTYPE_F32,
                            gt.MODE_WY if mode == "wy" else gt.MODE_FORK, max_depth)
        nbytes = gt.gdn_tree_workspace_bytes(desc)
        ver, com = [], []
        for ly in layers:
            ly["o_" + mode] = torch.empty_like(ly["v"])
            ly["ws_" + mode] = torch.empty(nbytes, dtype=torch.uint8, device=dev)
            ver.append(gt.prepare_verify(desc, offsets, parents, ly["q"], ly["k"], ly["v"],
                                         ly["alpha"], ly["beta"], ly["S"], ly["o_" + mode],
                                         ly["ws_" + mode], status))
            com.append(gt.prepare_commit(desc, offsets, parents, accepted, ly["k"], ly["S"], ly["S"],
                                         ly["ws_" + mode], status))
        if batched:
            # one launch per kernel for all layers (commit in place: S_out = S0)
            ios = [gt.make_layer_io(desc, q=ly["q"], k=ly["k"], v=ly["v"], alpha=ly["alpha"],
                                    beta=ly["beta"], S0=ly["S"], o=ly["o_" + mode], S_out=ly["S"],
                                    workspace=ly["ws_" + mode]) for ly in layers]
            ver = [gt.prepare_verify_layers(desc, offsets, parents, ios, nbytes, status, keep=layers)]
            com = [gt.prepare_commit_layers(desc, offsets, parents, accepted, ios, nbytes, status,
                                            keep=layers)]
        return desc, nbytes, ver, com

    def run(ver, com, steps, warmup):
        for _ in range(warmup):
            for f in ver:
                f()
            for f in com:
                f()
        torch.cuda.synchronize()
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True),
               torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
        torch.cuda.synchronize()
        t_start = time.perf_counter()
        for s in range(steps):
            ev[s][0].record()
            for f in ver:
                f()
            ev[s][1].record()
            for f in com:
                f()
            ev[s][2].record()
        torch.cuda.synchronize()
        elapsed = time.perf_counter() - t_start
        v_ms = sum(e[0].elapsed_time(e[1]) for e in ev) / steps
        c_ms = sum(e[1].elapsed_time(e[2]) for e in ev) / steps
        return elapsed, v_ms, c_ms

    # ------------------------------------------------------------------ main leg
    batched = args.mode == "wy" and args.launch == "layers"
    # a fused round is the headline step where it applies (WY, layer-batched)
    headline_fused = args.step in ("fused", "replay") and batched
    sep_steps = max(1, args.secondary_steps) if headline_fused else args.steps
    desc, nbytes, ver, com = make_calls(args.mode, batched)
    log(f"mode {args.mode}: workspace {nbytes / 2**20:.1f} MiB per layer, "
        f"{'all layers per launch' if batched else 'one launch per layer'}")
    elapsed, v_ms, c_ms = run(ver, com, sep_steps, args.warmup)
    st = status.cpu().numpy()
    if np.any(st != 0):
        raise RuntimeError(f"nonzero tree status {np.unique(st)}")
    ms_step = 1e3 * elapsed / sep_steps
    nodes_per_s = w.T * L * sep_steps / elapsed
    vb, cb, fvb, fcb = algorithmic_bytes(w, io_bytes, gi)
    if args.mode == "fork":
        vb, cb = fvb, fcb
    # per-layer figures (events around the step's launches / layers); with
    # batched launches one launch carries all L layers
    lpl = L if batched else 1
    v_us = 1e3 * v_ms / L
    c_us = 1e3 * c_ms / L
    kern = {
        "verify": {"avg_us": round(v_us, 3), "alg_bytes": int(vb),
                   "achieved_GBs": round(vb / v_us / 1e3, 1),
                   "frac_hbm": round(vb / v_us / 1e3 / HBM_PEAK_GBS, 4)},
        "commit": {"avg_us": round(c_us, 3), "alg_bytes": int(cb),
                   "achieved_GBs": round(cb / c_us / 1e3, 1),
                   "frac_hbm": round(cb / c_us / 1e3 / HBM_PEAK_GBS, 4)},
    }
    if batched and sep_steps > 0:
        # the commit by replay alone (gdn_tree_replay_commit_layers, in place):
        # the accepted path's gated delta rule steps from its own k, v,
        # alpha, beta; no workspace
        rc = gt.prepare_replay_commit_layers(
            desc, offsets, parents, accepted,
            [gt.make_layer_io(desc, k=ly["k"], v=ly["v"], alpha=ly["alpha"], beta=ly["beta"],
                              S0=ly["S"], S_out=ly["S"]) for ly in layers], status, keep=(layers,))
        for _ in range(args.warmup):
            rc()
        torch.cuda.synchronize()
        rev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(sep_steps)]
        for e0, e1 in rev:
            e0.record()
            rc()
            e1.record()
        torch.cuda.synchronize()
        if np.any(status.cpu().numpy() != 0):
            raise RuntimeError("nonzero status in the replay commit")
        r_us = 1e3 * sum(a.elapsed_time(b) for a, b in rev) / sep_steps / L
        path = sum(len(gi.path_to_root(p_, int(a_))) if a_ >= 0 else 0
                   for p_, a_ in zip(w.parents_list, w.accepted))
        rcb = (w.B * w.H * 2 * 4 * w.dv * w.dk + path * w.H * (io_bytes * (w.dk + w.dv) + 8)
               + 4 * (2 * w.B + 1 + w.T))
        kern["replay_commit"] = {"avg_us": round(r_us, 3), "alg_bytes": int(rcb),
                                 "achieved_GBs": round(rcb / r_us / 1e3, 1),
                                 "frac_hbm": round(rcb / r_us / 1e3 / HBM_PEAK_GBS, 4)}
        del rc
    for kind in [k_ for k_ in ("verify", "commit", "replay_commit") if k_ in kern]:
        t = recorded_traffic(kind, args.config) if args.mode == "wy" else None   # per layer
        k = kern[kind]
        k["layers_per_launch"] = lpl
        k["launch_us"] = round(k["avg_us"] * lpl, 3)
        k["alg_bytes_per_launch"] = k["alg_bytes"] * lpl
        k["traffic_bytes"] = t
        k["traffic_over_alg"] = round(t / k["alg_bytes"], 3) if t else None
    dom = "verify" if v_us >= c_us else "commit"
    roof = {"kernel": f"{'wy' if args.mode == 'wy' else 'fork'}_{dom}", "bound": "hbm",
            "achieved": kern[dom]["achieved_GBs"], "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": kern[dom]["frac_hbm"],
            "traffic": kern[dom]["traffic_bytes"] * lpl if kern[dom]["traffic_bytes"] else None,
            "layers_per_launch": lpl}
    log(f"{args.mode}: {ms_step:.3f} ms/step, verify {v_us:.2f} us, commit {c_us:.2f} us per layer")

    # ------------------------------------------ one launch per layer (secondary)
    # In a model forward layer l+1's q, k, v come from layer l's output, so
    # verify goes out one layer at a time; the commits of all layers follow
    # acceptance and batch freely. Both schedules are reported.
    per_layer = None
    if batched and args.per_layer_steps > 0:
        for ly in layers:
            ly.pop("o_wy"), ly.pop("ws_wy")
        ver = com = None
        _, _, pver, pcom = make_calls("wy", False)
        p_el, p_v, p_c = run(pver, pcom, args.per_layer_steps, 2)
        pv_us, pc_us = 1e3 * p_v / L, 1e3 * p_c / L
        per_layer = {
            "verify_us_per_layer": round(pv_us, 3), "commit_us_per_layer": round(pc_us, 3),
            "verify_frac_hbm": round(vb / pv_us / 1e3 / HBM_PEAK_GBS, 4),
            "commit_frac_hbm": round(cb / pc_us / 1e3 / HBM_PEAK_GBS, 4),
            "nodes_per_s_per_layer": round(w.T * L * args.per_layer_steps / p_el, 1),
            # verify per layer (as a forward issues it), commit of all layers batched
            "model_order_nodes_per_s_per_layer": round(w.T / ((pv_us + c_us) * 1e-6), 1),
            "steps": args.per_layer_steps,
            # HBM bytes of one single-layer launch (rocprofv3 counters)
            "traffic_bytes": {k: recorded_traffic(k, args.config + "_per_layer")
                              for k in ("verify", "commit", "commit_verify", "replay_verify")}}
        for ly in layers:
            ly.pop("o_wy"), ly.pop("ws_wy")
        pver = pcom = None
        torch.cuda.empty_cache()
        # the fused previous commit + verify, one launch per layer: in model
        # order every layer's commit rides on its next verify
        pf = fused_leg(args, gt, w, layers, offsets, parents, accepted, status, vb, cb, dev,
                       args.per_layer_steps, 5, per_layer=True)
        per_layer["fused_us_per_layer"] = pf["us_per_layer"]
        per_layer["fused_frac_hbm"] = pf["frac_hbm"]
        per_layer["model_order_fused_nodes_per_s_per_layer"] = pf["nodes_per_s_per_layer"]
        pr = fused_leg(args, gt, w, layers, offsets, parents, accepted, status, vb, cb, dev,
                       args.per_layer_steps, 5, per_layer=True, replay=True)
        per_layer["replay_us_per_layer"] = pr["us_per_layer"]
        per_layer["replay_frac_hbm"] = pr["frac_hbm"]
        per_layer["model_order_replay_nodes_per_s_per_layer"] = pr["nodes_per_s_per_layer"]
        log(f"one launch per layer: {per_layer}")

    # ---------------------------------------- previous commit fused into verify
    fused = replay = None
    for kind in ("fused", "replay"):
        f_steps = args.steps if headline_fused and args.step == kind else args.secondary_steps
        if not batched or f_steps <= 0:
            continue
        for ly in layers:
            ly.pop("o_wy", None), ly.pop("ws_wy", None)
        ver = com = None
        torch.cuda.empty_cache()
        leg = fused_leg(args, gt, w, layers, offsets, parents, accepted, status, vb, cb, dev,
                        f_steps, args.warmup, replay=kind == "replay")
        t = recorded_traffic("commit_verify" if kind == "fused" else "replay_verify",
                             args.config)                      # per layer
        leg["traffic_bytes"] = t
        leg["traffic_over_alg"] = round(t / leg["alg_bytes_per_layer"], 3) if t else None
        if kind == "fused":
            fused = leg
        else:
            replay = leg
    separate = None
    if headline_fused:
        head = fused if args.step == "fused" else replay
        kname = "commit_verify" if args.step == "fused" else "replay_verify"
        # the separate calls become the secondary figures; the fused kernel is
        # the headline step's only (and so dominant) kernel
        separate = {"value": round(nodes_per_s, 1), "ms_per_step": round(ms_step, 4),
                    "steps": sep_steps, "roofline": roof}
    for kn, leg in (("commit_verify", fused), ("replay_verify", replay)):
        if leg is not None:
            kern[kn] = {
                "avg_us": leg["us_per_layer"], "alg_bytes": leg["alg_bytes_per_layer"],
                "achieved_GBs": leg["achieved_GBs"], "frac_hbm": leg["frac_hbm"],
                "layers_per_launch": L, "launch_us": leg["launch_us_mean"],
                "alg_bytes_per_launch": leg["alg_bytes_per_layer"] * L,
                "traffic_bytes": leg["traffic_bytes"], "traffic_over_alg": leg["traffic_over_alg"]}
    if headline_fused:
        roof = {"kernel": "wy_" + kname, "bound": "hbm", "achieved": head["achieved_GBs"],
                "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": head["frac_hbm"],
                "traffic": head["traffic_bytes"] * L if head["traffic_bytes"] else None,
                "layers_per_launch": L}
        nodes_per_s = head["nodes_per_s_per_layer"]
        ms_step = head["ms_per_step"]

    # ------------------------------------------------------------- fork baseline
    fork = None
    if args.mode == "wy" and args.fork_steps > 0:
        for ly in layers:
            ly.pop("o_wy", None), ly.pop("ws_wy", None)
        ver = com = None
        torch.cuda.empty_cache()
        fdesc, fbytes, fver, fcom = make_calls("fork")
        f_el, f_v, f_c = run(fver, fcom, args.fork_steps, 1)
        fork = {"ms_per_step": round(1e3 * f_el / args.fork_steps, 3),
                "nodes_per_s_per_layer": round(w.T * L * args.fork_steps / f_el, 1),
                "verify_us_per_layer": round(1e3 * f_v / L, 2),
                "commit_us_per_layer": round(1e3 * f_c / L, 2),
                "workspace_bytes_per_layer": int(fbytes), "steps": args.fork_steps}
        log(f"fork: {fork}")
        for ly in layers:
            ly.pop("o_fork"), ly.pop("ws_fork")
        fver = fcom = None
        torch.cuda.empty_cache()
        fork["delta_checkpoints"] = fork_delta_leg(args, gt, gi, w, layers, offsets, parents,
                                                   accepted, status, max_depth, run, dev)
        fork["selective"] = selective_fork_leg(args, gt, gi, w, layers, offsets, parents,
                                               accepted, status, max_depth, run, dev)

    if args.pmc_calibration:
        pmc_calibration(dev)

    # speculative state per request (one sequence), summed over the layers
    n_req = w.T / w.B
    wy_state = n_req * L * w.H * (4 * w.dv + 4 + io_bytes * w.dk)
    fork_state = n_req * L * w.H * 4 * w.dv * w.dk
    # the replay round (the headline step) keeps no workspace: between its
    # acceptance and the next verify it retains the round's k, v, alpha, beta
    # rows (all nodes, as the call takes them; only the accepted path's rows
    # are read, so a caller that compacts them keeps the path alone)
    replay_state = n_req * L * w.H * (io_bytes * (w.dk + w.dv) + 8)
    mean_path = sum(len(gi.path_to_root(p, int(a))) if a >= 0 else 0
                    for p, a in zip(w.parents_list, w.accepted)) / w.B
    replay_path = mean_path * L * w.H * (io_bytes * (w.dk + w.dv) + 8)
    spec = {"wy_bytes": int(wy_state), "wy_bytes_without_keys": int(n_req * L * w.H * (4 * w.dv + 4)),
            # the fused rounds keep two WY workspaces per layer at once (the
            # previous round's until its commit has run, and this round's)
            "wy_bytes_fused_rounds": int(2 * wy_state),
            "replay_retained_bytes": int(replay_state),
            "replay_retained_path_bytes": int(replay_path),
            "fork_fp32_bytes": int(fork_state), "fork_over_wy": round(fork_state / wy_state, 1),
            # selective fork: the saved checkpoints of an average request
            "selective_fork_fp32_bytes": (int(fork["selective"]["saved_bytes_per_layer"] * L / w.B)
                                          if fork and "selective" in fork else None),
            "fork_over_replay": round(fork_state / replay_state, 1),
            "nodes_per_request": n_req, "mean_accepted_path": round(mean_path, 3), "layers": L}

    # --------------------------------------------------------------- CPU oracle
    cpu = None
    if args.cpu_seconds > 0:
        import oracle
        threads = oracle.threads()
        done_nodes, spent, used_layers = 0, 0.0, 0
        for layer in range(L):
            x = [np.ascontiguousarray(a[layer], np.float64) for a in (w.q, w.k, w.v, w.alpha, w.beta, w.S0)]
            t1 = time.perf_counter()
            oracle.verify(w.offsets, w.parents, *x)
            oracle.commit(w.offsets, w.parents, w.accepted, x[1], x[2], x[3], x[4], x[5])
            spent += time.perf_counter() - t1
            done_nodes += w.T
            used_layers += 1
            if spent >= args.cpu_seconds:
                break
        cpu = {"value": round(done_nodes / spent, 1), "unit": "nodes/s/layer", "cores": threads,
               "kind": "oracle",
               "sample": f"{used_layers} of {L} layers x {w.B} seqs x {w.H} heads, verify+commit, "
                         f"fp64 per-path replay, {spent:.1f} s",
               "cpu_model": cpu_model()}
        # the k=2 d=3 batch (32 sequences, one layer) on one host thread
        w3 = gi.make_config("c3")
        x3 = [np.ascontiguousarray(a[0], np.float64)
              for a in (w3.q, w3.k, w3.v, w3.alpha, w3.beta, w3.S0)]
        oracle.set_threads(1)
        try:
            t1 = time.perf_counter()
            oracle.verify(w3.offsets, w3.parents, *x3)
            oracle.commit(w3.offsets, w3.parents, w3.accepted, x3[1], x3[2], x3[3], x3[4], x3[5])
            one = time.perf_counter() - t1
        finally:
            oracle.set_threads(threads)
        cpu["single_thread_k2d3"] = {"value": round(w3.T / one, 1), "unit": "nodes/s/layer",
                                     "seconds": round(one, 3),
                                     "sample": "tree k=2 d=3, 32 seqs x 16 heads, one layer"}
        log(f"cpu oracle: {cpu}")

    fa = None
    for ly in layers:
        for key in [k for k in ly if k.startswith("o_") or k.startswith("ws_")]:
            ly.pop(key)
    ver = com = None
    torch.cuda.empty_cache()
    cfgs = config_legs(args, gt, gi, dev) if args.config_steps > 0 else None
    if args.attn_steps > 0:
        fa = attention_leg(args, gt, gi, w, dev)
        torch.cuda.empty_cache()
    rnd = None
    if args.round_steps > 0 and args.mode == "wy" and w.io == "bf16":
        rnd = round_leg(args, gt, gi, w, layers, offsets, parents, dev)
        torch.cuda.empty_cache()
        rnd["sampling_acceptance"] = sampling_accept_leg(args, gt, gi, w, offsets, parents, dev)

    out = {
        "metric": METRIC, "value": round(nodes_per_s, 1), "unit": "nodes/s/layer", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16" if w.io == "bf16" else "f32",
        "data": "synthetic",
        "config": {"workload": gi.CONFIGS[args.config]["desc"], "config_id": args.config,
                   "layers": L, "batch": w.B, "total_nodes": w.T, "heads": w.H, "dk": w.dk,
                   "dv": w.dv, "io": w.io, "state": "fp32", "mode": args.mode,
                   "step": ("previous round's accepted path replayed + verify, fused"
                            if headline_fused and args.step == "replay" else
                            "previous commit + verify, fused" if headline_fused
                            else "verify then commit"),
                   "launch": "all layers per launch" if batched else "one launch per layer",
                   "parallelism": "single-gpu"},
        "roofline": roof, "kernels": kern, "cpu_baseline": cpu, "fork_baseline": fork,
        "per_layer_launches": per_layer, "fused_rounds": fused, "replay_rounds": replay,
        "separate_calls": separate,
        "spec_state_per_request": spec, "configs": cfgs, "fa_layers": fa,
        "round": rnd,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()

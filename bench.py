#!/usr/bin/env python3
"""Tree-GDN verify + commit throughput on one MI355X.

One step = every GDN layer of the workload verified (gdn_tree_verify) and
then committed in place (gdn_tree_commit): the whole hot path over one batch.
Default workload: k=3 d=3 draft trees (40 nodes incl. root), 24 GDN layers
with independent inputs and states, batch 64, 16 heads, 128x128 fp32 state,
bf16 q/k/v (Qwen3.5-9B GDN shape). Inputs are seeded synthetic data resident
in HBM before timing starts; the 24 layers' states (1.5 GiB) are far larger
than the 256 MB Infinity Cache, so layer-to-layer traffic reaches HBM.

Prints ONE JSON line. The metric is verified draft nodes per second per GDN
layer (nodes of all trees, root included, times layers, per second), with the
dominant kernel's roofline fraction, the fork/checkpoint baseline's time and
memory, and the CPU oracle timed on a bounded sample as a reported baseline.
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
CSRC = os.path.join(ROOT, "gated_deltanet_tree_02_amd", "csrc")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "wy_verify_commit_c4_hbm_traffic.md")
# sources whose hash ties a recorded counter measurement to the kernels it measured
KERNEL_SOURCES = {"verify": ["wy_verify.hip", "device_common.h", "launch.h"],
                  "commit": ["wy_commit.hip", "device_common.h", "launch.h"]}


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
    if not os.path.exists(TRAFFIC_FILE):
        return None
    pat = re.compile(rf"^traffic\s+{kind}\s+{config}\s+(\w+)\s+(\d+)\s*$")
    with open(TRAFFIC_FILE) as fh:
        for line in fh:
            m = pat.match(line.strip().strip("`"))
            if m and m.group(1) == kernel_source_hash(kind):
                return int(m.group(2))
    return None


def log(*a):
    print("[bench]", *a, file=sys.stderr, flush=True)


def parse():
    p = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=5)
    p.add_argument("--config", default="c4", choices=["c1", "c2", "c3", "c4", "c5"])
    p.add_argument("--mode", default="wy", choices=["wy", "fork"])
    p.add_argument("--fork-steps", type=int, default=3, help="timed steps of the fork baseline (0 = skip)")
    p.add_argument("--cpu-seconds", type=float, default=10.0, help="oracle sample budget (0 = skip)")
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

    def make_calls(mode):
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
    desc, nbytes, ver, com = make_calls(args.mode)
    log(f"mode {args.mode}: workspace {nbytes / 2**20:.1f} MiB per layer")
    elapsed, v_ms, c_ms = run(ver, com, args.steps, args.warmup)
    st = status.cpu().numpy()
    if np.any(st != 0):
        raise RuntimeError(f"nonzero tree status {np.unique(st)}")
    ms_step = 1e3 * elapsed / args.steps
    nodes_per_s = w.T * L * args.steps / elapsed
    vb, cb, fvb, fcb = algorithmic_bytes(w, io_bytes, gi)
    if args.mode == "fork":
        vb, cb = fvb, fcb
    v_us = 1e3 * v_ms / L      # average launch duration (events around back-to-back launches)
    c_us = 1e3 * c_ms / L
    kern = {
        "verify": {"avg_us": round(v_us, 3), "alg_bytes": int(vb),
                   "achieved_GBs": round(vb / v_us / 1e3, 1),
                   "frac_hbm": round(vb / v_us / 1e3 / HBM_PEAK_GBS, 4)},
        "commit": {"avg_us": round(c_us, 3), "alg_bytes": int(cb),
                   "achieved_GBs": round(cb / c_us / 1e3, 1),
                   "frac_hbm": round(cb / c_us / 1e3 / HBM_PEAK_GBS, 4)},
    }
    dom = "verify" if v_us >= c_us else "commit"
    traffic = recorded_traffic(dom, args.config) if args.mode == "wy" else None
    for kind in ("verify", "commit"):
        t = recorded_traffic(kind, args.config) if args.mode == "wy" else None
        kern[kind]["traffic_bytes"] = t
        kern[kind]["traffic_over_alg"] = round(t / kern[kind]["alg_bytes"], 3) if t else None
    roof = {"kernel": f"{'wy' if args.mode == 'wy' else 'fork'}_{dom}", "bound": "hbm",
            "achieved": kern[dom]["achieved_GBs"], "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": kern[dom]["frac_hbm"], "traffic": traffic}
    log(f"{args.mode}: {ms_step:.3f} ms/step, verify {v_us:.2f} us, commit {c_us:.2f} us per layer")

    # ------------------------------------------------------------- fork baseline
    fork = None
    if args.mode == "wy" and args.fork_steps > 0:
        for ly in layers:
            ly.pop("o_wy"), ly.pop("ws_wy")
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

    if args.pmc_calibration:
        x = torch.ones(64 << 20, device=dev)
        y = torch.empty_like(x)
        for _ in range(3):
            torch.mul(x, 1.0, out=y)
        torch.cuda.synchronize()
        del x, y
        log("pmc calibration: 3 x copy of 256 MiB done")

    # speculative state per request (one sequence), summed over the layers
    n_req = w.T / w.B
    wy_state = n_req * L * w.H * (4 * w.dv + 4 + io_bytes * w.dk)
    fork_state = n_req * L * w.H * 4 * w.dv * w.dk
    spec = {"wy_bytes": int(wy_state), "wy_bytes_without_keys": int(n_req * L * w.H * (4 * w.dv + 4)),
            "fork_fp32_bytes": int(fork_state), "fork_over_wy": round(fork_state / wy_state, 1),
            "nodes_per_request": n_req, "layers": L}

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
                         f"fp64 per-path replay, {spent:.1f} s"}
        log(f"cpu oracle: {cpu}")

    out = {
        "metric": METRIC, "value": round(nodes_per_s, 1), "unit": "nodes/s/layer", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": gi.CONFIGS[args.config]["desc"], "config_id": args.config,
                   "layers": L, "batch": w.B, "total_nodes": w.T, "heads": w.H, "dk": w.dk,
                   "dv": w.dv, "io": w.io, "state": "fp32", "mode": args.mode,
                   "parallelism": "single-gpu"},
        "roofline": roof, "kernels": kern, "cpu_baseline": cpu, "fork_baseline": fork,
        "spec_state_per_request": spec,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()

#!/usr/bin/env python3
"""Benchmark of the chunked gated delta-rule forward on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--no-cpu]

A step is one gdn_fwd call on one batch of the workload: the whole hot path (gate cumsum,
WY solve, inter-chunk state pass and masked output, all inside the fused kernel).  Inputs
are synthetic (workloads.py), resident in HBM before timing starts, and rotated over several
copies so that no step reads its inputs from the 256 MB MALL left warm by the previous one.

Prints one JSON line: throughput (tokens*heads/s), the roofline of the dominant kernel
(algorithmic bytes per launch / average launch time from HIP events on the launch stream,
against 8 TB/s HBM), and the fp64 CPU oracle timed on the host cores as a reported baseline.
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

HBM_PEAK_GBS = 8000.0
METRIC = "tokens·heads/sec for chunked gated delta-rule fwd; % MFMA (or HBM) peak"
KERNEL_SOURCES = ["gated_delta_rule_29_amd/csrc/gdn_fwd.hip", "gated_delta_rule_29_amd/csrc/gdn_device.h"]
COUNTER_FILE = "profiles/gdn_fwd_kernel_b4h16t4096_hbm_counters.md"


def alg_bytes_per_launch(B, T, H, K, V, elt=2):
    """Minimum HBM bytes of one dense forward: read q, k, v (elt bytes), beta and g (fp32),
    write o (elt bytes) and the final fp32 state."""
    tokens_heads = B * T * H
    per_th = (2 * K + V) * elt + 4 + 4 + V * elt
    return tokens_heads * per_th + B * H * K * V * 4


def kernel_source_hash():
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def measured_traffic(launch_bytes):
    """HBM bytes per launch from the committed rocprofv3 counter summary, if it was taken on
    the current kernel source (else None)."""
    path = os.path.join(ROOT, COUNTER_FILE)
    if not os.path.exists(path):
        return None
    text = open(path).read()
    m_hash = re.search(r"kernel_source_sha256_16:\s*([0-9a-f]+)", text)
    m_b = re.search(r"hbm_bytes_per_launch:\s*([0-9.eE+]+)", text)
    if not m_hash or not m_b or m_hash.group(1) != kernel_source_hash():
        return None
    return float(m_b.group(1))


def cpu_baseline(inp, n_chains_max=64):
    """The fp64 oracle on a bounded sample of the same workload (the first chains of batch 0
    onwards), timed on this host's cores."""
    import numpy as np

    import oracle

    B, T, H, K = inp["q"].shape
    nb = max(1, min(B, n_chains_max // H))
    sub = {k: (v[:nb] if v is not None else None) for k, v in inp.items()}
    args = [sub["q"], sub["k"], sub["v"], sub["beta"]]
    conv = [oracle._f64(a) for a in args]
    g = oracle._f64(sub["g"])
    oracle.gdn(conv[0][:, :64], conv[1][:, :64], conv[2][:, :64], conv[3][:, :64],
               g=g[:, :64])  # warm-up (library load, page-in)
    t0 = time.perf_counter()
    oracle.gdn(*conv, g=g)
    dt = time.perf_counter() - t0
    th = nb * T * H
    return {"value": th / dt, "unit": "tokens·heads/s", "cores": oracle.max_threads(),
            "kind": "oracle",
            "sample": "fp64 token recurrence on %d of %d batch rows (%d chains x %d tokens = "
                      "%d token*heads), one run, %.2f s wall" % (nb, B, nb * H, T, th, dt)}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="gdn_bf16_b4h16t4096")
    ap.add_argument("--rotate", type=int, default=4, help="input copies cycled through")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="instead of the benchmark, run 5 plain device-to-device copies of MIB "
                         "MiB (the reference kernel for scaling HBM byte counters)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(--gpus %d requested)" % args.gpus, file=sys.stderr)
        sys.exit(2)

    import torch

    import gated_delta_rule_29_amd as gdn
    import workloads

    if args.copy_calibration:
        n = args.copy_calibration << 20
        src = torch.ones(n, dtype=torch.uint8, device="cuda:0")
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes": n, "copies": 5}))
        return

    spec = workloads.WORKLOADS[args.workload]
    if spec["kind"] != "gdn":
        raise SystemExit("bench.py times the dense gdn_fwd workloads")
    dev = torch.device("cuda:0")
    inp = workloads.make(args.workload)
    B, T, H, K = inp["q"].shape
    V = inp["v"].shape[-1]
    dt = inp["q"].dtype
    sets = []
    for r in range(max(1, args.rotate)):
        sets.append({k: (v.to(dev) if v is not None else None) for k, v in inp.items()})
    torch.cuda.synchronize()

    def step(i):
        s = sets[i % len(sets)]
        return gdn.gdn_fwd(s["q"], s["k"], s["v"], s["beta"], g=s["g"], gk=s["gk"])

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream(dev)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(args.steps)]
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_start.record(stream)
    for i in range(args.steps):
        ev[i][0].record(stream)
        step(i)
        ev[i][1].record(stream)
    t_end.record(stream)
    torch.cuda.synchronize()
    total_ms = t_start.elapsed_time(t_end)
    launch_ms = [a.elapsed_time(b) for a, b in ev]
    ms_per_step = total_ms / args.steps
    th = B * T * H
    value = th / (ms_per_step / 1e3)
    avg_launch_s = sum(launch_ms) / len(launch_ms) / 1e3
    elt = 2 if dt == torch.bfloat16 else 4
    alg = alg_bytes_per_launch(B, T, H, K, V, elt)
    achieved = alg / avg_launch_s / 1e9
    traffic = measured_traffic(alg)
    out = {
        "metric": METRIC,
        "value": value,
        "unit": "tokens·heads/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if dt == torch.bfloat16 else "f32",
        "data": "synthetic (seeded; q,k L2-normalised, beta=sigmoid(N), g=logsigmoid(N+%g))"
                % spec.get("g_shift", 3.0),
        "config": {"workload": args.workload, "B": B, "T": T, "H": H, "K": K, "V": V,
                   "chunk": 64, "state": "fp32", "input_copies_rotated": len(sets)},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS, "traffic": traffic,
                     "kernel": "gdn_fwd_kernel", "alg_bytes_per_launch": alg,
                     "avg_launch_ms": avg_launch_s * 1e3},
        "cpu_baseline": None,
    }
    if not args.no_cpu:
        out["cpu_baseline"] = cpu_baseline(inp)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()

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
BF16_MFMA_PEAK_TFLOPS = 2500.0  # published dense bf16 matrix-core peak
METRIC = "tokens·heads/sec for chunked gated delta-rule fwd; % MFMA (or HBM) peak"
KERNEL_SOURCE_DIR = "gated_delta_rule_29_amd/csrc"
# The kernels one forward call launches; the roofline covers the whole call (every kernel on
# the path), timed with HIP events around it on the launch stream.
KERNELS_FUSED = "gdn_fwd call: fused16_kernel"
KERNELS_FUSED_PACKED = "gdn_fwd_varlen call: rank_kernel + fused16_kernel"
KERNELS_BF16 = "gdn_fwd call: prep16_kernel + scan16_kernel"
KERNELS_BF16_PK = "gdn_fwd call: prep16pk_kernel + scan16_kernel"
KERNELS_F32 = "gdn_fwd call: chunk_prep_kernel + scan_kernel"


def kernels_of(dt, per_key, save):
    """Kernels one forward call launches: bf16 with a scalar gate and nothing saved per chunk
    runs the single fused kernel; per-key gates or saved states take the two-kernel path."""
    import torch

    if dt != torch.bfloat16:
        return KERNELS_F32
    if per_key:
        return KERNELS_BF16_PK
    return KERNELS_BF16 if save else KERNELS_FUSED
COUNTER_FILE = "profiles/all_workloads_counters.md"

# The .hip files that define and launch each workload's kernels; their hash (with every local
# header they include) stamps the counter summary, which is used only while it matches.
SOURCES = {
    KERNELS_FUSED: ["gdn_fwd.hip", "gdn_fused16.hip"],
    KERNELS_FUSED_PACKED: ["gdn_fwd.hip", "gdn_fused16.hip"],
    KERNELS_BF16: ["gdn_fwd.hip", "gdn_prep16.hip", "gdn_scan16.hip"],
    KERNELS_BF16_PK: ["gdn_fwd.hip", "gdn_prep16.hip", "gdn_scan16.hip"],
    KERNELS_F32: ["gdn_fwd.hip"],
    "bigdn": ["gdn_bigdn.hip"],
    "bigdn_merged": ["gdn_bigdn.hip"],
    "cam": ["gdn_cam.hip", "gdn_bigdn.hip"],
    "cam_bwd": ["gdn_cambwd.hip"],
    "bigdn_bwd": ["gdn_bigdnbwd.hip", "gdn_cambwd.hip"],
    "bigdn_block_bwd": ["gdn_bigdn.hip", "gdn_bigdnbwd.hip", "gdn_cambwd.hip", "gdn_prepbwd.hip"],
    "cam_branch_bwd": ["gdn_cam.hip", "gdn_cambwd.hip", "gdn_prepbwd.hip"],
    "summary": ["gdn_fwd.hip", "gdn_fused16.hip", "gdn_summary.hip"],
    "dhu": ["gdn_bwd.hip"],
}

def alg_bytes_per_launch(B, T, H, K, V, elt=2, per_key=False, save=False, n_states=None,
                         n_chunks=None):
    """Minimum HBM bytes of one forward: read q, k, v (elt bytes), beta and g (fp32) and gk
    (fp32, per-key gate); write o (elt bytes), the final fp32 states and, when saved, v_new
    (elt bytes) and the state entering every 64-token chunk (elt bytes)."""
    tokens_heads = B * T * H
    per_th = (2 * K + V) * elt + 4 + 4 + V * elt
    if per_key:
        per_th += 4 * K
    total = tokens_heads * per_th
    if save:
        n_chunks = B * H * ((T + 63) // 64) if n_chunks is None else n_chunks
        total += tokens_heads * V * elt + n_chunks * K * V * elt
    n_states = B * H if n_states is None else n_states
    total += n_states * K * V * 4
    return total


def alg_bytes_bigdn(B, F, S, H, D):
    """Minimum HBM bytes of one BiGDN block forward: read qkv once (bf16), beta, decay, the
    two RoPE tables and norm weights; write num (bf16) and den (bf16)."""
    N = F * S
    return (B * N * 3 * H * D * 2 + B * H * N * 4 + B * H * F * 4 + 2 * N * D * 4
            + 2 * H * D * 4 + B * N * H * D * 2 + B * H * N * 2)


def alg_bytes_cam(B, F, S, H, D):
    """Minimum HBM bytes of the camera branch step (fp32): the prep reads q, k, v, the camera
    matrices, the half-width RoPE tables and norm weights once and writes q_t, k_t, v_t and
    the inflation; the two scan directions together read q_t, k_t, v_t, beta and decay once
    and write their two outputs."""
    N = F * S
    C = H * D
    prep = 3 * B * N * C * 4 + 2 * B * N * 16 * 4 + 2 * N * (D // 2) * 4 + 2 * C * 4 \
        + 3 * B * N * C * 4 + B * H * N * 4
    scans = 3 * B * N * C * 4 + B * H * N * 4 + B * H * F * 4 + 2 * B * N * C * 4
    return prep + scans


def alg_bytes_cam_bwd(B, F, S, H, D):
    """Minimum HBM bytes of one camera-scan backward call (fp32): read q, k, v, dout, beta and
    decay once; write dq, dk, dv, dbeta and ddecay."""
    N = F * S
    return 7 * B * H * D * N * 4 + 2 * B * H * N * 4 + 2 * B * H * F * 4


def alg_bytes_bigdn_bwd(B, F, S, H, D):
    """Minimum HBM bytes of one BiGDN direction backward call: read the five prepped bf16
    tensors, dnum (fp32), beta, decay and dden once; write the five fp32 gradients, dbeta and
    ddecay."""
    N = F * S
    return (5 * 2 + 4 + 5 * 4) * B * H * N * D + 3 * B * H * N * 4 + 2 * B * H * F * 4


def alg_bytes_bigdn_block_bwd(B, F, S, H, D):
    """Minimum HBM bytes of the whole BiGDN block's backward: read qkv, num, den and the gate
    (bf16), dout (fp32), beta, decay, the RoPE tables and norm weights once; write dqkv,
    dgate (fp32), dbeta, ddecay and the two norm weights' gradients."""
    N = F * S
    C = H * D
    return (B * N * 3 * C * 2 + 2 * B * N * C * 2 + B * H * N * 2 + B * N * C * 4
            + B * H * N * 4 + B * H * F * 4 + 2 * N * D * 4 + 2 * C * 4
            + B * N * 3 * C * 4 + B * N * C * 4 + B * H * N * 4 + B * H * F * 4 + 2 * C * 4)


def alg_bytes_cam_branch_bwd(B, F, S, H, D):
    """Minimum HBM bytes of the camera branch's backward (fp32): read q, k, v, the camera
    matrices, the half-width RoPE tables, norm weights, beta, decay, the two scan outputs'
    gradients and the inflation's once; write dq, dk, dv, the norm weights' gradients, dbeta
    and ddecay."""
    N = F * S
    C = H * D
    return (3 * B * N * C * 4 + 2 * B * N * 16 * 4 + 2 * N * (D // 2) * 4 + 2 * C * 4
            + B * H * N * 4 + B * H * F * 4 + 2 * B * N * C * 4 + B * H * N * 4
            + 3 * B * N * C * 4 + 2 * C * 4 + B * H * N * 4 + B * H * F * 4)


def alg_bytes_dhu(B, T, H, K, V, elt):
    """Minimum HBM bytes of one state-gradient pass: read q, k, w, do, dv (input dtype), the
    gates and dht once; write dv2 (input dtype), the per-chunk state gradients and dh0 (fp32)."""
    NT = (T + 63) // 64
    return (3 * B * T * H * K * elt + 2 * B * T * H * V * elt + B * T * H * 4 + B * H * K * V * 4
            + B * T * H * V * elt + B * H * NT * K * V * 4 + B * H * K * V * 4)


def kernel_source_hash(files):
    """Hash of the given kernel sources and of every local header they include (transitively):
    a counter summary is valid only for the code it measured."""
    d = os.path.join(ROOT, KERNEL_SOURCE_DIR)
    seen, todo = set(), list(files)
    while todo:
        name = todo.pop()
        if name in seen:
            continue
        seen.add(name)
        with open(os.path.join(d, name)) as f:
            todo += re.findall(r'^#include "([^"]+)"', f.read(), flags=re.M)
    h = hashlib.sha256()
    for name in sorted(seen):
        h.update(name.encode())
        with open(os.path.join(d, name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def measured_traffic(workload, files):
    """HBM bytes per call from the committed rocprofv3 counter summary, if it was taken on the
    current sources of the workload's kernels (else None).  Lines of the form
    `traffic <workload> <bytes per call> <source hash>`."""
    path = os.path.join(ROOT, COUNTER_FILE)
    if not os.path.exists(path):
        return None
    m = re.search(r"^traffic %s ([0-9.eE+]+) ([0-9a-f]+)$" % re.escape(workload), open(path).read(),
                  flags=re.M)
    if not m or m.group(2) != kernel_source_hash(files):
        return None
    return float(m.group(1))


def _cpu_time(fn, sample, th):
    import oracle

    t0 = time.perf_counter()
    fn()
    dt = time.perf_counter() - t0
    return {"value": th / dt, "unit": "tokens·heads/s", "cores": oracle.max_threads(),
            "kind": "oracle", "sample": "%s; one run, %.2f s wall" % (sample, dt)}


def cpu_baseline(kind, inp, max_chains=64):
    """The fp64 oracle, as it stands, on a bounded sample of the same workload (whole
    independent chains, so the sample does the same per-token work), timed on this host."""
    import oracle
    import torch

    oracle.build()
    if kind == "bigdn_merged":
        B, N, _, H, D = inp["qkv"].shape
        return _cpu_time(lambda: oracle.bigdn_merged(
            inp["qkv"], inp["beta"], inp["decay"], inp["q_norm_w"], inp["k_norm_w"],
            inp["rope_cos"], inp["rope_sin"], inp["k_scale"], inp["eps"],
            decay_bwd=inp["decay_bwd"], gate=inp["gate"], merge_eps=1e-6),
            "whole merged block: prep + both directions + merge, %d heads x %d tokens"
            % (H, N), B * N * H)
    if kind == "dhu":
        B, T, H, K = inp["q"].shape
        hh = min(H, 8)
        ts = T if inp["gk"] is None else min(T, 4096)  # per-key: a bounded prefix of each chain
        sub = {k: (oracle._f64(v[:1, :ts, :hh]) if isinstance(v, torch.Tensor) and k != "dht"
                   else v) for k, v in inp.items()}
        return _cpu_time(lambda: oracle.gdn_dhu(sub["q"], sub["k"], sub["w"], sub["do"],
                                                sub["dv"], g=sub["g"],
                                                dht=oracle._f64(inp["dht"][:1, :hh]),
                                                scale=inp["scale"], gk=sub["gk"]),
                         "1 of %d batch rows x %d of %d heads (%d chains x %d of %d tokens)"
                         % (B, hh, H, hh, ts, T), hh * ts)
    if kind == "cam":
        B, N, H, D = inp["q"].shape
        F, S = inp["beta"].shape[2], inp["beta"].shape[3]
        fs = min(F, 4)
        n = fs * S
        sub = {k: oracle._f64(inp[k][:, :n]) for k in ("q", "k", "v", "proj_q", "proj_kv")}

        def run():
            qt, kt, vt, _ = oracle.cam_prep(sub["q"], sub["k"], sub["v"], inp["q_norm_w"],
                                            inp["k_norm_w"], sub["proj_q"], sub["proj_kv"],
                                            inp["rope_cos"][:n], inp["rope_sin"][:n],
                                            inp["k_scale"], inp["eps"])
            for rev in (False, True):
                oracle.cam_scan(qt, kt, vt, inp["beta"][:, :, :fs], inp["decay"][:, :, :fs],
                                reverse=rev)
        return _cpu_time(run, "camera prep + both scan directions on the first %d of %d frames, "
                         "all %d heads (%d tokens)" % (fs, F, H, n), B * n * H)
    if kind == "cam_bwd":
        B, H, D, N = inp["q"].shape
        F, S = inp["beta"].shape[2], inp["beta"].shape[3]
        fs = min(F, 4)
        n = fs * S
        sub = {k: inp[k][..., :n] for k in ("q", "k", "v", "dout")}
        sub["beta"], sub["decay"] = inp["beta"][:, :, :fs], inp["decay"][:, :, :fs]

        def run():
            for rev in (False, True):
                oracle.cam_scan_bwd(**sub, reverse=rev)
        return _cpu_time(run, "both scan directions' backward on the first %d of %d frames, "
                         "all %d heads (%d tokens)" % (fs, F, H, n), 2 * B * n * H)
    if kind == "cam_branch_bwd":
        B, N, H, D = inp["q"].shape
        F, S = inp["beta"].shape[2], inp["beta"].shape[3]
        fs = min(F, 4)
        n = fs * S
        sub = {k: oracle._f64(inp[k][:, :n]) for k in ("q", "k", "v", "proj_q", "proj_kv")}
        sub.update({k: oracle._f64(inp[k][..., :n]) for k in ("dout_fwd", "dout_rev", "dinfl")})
        sub.update(beta=oracle._f64(inp["beta"][:, :, :fs]),
                   decay=oracle._f64(inp["decay"][:, :, :fs]),
                   rope_cos=oracle._f64(inp["rope_cos"][:n]), rope_sin=oracle._f64(inp["rope_sin"][:n]))
        pw = (oracle._f64(inp["q_norm_w"]), oracle._f64(inp["k_norm_w"]))
        ks, eps = inp["k_scale"], inp["eps"]

        def run():
            qt, kt, vt, _ = oracle.cam_prep(sub["q"], sub["k"], sub["v"], *pw, sub["proj_q"],
                                            sub["proj_kv"], sub["rope_cos"], sub["rope_sin"],
                                            ks, eps)
            d = [oracle.cam_scan_bwd(qt, kt, vt, sub["beta"], sub["decay"],
                                     sub["dout_rev" if rev else "dout_fwd"], reverse=rev)
                 for rev in (False, True)]
            oracle.cam_prep_bwd(sub["q"], sub["k"], *pw, sub["proj_q"], sub["proj_kv"],
                                sub["rope_cos"], sub["rope_sin"], ks,
                                *(d[0][n] + d[1][n] for n in ("dq", "dk", "dv")), sub["dinfl"],
                                eps)
        return _cpu_time(run, "the branch's backward on the first %d of %d frames, all %d "
                         "heads (%d tokens)" % (fs, F, H, n), B * n * H)
    if kind == "bigdn_bwd":
        B, H, N, D = inp["q_rot"].shape
        F, S = inp["beta"].shape[2], inp["beta"].shape[3]
        fs = min(F, 4)
        n = fs * S
        names = ("q_rot", "k_rot", "q_pos", "k_pos", "v")
        sub = {k: inp[k][:, :, :n] for k in names}
        sub.update(beta=inp["beta"][:, :, :fs], decay=inp["decay"][:, :, :fs],
                   dnum=inp["dnum"][:, :n], dden=inp["dden"][:, :, :n])

        def run():
            for rev in (False, True):
                oracle.bigdn_dir_bwd(*(sub[k] for k in names + ("beta", "decay", "dnum", "dden")),
                                     reverse=rev)
        return _cpu_time(run, "both directions' backward on the first %d of %d frames, all %d "
                         "heads (%d tokens)" % (fs, F, H, n), 2 * B * n * H)
    if kind == "bigdn_block_bwd":
        import numpy as np

        B, N, _, H, D = inp["qkv"].shape
        F, S = inp["beta"].shape[2], inp["beta"].shape[3]
        fs = min(F, 4)
        n = fs * S
        sub = {k: oracle._f64(inp[k][:, :n]) for k in ("qkv", "gate", "dout")}
        sub.update(beta=oracle._f64(inp["beta"][:, :, :fs]), decay=oracle._f64(inp["decay"][:, :, :fs]),
                   rope_cos=oracle._f64(inp["rope_cos"][:n]), rope_sin=oracle._f64(inp["rope_sin"][:n]))
        pw = (oracle._f64(inp["q_norm_w"]), oracle._f64(inp["k_norm_w"]))
        ks, eps = inp["k_scale"], inp["eps"]
        _, num, den = oracle.bigdn_merged(sub["qkv"], sub["beta"], sub["decay"], *pw,
                                          sub["rope_cos"], sub["rope_sin"], ks, eps,
                                          gate=sub["gate"])  # the saved forward sums (not timed)
        names = ("q_rot", "k_rot", "q_pos", "k_pos", "v")

        def run():
            p = oracle.prep(sub["qkv"], *pw, sub["rope_cos"], sub["rope_sin"], ks, eps)
            m = oracle.bigdn_merge_bwd(num, den, sub["dout"], sub["gate"])
            d = [oracle.bigdn_dir_bwd(*(p[k] for k in names), sub["beta"], sub["decay"],
                                      m["dnum"], m["dden"], reverse=rev) for rev in (False, True)]
            oracle.prep_bwd(sub["qkv"], *pw, sub["rope_cos"], sub["rope_sin"], ks,
                            {"d" + k: np.stack([x["d" + k] for x in d]) for k in names}, eps)
        return _cpu_time(run, "the block's backward on the first %d of %d frames, all %d heads "
                         "(%d tokens)" % (fs, F, H, n), B * n * H)
    if kind == "bigdn":
        B, N, _, H, D = inp["qkv"].shape
        F, S = inp["beta"].shape[2], inp["beta"].shape[3]
        args = [oracle._f64(inp[n]) for n in ("qkv", "beta", "decay", "q_norm_w", "k_norm_w",
                                               "rope_cos", "rope_sin")]
        return _cpu_time(lambda: oracle.bigdn(*args, inp["k_scale"], inp["eps"]),
                         "whole block: prep + both directions, %d heads x %d tokens" % (H, N),
                         B * N * H)
    if kind == "summary":
        B, T, H, K = inp["k"].shape
        nb, hh = 1, min(H, 8)
        sub = {k: (oracle._f64(v[:nb, :, :hh]) if v is not None else None) for k, v in inp.items()}
        return _cpu_time(lambda: oracle.state_summary(sub["k"], sub["v"], sub["beta"], g=sub["g"]),
                         "1 of %d batch rows x %d of %d heads (%d chains x %d tokens)"
                         % (B, hh, H, hh, T), hh * T)
    if kind == "varlen":
        cu = inp["cu_seqlens"].numpy()
        n = 1
        H = inp["q"].shape[2]
        T1 = int(cu[n])
        sub = {k: (oracle._f64(v[:, :T1]) if v is not None and k != "cu_seqlens" else None)
               for k, v in inp.items()}
        return _cpu_time(lambda: oracle.gdn_varlen(cu[:n + 1], sub["q"], sub["k"], sub["v"],
                                                   sub["beta"], g=sub["g"]),
                         "first packed sequence (%d tokens) x %d heads" % (T1, H), T1 * H)
    B, T, H, K = inp["q"].shape
    nb = max(1, min(B, max_chains // H))
    hh = min(H, max_chains)
    sub = {k: (oracle._f64(v[:nb, :, :hh]) if v is not None else None) for k, v in inp.items()}
    return _cpu_time(lambda: oracle.gdn(sub["q"], sub["k"], sub["v"], sub["beta"], g=sub["g"],
                                        gk=sub["gk"]),
                     "%d of %d batch rows x %d of %d heads (%d chains x %d tokens)"
                     % (nb, B, hh, H, nb * hh, T), nb * hh * T)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="gdn_bf16_b4h16t4096")
    ap.add_argument("--rotate", type=int, default=0,
                    help="input copies cycled through (default: enough to exceed 1 GB)")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="instead of the benchmark, run 5 plain device-to-device copies of MIB "
                         "MiB (the reference kernel for scaling HBM byte counters)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
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
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(5):
            dst.copy_(src)
        e1.record()
        torch.cuda.synchronize()
        # bytes read plus bytes written over the five copies: what a plain streaming kernel
        # reaches on this device, beside the published 8 TB/s the rooflines are quoted against
        gbs = 5 * 2 * n / (e0.elapsed_time(e1) * 1e6)
        print(json.dumps({"copy_calibration_bytes": n, "copies": 5, "copy_GBps": round(gbs, 1)}))
        return

    spec = dict(workloads.WORKLOADS[args.workload])
    kind = spec["kind"]
    dev = torch.device("cuda:0")
    inp = workloads.make(args.workload)
    in_bytes = sum(v.numel() * v.element_size() for v in inp.values() if isinstance(v, torch.Tensor))
    rotate = args.rotate or max(2, min(8, -(-(1 << 30) // max(in_bytes, 1))))
    sets = []
    for r in range(rotate):
        sets.append({k: (v.to(dev) if isinstance(v, torch.Tensor) else v) for k, v in inp.items()})
    torch.cuda.synchronize()
    save = bool(spec.get("save", False))

    if kind == "gdn":
        B, T, H, K = inp["q"].shape
        V = inp["v"].shape[-1]
        dt = inp["q"].dtype
        th = B * T * H
        elt = 2 if dt == torch.bfloat16 else 4
        alg = alg_bytes_per_launch(B, T, H, K, V, elt, inp["gk"] is not None, save)
        kernel = kernels_of(dt, inp["gk"] is not None, save)
        config = {"workload": args.workload, "B": B, "T": T, "H": H, "K": K, "V": V,
                  "chunk": 64, "state": "fp32", "per_key_gate": inp["gk"] is not None,
                  "saves_h_and_v_new": save}

        def step(i):
            s = sets[i % len(sets)]
            return gdn.gdn_fwd(s["q"], s["k"], s["v"], s["beta"], g=s["g"], gk=s["gk"],
                               want_h=save, want_v_new=save)
    elif kind == "varlen":
        _, T, H, K = inp["q"].shape
        V = inp["v"].shape[-1]
        dt = inp["q"].dtype
        cu = inp["cu_seqlens"]
        N = cu.numel() - 1
        th = T * H
        elt = 2 if dt == torch.bfloat16 else 4
        alg = alg_bytes_per_launch(1, T, H, K, V, elt, False, False, n_states=N * H)
        kernel = kernels_of(dt, inp["gk"] is not None, False)
        kernel = KERNELS_FUSED_PACKED if kernel == KERNELS_FUSED else kernel + " (packed)"
        config = {"workload": args.workload, "T_total": T, "N": N, "H": H, "K": K, "V": V,
                  "lengths": (cu[1:] - cu[:-1]).tolist(), "chunk": 64, "state": "fp32"}

        cu_host = cu.to(torch.int32).contiguous()  # the host copy, made once

        def step(i):
            s = sets[i % len(sets)]
            return gdn.gdn_fwd_varlen(s["q"], s["k"], s["v"], s["beta"], s["cu_seqlens"],
                                      g=s["g"], want_tables=False, cu_seqlens_host=cu_host)
    elif kind == "summary":
        B, T, H, K = inp["q"].shape
        V = inp["v"].shape[-1]
        dt = inp["q"].dtype
        th = B * T * H
        # the transition's chunked products per token and chain: X = W M and M -= K^T X,
        # 2 K^2 flops each (the split-operand form takes 3 matrix-core products per product, 2
        # with bf16 keys; counted once here)
        alg = 4 * K * K * th
        kernel = ("gdn_state_summary call: fused16_kernel (zero-start state) + trans_wy_kernel + "
                  "trans_chain_kernel")
        config = {"workload": args.workload, "B": B, "T": T, "H": H, "K": K, "V": V,
                  "state": "fp32", "outputs": "state_ext [B,H,K,V] + transition [B,H,K,K]"}

        def step(i):
            s = sets[i % len(sets)]
            return gdn.gdn_state_summary(s["k"], s["v"], s["beta"], g=s["g"])
    elif kind == "bigdn_merged":
        B, N, _, H, D = inp["qkv"].shape
        F, S = inp["beta"].shape[2], inp["beta"].shape[3]
        dt = torch.bfloat16
        th = B * N * H
        # as the block above, plus the reverse decay and the gate read; out written instead of
        # num and den
        alg = (alg_bytes_bigdn(B, F, S, H, D) + B * H * F * 4 + B * N * H * D * 2
               - B * H * N * 2)
        kernel = "bigdn_fwd_merged (4 kernels, whole call)"
        config = {"workload": args.workload, "B": B, "F": F, "S": S, "N": N, "H": H, "D": D,
                  "state": "fp32", "reverse": "decay 0 at every 4th frame",
                  "merge": "num / (den + 1e-6) * SiLU(gate)"}

        def step(i):
            s = sets[i % len(sets)]
            return gdn.bigdn_fwd_merged(s["qkv"], s["beta"], s["decay"], s["q_norm_w"],
                                        s["k_norm_w"], s["rope_cos"], s["rope_sin"],
                                        s["k_scale"], s["eps"], decay_bwd=s["decay_bwd"],
                                        gate=s["gate"], merge_eps=1e-6)
    elif kind == "dhu":
        B, T, H, K = inp["q"].shape
        V = inp["do"].shape[-1]
        dt = inp["q"].dtype
        th = B * T * H
        alg = alg_bytes_dhu(B, T, H, K, V, 2 if dt == torch.bfloat16 else 4)
        if inp["gk"] is not None:
            alg += B * T * H * K * 4
        kernel = "gdn_bwd_dhu call: " + ("dhu16_kernel" if dt == torch.bfloat16 else "dhu_kernel")
        config = {"workload": args.workload, "B": B, "T": T, "H": H, "K": K, "V": V,
                  "chunk": 64, "per_key_gate": inp["gk"] is not None,
                  "outputs": "dv2, dh per chunk [B,H,NT,K,V] fp32, dh0"}

        def step(i):
            s = sets[i % len(sets)]
            return gdn.gdn_bwd_dhu(s["q"], s["k"], s["w"], s["do"], s["dv"], g=s["g"],
                                   dht=s["dht"], scale=s["scale"], gk=s["gk"])
    elif kind == "cam":
        B, N, H, D = inp["q"].shape
        F, S = inp["beta"].shape[2], inp["beta"].shape[3]
        dt = torch.float32
        th = B * N * H
        alg = alg_bytes_cam(B, F, S, H, D)
        kernel = "cam_prep + cam_scan_bidi (5 kernels, whole step)"
        config = {"workload": args.workload, "B": B, "F": F, "S": S, "N": N, "H": H, "D": D,
                  "state": "fp32", "products": "fp16 operands, fp32 accumulation",
                  "step": "camera prep, then the forward and the reverse frame scans (one "
                          "bidirectional call)"}

        def step(i):
            s = sets[i % len(sets)]
            qt, kt, vt, infl = gdn.cam_prep(s["q"], s["k"], s["v"], s["q_norm_w"],
                                            s["k_norm_w"], s["proj_q"], s["proj_kv"],
                                            s["rope_cos"], s["rope_sin"], s["k_scale"], s["eps"])
            fwd, rev = gdn.cam_scan_bidi(qt, kt, vt, s["beta"], s["decay"])
            return fwd, rev, infl
    elif kind == "cam_bwd":
        B, H, D, N = inp["q"].shape
        F, S = inp["beta"].shape[2], inp["beta"].shape[3]
        dt = torch.float32
        th = 2 * B * N * H  # tokens*heads of both directions
        alg = 2 * alg_bytes_cam_bwd(B, F, S, H, D)
        kernel = "cam_scan_bwd x 2 directions (3 kernels each, whole step)"
        config = {"workload": args.workload, "B": B, "F": F, "S": S, "N": N, "H": H, "D": D,
                  "state": "fp32", "products": "split bf16 (hi/lo) operands, fp32 accumulation",
                  "step": "gradients of the forward and of the reverse frame scan (two calls, "
                          "the second reusing the first's frame statistics; summing the two "
                          "directions' gradients is the caller's)"}

        ws = torch.empty(gdn._lib.load().cam_scan_bwd_workspace_bytes(B, H, D, F),
                         dtype=torch.uint8, device=dev)

        def step(i):
            s = sets[i % len(sets)]
            # the reverse call reuses the forward one's frame statistics (same q, k, v, beta)
            return [gdn.cam_scan_bwd(s["q"], s["k"], s["v"], s["beta"], s["decay"], s["dout"],
                                     reverse=rev, workspace=ws, reuse_stats=rev)
                    for rev in (False, True)]
    elif kind == "cam_branch_bwd":
        B, N, H, D = inp["q"].shape
        F, S = inp["beta"].shape[2], inp["beta"].shape[3]
        dt = torch.float32
        th = B * N * H
        alg = alg_bytes_cam_branch_bwd(B, F, S, H, D)
        kernel = ("cam_bwd: cam_prep, cam_scan_bwd x 2 directions, cam_prep_bwd (12 kernels, "
                  "whole step)")
        config = {"workload": args.workload, "B": B, "F": F, "S": S, "N": N, "H": H, "D": D,
                  "state": "fp32", "products": "split bf16 (hi/lo) operands, fp32 accumulation",
                  "step": "from the gradients of the two scan outputs and of the inflation to q, "
                          "k, v, the norm weights, beta and decay"}
        pre = ("q_norm_w", "k_norm_w", "proj_q", "proj_kv", "rope_cos", "rope_sin")

        def step(i):
            s = sets[i % len(sets)]
            return gdn.cam_bwd(s["q"], s["k"], s["v"], *(s[k] for k in pre), s["k_scale"],
                               s["beta"], s["decay"], s["dout_fwd"], s["dout_rev"], s["dinfl"],
                               s["eps"])
    elif kind == "bigdn_bwd":
        B, H, N, D = inp["q_rot"].shape
        F, S = inp["beta"].shape[2], inp["beta"].shape[3]
        dt = torch.bfloat16
        th = 2 * B * N * H  # tokens*heads of both directions
        alg = 2 * alg_bytes_bigdn_bwd(B, F, S, H, D)
        kernel = "bigdn_dir_bwd x 2 directions (5 kernels each, whole step)"
        config = {"workload": args.workload, "B": B, "F": F, "S": S, "N": N, "H": H, "D": D,
                  "state": "fp32", "products": "split bf16 (hi/lo) operands, fp32 accumulation",
                  "step": "gradients of the forward and of the reverse direction (two calls, the "
                          "second reusing the first's frame statistics; summing the two "
                          "directions' gradients is the caller's)"}
        names = ("q_rot", "k_rot", "q_pos", "k_pos", "v", "beta", "decay", "dnum", "dden")

        ws = torch.empty(gdn._lib.load().bigdn_dir_bwd_workspace_bytes(B, H, D, F),
                         dtype=torch.uint8, device=dev)

        def step(i):
            s = sets[i % len(sets)]
            # the reverse call reuses the forward one's frame statistics (same inputs)
            return [gdn.bigdn_dir_bwd(*(s[k] for k in names), reverse=rev, workspace=ws,
                                      reuse_stats=rev) for rev in (False, True)]
    elif kind == "bigdn_block_bwd":
        B, N, _, H, D = inp["qkv"].shape
        F, S = inp["beta"].shape[2], inp["beta"].shape[3]
        dt = torch.bfloat16
        th = B * N * H
        alg = alg_bytes_bigdn_block_bwd(B, F, S, H, D)
        kernel = ("bigdn_bwd: gdn_prep, bigdn_merge_bwd, bigdn_dir_bwd x 2 directions, "
                  "gdn_prep_bwd (15 kernels, whole step)")
        config = {"workload": args.workload, "B": B, "F": F, "S": S, "N": N, "H": H, "D": D,
                  "state": "fp32", "products": "split bf16 (hi/lo) operands, fp32 accumulation",
                  "step": "from the gated output's gradient to qkv, the norm weights, beta, "
                          "decay and the gate (num, den from one forward before timing)"}
        pre = ("q_norm_w", "k_norm_w", "rope_cos", "rope_sin")
        for s in sets:  # the forward's saved sums, as a training step would hold them
            _, s["num"], s["den"] = gdn.bigdn_fwd_merged(
                s["qkv"], s["beta"], s["decay"], *(s[k] for k in pre), s["k_scale"], s["eps"],
                gate=s["gate"], merge_eps=1e-6, want_num_den=True)
        torch.cuda.synchronize()

        def step(i):
            s = sets[i % len(sets)]
            return gdn.bigdn_bwd(s["qkv"], s["beta"], s["decay"], *(s[k] for k in pre),
                                 s["k_scale"], s["num"], s["den"], s["dout"], s["gate"], 1e-6,
                                 s["eps"])
    elif kind == "bigdn":
        B, N, _, H, D = inp["qkv"].shape
        F, S = inp["beta"].shape[2], inp["beta"].shape[3]
        dt = torch.bfloat16
        th = B * N * H
        alg = alg_bytes_bigdn(B, F, S, H, D)
        kernel = "bigdn_fwd (4 kernels, whole call)"
        config = {"workload": args.workload, "B": B, "F": F, "S": S, "N": N, "H": H, "D": D,
                  "state": "fp32"}

        def step(i):
            s = sets[i % len(sets)]
            return gdn.bigdn_fwd(s["qkv"], s["beta"], s["decay"], s["q_norm_w"], s["k_norm_w"],
                                 s["rope_cos"], s["rope_sin"], s["k_scale"], s["eps"])
    else:
        raise SystemExit("unknown workload kind %s" % kind)

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
    srt = sorted(launch_ms)

    def pct(q):  # nearest-rank percentile of the per-launch times
        return srt[min(len(srt) - 1, max(0, int(round(q * (len(srt) - 1)))))]
    value = th / (ms_per_step / 1e3)
    avg_launch_s = sum(launch_ms) / len(launch_ms) / 1e3
    achieved = alg / avg_launch_s / 1e9
    if kind == "summary":  # matrix-core work: alg counts flops, reported in TFLOP/s
        roof = {"bound": "mfma", "achieved": achieved / 1e3, "peak": BF16_MFMA_PEAK_TFLOPS,
                "unit": "TFLOP/s", "frac": achieved / 1e3 / BF16_MFMA_PEAK_TFLOPS}
    else:
        roof = {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": achieved / HBM_PEAK_GBS}
    files = SOURCES.get(kernel if kind in ("gdn", "varlen") else kind)
    traffic = measured_traffic(args.workload, files) if files else None
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
        "data": "synthetic (seeded workloads.py recipe: %s)" % args.workload,
        "config": dict(config, input_copies_rotated=len(sets)),
        "launch_ms": {"median": pct(0.5), "p10": pct(0.1), "p90": pct(0.9), "mean":
                      avg_launch_s * 1e3, "n": len(launch_ms),
                      "clock": "HIP events around each call on its stream"},
        "roofline": dict(roof, traffic=traffic, kernel=kernel,
                         **{("alg_flops_per_launch" if kind == "summary" else
                             "alg_bytes_per_launch"): alg},
                         avg_launch_ms=avg_launch_s * 1e3),
        "cpu_baseline": None,
    }
    if not args.no_cpu:
        out["cpu_baseline"] = cpu_baseline(kind, inp)
        if args.workload == "tiny_f32":
            # the small fp32 workload is also timed on one host thread (whole workload)
            import oracle

            n0 = oracle.max_threads()
            oracle.set_threads(1)
            one = cpu_baseline(kind, inp)
            oracle.set_threads(n0)
            out["cpu_baseline"]["single_thread"] = {"value": one["value"], "cores": 1,
                                                    "sample": one["sample"]}
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()

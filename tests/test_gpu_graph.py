"""HIP graph capture of library calls: a captured call, replayed several times with eager
library work and synchronisations between the replays, gives the eager call's results bit for
bit (the kernels are deterministic), for the dense and packed forward, the BiGDN block and the
BiGDN block backward.  Every replay is checked, not only the first."""
import pytest
import torch

import workloads
from tests.gpu_util import say

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _flat(out):
    if isinstance(out, dict):
        return [v for k, v in sorted(out.items()) if isinstance(v, torch.Tensor)]
    if isinstance(out, (tuple, list)):
        return [t for o in out for t in _flat(o)]
    return [out]


def _check_replays(call, other, n=3):
    """call: the library call to capture; other: unrelated eager library work run between
    replays (it also overwrites the caching allocator's free blocks)."""
    ref = [t.clone() for t in _flat(call())]
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        out = call()
    outs = _flat(out)
    for r in range(n):
        g.replay()
        torch.cuda.synchronize()
        for a, b in zip(outs, ref):
            assert torch.equal(a, b), "replay %d differs" % r
        other()
        torch.cuda.synchronize()


def test_graph_dense_forward():
    import gated_delta_rule_29_amd as g

    say("graph: dense bf16 forward")
    d = {k: (v.to(DEV) if v is not None else None)
         for k, v in workloads.gdn_inputs(2, 1000, 4, 128, 128, dtype="bf16", seed=1).items()}
    e = {k: (v.to(DEV) if v is not None else None)
         for k, v in workloads.gdn_inputs(1, 300, 2, 64, 64, dtype="bf16", seed=2).items()}
    _check_replays(lambda: g.gdn_fwd(d["q"], d["k"], d["v"], d["beta"], g=d["g"]),
                   lambda: g.gdn_fwd(e["q"], e["k"], e["v"], e["beta"], g=e["g"]))


def test_graph_packed_forward():
    import gated_delta_rule_29_amd as g

    say("graph: packed bf16 forward")
    inp = workloads.varlen_inputs(5, 40, 700, 4, 128, 128, dtype="bf16", seed=3)
    d = {k: (v.to(DEV) if isinstance(v, torch.Tensor) and k != "cu_seqlens_host" else v)
         for k, v in inp.items()}
    cuh = inp["cu_seqlens"].cpu()

    def call():
        return g.gdn_fwd_varlen(d["q"], d["k"], d["v"], d["beta"], d["cu_seqlens"], g=d["g"],
                                cu_seqlens_host=cuh)
    e = {k: (v.to(DEV) if v is not None else None)
         for k, v in workloads.gdn_inputs(1, 300, 2, 64, 64, dtype="bf16", seed=2).items()}
    _check_replays(call, lambda: g.gdn_fwd(e["q"], e["k"], e["v"], e["beta"], g=e["g"]))


def test_graph_bigdn_block_and_backward():
    import gated_delta_rule_29_amd as g

    say("graph: BiGDN block forward and backward")
    inp = workloads.bigdn_block_bwd_inputs(1, 3, 128, 2, 128, seed=4)
    d = {k: (v.to(DEV) if isinstance(v, torch.Tensor) else v) for k, v in inp.items()}
    pre = (d["q_norm_w"], d["k_norm_w"], d["rope_cos"], d["rope_sin"], d["k_scale"])
    fwd = lambda: g.bigdn_fwd_merged(d["qkv"], d["beta"], d["decay"], *pre, d["eps"],
                                     gate=d["gate"], want_num_den=True)
    _, num, den = fwd()
    bwd = lambda: g.bigdn_bwd(d["qkv"], d["beta"], d["decay"], *pre, num, den, d["dout"],
                              d["gate"], 1e-6, d["eps"])
    _check_replays(fwd, bwd)
    _check_replays(bwd, fwd)

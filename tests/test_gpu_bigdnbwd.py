"""GPU parity of bigdn_dir_bwd (backward of one BiGDN direction) against the fp64 oracle,
through the C ABI.  The S stream's products take split bf16 operands and the z stream is fp32
arithmetic, so every gradient is held to the split-operand rule (SPLIT_OPERAND_TOL)."""
import pytest
import torch

import oracle
import workloads
from tests.gpu_util import SPLIT_OPERAND_TOL, assert_close, say

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
IN = ("q_rot", "k_rot", "q_pos", "k_pos", "v", "beta", "decay", "dnum", "dden")
OUT = ("dq_rot", "dk_rot", "dq_pos", "dk_pos", "dv", "dbeta", "ddecay")


def _run(inp, reverse):
    import gated_delta_rule_29_amd as g

    d = {k: inp[k].to(DEV) for k in IN}
    out = g.bigdn_dir_bwd(*(d[k] for k in IN), reverse=reverse)
    torch.cuda.synchronize()
    return out


def _check(inp, reverse, heads=None):
    out = _run(inp, reverse)
    sub = dict(inp)
    if heads is not None:
        sub = {k: (v[:, :, heads] if k == "dnum" else v[:, heads]) for k, v in inp.items()}
    ref = oracle.bigdn_dir_bwd(*(sub[k] for k in IN), reverse=reverse)
    for name in OUT:
        assert bool(torch.isfinite(out[name]).all()), name
        got = out[name] if heads is None else out[name][:, heads]
        assert_close(name, got, ref[name], SPLIT_OPERAND_TOL)
    return out


@pytest.mark.parametrize("reverse", [False, True])
@pytest.mark.parametrize("D,F,S", [(128, 4, 128), (64, 3, 64), (128, 2, 192)])
def test_bigdn_dir_bwd_small(D, F, S, reverse):
    say("bigdn_dir_bwd D%d F%d S%d reverse %s" % (D, F, S, reverse))
    _check(workloads.bigdn_bwd_inputs(2, F, S, 2, D, seed=D + F + S + int(reverse)), reverse)


@pytest.mark.parametrize("reverse", [False, True])
def test_bigdn_dir_bwd_strong_decay(reverse):
    """decay = sigmoid(N(0,1) - 2) (most of the state forgotten at every frame)."""
    _check(workloads.bigdn_bwd_inputs(1, 5, 64, 2, 128, seed=91, decay_shift=-2.0), reverse)


def test_bigdn_dir_bwd_structural_zeros_and_determinism():
    inp = workloads.bigdn_bwd_inputs(1, 3, 64, 2, 64, seed=5)
    rev = _run(inp, True)
    for name in ("dk_rot", "dk_pos", "dv"):
        assert torch.count_nonzero(rev[name][:, :, :64]).item() == 0, name
    for name in ("dq_rot", "dq_pos"):
        assert torch.count_nonzero(rev[name][:, :, 128:]).item() == 0, name
    assert torch.count_nonzero(rev["dbeta"][:, :, 0]).item() == 0
    assert torch.count_nonzero(rev["ddecay"][:, :, 0]).item() == 0
    fwd = _run(inp, False)
    assert torch.count_nonzero(fwd["ddecay"][:, :, 0]).item() == 0
    again = _run(inp, False)
    for name in OUT:
        assert torch.equal(fwd[name], again[name]), name


@pytest.mark.parametrize("reverse", [False, True])
def test_bigdn_dir_bwd_video_shape_sampled(reverse):
    """B1 F16 S1024 H16 D128 (the video block's shape): every gradient finite, three heads
    against the oracle element by element."""
    inp = workloads.bigdn_bwd_inputs(1, 16, 1024, 16, 128, seed=33 + int(reverse))
    say("video-shape bigdn_dir_bwd reverse %s" % reverse)
    _check(inp, reverse, heads=[0, 9, 15])


@pytest.mark.parametrize("D", [64, 128])
def test_bigdn_dir_bwd_reused_statistics(D):
    """The reverse call with the forward call's frame statistics (GDN_BWD_REUSE_STATS) equals
    a call that forms them itself, bit for bit."""
    import gated_delta_rule_29_amd as g

    inp = workloads.bigdn_bwd_inputs(1, 3, 64, 2, D, seed=11 + D)
    d = {k: inp[k].to(DEV) for k in IN}
    B, H, N, D_ = d["q_rot"].shape
    ws = torch.empty(g._lib.load().bigdn_dir_bwd_workspace_bytes(B, H, D, 3), dtype=torch.uint8,
                     device=DEV)
    g.bigdn_dir_bwd(*(d[k] for k in IN), reverse=False, workspace=ws)
    reused = g.bigdn_dir_bwd(*(d[k] for k in IN), reverse=True, workspace=ws, reuse_stats=True)
    fresh = g.bigdn_dir_bwd(*(d[k] for k in IN), reverse=True)
    torch.cuda.synchronize()
    for name in OUT:
        assert torch.equal(reused[name], fresh[name]), name

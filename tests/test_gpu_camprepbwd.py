"""GPU parity of the camera-branch prep backward (cam_prep_bwd) against the fp64 oracle,
through the C ABI.

Every input is fp32 and reaches both sides exactly; the GPU path is fp32 arithmetic
throughout, so the results are held to the fp32 rule (1e-4 of RMS).  The oracle takes one
upstream gradient per output, so the directions are summed (in fp64) before the call."""
import numpy as np
import pytest
import torch

import oracle
import workloads
from tests.gpu_util import SPLIT_OPERAND_TOL, TOL, assert_close, say

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
FP32 = TOL[torch.float32]
PARAMS = ("q_norm_w", "k_norm_w", "proj_q", "proj_kv", "rope_cos", "rope_sin")
OUTS = ("dq", "dk", "dv", "dq_norm_w", "dk_norm_w")


def _gpu(inp, ndir):
    import gated_delta_rule_29_amd as g

    d = {k: (v.to(DEV) if isinstance(v, torch.Tensor) else v) for k, v in inp.items()}
    sq = (lambda t: t[0]) if ndir == 1 else (lambda t: t)
    out = g.cam_prep_bwd(d["q"], d["k"], *(d[k] for k in PARAMS), d["k_scale"], sq(d["dq_t"]),
                         sq(d["dk_t"]), sq(d["dv_t"]), d["dinfl"], d["eps"])
    torch.cuda.synchronize()
    return out


def _ref(inp):
    s = lambda t: t.double().sum(dim=0).numpy()
    return oracle.cam_prep_bwd(inp["q"], inp["k"], *(inp[k] for k in PARAMS), inp["k_scale"],
                               s(inp["dq_t"]), s(inp["dk_t"]), s(inp["dv_t"]), inp["dinfl"],
                               inp["eps"])


def _check(inp, ndir):
    out = _gpu(inp, ndir)
    ref = _ref(inp)
    for name in OUTS:
        assert bool(torch.isfinite(out[name]).all()), name
        assert_close(name, out[name], ref[name], FP32)
    return out


@pytest.mark.parametrize("H,D,F,S,ndir,infl", [
    (2, 64, 2, 64, 1, False), (2, 64, 2, 64, 1, True), (3, 128, 3, 36, 2, True),
    (4, 128, 1, 196, 2, False), (32, 128, 1, 100, 2, True), (48, 64, 2, 20, 1, True)])
def test_cam_prep_bwd(H, D, F, S, ndir, infl):
    """D 64 and 128, 128 to 4096 channels (one and two strips), ragged last token tiles
    (N = 72, 108, 196, 100, 40), one and two directions, with and without the inflation
    gradient."""
    say("cam_prep_bwd H%d D%d F%d S%d ndir %d infl %s" % (H, D, F, S, ndir, infl))
    inp = workloads.cam_prep_bwd_inputs(1, F, S, H, D, ndir=ndir, infl=infl, seed=H + D + S)
    _check(inp, ndir)


def test_cam_prep_bwd_batches_and_token_groups():
    """Two batches of 600 tokens: more tokens than the RMSNorm backward's token groups (1024),
    with a ragged last group."""
    say("cam_prep_bwd B2 N600")
    _check(workloads.cam_prep_bwd_inputs(2, 6, 100, 2, 64, ndir=2, seed=5), 2)


def test_cam_prep_bwd_video_shape_and_determinism():
    """The video block's shape (B1 F16 S1024 H16 D128), both directions and the inflation
    gradient, every element; two calls give bitwise-identical results."""
    say("cam_prep_bwd video shape")
    inp = workloads.cam_prep_bwd_inputs(1, 16, 1024, 16, 128, ndir=2, seed=3)
    a = _check(inp, 2)
    b = _gpu(inp, 2)
    for name in a:
        assert torch.equal(a[name], b[name]), name


def _branch(inp, dout_f, dout_r, decay_bwd=None):
    import gated_delta_rule_29_amd as g

    d = {k: (v.to(DEV) if isinstance(v, torch.Tensor) else v) for k, v in inp.items()}
    db = None if decay_bwd is None else decay_bwd.to(DEV)
    out = g.cam_bwd(d["q"], d["k"], d["v"], *(d[k] for k in PARAMS), d["k_scale"], d["beta"],
                    d["decay"], dout_f.to(DEV), dout_r.to(DEV), d["dinfl"], d["eps"],
                    decay_bwd=db)
    qt, kt, vt, _ = g.cam_prep(d["q"], d["k"], d["v"], *(d[k] for k in PARAMS), d["k_scale"],
                               d["eps"])
    torch.cuda.synchronize()
    return out, (qt.cpu(), kt.cpu(), vt.cpu())


@pytest.mark.parametrize("D,F,S,sep", [(64, 3, 64, False), (128, 2, 128, False),
                                       (64, 4, 64, True)])
def test_cam_branch_bwd(D, F, S, sep):
    """The camera branch's backward (cam_bwd: cam_prep, both scan directions' backward with
    the reverse call accumulating dbeta and ddecay, cam_prep_bwd over both directions) against
    the oracle's pieces composed on the GPU path's fp32 prepped tensors.  The scan backward
    takes split bf16 operands, so the split-operand rule applies."""
    say("cam_bwd D%d F%d S%d decay_bwd %s" % (D, F, S, sep))
    inp = workloads.cam_prep_bwd_inputs(1, F, S, 2, D, ndir=2, seed=D + F + int(sep))
    dout_f, dout_r = inp["dq_t"][0], inp["dq_t"][1]  # any N(0, 1) [B,H,D,N] pair
    decay_bwd = None
    if sep:
        decay_bwd = inp["decay"].clone() * 0.9
        decay_bwd[:, :, 1::2] = 0.0
    out, t = _branch(inp, dout_f, dout_r, decay_bwd)
    fwd = oracle.cam_scan_bwd(*t, inp["beta"], inp["decay"], dout_f, reverse=False)
    rev = oracle.cam_scan_bwd(*t, inp["beta"], inp["decay"] if decay_bwd is None else decay_bwd,
                              dout_r, reverse=True)
    ref = oracle.cam_prep_bwd(inp["q"], inp["k"], *(inp[k] for k in PARAMS), inp["k_scale"],
                              fwd["dq"] + rev["dq"], fwd["dk"] + rev["dk"], fwd["dv"] + rev["dv"],
                              inp["dinfl"], inp["eps"])
    ref["dbeta"] = fwd["dbeta"] + rev["dbeta"]
    if sep:
        ref["ddecay"], ref["ddecay_bwd"] = fwd["ddecay"], rev["ddecay"]
    else:
        ref["ddecay"] = fwd["ddecay"] + rev["ddecay"]
    assert set(out) == set(ref)
    for name in ref:
        assert bool(torch.isfinite(out[name]).all()), name
        assert_close(name, out[name], ref[name], SPLIT_OPERAND_TOL)

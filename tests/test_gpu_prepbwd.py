"""GPU parity of the BiGDN front-end backward (gdn_prep_bwd), the merge backward
(bigdn_merge_bwd) and the whole block's backward (bigdn_bwd: front end, merge, both scan
directions) against the fp64 oracle, through the C ABI.

The front end and merge backward are fp32 arithmetic on inputs that both sides see exactly
(bf16 qkv, num, den, gate; fp32 gradients), so they are held to the fp32 rule (1e-4 of RMS).
The whole block composes them with the scan backward, whose products take split bf16
operands: the split-operand rule (SPLIT_OPERAND_TOL) there, with the oracle fed the same bf16
prepped tensors and num / den sums the GPU path works from."""
import numpy as np
import pytest
import torch

import oracle
import workloads
from tests.gpu_util import SPLIT_OPERAND_TOL, TOL, assert_close, say

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
FP32 = TOL[torch.float32]
NAMES = ("dq_rot", "dk_rot", "dq_pos", "dk_pos", "dv")
PREP = ("q_norm_w", "k_norm_w", "rope_cos", "rope_sin")


def _prep_bwd(inp):
    import gated_delta_rule_29_amd as g

    d = {k: inp[k].to(DEV) for k in ("qkv",) + PREP}
    grads = {n: inp["grads"][n].to(DEV) for n in NAMES}
    out = g.gdn_prep_bwd(d["qkv"], *(d[k] for k in PREP), inp["k_scale"], grads, inp["eps"])
    torch.cuda.synchronize()
    return out


def _check_prep(inp):
    out = _prep_bwd(inp)
    ref = oracle.prep_bwd(inp["qkv"], inp["q_norm_w"], inp["k_norm_w"], inp["rope_cos"],
                          inp["rope_sin"], inp["k_scale"], inp["grads"], inp["eps"])
    for name in ("dqkv", "dq_norm_w", "dk_norm_w"):
        assert bool(torch.isfinite(out[name]).all()), name
        assert_close(name, out[name], ref[name], FP32)
    return out


@pytest.mark.parametrize("H,D,ndir", [(2, 64, 1), (3, 128, 2), (16, 128, 2), (32, 128, 1)])
def test_prep_bwd_channels(H, D, ndir):
    """C = H*D from 128 to 4096 channels (two 2048-channel strips), one and two directions."""
    say("gdn_prep_bwd H%d D%d ndir %d" % (H, D, ndir))
    _check_prep(workloads.prep_bwd_inputs(1, 2, 64, H, D, ndir=ndir, seed=H + D + ndir))


def test_prep_bwd_token_groups():
    """More tokens than token groups (1024), with a ragged last group: 2 x 750 tokens."""
    say("gdn_prep_bwd B2 N750")
    inp = workloads.prep_bwd_inputs(2, 5, 150, 2, 64, ndir=2, seed=7)
    _check_prep(inp)


def test_prep_bwd_video_shape_and_determinism():
    """The video block's shape (B1 F16 S1024 H16 D128), both directions, every element; two
    calls give bitwise-identical results (the weight gradients are summed in a fixed order)."""
    say("gdn_prep_bwd video shape")
    inp = workloads.prep_bwd_inputs(1, 16, 1024, 16, 128, ndir=2, seed=3)
    a = _check_prep(inp)
    b = _prep_bwd(inp)
    for name in a:
        assert torch.equal(a[name], b[name]), name


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("gated", [False, True])
def test_merge_bwd(D, gated):
    import gated_delta_rule_29_amd as g

    say("bigdn_merge_bwd D%d gated %s" % (D, gated))
    inp = workloads.merge_bwd_inputs(2, 96, 3, D, gated=gated, seed=D + int(gated))
    d = {k: (None if v is None else v.to(DEV)) for k, v in inp.items()}
    out = g.bigdn_merge_bwd(d["num"], d["den"], d["dout"], d["gate"], 1e-6)
    torch.cuda.synchronize()
    ref = oracle.bigdn_merge_bwd(inp["num"], inp["den"], inp["dout"], inp["gate"], 1e-6)
    for name in ("dnum", "dden", "dgate"):
        if ref[name] is None:
            assert out[name] is None
            continue
        assert bool(torch.isfinite(out[name]).all()), name
        assert_close(name, out[name], ref[name], FP32)


def _block(inp, beta_bwd=None, decay_bwd=None):
    import gated_delta_rule_29_amd as g

    d = {k: (v.to(DEV) if isinstance(v, torch.Tensor) else v) for k, v in inp.items()}
    bb = None if beta_bwd is None else beta_bwd.to(DEV)
    db = None if decay_bwd is None else decay_bwd.to(DEV)
    args = (d["qkv"], d["beta"], d["decay"]) + tuple(d[k] for k in PREP) + (d["k_scale"],)
    _, num, den = g.bigdn_fwd_merged(*args, d["eps"], gate=d["gate"], beta_bwd=bb, decay_bwd=db,
                                     want_num_den=True)
    out = g.bigdn_bwd(*args, num, den, d["dout"], d["gate"], 1e-6, d["eps"], beta_bwd=bb,
                      decay_bwd=db)
    p = g.gdn_prep(d["qkv"], *(d[k] for k in PREP), d["k_scale"], d["eps"],
                   outputs=("q_rot", "k_rot", "q_pos", "k_pos", "v"))
    torch.cuda.synchronize()
    return out, num, den, p


def _block_ref(inp, num, den, p, beta_bwd=None, decay_bwd=None):
    """The oracle's backward pieces, composed, on the GPU path's bf16 prepped tensors and
    num / den sums."""
    t = [p[k] for k in ("q_rot", "k_rot", "q_pos", "k_pos", "v")]
    m = oracle.bigdn_merge_bwd(num, den, inp["dout"], inp["gate"], 1e-6)
    fwd = oracle.bigdn_dir_bwd(*t, inp["beta"], inp["decay"], m["dnum"], m["dden"], reverse=False)
    rev = oracle.bigdn_dir_bwd(*t, inp["beta"] if beta_bwd is None else beta_bwd,
                               inp["decay"] if decay_bwd is None else decay_bwd, m["dnum"],
                               m["dden"], reverse=True)
    grads = {n: np.stack([fwd[n], rev[n]]) for n in NAMES}
    g = oracle.prep_bwd(inp["qkv"], inp["q_norm_w"], inp["k_norm_w"], inp["rope_cos"],
                        inp["rope_sin"], inp["k_scale"], grads, inp["eps"])
    ref = dict(g, dgate=m["dgate"])
    if beta_bwd is None and decay_bwd is None:
        ref["dbeta"], ref["ddecay"] = fwd["dbeta"] + rev["dbeta"], fwd["ddecay"] + rev["ddecay"]
    else:
        ref["dbeta"], ref["ddecay"] = fwd["dbeta"], fwd["ddecay"]
        ref["dbeta_bwd"], ref["ddecay_bwd"] = rev["dbeta"], rev["ddecay"]
    return ref


@pytest.mark.parametrize("D,F,S", [(64, 3, 64), (128, 2, 128)])
def test_block_bwd(D, F, S):
    say("bigdn_bwd D%d F%d S%d" % (D, F, S))
    inp = workloads.bigdn_block_bwd_inputs(1, F, S, 2, D, seed=D + F)
    out, num, den, p = _block(inp)
    ref = _block_ref(inp, num, den, p)
    for name in ("dqkv", "dq_norm_w", "dk_norm_w", "dbeta", "ddecay", "dgate"):
        assert bool(torch.isfinite(out[name]).all()), name
        assert_close(name, out[name], ref[name], SPLIT_OPERAND_TOL)


def test_block_bwd_chunk_causal_overrides():
    """Reverse-direction beta / decay overrides (zero decay at every second frame): the
    parameter gradients of the two directions come back separately."""
    say("bigdn_bwd with beta_bwd / decay_bwd")
    inp = workloads.bigdn_block_bwd_inputs(1, 4, 64, 2, 64, seed=13)
    beta_bwd = inp["beta"] * 0.5
    decay_bwd = inp["decay"].clone()
    decay_bwd[:, :, 1::2] = 0.0
    out, num, den, p = _block(inp, beta_bwd, decay_bwd)
    ref = _block_ref(inp, num, den, p, beta_bwd, decay_bwd)
    for name in ("dqkv", "dq_norm_w", "dk_norm_w", "dbeta", "ddecay", "dbeta_bwd", "ddecay_bwd",
                 "dgate"):
        assert bool(torch.isfinite(out[name]).all()), name
        assert_close(name, out[name], ref[name], SPLIT_OPERAND_TOL)

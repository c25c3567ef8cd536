"""GPU parity of gdn_prep and bigdn_fwd against the fp64 oracle, through the C ABI."""
import numpy as np
import pytest
import torch

import oracle
import workloads
from tests.gpu_util import assert_close, say

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _dev(w):
    return {k: (v.to(DEV) if isinstance(v, torch.Tensor) else v) for k, v in w.items()}


@pytest.mark.parametrize("B,N,H,D", [(2, 100, 3, 64), (1, 16384, 16, 128)])
def test_prep(B, N, H, D):
    """Every element: fp32 arithmetic then one rounding, so within 1e-4*RMS of the oracle
    under the bf16 storage rule; inverse RMS (fp32 out) within 1e-4*RMS."""
    import gated_delta_rule_29_amd as g

    w = workloads.bigdn_inputs(B, N // 64 if N % 64 == 0 else 1, 64 if N % 64 == 0 else N, H, D,
                               seed=B + H)
    say("prep B%d N%d H%d D%d" % (B, N, H, D))
    d = _dev(w)
    out = g.gdn_prep(d["qkv"], d["q_norm_w"], d["k_norm_w"], d["rope_cos"], d["rope_sin"],
                     w["k_scale"], w["eps"])
    torch.cuda.synchronize()
    ref = oracle.prep(w["qkv"], w["q_norm_w"], w["k_norm_w"], w["rope_cos"], w["rope_sin"],
                      w["k_scale"], w["eps"])
    for name in ("q_inv_rms", "k_inv_rms", "q_rot", "k_rot", "q_pos", "k_pos", "v"):
        assert_close(name, out[name], ref[name], 1e-4)


@pytest.mark.parametrize("B,F,S,H,D", [(1, 3, 64, 2, 64), (2, 5, 128, 3, 128), (1, 1, 64, 2, 128),
                                          (1, 2, 64, 1, 64), (1, 7, 64, 2, 128)])
def test_bigdn_small(B, F, S, H, D):
    import gated_delta_rule_29_amd as g

    w = workloads.bigdn_inputs(B, F, S, H, D, seed=F * S)
    say("bigdn B%d F%d S%d H%d D%d" % (B, F, S, H, D))
    d = _dev(w)
    num, den = g.bigdn_fwd(d["qkv"], d["beta"], d["decay"], d["q_norm_w"], d["k_norm_w"],
                           d["rope_cos"], d["rope_sin"], w["k_scale"], w["eps"])
    torch.cuda.synchronize()
    rn, rd = oracle.bigdn(w["qkv"], w["beta"], w["decay"], w["q_norm_w"], w["k_norm_w"],
                          w["rope_cos"], w["rope_sin"], w["k_scale"], w["eps"])
    assert_close("num", num, rn, 2e-2)
    assert_close("den", den, rd, 2e-2)


def test_bigdn_beta_zero_exact():
    import gated_delta_rule_29_amd as g

    w = workloads.bigdn_inputs(1, 4, 64, 2, 128, seed=5)
    d = _dev(w)
    num, den = g.bigdn_fwd(d["qkv"], torch.zeros_like(d["beta"]), d["decay"], d["q_norm_w"],
                           d["k_norm_w"], d["rope_cos"], d["rope_sin"], w["k_scale"], w["eps"])
    torch.cuda.synchronize()
    assert torch.count_nonzero(num).item() == 0 and torch.count_nonzero(den).item() == 0


def test_bigdn_video_workload():
    """qkv [1, 16 frames x 1024 tokens, 3, 16, 128] (the video-block workload): every element
    of num and den."""
    import gated_delta_rule_29_amd as g

    w = workloads.make("bigdn_video_f16x1024")
    say("bigdn video workload")
    d = _dev(w)
    num, den = g.bigdn_fwd(d["qkv"], d["beta"], d["decay"], d["q_norm_w"], d["k_norm_w"],
                           d["rope_cos"], d["rope_sin"], w["k_scale"], w["eps"])
    a, b = g.bigdn_fwd(d["qkv"], d["beta"], d["decay"], d["q_norm_w"], d["k_norm_w"],
                       d["rope_cos"], d["rope_sin"], w["k_scale"], w["eps"])
    torch.cuda.synchronize()
    assert torch.equal(num, a) and torch.equal(den, b), "not deterministic"
    rn, rd = oracle.bigdn(w["qkv"], w["beta"], w["decay"], w["q_norm_w"], w["k_norm_w"],
                          w["rope_cos"], w["rope_sin"], w["k_scale"], w["eps"])
    assert_close("num", num, rn, 2e-2)
    assert_close("den", den, rd, 2e-2)


@pytest.mark.parametrize("B,F,S,H,D,gated,override", [(1, 5, 128, 2, 128, True, 1),
                                                        (2, 3, 64, 3, 64, False, 1),
                                                        (1, 4, 64, 2, 128, True, 0),
                                                        (1, 1, 64, 1, 64, True, 1),
                                                        (1, 3, 128, 2, 128, True, 2),
                                                        (2, 2, 64, 3, 64, False, 2)])
def test_bigdn_merged(B, F, S, H, D, gated, override):
    """bigdn_fwd_merged: reverse-direction overrides (override 1: beta / decay with a zero
    reverse decay at one frame, chunk-causal; 2: also the reverse direction's own q, k, v, its k
    and v zero at that frame) and the fused merge epilogue, against the oracle's block."""
    import gated_delta_rule_29_amd as g

    w = workloads.bigdn_inputs(B, F, S, H, D, seed=F * S + H)
    gen = torch.Generator().manual_seed(F + D)
    N = F * S
    gate = torch.randn(B, N, H, D, generator=gen).to(torch.bfloat16) if gated else None
    bb = db = qb = None
    if override:
        bb = torch.sigmoid(torch.randn(B, H, F, S, generator=gen))
        db = w["decay"].clone()
        db[:, :, F // 2] = 0.0
    if override == 2:
        qb = workloads.bigdn_inputs(B, F, S, H, D, seed=F * S + H + 1)["qkv"].clone()
        qb[:, (F // 2) * S:(F // 2 + 1) * S, 1:] = 0
    say("bigdn merged B%d F%d S%d H%d D%d gate%d override%d" % (B, F, S, H, D, gated, override))
    d = _dev(w)
    out, num, den = g.bigdn_fwd_merged(
        d["qkv"], d["beta"], d["decay"], d["q_norm_w"], d["k_norm_w"], d["rope_cos"],
        d["rope_sin"], w["k_scale"], w["eps"], qkv_bwd=None if qb is None else qb.to(DEV),
        beta_bwd=None if bb is None else bb.to(DEV),
        decay_bwd=None if db is None else db.to(DEV), gate=None if gate is None else gate.to(DEV),
        merge_eps=1e-6, want_num_den=True)
    torch.cuda.synchronize()
    ro, rn, rd = oracle.bigdn_merged(w["qkv"], w["beta"], w["decay"], w["q_norm_w"],
                                     w["k_norm_w"], w["rope_cos"], w["rope_sin"], w["k_scale"],
                                     w["eps"], beta_bwd=bb, decay_bwd=db, gate=gate,
                                     merge_eps=1e-6, qkv_bwd=qb)
    assert_close("num", num, rn, 2e-2)
    assert_close("den", den, rd, 2e-2)
    assert_close("out", out, ro, 2e-2)
    out_only = g.bigdn_fwd_merged(
        d["qkv"], d["beta"], d["decay"], d["q_norm_w"], d["k_norm_w"], d["rope_cos"],
        d["rope_sin"], w["k_scale"], w["eps"], qkv_bwd=None if qb is None else qb.to(DEV),
        beta_bwd=None if bb is None else bb.to(DEV),
        decay_bwd=None if db is None else db.to(DEV), gate=None if gate is None else gate.to(DEV),
        merge_eps=1e-6)
    torch.cuda.synchronize()
    assert torch.equal(out_only, out)


def test_bigdn_video_merged_workload():
    """The merged video-block workload (chunk-causal reverse decay, SiLU gate): every element
    of out."""
    import gated_delta_rule_29_amd as g

    w = workloads.make("bigdn_video_merged_f16x1024")
    say("bigdn video merged workload")
    d = _dev(w)
    out = g.bigdn_fwd_merged(d["qkv"], d["beta"], d["decay"], d["q_norm_w"], d["k_norm_w"],
                             d["rope_cos"], d["rope_sin"], w["k_scale"], w["eps"],
                             decay_bwd=d["decay_bwd"], gate=d["gate"], merge_eps=1e-6)
    torch.cuda.synchronize()
    ro, _, _ = oracle.bigdn_merged(w["qkv"], w["beta"], w["decay"], w["q_norm_w"],
                                   w["k_norm_w"], w["rope_cos"], w["rope_sin"], w["k_scale"],
                                   w["eps"], decay_bwd=w["decay_bwd"], gate=w["gate"],
                                   merge_eps=1e-6)
    assert_close("out", out, ro, 2e-2)

"""GPU parity of the camera branch (cam_prep, cam_scan) against the fp64 oracle, through the
C ABI."""
import numpy as np
import pytest
import torch

import oracle
import workloads
from tests.gpu_util import FP16_OPERAND_TOL, assert_close, say

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _dev(w):
    return {k: (v.to(DEV) if isinstance(v, torch.Tensor) else v) for k, v in w.items()}


def _prep_args(w):
    return (w["q"], w["k"], w["v"], w["q_norm_w"], w["k_norm_w"], w["proj_q"], w["proj_kv"],
            w["rope_cos"], w["rope_sin"], w["k_scale"], w["eps"])


@pytest.mark.parametrize("B,F,S,H,D", [(2, 1, 200, 3, 64), (1, 3, 44, 2, 128), (1, 1, 4, 1, 64),
                                          (1, 2, 64, 16, 128)])
def test_cam_prep(B, F, S, H, D):
    """Every element of q_t, k_t, v_t and inflation: fp32 arithmetic, 1e-4 * RMS.  N = 200 and
    132 leave a ragged last 64-token tile; N = 4 is a single quad."""
    import gated_delta_rule_29_amd as g

    w = workloads.cam_inputs(B, F, S, H, D, seed=B + H + D)
    say("cam prep B%d N%d H%d D%d" % (B, F * S, H, D))
    d = _dev(w)
    got = g.cam_prep(*_prep_args(d))
    torch.cuda.synchronize()
    ref = oracle.cam_prep(*_prep_args(w))
    for name, x, r in zip(("q_t", "k_t", "v_t", "inflation"), got, ref):
        assert_close(name, x, r, 1e-4)


@pytest.mark.parametrize("B,F,S,H,D,reverse", [(1, 5, 128, 2, 128, False),
                                                (1, 5, 128, 2, 128, True),
                                                (2, 3, 64, 3, 64, False),
                                                (2, 3, 64, 3, 64, True),
                                                (1, 1, 64, 1, 128, False),
                                                (1, 1, 64, 1, 128, True),
                                                (1, 9, 64, 8, 64, False)])
def test_cam_scan(B, F, S, H, D, reverse):
    """Every output element, both directions, against the oracle's frame recurrence."""
    import gated_delta_rule_29_amd as g

    w = workloads.cam_scan_inputs(B, F, S, H, D, seed=F * S + H + int(reverse))
    say("cam scan B%d F%d S%d H%d D%d reverse%d" % (B, F, S, H, D, reverse))
    d = _dev(w)
    out = g.cam_scan(d["q"], d["k"], d["v"], d["beta"], d["decay"], reverse=reverse)
    torch.cuda.synchronize()
    ref = oracle.cam_scan(w["q"], w["k"], w["v"], w["beta"], w["decay"], reverse=reverse)
    assert_close("out", out, ref, FP16_OPERAND_TOL)
    if reverse:  # the last frame reads the zero state
        assert torch.count_nonzero(out[..., (F - 1) * S:]).item() == 0


@pytest.mark.parametrize("D", [64, 128])
def test_cam_scan_state_io(D):
    """init_state and final_state against the oracle; a scan split after two frames and
    resumed from its final state reproduces the whole scan bit for bit (the state crosses
    the split in fp32)."""
    import gated_delta_rule_29_amd as g

    B, F, S, H = 1, 5, 64, 2
    w = workloads.cam_scan_inputs(B, F, S, H, D, seed=D)
    h0 = 0.3 * torch.randn(B * H, D, D, generator=torch.Generator().manual_seed(D))
    say("cam scan state io D%d" % D)
    d = _dev(w)
    out, fin = g.cam_scan(d["q"], d["k"], d["v"], d["beta"], d["decay"],
                          init_state=h0.to(DEV), save_final_state=True)
    torch.cuda.synchronize()
    ro, rf = oracle.cam_scan(w["q"], w["k"], w["v"], w["beta"], w["decay"], init_state=h0,
                             want_final=True)
    assert_close("out", out, ro, FP16_OPERAND_TOL)
    assert_close("final", fin, rf, FP16_OPERAND_TOL)
    c = 2
    cut = lambda x, a, b: x[..., a * S:b * S].contiguous()
    o1, f1 = g.cam_scan(cut(d["q"], 0, c), cut(d["k"], 0, c), cut(d["v"], 0, c),
                        d["beta"][:, :, :c].contiguous(), d["decay"][:, :, :c].contiguous(),
                        init_state=h0.to(DEV), save_final_state=True)
    o2, f2 = g.cam_scan(cut(d["q"], c, F), cut(d["k"], c, F), cut(d["v"], c, F),
                        d["beta"][:, :, c:].contiguous(), d["decay"][:, :, c:].contiguous(),
                        init_state=f1, save_final_state=True)
    torch.cuda.synchronize()
    assert torch.equal(torch.cat([o1, o2], dim=-1), out)
    assert torch.equal(f2, fin)


def test_cam_scan_reverse_rejects_state():
    import gated_delta_rule_29_amd as g

    w = _dev(workloads.cam_scan_inputs(1, 2, 64, 1, 64))
    with pytest.raises(NotImplementedError):
        g.cam_scan(w["q"], w["k"], w["v"], w["beta"], w["decay"], reverse=True,
                   save_final_state=True)


def test_cam_video_workload():
    """The camera branch of the 16-frame video block (B1 F16 S1024 H16 D128): prep of every
    token, then both scan directions; every prep output, and the scans on heads 0 and 11."""
    import gated_delta_rule_29_amd as g

    w = workloads.make("cam_video_f16x1024")
    say("cam video workload")
    d = _dev(w)
    qt, kt, vt, infl = g.cam_prep(*_prep_args(d))
    fwd = g.cam_scan(qt, kt, vt, d["beta"], d["decay"])
    rev = g.cam_scan(qt, kt, vt, d["beta"], d["decay"], reverse=True)
    torch.cuda.synchronize()
    rq, rk, rv, ri = oracle.cam_prep(*_prep_args(w))
    for name, x, r in (("q_t", qt, rq), ("k_t", kt, rk), ("v_t", vt, rv), ("inflation", infl, ri)):
        assert_close(name, x, r, 1e-4)
    for h in (0, 11):
        sl = slice(h, h + 1)
        args = (rq[:, sl], rk[:, sl], rv[:, sl], w["beta"][:, sl], w["decay"][:, sl])
        assert_close("fwd h%d" % h, fwd[:, sl], oracle.cam_scan(*args), FP16_OPERAND_TOL)
        assert_close("rev h%d" % h, rev[:, sl], oracle.cam_scan(*args, reverse=True),
                     FP16_OPERAND_TOL)


@pytest.mark.parametrize("B,F,S,H,D", [(1, 6, 128, 2, 128), (2, 3, 64, 3, 64)])
def test_cam_scan_bidi(B, F, S, H, D):
    """Both directions in one call: against the oracle (the reverse with its own decay, zero
    at one frame: chunk-causal), and bit for bit equal to the two single-direction calls."""
    import gated_delta_rule_29_amd as g

    w = workloads.cam_scan_inputs(B, F, S, H, D, seed=3 * F + D)
    db = w["decay"].clone()
    db[:, :, F // 2] = 0.0
    h0 = 0.3 * torch.randn(B * H, D, D, generator=torch.Generator().manual_seed(F))
    say("cam scan bidi B%d F%d S%d H%d D%d" % (B, F, S, H, D))
    d = _dev(w)
    of, orv, fin = g.cam_scan_bidi(d["q"], d["k"], d["v"], d["beta"], d["decay"],
                                   decay_bwd=db.to(DEV), init_state=h0.to(DEV),
                                   save_final_state=True)
    sf, sfin = g.cam_scan(d["q"], d["k"], d["v"], d["beta"], d["decay"], init_state=h0.to(DEV),
                          save_final_state=True)
    sr = g.cam_scan(d["q"], d["k"], d["v"], d["beta"], db.to(DEV), reverse=True)
    torch.cuda.synchronize()
    rf, rfin = oracle.cam_scan(w["q"], w["k"], w["v"], w["beta"], w["decay"], init_state=h0,
                               want_final=True)
    rr = oracle.cam_scan(w["q"], w["k"], w["v"], w["beta"], db, reverse=True)
    assert_close("fwd", of, rf, FP16_OPERAND_TOL)
    assert_close("final", fin, rfin, FP16_OPERAND_TOL)
    assert_close("rev", orv, rr, FP16_OPERAND_TOL)
    assert torch.equal(of, sf) and torch.equal(orv, sr) and torch.equal(fin, sfin)


def test_cam_deterministic():
    """Two identical calls give bitwise-identical outputs (no atomics anywhere)."""
    import gated_delta_rule_29_amd as g

    w = _dev(workloads.cam_inputs(1, 4, 128, 4, 128, seed=7))
    a = g.cam_prep(*_prep_args(w))
    b = g.cam_prep(*_prep_args(w))
    ra = g.cam_scan_bidi(a[0], a[1], a[2], w["beta"], w["decay"])
    rb = g.cam_scan_bidi(b[0], b[1], b[2], w["beta"], w["decay"])
    torch.cuda.synchronize()
    for x, y in zip(a + ra, b + rb):
        assert torch.equal(x, y)

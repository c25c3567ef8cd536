"""Pins of the BiGDN direction backward oracle (oracle.bigdn_dir_bwd), CPU only.

Every gradient element is checked against central differences of the forward oracle
(oracle.bigdn_dir, separate code) for L = sum(num * dnum) + sum(den * dden): the forward is
smooth in every input, so (L(x + e) - L(x - e)) / 2e matches the analytic gradient to about
e^2.  Structural zeros of the reverse direction (frame 0 is never absorbed; the last frame is
emitted from the zero state) and of the forward one (the first decay multiplies the zero
state) are pinned exactly.
"""
import numpy as np
import pytest

import oracle

NAMES = ("q_rot", "k_rot", "q_pos", "k_pos", "v", "beta", "decay")


def _inputs(B, H, D, F, S, seed):
    rng = np.random.default_rng(seed)
    N = F * S
    x = dict(q_rot=rng.normal(0, 0.7, (B, H, N, D)), k_rot=rng.normal(0, 0.5, (B, H, N, D)),
             q_pos=np.abs(rng.normal(0, 0.7, (B, H, N, D))),
             k_pos=np.abs(rng.normal(0, 0.4, (B, H, N, D))), v=rng.normal(0, 1.0, (B, H, N, D)),
             beta=rng.uniform(0.2, 0.9, (B, H, F, S)), decay=rng.uniform(0.4, 1.0, (B, H, F)))
    x["dnum"] = rng.normal(0, 1.0, (B, N, H, D))
    x["dden"] = rng.normal(0, 1.0, (B, H, N))
    return x


def _loss(x, reverse):
    num, den = oracle.bigdn_dir(*(x[n] for n in NAMES), reverse=reverse)
    return float((num * x["dnum"]).sum() + (den * x["dden"]).sum())


@pytest.mark.parametrize("reverse", [False, True])
def test_every_gradient_element_matches_central_differences(reverse):
    x = _inputs(1, 2, 4, 3, 2, seed=3 + int(reverse))
    g = oracle.bigdn_dir_bwd(*(x[n] for n in NAMES), x["dnum"], x["dden"], reverse=reverse)
    eps = 1e-5
    for name in NAMES:
        fd = np.zeros_like(x[name])
        for idx in np.ndindex(x[name].shape):
            xp = {k: v.copy() for k, v in x.items()}
            xm = {k: v.copy() for k, v in x.items()}
            xp[name][idx] += eps
            xm[name][idx] -= eps
            fd[idx] = (_loss(xp, reverse) - _loss(xm, reverse)) / (2 * eps)
        key = "d" + name
        np.testing.assert_allclose(g[key], fd, rtol=1e-6, atol=1e-8, err_msg=key)


def test_structural_zeros():
    x = _inputs(1, 2, 4, 3, 2, seed=9)
    F, S = 3, 2
    rev = oracle.bigdn_dir_bwd(*(x[n] for n in NAMES), x["dnum"], x["dden"], reverse=True)
    for name in ("dk_rot", "dk_pos", "dv"):
        assert np.all(rev[name][:, :, :S] == 0.0), name          # frame 0 never absorbed
    assert np.all(rev["dbeta"][:, :, 0] == 0.0)
    assert np.all(rev["ddecay"][:, :, 0] == 0.0)
    for name in ("dq_rot", "dq_pos"):
        assert np.all(rev[name][:, :, (F - 1) * S:] == 0.0), name  # emitted from zero
    fwd = oracle.bigdn_dir_bwd(*(x[n] for n in NAMES), x["dnum"], x["dden"], reverse=False)
    assert np.all(fwd["ddecay"][:, :, 0] == 0.0)


def test_the_s_stream_is_the_camera_scan_backward():
    """Without the z stream (dden = 0, q_pos = k_pos = 0), the BiGDN direction is the camera
    scan on transposed slabs, so its gradients are oracle.cam_scan_bwd's."""
    x = _inputs(1, 2, 4, 3, 2, seed=5)
    x["dden"][:] = 0.0
    x["q_pos"][:] = 0.0
    x["k_pos"][:] = 0.0
    for reverse in (False, True):
        g = oracle.bigdn_dir_bwd(*(x[n] for n in NAMES), x["dnum"], x["dden"], reverse=reverse)
        t = lambda a: np.ascontiguousarray(np.swapaxes(a, 2, 3))   # [B,H,N,D] -> [B,H,D,N]
        dout = t(np.transpose(x["dnum"], (0, 2, 1, 3)))
        c = oracle.cam_scan_bwd(t(x["q_rot"]), t(x["k_rot"]), t(x["v"]), x["beta"], x["decay"],
                                dout, reverse=reverse)
        np.testing.assert_allclose(t(g["dq_rot"]), c["dq"], rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(t(g["dk_rot"]), c["dk"], rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(t(g["dv"]), c["dv"], rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(g["dbeta"], c["dbeta"], rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(g["ddecay"], c["ddecay"], rtol=1e-12, atol=1e-12)

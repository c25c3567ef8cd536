"""Pins of the camera-scan backward oracle (oracle.cam_scan_bwd), CPU only.

The backward is checked element by element against central differences of the forward
oracle (oracle.cam_scan, separate code): L = sum(out * dout) is smooth in every input, so
(L(x + e) - L(x - e)) / 2e matches the analytic gradient to about e^2 in fp64.  Structural
zeros from the pages' backward (frame 0 of the reverse scan is never absorbed; a decay applied
to the zero initial state has no gradient) are pinned exactly.
"""
import numpy as np
import pytest

import oracle


def _inputs(B, H, D, F, S, seed):
    rng = np.random.default_rng(seed)
    N = F * S
    return dict(q=rng.normal(0, 0.7, (B, H, D, N)), k=rng.normal(0, 0.5, (B, H, D, N)),
                v=rng.normal(0, 1.0, (B, H, D, N)), beta=rng.uniform(0.2, 0.9, (B, H, F, S)),
                decay=rng.uniform(0.4, 1.0, (B, H, F)), dout=rng.normal(0, 1.0, (B, H, D, N)))


def _loss(inp, reverse):
    out = oracle.cam_scan(inp["q"], inp["k"], inp["v"], inp["beta"], inp["decay"],
                          reverse=reverse)
    return float((out * inp["dout"]).sum())


@pytest.mark.parametrize("reverse", [False, True])
def test_every_gradient_element_matches_central_differences(reverse):
    inp = _inputs(1, 2, 4, 3, 2, seed=7 + int(reverse))
    g = oracle.cam_scan_bwd(inp["q"], inp["k"], inp["v"], inp["beta"], inp["decay"],
                            inp["dout"], reverse=reverse)
    eps = 1e-5
    for name, gname in (("q", "dq"), ("k", "dk"), ("v", "dv"), ("beta", "dbeta"),
                        ("decay", "ddecay")):
        x = inp[name]
        fd = np.empty_like(x)
        for idx in np.ndindex(x.shape):
            old = x[idx]
            x[idx] = old + eps
            lp = _loss(inp, reverse)
            x[idx] = old - eps
            lm = _loss(inp, reverse)
            x[idx] = old
            fd[idx] = (lp - lm) / (2 * eps)
        err = np.abs(fd - g[gname]).max()
        assert err <= 1e-7 * (1 + np.abs(fd).max()), (name, err)


@pytest.mark.parametrize("reverse", [False, True])
def test_larger_case_random_directions(reverse):
    """D=16, F=5, S=7 (ragged frame length), two heads: each gradient against central
    differences along random directions."""
    inp = _inputs(1, 2, 16, 5, 7, seed=21 + int(reverse))
    g = oracle.cam_scan_bwd(inp["q"], inp["k"], inp["v"], inp["beta"], inp["decay"],
                            inp["dout"], reverse=reverse)
    rng = np.random.default_rng(3)
    eps = 1e-5
    for name, gname in (("q", "dq"), ("k", "dk"), ("v", "dv"), ("beta", "dbeta"),
                        ("decay", "ddecay")):
        for _ in range(3):
            e = rng.normal(size=inp[name].shape)
            x0 = inp[name].copy()
            inp[name] = x0 + eps * e
            lp = _loss(inp, reverse)
            inp[name] = x0 - eps * e
            lm = _loss(inp, reverse)
            inp[name] = x0
            fd = (lp - lm) / (2 * eps)
            an = float((g[gname] * e).sum())
            assert abs(fd - an) <= 1e-7 * (1 + abs(an)), (name, fd, an)


def test_structural_zeros():
    inp = _inputs(1, 1, 6, 4, 3, seed=5)
    fwd = oracle.cam_scan_bwd(inp["q"], inp["k"], inp["v"], inp["beta"], inp["decay"],
                              inp["dout"], reverse=False)
    assert fwd["ddecay"][0, 0, 0] == 0.0  # decay of frame 0 multiplies the zero state
    rev = oracle.cam_scan_bwd(inp["q"], inp["k"], inp["v"], inp["beta"], inp["decay"],
                              inp["dout"], reverse=True)
    S = 3
    for name in ("dk", "dv"):
        assert np.all(rev[name][..., :S] == 0.0)  # frame 0 is never absorbed in reverse
    assert np.all(rev["dbeta"][:, :, 0] == 0.0) and rev["ddecay"][0, 0, 0] == 0.0
    # beta = 0: the states stay zero, so q, k, v have no gradient
    inp["beta"][:] = 0.0
    z = oracle.cam_scan_bwd(inp["q"], inp["k"], inp["v"], inp["beta"], inp["decay"],
                            inp["dout"], reverse=False)
    for name in ("dq", "dk", "dv", "ddecay"):
        assert np.all(z[name] == 0.0), name

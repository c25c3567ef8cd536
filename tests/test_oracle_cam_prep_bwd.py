"""Pins of the camera-branch prep backward oracle (oracle.cam_prep_bwd), CPU only.

Every gradient element (raw q, k, v and both norm weights) is checked against central
differences of the forward oracle oracle.cam_prep, which is separate code, for a loss that
weights q_t, k_t, v_t and (optionally) the inflation with random tensors.  The camera matrices
and the RoPE tables are random (not orthogonal, not a valid rotation), so a transposed 4x4 block
or a swapped sine index changes the result; every map is smooth at the drawn inputs (no
pre-ReLU value is within 1e-4 of zero, which the tests assert), so the central difference
matches the analytic gradient to about e^2.
"""
import numpy as np
import pytest

import oracle


def _inputs(B, N, H, D, seed):
    rng = np.random.default_rng(seed)
    x = dict(q=rng.normal(0, 1.0, (B, N, H, D)), k=rng.normal(0, 1.0, (B, N, H, D)),
             v=rng.normal(0, 1.0, (B, N, H, D)), qw=1.0 + 0.3 * rng.normal(0, 1.0, H * D),
             kw=1.0 + 0.3 * rng.normal(0, 1.0, H * D),
             pq=rng.normal(0, 1.0, (B, N, 4, 4)), pkv=rng.normal(0, 1.0, (B, N, 4, 4)),
             cos=rng.normal(0, 1.0, (N, D // 2)), sin=rng.normal(0, 1.0, (N, D // 2)))
    return x


def _margin(x, eps=1e-5):
    m = np.inf
    for name, w in (("q", x["qw"]), ("k", x["kw"])):
        B, N, H, D = x[name].shape
        raw = x[name].reshape(B, N, H * D)
        r = 1.0 / np.sqrt((raw * raw).mean(axis=-1, keepdims=True) + eps)
        m = min(m, float(np.abs(raw * r * w).min()))
    return m


def _fwd(x, k_scale):
    return oracle.cam_prep(x["q"], x["k"], x["v"], x["qw"], x["kw"], x["pq"], x["pkv"], x["cos"],
                           x["sin"], k_scale)


@pytest.mark.parametrize("with_infl", [False, True])
def test_cam_prep_bwd_matches_central_differences(with_infl):
    B, N, H, D, k_scale = 1, 3, 2, 8, 0.6
    x = _inputs(B, N, H, D, seed=41 + int(with_infl))
    assert _margin(x) > 1e-4
    rng = np.random.default_rng(43 + int(with_infl))
    G = [rng.normal(0, 1.0, (B, H, D, N)) for _ in range(3)]
    Gi = rng.normal(0, 1.0, (B, H, N)) if with_infl else None

    def loss(y):
        qt, kt, vt, infl = _fwd(y, k_scale)
        s = float((qt * G[0]).sum() + (kt * G[1]).sum() + (vt * G[2]).sum())
        return s + (float((infl * Gi).sum()) if with_infl else 0.0)

    g = oracle.cam_prep_bwd(x["q"], x["k"], x["qw"], x["kw"], x["pq"], x["pkv"], x["cos"],
                            x["sin"], k_scale, G[0], G[1], G[2], Gi)
    e = 1e-6
    for name, key in (("q", "dq"), ("k", "dk"), ("v", "dv"), ("qw", "dq_norm_w"),
                      ("kw", "dk_norm_w")):
        fd = np.zeros_like(x[name])
        for idx in np.ndindex(x[name].shape):
            xp = {k: v.copy() for k, v in x.items()}
            xm = {k: v.copy() for k, v in x.items()}
            xp[name][idx] += e
            xm[name][idx] -= e
            fd[idx] = (loss(xp) - loss(xm)) / (2 * e)
        np.testing.assert_allclose(g[key], fd, rtol=1e-6, atol=1e-8, err_msg=key)


def test_cam_prep_bwd_rotation_camera_inflation_gradient_vanishes():
    """A rigid-motion camera (orthogonal 3x3 block, zero translation) with a valid RoPE keeps
    |k_t| = |k|, so the inflation is 1 everywhere and its gradient adds nothing: the result
    with a random inflation gradient equals the one without."""
    B, N, H, D = 1, 4, 2, 16
    x = _inputs(B, N, H, D, seed=47)
    rng = np.random.default_rng(48)
    for b in range(B):
        for n in range(N):
            rot, _ = np.linalg.qr(rng.normal(0, 1.0, (3, 3)))
            m = np.eye(4)
            m[:3, :3] = rot
            x["pkv"][b, n] = m
    th = rng.uniform(0, 2 * np.pi, (N, D // 4))
    x["cos"] = np.repeat(np.cos(th), 2, axis=1)
    x["sin"] = np.stack([-np.sin(th), np.sin(th)], axis=-1).reshape(N, D // 2)
    _, _, _, infl = _fwd(x, 0.5)
    np.testing.assert_allclose(infl, 1.0, rtol=1e-12)
    G = [rng.normal(0, 1.0, (B, H, D, N)) for _ in range(3)]
    args = (x["q"], x["k"], x["qw"], x["kw"], x["pq"], x["pkv"], x["cos"], x["sin"], 0.5) + tuple(G)
    a = oracle.cam_prep_bwd(*args, rng.normal(0, 1.0, (B, H, N)))
    b = oracle.cam_prep_bwd(*args, None)
    for key in a:
        np.testing.assert_allclose(a[key], b[key], rtol=1e-9, atol=1e-11, err_msg=key)

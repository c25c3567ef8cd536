"""Pins of the camera-branch oracle (oracle.cam_prep, oracle.cam_scan) against facts fixed by
the SANA fused_cam_gdn.py page and by the mathematics: library routines (torch rms_norm,
complex multiplication, block-diagonal matrices), norm invariants, the token recurrence
(one token per frame), the affine product form of oracle/forms.py, flip-and-shift for the
reverse scan, and split/resume of the state.  None of them retypes the oracle's loops.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads
from oracle import forms

pytestmark = pytest.mark.filterwarnings("ignore::DeprecationWarning")


def _prep(w, **over):
    a = dict(w, **over)
    return oracle.cam_prep(a["q"], a["k"], a["v"], a["q_norm_w"], a["k_norm_w"], a["proj_q"],
                           a["proj_kv"], a["rope_cos"], a["rope_sin"], a["k_scale"], a["eps"])


def _to_bhdn(x):  # [B,N,H,D] -> [B,H,D,N]
    return np.ascontiguousarray(np.transpose(np.asarray(x, np.float64), (0, 2, 3, 1)))


def test_cam_prep_identity_camera_is_rmsnorm_relu():
    # P = I and a zero angle: the prep reduces to the full-channel RMSNorm (torch's own
    # rms_norm over all H*D channels), ReLU, k_scale on k, v untouched; inflation 1
    w = workloads.cam_inputs(2, 2, 8, 3, 16, seed=1)
    B, N, H, D = w["q"].shape
    eye = torch.eye(4).expand(B, N, 4, 4).contiguous()
    qt, kt, vt, infl = _prep(w, proj_q=eye, proj_kv=eye,
                             rope_cos=torch.ones(N, D // 2), rope_sin=torch.zeros(N, D // 2))

    def ref(x, wt):
        y = torch.nn.functional.rms_norm(x.double().reshape(B, N, H * D), (H * D,),
                                         weight=wt.double(), eps=w["eps"])
        return torch.relu(y).reshape(B, N, H, D).numpy()

    np.testing.assert_allclose(qt, _to_bhdn(ref(w["q"], w["q_norm_w"])), rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(kt, _to_bhdn(ref(w["k"], w["k_norm_w"]) * w["k_scale"]),
                               rtol=1e-12, atol=1e-16)
    np.testing.assert_array_equal(vt, _to_bhdn(w["v"].double().numpy()))
    np.testing.assert_allclose(infl, 1.0, rtol=1e-12)


def test_cam_prep_halves_are_block_projection_and_complex_rotation():
    # first half: block_diag(P, ..., P) applied to the normalised vector; second half: the
    # pairs (x[2i], x[2i+1]) as complex numbers times exp(i theta) -- the tables' sin sign
    # convention is fixed by this
    w = workloads.cam_inputs(1, 2, 4, 2, 16, seed=2)
    B, N, H, D = w["q"].shape
    Dh = D // 2
    qt, kt, vt, _ = _prep(w)
    # the normalised inputs, from the identity-camera, zero-angle prep (pinned above)
    eye = torch.eye(4).expand(B, N, 4, 4).contiguous()
    qn, kn, vn, _ = _prep(w, proj_q=eye, proj_kv=eye, rope_cos=torch.ones(N, Dh),
                          rope_sin=torch.zeros(N, Dh))
    theta = torch.arange(N, dtype=torch.float64)[:, None] * torch.pow(
        10000.0, -2.0 * torch.arange(Dh // 2, dtype=torch.float64) / Dh)[None, :]
    rot = torch.polar(torch.ones_like(theta), theta)  # [N, Dh/2]
    for got, base, P in ((qt, qn, w["proj_q"]), (kt, kn, w["proj_kv"]), (vt, vn, w["proj_kv"])):
        for n in range(N):
            bd = torch.block_diag(*([P[0, n].double()] * (Dh // 4))).numpy()
            for h in range(H):
                x = base[0, h, :, n]
                np.testing.assert_allclose(got[0, h, :Dh, n], bd @ x[:Dh], rtol=1e-12, atol=1e-14)
                z = torch.complex(torch.tensor(x[Dh::2]), torch.tensor(x[Dh + 1::2])) * rot[n]
                np.testing.assert_allclose(got[0, h, Dh::2, n], z.real.numpy(), rtol=1e-6, atol=1e-7)
                np.testing.assert_allclose(got[0, h, Dh + 1::2, n], z.imag.numpy(), rtol=1e-6, atol=1e-7)


def test_cam_prep_inflation_is_one_for_a_rotation_camera():
    # a pure rotation (no translation) keeps |k| in the first half, RoPE keeps it in the
    # second, so the inflation ratio is exactly 1; a translation changes it
    w = workloads.cam_inputs(1, 2, 8, 2, 16, seed=3, translate=0.0)
    _, _, _, infl = _prep(w)
    np.testing.assert_allclose(infl, 1.0, rtol=1e-6)
    w2 = workloads.cam_inputs(1, 2, 8, 2, 16, seed=3, translate=0.5)
    _, _, _, infl2 = _prep(w2)
    assert np.abs(infl2 - 1.0).max() > 1e-2
    # P = c I for k, zero angle: the first half's squared norm scales by c^2, the second's not
    B, N, H, D = w["q"].shape
    eye = torch.eye(4).expand(B, N, 4, 4).contiguous()
    flat = dict(rope_cos=torch.ones(N, D // 2), rope_sin=torch.zeros(N, D // 2))
    _, kn, _, _ = _prep(w, proj_q=eye, proj_kv=eye, **flat)
    _, _, _, infl3 = _prep(w, proj_q=eye, proj_kv=3.0 * eye, **flat)
    a = (kn[:, :, :D // 2] ** 2).sum(axis=2)
    b = (kn[:, :, D // 2:] ** 2).sum(axis=2)
    np.testing.assert_allclose(infl3, (9.0 * a + b) / (a + b), rtol=1e-12)


def _scan_inputs(F=4, S=6, H=2, D=8, B=1, seed=5):
    return workloads.cam_scan_inputs(B, F, S, H, D, seed=seed)


def test_cam_scan_one_token_frames_is_the_token_rule():
    # S = 1: the frame-level rule is the token recurrence with log gate log(decay)
    w = _scan_inputs(F=9, S=1, D=8)
    out = oracle.cam_scan(w["q"], w["k"], w["v"], w["beta"], w["decay"])
    B, H, D, N = w["q"].shape
    tok = lambda x: np.transpose(x.double().numpy(), (0, 3, 1, 2))  # [B,N,H,D]
    r = oracle.gdn(tok(w["q"]), tok(w["k"]), tok(w["v"]),
                   np.transpose(w["beta"][..., 0].double().numpy(), (0, 2, 1)),
                   g=np.transpose(np.log(w["decay"].double().numpy()), (0, 2, 1)))
    np.testing.assert_allclose(out, np.transpose(r["o"], (0, 2, 3, 1)), rtol=1e-10, atol=1e-12)


def test_cam_scan_forward_is_the_product_form():
    # S_f = decay_f (I - K_f^T diag(beta_f) K_f) S_{f-1} + K_f^T diag(beta_f) V_f; out = Q S_f
    w = _scan_inputs(F=5, S=7, H=2, D=8)
    out = oracle.cam_scan(w["q"], w["k"], w["v"], w["beta"], w["decay"])
    B, H, D, N = w["q"].shape
    for h in range(H):
        t = lambda x: x[0, h].double().numpy().T  # [N, D]
        num, _ = forms.bigdn_product(t(w["q"]), t(w["k"]), t(w["q"]), t(w["k"]), t(w["v"]),
                                     w["beta"][0, h].double().numpy(),
                                     w["decay"][0, h].double().numpy())
        np.testing.assert_allclose(out[0, h].T, num, rtol=1e-10, atol=1e-12)


def test_cam_scan_reverse_is_flip_and_shift():
    # the page's reference: q flipped along frames, k, v, beta flip-and-shifted with 0,
    # decay with 1, a forward scan, the output flipped back
    w = _scan_inputs(F=5, S=3, H=2, D=8)
    out = oracle.cam_scan(w["q"], w["k"], w["v"], w["beta"], w["decay"], reverse=True)
    B, H, D, N = w["q"].shape
    F, S = w["beta"].shape[2:]
    fr = lambda x: x.double().numpy().reshape(B, H, D, F, S)
    unf = lambda x: np.ascontiguousarray(x.reshape(B, H, D, N))
    qf = unf(np.flip(fr(w["q"]), axis=3))
    kf = unf(forms.flip_and_shift(fr(w["k"]), 3, 0.0))
    vf = unf(forms.flip_and_shift(fr(w["v"]), 3, 0.0))
    bf = forms.flip_and_shift(w["beta"].double().numpy(), 2, 0.0)
    df = forms.flip_and_shift(w["decay"].double().numpy(), 2, 1.0)
    fwd = oracle.cam_scan(qf, kf, vf, bf, df)
    np.testing.assert_allclose(out, unf(np.flip(fwd.reshape(B, H, D, F, S), axis=3)),
                               rtol=1e-12, atol=1e-14)
    # the last frame reads the zero state
    assert np.abs(out[..., (F - 1) * S:]).max() == 0.0


def test_cam_scan_split_resume():
    # frames [0, c) with the final state out, then [c, F) from it: the whole scan's outputs
    # and final state
    w = _scan_inputs(F=6, S=4, H=3, D=8, B=2)
    out, fin = oracle.cam_scan(w["q"], w["k"], w["v"], w["beta"], w["decay"], want_final=True)
    c, S = 2, 4
    cut = lambda x, a, b: x[..., a * S:b * S]
    o1, f1 = oracle.cam_scan(cut(w["q"], 0, c), cut(w["k"], 0, c), cut(w["v"], 0, c),
                             w["beta"][:, :, :c], w["decay"][:, :, :c], want_final=True)
    o2, f2 = oracle.cam_scan(cut(w["q"], c, 6), cut(w["k"], c, 6), cut(w["v"], c, 6),
                             w["beta"][:, :, c:], w["decay"][:, :, c:], init_state=f1,
                             want_final=True)
    np.testing.assert_allclose(np.concatenate([o1, o2], axis=-1), out, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(f2, fin, rtol=1e-12, atol=1e-14)


def test_cam_scan_zero_beta_only_decays_the_initial_state():
    # beta = 0: the state is the initial one times the running product of decays
    w = _scan_inputs(F=4, S=3, H=2, D=8)
    B, H, D, N = w["q"].shape
    rng = np.random.default_rng(0)
    h0 = rng.standard_normal((B * H, D, D))
    out, fin = oracle.cam_scan(w["q"], w["k"], w["v"], torch.zeros_like(w["beta"]),
                               w["decay"], init_state=h0, want_final=True)
    dec = np.cumprod(w["decay"].double().numpy(), axis=-1)  # [B,H,F]
    for b in range(B):
        for h in range(H):
            for f in range(4):
                st = dec[b, h, f] * h0[b * H + h]
                qq = w["q"][b, h, :, f * 3:(f + 1) * 3].double().numpy()
                np.testing.assert_allclose(out[b, h, :, f * 3:(f + 1) * 3], st.T @ qq,
                                           rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(fin.reshape(B, H, D, D), dec[..., -1, None, None] * h0.reshape(B, H, D, D),
                               rtol=1e-12)


def test_cam_scan_reverse_rejects_state_io():
    w = _scan_inputs()
    with pytest.raises(NotImplementedError):
        oracle.cam_scan(w["q"], w["k"], w["v"], w["beta"], w["decay"], reverse=True,
                        want_final=True)

"""Pins of the state-gradient pass (oracle.gdn_dhu) against derivatives of the token-level
forward oracle taken by central differences.

The forward is affine in the initial state and in v, so central differences give its
gradients up to rounding.  With L = sum o . do + sum ht . dht:
  * dh0 must be dL/dh0;
  * dh[n] must be dL/dh[n] for the state entering chunk n, obtained by running the tokens
    after nC from a perturbed state (the tokens before nC do not see it);
  * dv2 (the gradient of v_new) must satisfy dL/dv = diag(beta) Tm^T dv2 per chunk, since
    v_new = Tm diag(beta) v - w h.
The inputs w and dv of the pass are formed here from their definitions (the WY w and the
intra-chunk gradient P^T do); a slip in either, or in the pass, breaks a pin.
"""
import numpy as np
import pytest

import oracle

pytestmark = pytest.mark.filterwarnings("ignore::DeprecationWarning")
C = 4


def _setup(T=11, H=2, K=4, V=3, seed=0, gated=True, per_key=False):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((1, T, H, K))
    k = rng.standard_normal((1, T, H, K))
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = rng.standard_normal((1, T, H, V))
    beta = 1.0 / (1.0 + np.exp(-rng.standard_normal((1, T, H))))
    g = np.log(1.0 / (1.0 + np.exp(-(rng.standard_normal((1, T, H)) + 2.0)))) if gated else None
    h0 = rng.standard_normal((1, H, K, V))
    do = rng.standard_normal((1, T, H, V))
    dht = rng.standard_normal((1, H, K, V))
    gk = (np.log(1.0 / (1.0 + np.exp(-(rng.standard_normal((1, T, H, K)) + 2.0))))
          if per_key else None)
    return dict(q=q, k=k, v=v, beta=beta, g=g, gk=gk, h0=h0, do=do, dht=dht, scale=0.7)


def _loss(s, v=None, h0=None, t0=0):
    """L over tokens t0.. run from the state h0 (the state entering token t0)."""
    v = s["v"] if v is None else v
    h0 = s["h0"] if h0 is None else h0
    sl = slice(t0, None)
    g = None if s["g"] is None else s["g"][:, sl]
    gk = None if s["gk"] is None else s["gk"][:, sl]
    r = oracle.gdn(s["q"][:, sl], s["k"][:, sl], v[:, sl], s["beta"][:, sl], g=g, gk=gk,
                   scale=s["scale"], h0=h0)
    return float(np.sum(r["o"] * s["do"][:, sl]) + np.sum(r["ht"] * s["dht"]))


def _wy_inputs(s):
    """w (the WY w) and dv (P^T do) per chunk, from their definitions."""
    q, k, beta, do = s["q"], s["k"], s["beta"], s["do"]
    _, T, H, K = q.shape
    w = np.zeros_like(k)
    dv = np.zeros_like(do)
    tms = {}
    for h in range(H):
        for t0 in range(0, T, C):
            L = min(C, T - t0)
            sl = slice(t0, t0 + L)
            gg = np.zeros(L) if s["g"] is None else s["g"][0, sl, h]
            lam = gg[:, None] + (0.0 if s["gk"] is None else s["gk"][0, sl, h])  # [L, K]
            gam = np.cumsum(lam * np.ones((L, K)), axis=0)
            kk, qq, bt = k[0, sl, h], q[0, sl, h], beta[0, sl, h]
            # sum_d x_{r,d} y_{s,d} e^{gamma_{r,d} - gamma_{s,d}}
            gram = lambda x, y: np.einsum("rd,sd,rsd->rs", x, y,
                                          np.exp(gam[:, None, :] - gam[None, :, :]))
            A = np.tril(bt[:, None] * gram(kk, kk), -1)
            Tm = np.linalg.inv(np.eye(L) + A)
            w[0, sl, h] = Tm @ (bt[:, None] * kk * np.exp(gam))
            P = s["scale"] * np.tril(gram(qq, kk))
            dv[0, sl, h] = P.T @ do[0, sl, h]
            tms[(h, t0)] = Tm
    return w, dv, tms


def _central(f, x, eps=1e-3):
    gr = np.zeros_like(x)
    for idx in np.ndindex(x.shape):
        xp = x.copy()
        xp[idx] += eps
        xm = x.copy()
        xm[idx] -= eps
        gr[idx] = (f(xp) - f(xm)) / (2 * eps)
    return gr


@pytest.mark.parametrize("gated,per_key", [(True, False), (False, False), (True, True),
                                           (False, True)])
def test_dhu_dh0_and_chunk_states_are_gradients(gated, per_key):
    s = _setup(gated=gated, per_key=per_key)
    w, dv, _ = _wy_inputs(s)
    r = oracle.gdn_dhu(s["q"], s["k"], w, s["do"], dv, g=s["g"], dht=s["dht"], scale=s["scale"],
                       chunk=C, gk=s["gk"])
    np.testing.assert_allclose(r["dh0"], _central(lambda h: _loss(s, h0=h), s["h0"]),
                               rtol=1e-7, atol=1e-8)
    T = s["q"].shape[1]
    for n in range(1, (T + C - 1) // C):
        pre = oracle.gdn(s["q"][:, :n * C], s["k"][:, :n * C], s["v"][:, :n * C],
                         s["beta"][:, :n * C], g=None if s["g"] is None else s["g"][:, :n * C],
                         gk=None if s["gk"] is None else s["gk"][:, :n * C],
                         scale=s["scale"], h0=s["h0"])
        hn = pre["ht"]
        fd = _central(lambda h: _loss(s, h0=h, t0=n * C), hn)
        np.testing.assert_allclose(r["dh"][:, :, n], fd, rtol=1e-7, atol=1e-8)
    np.testing.assert_array_equal(r["dh"][:, :, 0], r["dh0"])


@pytest.mark.parametrize("per_key", [False, True])
def test_dhu_dv2_is_the_gradient_of_v_new(per_key):
    s = _setup(seed=1, per_key=per_key)
    w, dv, tms = _wy_inputs(s)
    r = oracle.gdn_dhu(s["q"], s["k"], w, s["do"], dv, g=s["g"], dht=s["dht"], scale=s["scale"],
                       chunk=C, gk=s["gk"])
    dl_dv = _central(lambda x: _loss(s, v=x), s["v"])
    _, T, H, _ = s["q"].shape
    for (h, t0), Tm in tms.items():
        sl = slice(t0, t0 + Tm.shape[0])
        want = s["beta"][0, sl, h][:, None] * (Tm.T @ r["dv2"][0, sl, h])
        np.testing.assert_allclose(dl_dv[0, sl, h], want, rtol=1e-7, atol=1e-8)


def test_dhu_without_final_gradient():
    # dht = None is a zero final-state gradient
    s = _setup(seed=2)
    w, dv, _ = _wy_inputs(s)
    a = oracle.gdn_dhu(s["q"], s["k"], w, s["do"], dv, g=s["g"], scale=s["scale"], chunk=C)
    b = oracle.gdn_dhu(s["q"], s["k"], w, s["do"], dv, g=s["g"], dht=np.zeros_like(s["dht"]),
                       scale=s["scale"], chunk=C)
    for key in ("dh", "dv2", "dh0"):
        np.testing.assert_array_equal(a[key], b[key])


@pytest.mark.parametrize("gated,per_key", [(True, False), (False, False), (True, True)])
def test_bwd_prep_forms_the_inputs_whose_pass_gives_the_gradient(gated, per_key):
    """oracle.gdn_bwd_prep (w and P^T do from the forward's inputs) feeds oracle.gdn_dhu, and
    the result must be dL/dh0 by central differences of the token-level forward."""
    s = _setup(T=13, seed=3, gated=gated, per_key=per_key)
    w, dv = oracle.gdn_bwd_prep(s["q"], s["k"], s["beta"], s["do"], g=s["g"], gk=s["gk"],
                                scale=s["scale"], chunk=C)
    r = oracle.gdn_dhu(s["q"], s["k"], w, s["do"], dv, g=s["g"], dht=s["dht"], scale=s["scale"],
                       chunk=C, gk=s["gk"])
    np.testing.assert_allclose(r["dh0"], _central(lambda h: _loss(s, h0=h), s["h0"]),
                               rtol=1e-7, atol=1e-8)
    # and the same w, dv as the definitions written out above (einsum form)
    w2, dv2, _ = _wy_inputs(s)
    np.testing.assert_allclose(w, w2, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(dv, dv2, rtol=1e-12, atol=1e-13)


@pytest.mark.parametrize("per_key", [False, True])
def test_reverse_summaries_join_to_the_whole_gradient(per_key):
    """Context-parallel backward: fragments cut at any token (each with its own chunk grid)
    give grad_state_ext = dh0 of the pass from a zero final gradient; walking the fragments
    from the right with grad_in <- grad_ext + M^T grad_in (M the fragment's forward transition)
    must give dL/dh0 of the whole run."""
    s = _setup(T=23, seed=4, per_key=per_key)
    cuts = [0, 6, 15, 23]
    sl = lambda x, a, b: None if x is None else x[:, a:b]
    g_in = s["dht"]
    for a, b in reversed(list(zip(cuts[:-1], cuts[1:]))):
        q, k, beta, do = (sl(s[n], a, b) for n in ("q", "k", "beta", "do"))
        g, gk = sl(s["g"], a, b), sl(s["gk"], a, b)
        w, dv = oracle.gdn_bwd_prep(q, k, beta, do, g=g, gk=gk, scale=s["scale"], chunk=C)
        ext = oracle.gdn_dhu(q, k, w, do, dv, g=g, scale=s["scale"], chunk=C, gk=gk)["dh0"]
        M = oracle.transition(k, beta, g=g, gk=gk)
        g_in = oracle.apply_grad_summary(ext, M, g_in)
    np.testing.assert_allclose(g_in, _central(lambda h: _loss(s, h0=h), s["h0"]),
                               rtol=1e-7, atol=1e-8)

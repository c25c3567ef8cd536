"""Independent numpy forms used only to pin the C oracle (TEST INFRASTRUCTURE ONLY).

Each function below reaches the oracle's result by a different algorithm, so an error in
either one (a dropped term, a wrong sign, index or transpose) shows up as a disagreement.
They work on one chain at a time, in float64, and are meant for small sizes.

  naive_global   -- the whole sequence at once: the deltas solve one T x T unit-lower-
                    triangular system and the outputs are a masked, decay-weighted
                    attention over those deltas.  Obtained by unrolling the recurrence.
  chunked_wy     -- the chunkwise form: per chunk a WY representation (w, u) from a
                    triangular solve, the state pass v_new = u - w h and
                    h <- diag(e^{gamma_last}) h + (k * e^{gamma_last - gamma})^T v_new
                    (the state-pass fragments on the hyper-parallel "Diff Coverage" page),
                    and the masked intra-chunk output.
  bigdn_product  -- the frame-level scan as a product of per-frame affine maps
                    state <- W_f state + U_f, the form of _torch_cam_scan_single_chunk on
                    the SANA fused_cam_gdn.py page (torch reference section).
  flip_and_shift -- _flip_and_shift on the same page: reverse along frames, shift right by
                    one, pad with a given value.
"""
from __future__ import annotations

import numpy as np


def _lam(T, K, g, gk):
    lam = np.zeros((T, K))
    if g is not None:
        lam += np.asarray(g, np.float64)[:, None]
    if gk is not None:
        lam += np.asarray(gk, np.float64)
    return lam


def naive_global(q, k, v, beta, g=None, gk=None, scale=1.0, h0=None):
    """One chain, q,k [T,K], v [T,V], beta,g [T], gk [T,K], h0 [K,V].  Returns (o, ht).

    With Gam = cumsum of the log decays over the whole sequence and
    E[r,s,d] = exp(Gam[r,d] - Gam[s,d]) (the decay applied between tokens s and r):
        delta + A delta = beta*v - beta*((exp(Gam)*k) @ h0),  A[s,j] = beta_s sum_d k_s k_j E[s,j]  (j<s)
        o_r = scale * ( (exp(Gam_r)*q_r) @ h0 + sum_{s<=r} (sum_d q_r k_s E[r,s]) delta_s )
        ht  = diag(exp(Gam_T)) h0 + sum_s (exp(Gam_T - Gam_s) * k_s) delta_s^T
    """
    q, k, v, beta = (np.asarray(x, np.float64) for x in (q, k, v, beta))
    T, K = k.shape
    V = v.shape[1]
    h0 = np.zeros((K, V)) if h0 is None else np.asarray(h0, np.float64)
    Gam = np.cumsum(_lam(T, K, g, gk), axis=0)
    E = np.exp(Gam[:, None, :] - Gam[None, :, :])  # [r, s, d]
    kk = np.einsum("sd,jd,sjd->sj", k, k, E)
    A = np.tril(beta[:, None] * kk, -1)
    rhs = beta[:, None] * (v - (np.exp(Gam) * k) @ h0)
    delta = np.linalg.solve(np.eye(T) + A, rhs)
    qk = np.tril(np.einsum("rd,sd,rsd->rs", q, k, E))
    o = scale * ((np.exp(Gam) * q) @ h0 + qk @ delta)
    ht = np.exp(Gam[-1])[:, None] * h0 + (np.exp(Gam[-1][None, :] - Gam) * k).T @ delta
    return o, ht


def chunked_wy(q, k, v, beta, g=None, gk=None, scale=1.0, h0=None, chunk=64):
    """One chain in the chunkwise WY form.  Returns dict(o, ht, h [NT,K,V], v_new [T,V]).

    Per chunk (local index r, inclusive local cumsum gam of the log decays, gl = gam at the
    chunk's last token, h = state entering the chunk):
        A[r,s] = beta_r sum_d k_r k_s exp(gam_r - gam_s)   (s < r),   Tm = (I + A)^-1
        w = Tm (beta * exp(gam) * k),  u = Tm (beta * v),   v_new = u - w h
        o_r = scale * ( (exp(gam_r) * q_r) h + sum_{s<=r} (sum_d q_r k_s exp(gam_r - gam_s)) v_new_s )
        h  <- diag(exp(gl)) h + (exp(gl - gam) * k)^T v_new
    """
    q, k, v, beta = (np.asarray(x, np.float64) for x in (q, k, v, beta))
    T, K = k.shape
    V = v.shape[1]
    lam = _lam(T, K, g, gk)
    h = np.zeros((K, V)) if h0 is None else np.array(h0, np.float64)
    NT = (T + chunk - 1) // chunk
    o = np.zeros((T, V))
    vnew = np.zeros((T, V))
    hs = np.zeros((NT, K, V))
    for n in range(NT):
        sl = slice(n * chunk, min((n + 1) * chunk, T))
        kc, qc, vc, bc = k[sl], q[sl], v[sl], beta[sl]
        L = kc.shape[0]
        gam = np.cumsum(lam[sl], axis=0)
        gl = gam[-1]
        E = np.exp(gam[:, None, :] - gam[None, :, :])
        A = np.tril(bc[:, None] * np.einsum("rd,sd,rsd->rs", kc, kc, E), -1)
        Tm = np.linalg.inv(np.eye(L) + A)
        w = Tm @ (bc[:, None] * np.exp(gam) * kc)
        u = Tm @ (bc[:, None] * vc)
        hs[n] = h
        vn = u - w @ h
        P = np.tril(np.einsum("rd,sd,rsd->rs", qc, kc, E))
        o[sl] = scale * ((np.exp(gam) * qc) @ h + P @ vn)
        vnew[sl] = vn
        h = np.exp(gl)[:, None] * h + (np.exp(gl[None, :] - gam) * kc).T @ vn
    return {"o": o, "ht": h, "h": hs, "v_new": vnew}


def flip_and_shift(x, axis, pad):
    """Reverse ``x`` along ``axis``, drop the last entry, and put ``pad`` in front."""
    x = np.asarray(x, np.float64)
    xf = np.flip(x, axis=axis)
    body = np.take(xf, np.arange(x.shape[axis] - 1), axis=axis)
    shape = list(x.shape)
    shape[axis] = 1
    return np.concatenate([np.full(shape, pad), body], axis=axis)


def bigdn_product(q_rot, k_rot, q_pos, k_pos, v, beta, decay):
    """One (b,h) forward direction as affine maps.  Inputs [N,D] (N = F*S), beta [F,S],
    decay [F].  Returns (num [N,D], den [N]).

        W_f = decay_f * (I - K_f^T diag(beta_f) K_f),   U_f = K_f^T diag(beta_f) V_f
        S_f = W_f S_{f-1} + U_f,   z_f = W'_f z_{f-1} + K'_f^T beta_f   (primes: k_pos)
        num = Q_rot,f S_f,  den = Q_pos,f z_f
    """
    F, S = beta.shape
    D = q_rot.shape[1]
    St = np.zeros((D, D))
    z = np.zeros(D)
    num = np.zeros((F * S, D))
    den = np.zeros(F * S)
    I = np.eye(D)
    for f in range(F):
        sl = slice(f * S, (f + 1) * S)
        kr, kp, vv, bt = k_rot[sl], k_pos[sl], v[sl], beta[f]
        W = decay[f] * (I - kr.T @ (bt[:, None] * kr))
        U = kr.T @ (bt[:, None] * vv)
        Wz = decay[f] * (I - kp.T @ (bt[:, None] * kp))
        St = W @ St + U
        z = Wz @ z + kp.T @ bt
        num[sl] = q_rot[sl] @ St
        den[sl] = q_pos[sl] @ z
    return num, den


def bigdn_reverse_by_flip(q_rot, k_rot, q_pos, k_pos, v, beta, decay):
    """Reverse direction of one (b,h) via flip-and-shift of the inputs and a forward scan:
    q is flipped along frames; k, v, beta are flip-and-shifted with pad 0; decay with pad
    1; the forward result is flipped back."""
    F, S = beta.shape
    D = q_rot.shape[1]

    def frames(x):
        return np.asarray(x, np.float64).reshape(F, S, D)

    def unframes(x):
        return x.reshape(F * S, D)

    qr = unframes(np.flip(frames(q_rot), axis=0))
    qp = unframes(np.flip(frames(q_pos), axis=0))
    kr = unframes(flip_and_shift(frames(k_rot), 0, 0.0))
    kp = unframes(flip_and_shift(frames(k_pos), 0, 0.0))
    vv = unframes(flip_and_shift(frames(v), 0, 0.0))
    bt = flip_and_shift(beta, 0, 0.0)
    dc = flip_and_shift(decay, 0, 1.0)
    num, den = bigdn_product(qr, kr, qp, kp, vv, bt, dc)
    num = unframes(np.flip(frames(num), axis=0))
    den = np.flip(den.reshape(F, S), axis=0).reshape(F * S)
    return num, den

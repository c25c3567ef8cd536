"""Pins of the fp64 CPU oracle against facts fixed by the pages and by the mathematics.

None of these compare the oracle with a retyped copy of itself: each check is a closed
form, an invariant, a hand-derived example (tests/golden), a textbook/library routine, or
an independently derived algorithm (oracle/forms.py) that reaches the same result by a
different route.  A dropped term, a wrong sign, index or transpose in the oracle breaks at
least one of them.
"""
import math
import os

import numpy as np
import pytest
import torch

import oracle
from oracle import forms

pytestmark = pytest.mark.filterwarnings("ignore::DeprecationWarning")
HERE = os.path.dirname(os.path.abspath(__file__))


def _rand_chain(rng, T, K, V, per_key=False, unit_keys=True, g_shift=2.0):
    q = rng.standard_normal((1, T, 1, K))
    k = rng.standard_normal((1, T, 1, K))
    if unit_keys:
        k /= np.linalg.norm(k, axis=-1, keepdims=True)
        q /= np.linalg.norm(q, axis=-1, keepdims=True)
    v = rng.standard_normal((1, T, 1, V))
    beta = 1.0 / (1.0 + np.exp(-rng.standard_normal((1, T, 1))))
    g = -np.log1p(np.exp(-(rng.standard_normal((1, T, 1)) + g_shift)))
    gk = -np.log1p(np.exp(-(rng.standard_normal((1, T, 1, K)) + 3.0))) if per_key else None
    return q, k, v, beta, g, gk


def _read_golden(path):
    vals = {}
    with open(path) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            name, *nums = line.split()
            vals[name] = np.array([float(x) for x in nums])
    return vals


# ---------------------------------------------------------------- hand-derived examples
def test_golden_hand_examples():
    gold = _read_golden(os.path.join(HERE, "golden", "gdn_hand_example.txt"))
    q = np.array([[1, 1], [0, 1]], float).reshape(1, 2, 1, 2)
    k = np.array([[1, 0], [0.6, 0.8]], float).reshape(1, 2, 1, 2)
    v = np.array([[2, 3], [1, -1]], float).reshape(1, 2, 1, 2)
    beta = np.array([0.5, 1.0]).reshape(1, 2, 1)
    g = np.array([0.0, math.log(0.5)]).reshape(1, 2, 1)
    r = oracle.gdn(q, k, v, beta, g=g, want_vnew=True)
    np.testing.assert_allclose(r["o"].ravel(), gold["A.o"], atol=1e-14)
    np.testing.assert_allclose(r["v_new"].ravel(), gold["A.v_new"], atol=1e-14)
    np.testing.assert_allclose(r["ht"].ravel(), gold["A.ht"], atol=1e-14)

    q = np.array([1.0, 0.0]).reshape(1, 1, 1, 2)
    k = np.array([0.6, 0.8]).reshape(1, 1, 1, 2)
    v = np.array([1.0, 1.0]).reshape(1, 1, 1, 2)
    beta = np.array([0.5]).reshape(1, 1, 1)
    g = np.array([math.log(0.8)]).reshape(1, 1, 1)
    gk = np.array([math.log(0.5), math.log(0.25)]).reshape(1, 1, 1, 2)
    h0 = np.array([[1.0, 2.0], [3.0, 4.0]]).reshape(1, 1, 2, 2)
    r = oracle.gdn(q, k, v, beta, g=g, gk=gk, scale=2.0, h0=h0, want_vnew=True)
    np.testing.assert_allclose(r["o"].ravel(), gold["B.o"], atol=1e-14)
    np.testing.assert_allclose(r["v_new"].ravel(), gold["B.v_new"], atol=1e-14)
    np.testing.assert_allclose(r["ht"].ravel(), gold["B.ht"], atol=1e-14)


# ---------------------------------------------------------------- invariants / closed forms
@pytest.mark.parametrize("per_key", [False, True])
def test_beta_zero_keeps_state(per_key):
    """beta = 0: no write ever happens.  From zero the output is exactly zero; from h0 the
    state is only decayed, S_t = diag(exp(cumsum of log decays)) h0."""
    rng = np.random.default_rng(1)
    q, k, v, beta, g, gk = _rand_chain(rng, 77, 16, 8, per_key=per_key)
    beta = np.zeros_like(beta)
    r = oracle.gdn(q, k, v, beta, g=g, gk=gk)
    assert np.all(r["o"] == 0.0) and np.all(r["ht"] == 0.0)
    h0 = rng.standard_normal((1, 1, 16, 8))
    r = oracle.gdn(q, k, v, beta, g=g, gk=gk, scale=0.7, h0=h0)
    lam = np.repeat(g[0, :, 0][:, None], 16, axis=1) + (gk[0, :, 0] if per_key else 0.0)
    cum = np.cumsum(lam, axis=0)
    want = 0.7 * np.einsum("td,tdv->tv", q[0, :, 0], np.exp(cum)[:, :, None] * h0[0, 0][None])
    np.testing.assert_allclose(r["o"][0, :, 0], want, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(r["ht"][0, 0], np.exp(cum[-1])[:, None] * h0[0, 0], rtol=1e-12)


def test_orthonormal_keys_recall():
    """alpha = beta = 1 with orthonormal keys: every write lands in its own direction, so
    querying with k_i returns v_i (both right after the write and at the end)."""
    rng = np.random.default_rng(2)
    K = V = 64
    T = 64
    Q, _ = np.linalg.qr(rng.standard_normal((K, K)))
    k = Q.T.reshape(1, T, 1, K)  # rows orthonormal
    v = rng.standard_normal((1, T, 1, V))
    beta = np.ones((1, T, 1))
    g = np.zeros((1, T, 1))
    r = oracle.gdn(k, k, v, beta, g=g)
    np.testing.assert_allclose(r["o"], v, atol=1e-12)
    ht = r["ht"][0, 0]
    np.testing.assert_allclose(k[0, :, 0] @ ht, v[0, :, 0], atol=1e-12)


@pytest.mark.parametrize("per_key", [False, True])
def test_per_step_closed_form(per_key):
    """Unit keys: S_t^T k_t = (1 - beta_t) (diag(a_t) S_{t-1})^T k_t + beta_t v_t, checked at
    every step with S_{t-1} taken from a prefix run's final state (q = k gives S_t^T k_t)."""
    rng = np.random.default_rng(3)
    T, K, V = 40, 8, 5
    q, k, v, beta, g, gk = _rand_chain(rng, T, K, V, per_key=per_key)
    h0 = rng.standard_normal((1, 1, K, V))
    full = oracle.gdn(k, k, v, beta, g=g, gk=gk, h0=h0)
    prev = h0[0, 0]
    for t in range(T):
        if t > 0:
            prev = oracle.gdn(k[:, :t], k[:, :t], v[:, :t], beta[:, :t], g=g[:, :t],
                              gk=None if gk is None else gk[:, :t], h0=h0)["ht"][0, 0]
        lam = g[0, t, 0] + (gk[0, t, 0] if per_key else np.zeros(K))
        Sp = np.exp(lam)[:, None] * prev
        kt = k[0, t, 0]
        want = (1 - beta[0, t, 0]) * (Sp.T @ kt) + beta[0, t, 0] * v[0, t, 0]
        np.testing.assert_allclose(full["o"][0, t, 0], want, atol=1e-12)


def test_reset_gate():
    """alpha = 0 (g = -inf) erases the state before each write: o_t = scale beta_t (q_t.k_t) v_t."""
    rng = np.random.default_rng(4)
    q, k, v, beta, g, _ = _rand_chain(rng, 33, 12, 7, unit_keys=False)
    g = np.full_like(g, -np.inf)
    r = oracle.gdn(q, k, v, beta, g=g, scale=1.5)
    want = 1.5 * beta[0, :, 0, None] * np.sum(q[0, :, 0] * k[0, :, 0], -1)[:, None] * v[0, :, 0]
    np.testing.assert_allclose(r["o"][0, :, 0], want, rtol=1e-13, atol=1e-14)


def test_single_token_rank_one():
    """One token from zero: S = beta k v^T, so o = scale beta (k.q) v, v_new = beta v."""
    rng = np.random.default_rng(5)
    q, k, v, beta, g, gk = _rand_chain(rng, 1, 9, 4, per_key=True, unit_keys=False)
    r = oracle.gdn(q, k, v, beta, g=g, gk=gk, scale=0.3, want_vnew=True)
    b = beta[0, 0, 0]
    np.testing.assert_allclose(r["o"][0, 0, 0], 0.3 * b * (q[0, 0, 0] @ k[0, 0, 0]) * v[0, 0, 0],
                               rtol=1e-13)
    np.testing.assert_allclose(r["v_new"][0, 0, 0], b * v[0, 0, 0], rtol=1e-14)
    np.testing.assert_allclose(r["ht"][0, 0], b * np.outer(k[0, 0, 0], v[0, 0, 0]), rtol=1e-14)


# ---------------------------------------------------------------- independent algorithms
@pytest.mark.parametrize("per_key,with_h0,T", [(False, False, 64), (False, True, 97),
                                              (True, True, 128), (True, False, 37)])
def test_naive_global_form_agrees(per_key, with_h0, T):
    rng = np.random.default_rng(6 + T)
    K, V = 16, 12
    q, k, v, beta, g, gk = _rand_chain(rng, T, K, V, per_key=per_key)
    h0 = rng.standard_normal((1, 1, K, V)) if with_h0 else None
    r = oracle.gdn(q, k, v, beta, g=g, gk=gk, scale=0.8, h0=h0)
    o, ht = forms.naive_global(q[0, :, 0], k[0, :, 0], v[0, :, 0], beta[0, :, 0], g[0, :, 0],
                               None if gk is None else gk[0, :, 0], 0.8,
                               None if h0 is None else h0[0, 0])
    np.testing.assert_allclose(r["o"][0, :, 0], o, atol=1e-12)
    np.testing.assert_allclose(r["ht"][0, 0], ht, atol=1e-12)


@pytest.mark.parametrize("chunk,T,per_key", [(64, 256, False), (64, 200, True),
                                             (16, 130, False), (16, 77, True), (64, 5, False)])
def test_chunked_wy_form_agrees(chunk, T, per_key):
    rng = np.random.default_rng(100 + T)
    K, V = 32, 24
    q, k, v, beta, g, gk = _rand_chain(rng, T, K, V, per_key=per_key)
    h0 = rng.standard_normal((1, 1, K, V))
    r = oracle.gdn(q, k, v, beta, g=g, gk=gk, scale=1.1, h0=h0, chunk=chunk, want_h=True,
                   want_vnew=True)
    c = forms.chunked_wy(q[0, :, 0], k[0, :, 0], v[0, :, 0], beta[0, :, 0], g[0, :, 0],
                         None if gk is None else gk[0, :, 0], 1.1, h0[0, 0], chunk)
    np.testing.assert_allclose(r["o"][0, :, 0], c["o"], atol=1e-12)
    np.testing.assert_allclose(r["ht"][0, 0], c["ht"], atol=1e-12)
    np.testing.assert_allclose(r["h"][0, 0], c["h"], atol=1e-12)
    np.testing.assert_allclose(r["v_new"][0, :, 0], c["v_new"], atol=1e-12)


def test_batch_layout_matches_single_chains():
    """[B,T,H,.] indexing: every (b,h) of a batched call equals a one-chain call."""
    rng = np.random.default_rng(7)
    B, T, H, K, V = 2, 70, 3, 8, 6
    q = rng.standard_normal((B, T, H, K))
    k = rng.standard_normal((B, T, H, K)) / 3
    v = rng.standard_normal((B, T, H, V))
    beta = rng.uniform(0, 1, (B, T, H))
    g = -rng.uniform(0, 0.3, (B, T, H))
    gk = -rng.uniform(0, 0.3, (B, T, H, K))
    h0 = rng.standard_normal((B, H, K, V))
    r = oracle.gdn(q, k, v, beta, g=g, gk=gk, h0=h0, want_h=True, want_vnew=True)
    for b in range(B):
        for h in range(H):
            s = oracle.gdn(q[b:b + 1, :, h:h + 1], k[b:b + 1, :, h:h + 1], v[b:b + 1, :, h:h + 1],
                           beta[b:b + 1, :, h:h + 1], g=g[b:b + 1, :, h:h + 1],
                           gk=gk[b:b + 1, :, h:h + 1], h0=h0[b:b + 1, h:h + 1], want_h=True,
                           want_vnew=True)
            np.testing.assert_array_equal(r["o"][b, :, h], s["o"][0, :, 0])
            np.testing.assert_array_equal(r["ht"][b, h], s["ht"][0, 0])
            np.testing.assert_array_equal(r["h"][b, h], s["h"][0, 0])
            np.testing.assert_array_equal(r["v_new"][b, :, h], s["v_new"][0, :, 0])


def test_split_resume():
    """Running [0,T1) then resuming [T1,T) from its final state equals one run."""
    rng = np.random.default_rng(8)
    q, k, v, beta, g, gk = _rand_chain(rng, 150, 16, 16, per_key=True)
    full = oracle.gdn(q, k, v, beta, g=g, gk=gk)
    T1 = 61
    a = oracle.gdn(q[:, :T1], k[:, :T1], v[:, :T1], beta[:, :T1], g=g[:, :T1], gk=gk[:, :T1])
    b = oracle.gdn(q[:, T1:], k[:, T1:], v[:, T1:], beta[:, T1:], g=g[:, T1:], gk=gk[:, T1:],
                   h0=a["ht"])
    np.testing.assert_allclose(np.concatenate([a["o"], b["o"]], axis=1), full["o"], atol=1e-13)
    np.testing.assert_allclose(b["ht"], full["ht"], atol=1e-13)


def test_thread_count_does_not_change_results():
    rng = np.random.default_rng(9)
    B, T, H, K, V = 2, 50, 4, 8, 8
    args = (rng.standard_normal((B, T, H, K)), rng.standard_normal((B, T, H, K)) / 3,
            rng.standard_normal((B, T, H, V)), rng.uniform(0, 1, (B, T, H)))
    g = -rng.uniform(0, 0.3, (B, T, H))
    n0 = oracle.max_threads()
    r1 = oracle.gdn(*args, g=g)
    oracle.set_threads(1)
    try:
        r2 = oracle.gdn(*args, g=g)
    finally:
        oracle.set_threads(n0)
    np.testing.assert_array_equal(r1["o"], r2["o"])


# ---------------------------------------------------------------- varlen
def test_varlen_tables_properties():
    """The chunk tables tile every sequence exactly: chunk c of sequence i covers tokens
    [cu[i] + 64c, min(cu[i] + 64(c+1), cu[i+1])), chunks appear in order, and together they
    cover [0, T_total) once."""
    rng = np.random.default_rng(10)
    for trial in range(20):
        n = int(rng.integers(1, 12))
        lens = rng.integers(1, 300, n)
        cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
        offs, idx = oracle.varlen_tables(cu)
        assert offs.dtype == np.int32 and idx.dtype == np.int32
        covered = np.zeros(cu[-1], np.int32)
        for row, (i, c) in enumerate(idx):
            assert offs[i] <= row < offs[i + 1]
            assert row - offs[i] == c
            lo, hi = cu[i] + 64 * c, min(cu[i] + 64 * (c + 1), cu[i + 1])
            assert lo < hi
            covered[lo:hi] += 1
        assert np.all(covered == 1)
        assert offs[0] == 0 and offs[-1] == len(idx)
    with pytest.raises(ValueError):
        oracle.varlen_tables(np.array([0, 5, 5, 9], np.int32))  # empty sequence
    with pytest.raises(ValueError):
        oracle.varlen_tables(np.array([1, 5], np.int32))  # does not start at 0


def test_varlen_equals_separate_runs():
    rng = np.random.default_rng(11)
    lens = [70, 1, 128, 64, 33]
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    T, H, K, V = int(cu[-1]), 2, 8, 8
    q = rng.standard_normal((1, T, H, K))
    k = rng.standard_normal((1, T, H, K)) / 3
    v = rng.standard_normal((1, T, H, V))
    beta = rng.uniform(0, 1, (1, T, H))
    g = -rng.uniform(0, 0.3, (1, T, H))
    gk = -rng.uniform(0, 0.3, (1, T, H, K))
    h0 = rng.standard_normal((len(lens), H, K, V))
    r = oracle.gdn_varlen(cu, q, k, v, beta, g=g, gk=gk, h0=h0, want_h=True, want_vnew=True)
    offs, _ = oracle.varlen_tables(cu)
    for i in range(len(lens)):
        sl = slice(cu[i], cu[i + 1])
        s = oracle.gdn(q[:, sl], k[:, sl], v[:, sl], beta[:, sl], g=g[:, sl], gk=gk[:, sl],
                       h0=h0[i:i + 1], want_h=True, want_vnew=True)
        np.testing.assert_array_equal(r["o"][:, sl], s["o"])
        np.testing.assert_array_equal(r["v_new"][:, sl], s["v_new"])
        np.testing.assert_array_equal(r["ht"][i], s["ht"][0])
        np.testing.assert_array_equal(r["h"][0, :, offs[i]:offs[i + 1]], s["h"][0])


# ---------------------------------------------------------------- BiGDN front end
def _prep_inputs(seed, B=1, N=24, H=3, D=8):
    gen = torch.Generator().manual_seed(seed)
    qkv = torch.randn(B, N, 3, H, D, generator=gen, dtype=torch.float64)
    qw = 1 + 0.1 * torch.randn(H * D, generator=gen, dtype=torch.float64)
    kw = 1 + 0.1 * torch.randn(H * D, generator=gen, dtype=torch.float64)
    return qkv, qw, kw


def test_prep_identity_rope_and_library_rmsnorm():
    """With cos = 1, sin = 0 the rotation is the identity; the normalised, rectified q/k
    equal torch's rms_norm over the H*D channels of each token, then ReLU (and the k-scale
    on k only)."""
    B, N, H, D = 2, 24, 3, 8
    qkv, qw, kw = _prep_inputs(0, B, N, H, D)
    cos = np.ones((N, D))
    sin = np.zeros((N, D))
    r = oracle.prep(qkv, qw, kw, cos, sin, k_scale=0.25, eps=1e-5)
    np.testing.assert_array_equal(r["q_rot"], r["q_pos"])
    np.testing.assert_array_equal(r["k_rot"], r["k_pos"])
    C = H * D
    for which, w, ks, name in ((0, qw, 1.0, "q_pos"), (1, kw, 0.25, "k_pos")):
        x = qkv[:, :, which].reshape(B, N, C)
        y = torch.relu(torch.nn.functional.rms_norm(x, (C,), weight=w, eps=1e-5)) * ks
        want = y.reshape(B, N, H, D).permute(0, 2, 1, 3).numpy()
        np.testing.assert_allclose(r[name], want, rtol=1e-12, atol=1e-14)
        # rms_norm(x) = x * inv_rms, so any channel's ratio gives inv_rms
        inv = (torch.nn.functional.rms_norm(x, (C,), eps=1e-5) / x)[..., 0]
        np.testing.assert_allclose(r["q_inv_rms" if which == 0 else "k_inv_rms"], inv.numpy(),
                                   rtol=1e-12)
    np.testing.assert_array_equal(r["v"], qkv[:, :, 2].permute(0, 2, 1, 3).numpy())
    assert np.all(r["q_pos"] >= 0) and np.all(r["k_pos"] >= 0)


def test_prep_rope_is_complex_rotation():
    """The expanded-table rotation equals multiplying each pair (x[2i] + i x[2i+1]) by
    exp(i theta[n, i]) (numpy complex arithmetic), so pair norms are preserved."""
    import workloads

    B, N, H, D = 1, 40, 2, 16
    qkv, qw, kw = _prep_inputs(1, B, N, H, D)
    cos, sin = workloads.rope_tables(N, D)
    r = oracle.prep(qkv, qw, kw, cos, sin, k_scale=1.0)
    theta = np.arange(N)[:, None] * np.power(10000.0, -2.0 * np.arange(D // 2) / D)[None, :]
    for pos, out in (("q_pos", "q_rot"), ("k_pos", "k_rot")):
        x = r[pos]
        z = (x[..., 0::2] + 1j * x[..., 1::2]) * np.exp(1j * theta)[None, None]
        np.testing.assert_allclose(r[out][..., 0::2], z.real, atol=1e-6)
        np.testing.assert_allclose(r[out][..., 1::2], z.imag, atol=1e-6)
        np.testing.assert_allclose(r[out][..., 0::2] ** 2 + r[out][..., 1::2] ** 2,
                                   x[..., 0::2] ** 2 + x[..., 1::2] ** 2, rtol=2e-6, atol=1e-12)


# ---------------------------------------------------------------- BiGDN frame scan
def _bigdn_prepped(seed, B, F, S, H, D):
    rng = np.random.default_rng(seed)
    N = F * S
    q_rot = rng.standard_normal((B, H, N, D)) * 0.3
    k_rot = rng.standard_normal((B, H, N, D)) * 0.3
    q_pos = np.abs(rng.standard_normal((B, H, N, D))) * 0.3
    k_pos = np.abs(rng.standard_normal((B, H, N, D))) * 0.3
    v = rng.standard_normal((B, H, N, D))
    beta = rng.uniform(0, 1, (B, H, F, S))
    decay = rng.uniform(0.5, 1.0, (B, H, F))
    return q_rot, k_rot, q_pos, k_pos, v, beta, decay


def test_bigdn_single_token_frames_reduce_to_token_rule():
    """S = 1: the frame rule is the token rule.  num = token GDN on (q_rot, k_rot, v,
    alpha = decay); den = the token delta rule with v = 1 on (q_pos, k_pos)."""
    B, F, S, H, D = 1, 30, 1, 2, 6
    q_rot, k_rot, q_pos, k_pos, v, beta, decay = _bigdn_prepped(12, B, F, S, H, D)
    num, den = oracle.bigdn_dir(q_rot, k_rot, q_pos, k_pos, v, beta, decay, reverse=False)
    tr = lambda x: np.transpose(x, (0, 2, 1, 3))  # [B,H,N,D] -> [B,N,H,D]
    lg = np.log(decay).transpose(0, 2, 1)  # [B,F=N,H]
    bt = beta[..., 0].transpose(0, 2, 1)
    r = oracle.gdn(tr(q_rot), tr(k_rot), tr(v), bt, g=lg)
    np.testing.assert_allclose(num, r["o"], atol=1e-13)
    r1 = oracle.gdn(tr(q_pos), tr(k_pos), np.ones((B, F, H, 1)), bt, g=lg)
    np.testing.assert_allclose(den, r1["o"][..., 0].transpose(0, 2, 1), atol=1e-13)


def test_bigdn_forward_matches_product_form():
    B, F, S, H, D = 1, 5, 7, 2, 6
    ins = _bigdn_prepped(13, B, F, S, H, D)
    num, den = oracle.bigdn_dir(*ins, reverse=False)
    q_rot, k_rot, q_pos, k_pos, v, beta, decay = ins
    for h in range(H):
        n2, d2 = forms.bigdn_product(q_rot[0, h], k_rot[0, h], q_pos[0, h], k_pos[0, h], v[0, h],
                                     beta[0, h], decay[0, h])
        np.testing.assert_allclose(num[0, :, h], n2, atol=1e-13)
        np.testing.assert_allclose(den[0, h], d2, atol=1e-13)


def test_bigdn_reverse_is_flip_and_shift():
    B, F, S, H, D = 1, 6, 4, 2, 6
    ins = _bigdn_prepped(14, B, F, S, H, D)
    num, den = oracle.bigdn_dir(*ins, reverse=True)
    q_rot, k_rot, q_pos, k_pos, v, beta, decay = ins
    for h in range(H):
        n2, d2 = forms.bigdn_reverse_by_flip(q_rot[0, h], k_rot[0, h], q_pos[0, h], k_pos[0, h],
                                             v[0, h], beta[0, h], decay[0, h])
        np.testing.assert_allclose(num[0, :, h], n2, atol=1e-13)
        np.testing.assert_allclose(den[0, h], d2, atol=1e-13)


def test_bigdn_degenerate_cases():
    B, F, S, H, D = 1, 4, 3, 2, 4
    q_rot, k_rot, q_pos, k_pos, v, beta, decay = _bigdn_prepped(15, B, F, S, H, D)
    for rev in (False, True):
        num, den = oracle.bigdn_dir(q_rot, k_rot, q_pos, k_pos, v, np.zeros_like(beta), decay, rev)
        assert np.all(num == 0) and np.all(den == 0)
    # one frame: the reverse direction sees no future frame and emits zeros
    ins1 = _bigdn_prepped(16, B, 1, S, H, D)
    num, den = oracle.bigdn_dir(*ins1, reverse=True)
    assert np.all(num == 0) and np.all(den == 0)


def test_bigdn_block_is_prep_plus_both_directions():
    import workloads

    w = workloads.bigdn_inputs(1, 3, 8, 2, 8, seed=3)
    num, den = oracle.bigdn(w["qkv"], w["beta"], w["decay"], w["q_norm_w"], w["k_norm_w"],
                            w["rope_cos"], w["rope_sin"], w["k_scale"], w["eps"])
    p = oracle.prep(w["qkv"], w["q_norm_w"], w["k_norm_w"], w["rope_cos"], w["rope_sin"],
                    w["k_scale"], w["eps"])
    ins = (p["q_rot"], p["k_rot"], p["q_pos"], p["k_pos"], p["v"], w["beta"], w["decay"])
    nf, df = oracle.bigdn_dir(*ins, reverse=False)
    nr, dr = oracle.bigdn_dir(*ins, reverse=True)
    np.testing.assert_allclose(num, nf + nr, atol=1e-14)
    np.testing.assert_allclose(den, df + dr, atol=1e-14)


# ------------------------------------------------- fragment state summaries (transition)
# The final state of a fragment is affine in its initial state: ht(h0) = M h0 + ht(0).  These
# pin M against closed forms and against the separately pinned recurrence.
@pytest.mark.parametrize("per_key", [False, True])
def test_transition_beta_zero_is_total_decay(per_key):
    # beta = 0 makes every token map diagonal: M = diag(exp(sum_t (g_t + gk_t)))
    rng = np.random.default_rng(11)
    q, k, v, beta, g, gk = _rand_chain(rng, 37, 16, 8, per_key=per_key)
    beta = np.zeros_like(beta)
    M = oracle.transition(k, beta, g=g, gk=gk)[0, 0]
    lam = g[0, :, 0].sum() + (gk[0, :, 0, :].sum(axis=0) if per_key else np.zeros(16))
    np.testing.assert_allclose(M, np.diag(np.exp(lam)), rtol=1e-12, atol=0.0)


def test_transition_orthonormal_keys_is_projection():
    # no decay, beta = 1, orthonormal keys: the token maps I - k_t k_t^T are commuting
    # projections, so M = I - sum_t k_t k_t^T, the projection onto the keys' complement
    rng = np.random.default_rng(12)
    K, T = 16, 6
    Q, _ = np.linalg.qr(rng.standard_normal((K, K)))
    k = Q[:, :T].T.reshape(1, T, 1, K)
    M = oracle.transition(k, np.ones((1, T, 1)))[0, 0]
    np.testing.assert_allclose(M, np.eye(K) - Q[:, :T] @ Q[:, :T].T, atol=1e-13)


@pytest.mark.parametrize("per_key", [False, True])
def test_transition_is_linear_part_of_the_recurrence(per_key):
    # ht(h0) from the recurrence equals M h0 + state_ext for a random h0
    rng = np.random.default_rng(13)
    q, k, v, beta, g, gk = _rand_chain(rng, 70, 16, 12, per_key=per_key)
    h0 = rng.standard_normal((1, 1, 16, 12))
    s = oracle.state_summary(k, v, beta, g=g, gk=gk)
    full = oracle.gdn(q, k, v, beta, g=g, gk=gk, h0=h0)["ht"]
    np.testing.assert_allclose(oracle.apply_summary(s["state_ext"], s["transition"], h0), full,
                               rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(oracle.apply_summary(s["state_ext"], s["transition"]),
                               oracle.gdn(q, k, v, beta, g=g, gk=gk)["ht"], atol=0.0)


@pytest.mark.parametrize("per_key", [False, True])
def test_summaries_compose_over_fragments(per_key):
    # cut a chain into fragments: composing the fragments' summaries in order gives the whole
    # chain's final state, and the whole chain's M is the ordered product of the fragments'
    rng = np.random.default_rng(14)
    q, k, v, beta, g, gk = _rand_chain(rng, 150, 16, 8, per_key=per_key)
    cuts = [0, 41, 64, 130, 150]
    h, m_all = None, np.eye(16)
    for a, b in zip(cuts[:-1], cuts[1:]):
        sl = (slice(None), slice(a, b))
        s = oracle.state_summary(k[sl], v[sl], beta[sl], g=g[sl],
                                 gk=None if gk is None else gk[sl])
        h = oracle.apply_summary(s["state_ext"], s["transition"], h)
        m_all = s["transition"][0, 0] @ m_all
    np.testing.assert_allclose(h, oracle.gdn(q, k, v, beta, g=g, gk=gk)["ht"], rtol=1e-11,
                               atol=1e-12)
    np.testing.assert_allclose(m_all, oracle.transition(k, beta, g=g, gk=gk)[0, 0], rtol=1e-11,
                               atol=1e-13)


# ------------------------------------------------- BiGDN block: overrides and merge epilogue
def _merged_inputs(F=4, S=8, H=2, D=8, seed=21):
    import workloads

    return workloads.bigdn_inputs(1, F, S, H, D, seed=seed)


def _bm(w, **kw):
    return oracle.bigdn_merged(w["qkv"], w["beta"], w["decay"], w["q_norm_w"], w["k_norm_w"],
                               w["rope_cos"], w["rope_sin"], w["k_scale"], w["eps"], **kw)


def test_bigdn_merged_without_overrides_is_the_block():
    w = _merged_inputs()
    out, num, den = _bm(w)
    rn, rd = oracle.bigdn(w["qkv"], w["beta"], w["decay"], w["q_norm_w"], w["k_norm_w"],
                          w["rope_cos"], w["rope_sin"], w["k_scale"], w["eps"])
    np.testing.assert_allclose(num, rn, atol=1e-14)
    np.testing.assert_allclose(den, rd, atol=1e-14)
    out2, _, _ = _bm(w, beta_bwd=w["beta"], decay_bwd=w["decay"])
    np.testing.assert_array_equal(out, out2)


def test_bigdn_zero_reverse_decay_cuts_the_reverse_direction():
    # decay_bwd = 0 at frame c: absorbing frame c wipes the reverse state, so frames before c
    # see nothing after c (chunk-causal); the plain reverse direction does see it
    w = _merged_inputs(F=5)
    c, S = 2, w["beta"].shape[3]
    dbwd = w["decay"].clone()
    dbwd[:, :, c] = 0.0
    w2 = dict(w)
    qkv2 = w["qkv"].clone()
    qkv2[:, (c + 1) * S:] = torch.randn(qkv2[:, (c + 1) * S:].shape, generator=torch.Generator().manual_seed(9)).to(qkv2.dtype)
    w2["qkv"] = qkv2
    _, n1, d1 = _bm(w, decay_bwd=dbwd)
    _, n2, d2 = _bm(w2, decay_bwd=dbwd)
    np.testing.assert_allclose(n1[:, :c * S], n2[:, :c * S], atol=1e-13)
    np.testing.assert_allclose(d1[:, :, :c * S], d2[:, :, :c * S], atol=1e-13)
    _, m1, _ = _bm(w)
    _, m2, _ = _bm(w2)
    assert np.abs(m1[:, :c * S] - m2[:, :c * S]).max() > 1e-3


def test_bigdn_reverse_beta_override_reaches_only_the_reverse():
    # beta_bwd = 0: the reverse direction absorbs nothing, leaving the forward direction alone
    w = _merged_inputs()
    _, num, den = _bm(w, beta_bwd=torch.zeros_like(w["beta"]))
    p = oracle.prep(w["qkv"], w["q_norm_w"], w["k_norm_w"], w["rope_cos"], w["rope_sin"],
                    w["k_scale"], w["eps"])
    nf, df = oracle.bigdn_dir(p["q_rot"], p["k_rot"], p["q_pos"], p["k_pos"], p["v"], w["beta"],
                              w["decay"], reverse=False)
    np.testing.assert_allclose(num, nf, atol=1e-14)
    np.testing.assert_allclose(den, df, atol=1e-14)


def test_bigdn_merge_gate_is_silu():
    # SiLU(x) - SiLU(-x) = x and SiLU(0) = 0: a sigmoid gate or a sign slip fails these
    w = _merged_inputs()
    B, N, _, H, D = w["qkv"].shape
    g = torch.randn(B, N, H, D, generator=torch.Generator().manual_seed(4))
    base, _, _ = _bm(w)
    up, _, _ = _bm(w, gate=g)
    dn, _, _ = _bm(w, gate=-g)
    np.testing.assert_allclose(up - dn, base * g.double().numpy(), rtol=1e-12, atol=1e-13)
    zero, _, _ = _bm(w, gate=torch.zeros_like(g))
    assert np.abs(zero).max() == 0.0


def test_bigdn_reverse_qkv_override():
    # the reverse direction's q, k, v and their inverse RMS come from qkv_bwd
    w = _merged_inputs()
    base, num, den = _bm(w)
    # the same tensor as override: the same block
    same, n1, d1 = _bm(w, qkv_bwd=w["qkv"].clone())
    np.testing.assert_array_equal(same, base)
    # q and k scaled by 4 (exact in bf16): the RMS norm of qkv_bwd's own channels removes it
    # (a negligible norm eps, so that the scaling is exactly invisible)
    wt = dict(w, eps=1e-30)
    _, nt, dt = _bm(wt)
    sc = w["qkv"].clone()
    sc[:, :, :2] *= 4
    _, n2, d2 = _bm(wt, qkv_bwd=sc)
    np.testing.assert_allclose(n2, nt, rtol=1e-9, atol=1e-12)
    np.testing.assert_allclose(d2, dt, rtol=1e-9, atol=1e-12)
    # q of qkv_bwd zero: the reverse direction adds nothing to num and den, which then match a
    # reverse direction with beta_bwd = 0 (no state at all)
    zq = w["qkv"].clone()
    zq[:, :, 0] = 0
    _, n3, d3 = _bm(w, qkv_bwd=zq)
    _, n4, d4 = _bm(w, beta_bwd=torch.zeros_like(w["beta"]))
    np.testing.assert_allclose(n3, n4, atol=1e-14)
    np.testing.assert_allclose(d3, d4, atol=1e-14)
    # k and v of qkv_bwd zero: the reverse state stays zero, the same result again
    zkv = w["qkv"].clone()
    zkv[:, :, 1:] = 0
    _, n5, d5 = _bm(w, qkv_bwd=zkv)
    np.testing.assert_allclose(n5, n4, atol=1e-14)
    np.testing.assert_allclose(d5, d4, atol=1e-14)
    assert np.abs(n4 - num).max() > 1e-3

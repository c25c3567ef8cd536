"""Pins of the BiGDN front-end and merge backward oracles (oracle.prep_bwd,
oracle.bigdn_merge_bwd), CPU only.

Every gradient element is checked against central differences of the forward oracles, which
are separate code: oracle.prep (C) for the front end, oracle.bigdn_merge (numpy) for the
merge, and oracle.bigdn_merged (the whole block: front end, both scan directions, merge) for
the composed backward merge -> bigdn_dir_bwd in both directions -> prep_bwd.  Every map
involved is smooth at the drawn inputs (no pre-ReLU value is within 1e-4 of zero, which the
tests assert), so (L(x + e) - L(x - e)) / 2e matches the analytic gradient to about e^2.
"""
import numpy as np
import pytest

import oracle

PREP_OUT = ("q_rot", "k_rot", "q_pos", "k_pos", "v")


def _tables(N, D):
    n = np.arange(N, dtype=np.float64)[:, None]
    i = np.arange(D // 2, dtype=np.float64)[None, :]
    theta = n * np.power(10000.0, -2.0 * i / D)
    cos_t = np.repeat(np.cos(theta), 2, axis=1)
    sin_t = np.stack([-np.sin(theta), np.sin(theta)], axis=-1).reshape(N, D)
    return np.ascontiguousarray(cos_t), np.ascontiguousarray(sin_t)


def _prep_inputs(B, N, H, D, seed):
    rng = np.random.default_rng(seed)
    x = dict(qkv=rng.normal(0, 1.0, (B, N, 3, H, D)), qw=1.0 + 0.3 * rng.normal(0, 1.0, H * D),
             kw=1.0 + 0.3 * rng.normal(0, 1.0, H * D))
    x["cos"], x["sin"] = _tables(N, D)
    return x


def _margin(x, k_scale=0.7, eps=1e-5):
    """Smallest |pre-ReLU value| of q and k (the front end is smooth away from zero)."""
    qkv = x["qkv"]
    C = qkv.shape[3] * qkv.shape[4]
    m = np.inf
    for which, w in ((0, x["qw"]), (1, x["kw"])):
        raw = qkv[:, :, which].reshape(qkv.shape[0], qkv.shape[1], C)
        r = 1.0 / np.sqrt((raw * raw).mean(axis=-1, keepdims=True) + eps)
        m = min(m, float(np.abs(raw * r * w).min()))
    return m


def _prep_loss(x, G, k_scale):
    p = oracle.prep(x["qkv"], x["qw"], x["kw"], x["cos"], x["sin"], k_scale)
    return float(sum((p[n] * G[n].sum(axis=0)).sum() for n in PREP_OUT))


@pytest.mark.parametrize("ndir", [1, 2])
def test_prep_bwd_matches_central_differences(ndir):
    B, N, H, D, k_scale = 1, 3, 2, 4, 0.7
    x = _prep_inputs(B, N, H, D, seed=11 + ndir)
    assert _margin(x, k_scale) > 1e-4
    rng = np.random.default_rng(5 + ndir)
    G = {n: rng.normal(0, 1.0, (ndir, B, H, N, D)) for n in PREP_OUT}
    grads = {"d" + n: G[n] for n in PREP_OUT}
    g = oracle.prep_bwd(x["qkv"], x["qw"], x["kw"], x["cos"], x["sin"], k_scale, grads)
    e = 1e-6
    for name, key in (("qkv", "dqkv"), ("qw", "dq_norm_w"), ("kw", "dk_norm_w")):
        fd = np.zeros_like(x[name])
        for idx in np.ndindex(x[name].shape):
            xp = {k: v.copy() for k, v in x.items()}
            xm = {k: v.copy() for k, v in x.items()}
            xp[name][idx] += e
            xm[name][idx] -= e
            fd[idx] = (_prep_loss(xp, G, k_scale) - _prep_loss(xm, G, k_scale)) / (2 * e)
        np.testing.assert_allclose(g[key], fd, rtol=1e-6, atol=1e-8, err_msg=key)


@pytest.mark.parametrize("gated", [False, True])
def test_merge_bwd_matches_central_differences(gated):
    B, N, H, D, meps = 1, 3, 2, 4, 1e-6
    rng = np.random.default_rng(21 + int(gated))
    x = dict(num=rng.normal(0, 1.0, (B, N, H, D)), den=rng.uniform(0.5, 2.0, (B, H, N)),
             gate=rng.normal(0, 1.0, (B, N, H, D)) if gated else None)
    dout = rng.normal(0, 1.0, (B, N, H, D))
    loss = lambda y: float((oracle.bigdn_merge(y["num"], y["den"], y["gate"], meps) * dout).sum())
    g = oracle.bigdn_merge_bwd(x["num"], x["den"], dout, x["gate"], meps)
    e = 1e-6
    for name in ("num", "den", "gate"):
        if x[name] is None:
            assert g["d" + name] is None
            continue
        fd = np.zeros_like(x[name])
        for idx in np.ndindex(x[name].shape):
            xp = {k: (None if v is None else v.copy()) for k, v in x.items()}
            xm = {k: (None if v is None else v.copy()) for k, v in x.items()}
            xp[name][idx] += e
            xm[name][idx] -= e
            fd[idx] = (loss(xp) - loss(xm)) / (2 * e)
        np.testing.assert_allclose(g["d" + name], fd, rtol=1e-6, atol=1e-8, err_msg=name)


def _block_backward(x, dout, k_scale, meps):
    """Composed backward of the whole block from the oracle's backward pieces."""
    p = oracle.prep(x["qkv"], x["qw"], x["kw"], x["cos"], x["sin"], k_scale)
    t = [p[n] for n in PREP_OUT]
    _, num, den = oracle.bigdn_merged(x["qkv"], x["beta"], x["decay"], x["qw"], x["kw"], x["cos"],
                                      x["sin"], k_scale, gate=x["gate"], merge_eps=meps)
    m = oracle.bigdn_merge_bwd(num, den, dout, x["gate"], meps)
    dirs = [oracle.bigdn_dir_bwd(*t, x["beta"], x["decay"], m["dnum"], m["dden"], reverse=r)
            for r in (False, True)]
    grads = {"d" + n: np.stack([d["d" + n] for d in dirs]) for n in PREP_OUT}
    g = oracle.prep_bwd(x["qkv"], x["qw"], x["kw"], x["cos"], x["sin"], k_scale, grads)
    return dict(qkv=g["dqkv"], qw=g["dq_norm_w"], kw=g["dk_norm_w"],
                beta=dirs[0]["dbeta"] + dirs[1]["dbeta"],
                decay=dirs[0]["ddecay"] + dirs[1]["ddecay"], gate=m["dgate"])


def test_whole_block_backward_matches_central_differences():
    """merge_bwd -> bigdn_dir_bwd (both directions) -> prep_bwd against central differences of
    the block forward oracle.bigdn_merged, for every input: qkv, norm weights, beta, decay and
    the gate."""
    B, F, S, H, D, k_scale, meps = 1, 2, 2, 2, 4, 0.7, 1e-6
    N = F * S
    x = _prep_inputs(B, N, H, D, seed=31)
    assert _margin(x, k_scale) > 1e-4
    rng = np.random.default_rng(32)
    x["beta"] = rng.uniform(0.2, 0.9, (B, H, F, S))
    x["decay"] = rng.uniform(0.4, 1.0, (B, H, F))
    x["gate"] = rng.normal(0, 1.0, (B, N, H, D))
    dout = rng.normal(0, 1.0, (B, N, H, D))

    def loss(y):
        out, _, _ = oracle.bigdn_merged(y["qkv"], y["beta"], y["decay"], y["qw"], y["kw"],
                                        y["cos"], y["sin"], k_scale, gate=y["gate"], merge_eps=meps)
        return float((out * dout).sum())

    g = _block_backward(x, dout, k_scale, meps)
    e = 1e-6
    for name in ("qkv", "qw", "kw", "beta", "decay", "gate"):
        fd = np.zeros_like(x[name])
        for idx in np.ndindex(x[name].shape):
            xp = {k: v.copy() for k, v in x.items()}
            xm = {k: v.copy() for k, v in x.items()}
            xp[name][idx] += e
            xm[name][idx] -= e
            fd[idx] = (loss(xp) - loss(xm)) / (2 * e)
        np.testing.assert_allclose(g[name], fd, rtol=1e-5, atol=1e-7, err_msg=name)

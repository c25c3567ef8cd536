"""GPU parity of the fragment state summary (gdn_state_summary) and of joining fragments
(gdn_state_apply) against the fp64 oracle, through the C ABI."""
import numpy as np
import pytest
import torch

import oracle
import workloads
from tests.gpu_util import TOL, assert_close, say

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def _gpu():
    import gated_delta_rule_29_amd as g
    return g


def _to(d, dev=DEV):
    return {k: (v.to(dev) if isinstance(v, torch.Tensor) else v) for k, v in d.items()}


def _cut(inp, a, b):
    return {k: (v[:, a:b].contiguous() if isinstance(v, torch.Tensor) else v) for k, v in inp.items()}


@pytest.mark.parametrize("dtype,K,V,T,per_key", [("bf16", 128, 128, 300, False),
                                                 ("bf16", 64, 128, 131, False),
                                                 ("bf16", 128, 64, 64, True),
                                                 ("bf16", 128, 128, 1, False),
                                                 ("f32", 64, 128, 190, False),
                                                 ("f32", 64, 64, 77, False)])
def test_summary_parity(dtype, K, V, T, per_key):
    g = _gpu()
    inp = workloads.gdn_inputs(2, T, 3, K, V, dtype=dtype, seed=T + K + V, g_shift=3.0,
                               per_key=per_key)
    say("summary %s K%d V%d T%d pk%d" % (dtype, K, V, T, per_key))
    d = _to(inp)
    st, tr = g.gdn_state_summary(d["k"], d["v"], d["beta"], g=d["g"], gk=d["gk"])
    torch.cuda.synchronize()
    ref = oracle.state_summary(inp["k"], inp["v"], inp["beta"], g=inp["g"], gk=inp["gk"])
    tol = TOL[inp["k"].dtype]
    assert_close("state_ext", st, ref["state_ext"], tol)
    _check_transition("transition", tr, ref["transition"], tol)
    st2, tr2 = g.gdn_state_summary(d["k"], d["v"], d["beta"], g=d["g"], gk=d["gk"],
                                   want_transition=False)
    torch.cuda.synchronize()
    assert tr2 is None
    assert torch.equal(st2, st)


@pytest.mark.parametrize("dtype,per_key", [("bf16", False), ("bf16", True), ("f32", False)])
def test_fragments_join_to_the_whole_run(dtype, per_key):
    """A chain cut into ragged fragments: summaries joined in order give the whole run's final
    state, and the last fragment re-run from the joined state gives the whole run's output
    on its tokens."""
    g = _gpu()
    K, V, T = (128, 128, 700) if dtype == "bf16" else (64, 64, 700)
    cuts = [0, 190, 449, 700]
    inp = workloads.gdn_inputs(1, T, 2, K, V, dtype=dtype, seed=77, g_shift=3.0, per_key=per_key)
    say("join %s pk%d cuts %s" % (dtype, per_key, cuts))
    d = _to(inp)
    h = None
    for a, b in zip(cuts[:-2], cuts[1:-1]):
        f = _cut(d, a, b)
        st, tr = g.gdn_state_summary(f["k"], f["v"], f["beta"], g=f["g"], gk=f["gk"])
        h = g.gdn_state_apply(st, tr, h)
    last = _cut(d, cuts[-2], cuts[-1])
    out = g.gdn_fwd(last["q"], last["k"], last["v"], last["beta"], g=last["g"], gk=last["gk"],
                    h0=h)
    torch.cuda.synchronize()
    ref = oracle.gdn(inp["q"], inp["k"], inp["v"], inp["beta"], g=inp["g"], gk=inp["gk"],
                     want_h=False)
    tol = TOL[inp["k"].dtype]
    assert_close("ht", out["ht"], ref["ht"], tol)
    assert_close("o(last fragment)", out["o"], ref["o"][:, cuts[-2]:], tol)


def test_apply_is_affine_map():
    g = _gpu()
    gen = torch.Generator().manual_seed(5)
    for K, V, BH in ((128, 128, 6), (64, 128, 3), (48, 80, 2)):
        c = torch.randn(BH, K, V, generator=gen)
        M = torch.randn(BH, K, K, generator=gen) / K ** 0.5
        h = torch.randn(BH, K, V, generator=gen)
        out = g.gdn_state_apply(c.to(DEV), M.to(DEV), h.to(DEV))
        out0 = g.gdn_state_apply(c.to(DEV), M.to(DEV), None)
        torch.cuda.synchronize()
        ref = np.matmul(M.double().numpy(), h.double().numpy()) + c.double().numpy()
        assert_close("apply K%d V%d" % (K, V), out, ref, 1e-5)
        assert torch.equal(out0.cpu(), c)


def _check_transition(name, got, ref, tol):
    """Transitions decay like the product of all of a fragment's decays; where the exact
    value is below the fp32 range the stored fp32 result must be (nearly) zero instead."""
    if np.abs(ref).max() < 1e-36:
        assert float(got.abs().max()) <= 1e-36, name
        print("  %-10s below fp32 range (oracle max %.1e), stored max %.1e" % (
            name, np.abs(ref).max(), float(got.abs().max())), flush=True)
    else:
        assert_close(name, got, ref, tol)


@pytest.mark.parametrize("g_shift", [3.0, 8.0])
def test_summary_at_the_dense_bf16_workload_shape_sampled(g_shift):
    """B=4 H=16 T=4096 K=V=128 bf16: the summary of every chain (all finite), checked against
    the oracle on 16 sampled chains.  g_shift 3 is the dense bf16 workload itself (its transitions are
    far below fp32 range); g_shift 8 keeps the total decay of 4096 tokens representable."""
    g = _gpu()
    inp = workloads.gdn_inputs(4, 4096, 16, 128, 128, dtype="bf16", seed=0, g_shift=g_shift)
    d = _to(inp)
    say("summary at B4 H16 T4096, g_shift %.0f" % g_shift)
    st, tr = g.gdn_state_summary(d["k"], d["v"], d["beta"], g=d["g"])
    torch.cuda.synchronize()
    assert bool(torch.isfinite(st).all()) and bool(torch.isfinite(tr).all())
    for b, h in [(b, h) for b in range(4) for h in (0, 5, 11, 15)]:
        sl = lambda x: x[b:b + 1, :, h:h + 1]
        ref = oracle.state_summary(sl(inp["k"]), sl(inp["v"]), sl(inp["beta"]), g=sl(inp["g"]))
        assert_close("state_ext[%d,%d]" % (b, h), st[b, h], ref["state_ext"][0, 0],
                     TOL[torch.bfloat16])
        _check_transition("transition[%d,%d]" % (b, h), tr[b, h], ref["transition"][0, 0],
                          TOL[torch.bfloat16])

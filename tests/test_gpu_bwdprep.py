"""GPU parity of the backward's inputs (gdn_bwd_prep: the WY w and P^T do per chunk), of the
chain forward inputs -> gdn_bwd_prep -> gdn_bwd_dhu, and of the reverse (gradient) state
summary joined over fragments, against the fp64 oracle through the C ABI.

gdn_bwd_prep's products take split bf16 operands, so its outputs are held to the
split-operand rule (SPLIT_OPERAND_TOL) after their own storage rounding; anything that then
passes through gdn_bwd_dhu (fp16 operands for bf16 inputs) is held to that pass's rule."""
import numpy as np
import pytest
import torch

import oracle
import workloads
from tests.gpu_util import SPLIT_OPERAND_TOL, TOL, assert_close, say

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _gpu():
    import gated_delta_rule_29_amd as g
    return g


def _to(d):
    return {k: (v.to(DEV) if isinstance(v, torch.Tensor) else v) for k, v in d.items()}


@pytest.mark.parametrize("dtype,K,V,T,gated", [("bf16", 128, 128, 300, True),
                                               ("bf16", 128, 64, 64, True),
                                               ("bf16", 64, 128, 131, False),
                                               ("f32", 64, 64, 77, True),
                                               ("f32", 128, 128, 200, True),
                                               ("bf16", 128, 128, 1, True)])
def test_bwd_prep_parity(dtype, K, V, T, gated):
    g = _gpu()
    inp = workloads.bwd_inputs(2, T, 3, K, V, dtype=dtype, seed=T + K + V)
    if not gated:
        inp["g"] = None
    say("bwd_prep %s K%d V%d T%d gated %s" % (dtype, K, V, T, gated))
    d = _to(inp)
    w, dv = g.gdn_bwd_prep(d["q"], d["k"], d["beta"], d["do"], g=d["g"], scale=inp["scale"])
    torch.cuda.synchronize()
    rw, rdv = oracle.gdn_bwd_prep(inp["q"], inp["k"], inp["beta"], inp["do"], g=inp["g"],
                                  scale=inp["scale"])
    assert_close("w", w, rw, SPLIT_OPERAND_TOL)
    assert_close("dv", dv, rdv, SPLIT_OPERAND_TOL)


def test_bwd_prep_refuses_per_key_gates():
    g = _gpu()
    inp = _to(workloads.bwd_inputs(1, 64, 1, 128, 128, seed=1))
    gk = torch.zeros(1, 64, 1, 128, device=DEV)
    with pytest.raises(NotImplementedError):
        g.gdn_bwd_prep(inp["q"], inp["k"], inp["beta"], inp["do"], g=inp["g"], gk=gk)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_forward_inputs_to_state_gradients(dtype):
    """w and P^T do from gdn_bwd_prep feed gdn_bwd_dhu: dh0 and every chunk's dh against the
    oracle's pass fed by the oracle's w and P^T do (whose dh0 is dL/dh0 of the forward)."""
    g = _gpu()
    inp = workloads.bwd_inputs(2, 300, 2, 128, 128, dtype=dtype, seed=11)
    d = _to(inp)
    say("forward inputs -> gdn_bwd_prep -> gdn_bwd_dhu (%s)" % dtype)
    w, dv = g.gdn_bwd_prep(d["q"], d["k"], d["beta"], d["do"], g=d["g"], scale=inp["scale"])
    r = g.gdn_bwd_dhu(d["q"], d["k"], w, d["do"], dv, g=d["g"], dht=d["dht"], scale=inp["scale"])
    torch.cuda.synchronize()
    rw, rdv = oracle.gdn_bwd_prep(inp["q"], inp["k"], inp["beta"], inp["do"], g=inp["g"],
                                  scale=inp["scale"])
    ref = oracle.gdn_dhu(inp["q"], inp["k"], rw, inp["do"], rdv, g=inp["g"], dht=inp["dht"],
                         scale=inp["scale"])
    tol = TOL[inp["q"].dtype]
    assert_close("dh0", r["dh0"], ref["dh0"], tol)
    assert_close("dh", r["dh"], ref["dh"], tol)


def test_gradient_summaries_join_to_the_whole_run():
    """A chain cut into ragged fragments: each fragment's gradient summary (gdn_bwd_prep on the
    fragment, then gdn_state_grad_summary), joined from the right with gdn_state_grad_apply and
    the fragment's forward transition, gives the whole run's dL/dh0."""
    g = _gpu()
    T, cuts = 700, [0, 190, 449, 700]
    inp = workloads.bwd_inputs(1, T, 2, 128, 128, dtype="bf16", seed=77)
    d = _to(inp)
    say("gradient summaries, cuts %s" % cuts)
    g_in = d["dht"]
    for a, b in reversed(list(zip(cuts[:-1], cuts[1:]))):
        f = {k: (v[:, a:b].contiguous() if isinstance(v, torch.Tensor) and k != "dht" else v)
             for k, v in d.items()}
        w, dv = g.gdn_bwd_prep(f["q"], f["k"], f["beta"], f["do"], g=f["g"], scale=inp["scale"])
        ext = g.gdn_state_grad_summary(f["q"], f["k"], w, f["do"], dv, g=f["g"],
                                       scale=inp["scale"])
        _, M = g.gdn_state_summary(f["k"], f["v"], f["beta"], g=f["g"])
        g_in = g.gdn_state_grad_apply(ext, M, g_in)
    torch.cuda.synchronize()
    rw, rdv = oracle.gdn_bwd_prep(inp["q"], inp["k"], inp["beta"], inp["do"], g=inp["g"],
                                  scale=inp["scale"])
    ref = oracle.gdn_dhu(inp["q"], inp["k"], rw, inp["do"], rdv, g=inp["g"], dht=inp["dht"],
                         scale=inp["scale"])
    assert_close("dh0 (joined)", g_in, ref["dh0"], TOL[torch.bfloat16])


def test_grad_apply_is_the_transposed_map():
    g = _gpu()
    gen = torch.Generator().manual_seed(9)
    for K, V, BH in ((128, 128, 6), (64, 128, 3), (48, 80, 2)):
        c = torch.randn(BH, K, V, generator=gen)
        M = torch.randn(BH, K, K, generator=gen) / K ** 0.5
        h = torch.randn(BH, K, V, generator=gen)
        out = g.gdn_state_grad_apply(c.to(DEV), M.to(DEV), h.to(DEV))
        out0 = g.gdn_state_grad_apply(c.to(DEV), M.to(DEV), None)
        torch.cuda.synchronize()
        ref = np.matmul(np.swapaxes(M.double().numpy(), 1, 2), h.double().numpy()) + c.double().numpy()
        assert_close("grad apply K%d V%d" % (K, V), out, ref, 1e-5)
        assert torch.equal(out0.cpu(), c)

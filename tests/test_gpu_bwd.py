"""GPU parity of the state-gradient pass (gdn_bwd_dhu) against the fp64 oracle, through the C
ABI.  fp32 inputs: fp32 arithmetic, 1e-4 * RMS.  bf16 inputs: fp16 matrix-core operands (dh
and dv2 rounded to fp16 where they enter a product) with fp32 accumulation, held to the
fp16-operand rule; dv2 stored in bf16 under the storage rule."""
import numpy as np
import pytest
import torch

import oracle
import workloads
from tests.gpu_util import FP16_OPERAND_TOL, assert_close, say

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _dev(w):
    return {k: (v.to(DEV) if isinstance(v, torch.Tensor) else v) for k, v in w.items()}


@pytest.mark.parametrize("B,T,H,V,dtype,gated,final,per_key",
                         [(1, 200, 2, 64, "f32", True, True, False),
                          (2, 128, 3, 32, "bf16", False, False, False),
                          (1, 64, 1, 128, "f32", True, False, False),
                          (1, 1, 2, 32, "bf16", True, True, False),
                          (1, 333, 2, 96, "bf16", True, True, False),
                          (1, 200, 2, 64, "bf16", True, True, True),
                          (2, 130, 3, 32, "bf16", False, False, True)])
def test_dhu(B, T, H, V, dtype, gated, final, per_key):
    import gated_delta_rule_29_amd as g

    w = workloads.dhu_inputs(B, T, H, 128, V, dtype=dtype, seed=T + V, per_key=per_key)
    gg = w["g"] if gated else None
    dht = w["dht"] if final else None
    say("dhu B%d T%d H%d V%d %s gated%d final%d per_key%d" % (B, T, H, V, dtype, gated, final,
                                                              per_key))
    d = _dev(w)
    r = g.gdn_bwd_dhu(d["q"], d["k"], d["w"], d["do"], d["dv"], g=None if gg is None else d["g"],
                      dht=None if dht is None else d["dht"], scale=w["scale"],
                      gk=d["gk"] if per_key else None)
    torch.cuda.synchronize()
    ref = oracle.gdn_dhu(w["q"], w["k"], w["w"], w["do"], w["dv"], g=gg, dht=dht,
                         scale=w["scale"], gk=w["gk"])
    tol = 1e-4 if dtype == "f32" else FP16_OPERAND_TOL
    for name in ("dv2", "dh", "dh0"):
        assert_close(name, r[name], ref[name], tol)


def test_dhu_workload_sampled():
    """The dense bf16 shape (B4 H16 T4096 V128) in the launch configuration the benchmark
    times; chains (0, 0), (1, 7) and (3, 15) against the oracle."""
    import gated_delta_rule_29_amd as g

    w = workloads.make("dhu_bf16_b4h16t4096")
    say("dhu workload")
    d = _dev(w)
    r = g.gdn_bwd_dhu(d["q"], d["k"], d["w"], d["do"], d["dv"], g=d["g"], dht=d["dht"],
                      scale=w["scale"])
    torch.cuda.synchronize()
    for b, h in ((0, 0), (1, 7), (3, 15)):
        sl = lambda x: x[b:b + 1, :, h:h + 1]
        ref = oracle.gdn_dhu(sl(w["q"]), sl(w["k"]), sl(w["w"]), sl(w["do"]), sl(w["dv"]),
                             g=sl(w["g"]), dht=w["dht"][b:b + 1, h:h + 1], scale=w["scale"])
        tol = FP16_OPERAND_TOL
        assert_close("dv2 %d,%d" % (b, h), r["dv2"][b:b + 1, :, h:h + 1], ref["dv2"], tol)
        assert_close("dh %d,%d" % (b, h), r["dh"][b:b + 1, h:h + 1], ref["dh"], tol)
        assert_close("dh0 %d,%d" % (b, h), r["dh0"][b:b + 1, h:h + 1], ref["dh0"], tol)


@pytest.mark.parametrize("dtype,per_key", [("f32", False), ("bf16", False), ("bf16", True)])
def test_dhu_varlen(dtype, per_key):
    """Packed sequences (1, 70, 128, 200 and 5 tokens): every sequence against the oracle run
    on it alone, and bit for bit equal to the dense pass run on each sequence separately."""
    import gated_delta_rule_29_amd as g

    lens = [1, 70, 128, 200, 5]
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    T, H, V = int(cu[-1]), 2, 64
    w = workloads.dhu_inputs(1, T, H, 128, V, dtype=dtype, seed=11, per_key=per_key)
    gk = d_gk = None
    dht = torch.randn(len(lens), H, 128, V, generator=torch.Generator().manual_seed(3))
    say("dhu varlen %s lengths %s" % (dtype, lens))
    d = _dev(w)
    if per_key:
        gk, d_gk = w["gk"], d["gk"]
    r = g.gdn_bwd_dhu_varlen(d["q"], d["k"], d["w"], d["do"], d["dv"], torch.from_numpy(cu),
                             g=d["g"], dht=dht.to(DEV), scale=w["scale"], gk=d_gk)
    torch.cuda.synchronize()
    tol = 1e-4 if dtype == "f32" else FP16_OPERAND_TOL
    c0 = 0
    for i, L in enumerate(lens):
        sl = slice(int(cu[i]), int(cu[i + 1]))
        nt = (L + 63) // 64
        ref = oracle.gdn_dhu(w["q"][:, sl], w["k"][:, sl], w["w"][:, sl], w["do"][:, sl],
                             w["dv"][:, sl], g=w["g"][:, sl], dht=dht[i:i + 1], scale=w["scale"],
                             gk=None if gk is None else gk[:, sl])
        assert_close("dv2 s%d" % i, r["dv2"][:, sl], ref["dv2"], tol)
        assert_close("dh s%d" % i, r["dh"][:, :, c0:c0 + nt], ref["dh"], tol)
        assert_close("dh0 s%d" % i, r["dh0"][i:i + 1], ref["dh0"], tol)
        one = g.gdn_bwd_dhu(d["q"][:, sl].contiguous(), d["k"][:, sl].contiguous(),
                            d["w"][:, sl].contiguous(), d["do"][:, sl].contiguous(),
                            d["dv"][:, sl].contiguous(), g=d["g"][:, sl].contiguous(),
                            dht=dht[i:i + 1].to(DEV), scale=w["scale"],
                            gk=None if d_gk is None else d_gk[:, sl].contiguous())
        torch.cuda.synchronize()
        assert torch.equal(one["dv2"], r["dv2"][:, sl])
        assert torch.equal(one["dh"], r["dh"][:, :, c0:c0 + nt])
        assert torch.equal(one["dh0"], r["dh0"][i:i + 1])
        c0 += nt


def test_dhu_perkey_workload_sampled():
    """The long-context per-key shape (B2 H32 T32768 V128, bf16, per-key gates) in the launch
    configuration the benchmark times; chains (0, 0) and (1, 31) against the oracle."""
    import gated_delta_rule_29_amd as g

    w = workloads.make("dhu_perkey_b2h32t32768")
    say("dhu per-key workload")
    d = _dev(w)
    r = g.gdn_bwd_dhu(d["q"], d["k"], d["w"], d["do"], d["dv"], g=d["g"], dht=d["dht"],
                      scale=w["scale"], gk=d["gk"])
    torch.cuda.synchronize()
    for b, h in ((0, 0), (1, 31)):
        sl = lambda x: x[b:b + 1, :, h:h + 1]
        ref = oracle.gdn_dhu(sl(w["q"]), sl(w["k"]), sl(w["w"]), sl(w["do"]), sl(w["dv"]),
                             g=sl(w["g"]), dht=w["dht"][b:b + 1, h:h + 1], scale=w["scale"],
                             gk=sl(w["gk"]))
        tol = FP16_OPERAND_TOL
        assert_close("dv2 %d,%d" % (b, h), r["dv2"][b:b + 1, :, h:h + 1], ref["dv2"], tol)
        assert_close("dh %d,%d" % (b, h), r["dh"][b:b + 1, h:h + 1], ref["dh"], tol)
        assert_close("dh0 %d,%d" % (b, h), r["dh0"][b:b + 1, h:h + 1], ref["dh0"], tol)


def test_dhu_deterministic():
    """Two identical calls give bitwise-identical outputs (no atomics anywhere)."""
    import gated_delta_rule_29_amd as g

    w = _dev(workloads.dhu_inputs(2, 300, 3, 128, 64, seed=5, per_key=True))
    args = (w["q"], w["k"], w["w"], w["do"], w["dv"])
    ra = g.gdn_bwd_dhu(*args, g=w["g"], dht=w["dht"], scale=w["scale"], gk=w["gk"])
    rb = g.gdn_bwd_dhu(*args, g=w["g"], dht=w["dht"], scale=w["scale"], gk=w["gk"])
    torch.cuda.synchronize()
    for key in ("dv2", "dh", "dh0"):
        assert torch.equal(ra[key], rb[key])

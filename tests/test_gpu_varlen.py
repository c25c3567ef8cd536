"""GPU parity of gdn_fwd_varlen (packed sequences) against the fp64 oracle."""
import numpy as np
import pytest
import torch

import oracle
import workloads
from tests.gpu_util import TOL, assert_close, say

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _run(inp, h0=None, want_h=True, label=""):
    import gated_delta_rule_29_amd as g

    say("case %s: T_total %d, N %d" % (label, inp["q"].shape[1], inp["cu_seqlens"].numel() - 1))
    d = {k: (v.to(DEV) if isinstance(v, torch.Tensor) else v) for k, v in inp.items()}
    out = g.gdn_fwd_varlen(d["q"], d["k"], d["v"], d["beta"], d["cu_seqlens"], g=d["g"],
                           gk=d["gk"], h0=None if h0 is None else h0.to(DEV), want_h=want_h,
                           want_v_new=want_h)
    torch.cuda.synchronize()
    cu = inp["cu_seqlens"].numpy()
    ref = oracle.gdn_varlen(cu, inp["q"], inp["k"], inp["v"], inp["beta"], g=inp["g"],
                            gk=inp["gk"], h0=h0, want_h=want_h, want_vnew=want_h)
    offs, idx = oracle.varlen_tables(cu)
    assert np.array_equal(out["chunk_offsets"].cpu().numpy(), offs)
    assert np.array_equal(out["chunk_indices"].cpu().numpy(), idx)
    tol = TOL[inp["q"].dtype]
    assert_close("o", out["o"], ref["o"], tol)
    assert_close("ht", out["ht"], ref["ht"], tol)
    if want_h:
        assert_close("h", out["h"], ref["h"], tol)
        assert_close("v_new", out["v_new"], ref["v_new"], tol)
    return out


@pytest.mark.parametrize("want_h", [True, False])
@pytest.mark.parametrize("lengths,K,dtype", [([1, 64, 65, 200, 7], 128, "bf16"),
                                             ([130, 3, 64], 64, "bf16"),
                                             # 24 sequences x 3 heads: longest-first order dealt
                                             # round-robin to the XCDs (72 chains)
                                             ([37, 300, 5, 64, 129, 1, 250, 77, 64, 190, 12, 3,
                                               280, 65, 99, 140, 2, 31, 222, 128, 45, 160, 9, 300],
                                              128, "bf16"),
                                             ([100, 28, 129], 64, "f32")])
def test_packed_small(lengths, K, dtype, want_h):
    """Packed sequences with h0; with and without saved h / v_new (bf16 without saves runs
    the single-kernel path)."""
    gen = torch.Generator().manual_seed(sum(lengths))
    cu = torch.zeros(len(lengths) + 1, dtype=torch.int32)
    cu[1:] = torch.cumsum(torch.tensor(lengths), 0)
    T = int(cu[-1])
    inp = workloads.gdn_inputs(1, T, 3, K, 128, dtype=dtype, seed=len(lengths), g_shift=2.0)
    inp["cu_seqlens"] = cu
    h0 = torch.randn(len(lengths), 3, K, 128, generator=gen) * 0.3
    _run(inp, h0=h0, want_h=want_h, label="lengths %s K%d %s saves %s" % (lengths, K, dtype, want_h))


def test_packed_equals_separate_runs_bitwise():
    """Each packed sequence gives bit-identical results to a dense call on that sequence."""
    import gated_delta_rule_29_amd as g

    lengths = [90, 64, 1, 150]
    cu = torch.zeros(5, dtype=torch.int32)
    cu[1:] = torch.cumsum(torch.tensor(lengths), 0)
    inp = workloads.gdn_inputs(1, int(cu[-1]), 2, 128, 128, dtype="bf16", seed=9)
    d = {k: (v.to(DEV) if isinstance(v, torch.Tensor) else v) for k, v in inp.items()}
    packed = g.gdn_fwd_varlen(d["q"], d["k"], d["v"], d["beta"], cu, g=d["g"])
    for i in range(4):
        a, b = int(cu[i]), int(cu[i + 1])
        sl = lambda x: x[:, a:b].contiguous()
        one = g.gdn_fwd(sl(d["q"]), sl(d["k"]), sl(d["v"]), sl(d["beta"]), g=sl(d["g"]))
        torch.cuda.synchronize()
        assert torch.equal(packed["o"][:, a:b], one["o"])
        assert torch.equal(packed["ht"][i], one["ht"][0])


def test_varlen_workload_full():
    """8 sequences with lengths uniform in [512, 8192], H=16, K=V=128, bf16: every element."""
    inp = workloads.make("varlen_bf16_8seq")
    _run(inp, want_h=False, label="varlen_bf16_8seq")


@pytest.mark.parametrize("want_h", [True, False])
def test_packed_per_key_strong_decay(want_h):
    """Packed sequences with a fast-forgetting per-key gate (gk = logsigmoid(N(0,1) - 2)) and a
    per-key reset (gk = -30) inside a chunk, with and without saves."""
    lengths = [70, 1, 200, 64, 33]
    cu = torch.zeros(len(lengths) + 1, dtype=torch.int32)
    cu[1:] = torch.cumsum(torch.tensor(lengths), 0)
    T = int(cu[-1])
    inp = workloads.gdn_inputs(1, T, 2, 128, 128, dtype="bf16", seed=41, g_shift=3.0,
                               per_key=True, gk_shift=-2.0)
    inp["gk"][0, 150] = -30.0
    inp["cu_seqlens"] = cu
    h0 = torch.randn(len(lengths), 2, 128, 128, generator=torch.Generator().manual_seed(5)) * 0.3
    _run(inp, h0=h0, want_h=want_h, label="packed per-key strong decay saves %s" % want_h)

"""gdn_fwd_varlen_noalloc (the packed forward whose scratch is the library's static device
array, for callers that cannot allocate) against gdn_fwd_varlen, through the C ABI: two
calls in a row, the second with a smaller input, on the single-kernel path and on the
two-kernel path (per-key gate, saved h and v_new).  Results must be bitwise equal (the same
kernels run on the same inputs), and the first call is also checked against the oracle."""
import pytest
import torch

import oracle
import workloads
from tests.gpu_util import TOL, assert_close, say

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _packed(lengths, H, per_key, seed):
    cu = torch.zeros(len(lengths) + 1, dtype=torch.int32)
    cu[1:] = torch.cumsum(torch.tensor(lengths), 0)
    inp = workloads.gdn_inputs(1, int(cu[-1]), H, 128, 128, dtype="bf16", seed=seed,
                               g_shift=2.0, per_key=per_key, gk_shift=0.0)
    inp["cu_seqlens"] = cu
    return inp


def _both(inp, saves):
    import gated_delta_rule_29_amd as g

    d = {k: (v.to(DEV) if isinstance(v, torch.Tensor) else v) for k, v in inp.items()}
    cu_host = inp["cu_seqlens"]
    kw = dict(g=d["g"], gk=d["gk"], want_h=saves, want_v_new=saves, cu_seqlens_host=cu_host)
    ref = g.gdn_fwd_varlen(d["q"], d["k"], d["v"], d["beta"], d["cu_seqlens"], **kw)
    out = g.gdn_fwd_varlen(d["q"], d["k"], d["v"], d["beta"], d["cu_seqlens"], no_alloc=True,
                           **kw)
    torch.cuda.synchronize()
    for name, t in ref.items():
        assert torch.equal(out[name], t), "%s differs from gdn_fwd_varlen" % name
    return out


@pytest.mark.parametrize("per_key", [False, True])
def test_noalloc_matches_gdn_fwd_varlen(per_key):
    saves = per_key
    big = _packed([300, 64, 1, 129, 200], 4, per_key, seed=51)
    small = _packed([70, 5], 2, per_key, seed=52)
    say("noalloc %s: first call %d tokens" % ("two-kernel" if per_key else "single-kernel",
                                             big["q"].shape[1]))
    out = _both(big, saves)
    ref = oracle.gdn_varlen(big["cu_seqlens"].numpy(), big["q"], big["k"], big["v"], big["beta"],
                            g=big["g"], gk=big["gk"], want_h=saves, want_vnew=saves)
    assert_close("o", out["o"], ref["o"], TOL[torch.bfloat16])
    assert_close("ht", out["ht"], ref["ht"], TOL[torch.bfloat16])
    say("second call, %d tokens" % small["q"].shape[1])
    _both(small, saves)


def test_noalloc_rejects_beyond_its_scratch():
    """A per-key call whose per-chunk slots exceed the static scratch is refused before any
    launch, with a message naming the limit."""
    import gated_delta_rule_29_amd as g

    inp = _packed([64 * 40] * 4, 4, True, seed=53)  # 4 heads x 160 chunks x 74 KB > 32 MiB
    d = {k: (v.to(DEV) if isinstance(v, torch.Tensor) else v) for k, v in inp.items()}
    with pytest.raises(ValueError, match="static scratch"):
        g.gdn_fwd_varlen(d["q"], d["k"], d["v"], d["beta"], d["cu_seqlens"], g=d["g"], gk=d["gk"],
                         cu_seqlens_host=inp["cu_seqlens"], no_alloc=True)

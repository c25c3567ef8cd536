"""CPU-only checks of the C ABI: the library loads, exports every declared entry point, and
rejects bad arguments before launching anything (no GPU is touched by these calls)."""
import ctypes
import os
import re

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _lib():
    from gated_delta_rule_29_amd import _lib as L

    return L, L.load()


def _declared():
    names = []
    for path in sorted(os.listdir(os.path.join(ROOT, "include"))):
        if path.endswith(".h"):
            # every declaration (not the macro's own definition): GDN_API <return type> <name>(
            src = "\n".join(l for l in open(os.path.join(ROOT, "include", path))
                            if not l.lstrip().startswith("#"))
            names += re.findall(r"GDN_API\s+(?:const\s+)?\w+\s*\**\s*([A-Za-z]\w*)\s*\(", src)
    return names


def test_exports_every_declared_symbol():
    L, lib = _lib()
    names = _declared()
    assert len(names) >= 22
    for n in ("cam_prep", "cam_scan", "cam_scan_bidi", "gdn_bwd_dhu", "bigdn_fwd_merged"):
        assert n in names, n
    for n in names:
        assert hasattr(lib, n), n
        assert n in L.SIGNATURES, "binding lacks %s" % n
    assert lib.gdn_abi_version() == 6


FAKE = ctypes.c_void_p(0x1000)  # never dereferenced: every call below fails validation first


def _fwd(lib, **kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, g=None, gk=None, beta=FAKE, scale=1.0, h0=None, o=FAKE,
             ht=None, hch=None, vn=None, B=1, T=64, H=2, K=128, V=128, dtype=1)
    a.update(kw)
    return lib.gdn_fwd(a["q"], a["k"], a["v"], a["g"], a["gk"], a["beta"], a["scale"], a["h0"],
                       a["o"], a["ht"], a["hch"], a["vn"], a["B"], a["T"], a["H"], a["K"], a["V"],
                       a["dtype"], None, 0, None)


def test_fwd_validation_codes():
    L, lib = _lib()
    assert _fwd(lib, q=None) == L.ERR_INVALID
    assert "non-null" in L.last_error()
    assert _fwd(lib, T=0) == L.ERR_INVALID
    assert _fwd(lib, B=-1) == L.ERR_INVALID
    assert _fwd(lib, dtype=7) == L.ERR_INVALID
    assert _fwd(lib, K=32) == L.ERR_UNSUPPORTED
    assert _fwd(lib, V=96) == L.ERR_UNSUPPORTED
    assert _fwd(lib, dtype=0, K=128) == L.ERR_UNSUPPORTED
    assert _fwd(lib, B=1 << 20, H=1 << 12) == L.ERR_INVALID  # grid too large


def test_fwd_workspace_sizes_follow_the_flags():
    """The single fused kernel (bf16, no per-key gate, nothing saved) needs no workspace for
    a dense call and only its rank table (4 bytes per sequence, 256-byte rounded) for a packed
    one; per-key gates, saves and fp32 need per-chunk slots."""
    L, lib = _lib()
    PK, SV = L.FWD_PER_KEY, L.FWD_SAVES
    assert lib.gdn_fwd_workspace_bytes(2, 300, 4, 128, 128, 1, 0) == 0
    n_pk = lib.gdn_fwd_workspace_bytes(2, 300, 4, 128, 128, 1, PK)
    n_sv = lib.gdn_fwd_workspace_bytes(2, 300, 4, 128, 128, 1, SV)
    assert n_pk > n_sv > 0 and n_pk == lib.gdn_fwd_workspace_bytes(2, 300, 4, 128, 128, 1, PK | SV)
    assert n_sv % (2 * 4 * 5) == 0  # one slot per chunk: B * H * ceil(300 / 64)
    assert lib.gdn_fwd_workspace_bytes(1, 64, 2, 64, 64, 0, 0) > 0  # fp32: two-kernel path
    assert lib.gdn_fwd_workspace_bytes(1, 64, 2, 128, 128, 0, 0) == 0  # fp32 K=128 unsupported
    # packed: exact with NT_total, a bound without it
    assert lib.gdn_fwd_varlen_workspace_bytes(1000, 3, 17, 4, 128, 128, 1, 0) == 256
    assert lib.gdn_fwd_varlen_workspace_bytes(1000, 100, 100, 4, 128, 128, 1, 0) == 512
    exact = lib.gdn_fwd_varlen_workspace_bytes(1000, 3, 17, 4, 128, 128, 1, SV)
    bound = lib.gdn_fwd_varlen_workspace_bytes(1000, 3, 0, 4, 128, 128, 1, SV)
    assert 0 < exact < bound
    # a dense bf16 call on the fused path accepts a NULL workspace; the others do not
    assert _fwd(lib, ht=FAKE, hch=FAKE) == L.ERR_WORKSPACE
    assert _fwd(lib, gk=FAKE) == L.ERR_WORKSPACE


def test_varlen_num_chunks():
    L, lib = _lib()
    cu = np.array([0, 1, 64, 65, 300], np.int32)
    p = cu.ctypes.data_as(ctypes.c_void_p)
    assert lib.gdn_varlen_num_chunks(p, 4) == 1 + 1 + 1 + 4
    bad = np.array([0, 5, 5], np.int32)
    assert lib.gdn_varlen_num_chunks(bad.ctypes.data_as(ctypes.c_void_p), 2) == -1
    bad = np.array([2, 5], np.int32)
    assert lib.gdn_varlen_num_chunks(bad.ctypes.data_as(ctypes.c_void_p), 1) == -1


def test_varlen_validation_codes():
    L, lib = _lib()

    def call(cu, N, T_total):
        cu = np.asarray(cu, np.int32)
        return lib.gdn_fwd_varlen(FAKE, FAKE, FAKE, None, None, FAKE, 1.0, FAKE,
                                  cu.ctypes.data_as(ctypes.c_void_p), N, None, FAKE, None, None,
                                  None, None, None, T_total, 2, 128, 128, 1, None, 0, None)

    assert call([0, 10, 10, 20], 3, 20) == L.ERR_INVALID  # empty sequence
    assert call([1, 10, 20], 2, 20) == L.ERR_INVALID  # does not start at 0
    assert call([0, 10, 20], 2, 21) == L.ERR_INVALID  # last offset != T_total
    assert call([0, 10, 20], 0, 20) == L.ERR_INVALID  # no sequences


def test_binding_fails_loudly_without_library(tmp_path, monkeypatch):
    from gated_delta_rule_29_amd import _lib as L

    monkeypatch.setattr(L, "_lib", None)
    monkeypatch.setattr(L, "LIB_PATH", str(tmp_path / "missing.so"))
    with pytest.raises(RuntimeError, match="not built"):
        L.load()


def test_state_summary_validation_codes():
    L, lib = _lib()

    def call(**kw):
        a = dict(k=FAKE, v=FAKE, g=None, gk=None, beta=FAKE, st=FAKE, tr=FAKE, B=1, T=64, H=2,
                 K=128, V=128, dtype=1, ws=None, wsn=0)
        a.update(kw)
        return lib.gdn_state_summary(a["k"], a["v"], a["g"], a["gk"], a["beta"], a["st"], a["tr"],
                                     a["B"], a["T"], a["H"], a["K"], a["V"], a["dtype"], a["ws"],
                                     a["wsn"], None)

    assert call(k=None) == L.ERR_INVALID
    assert call(st=None) == L.ERR_INVALID
    assert call(T=0) == L.ERR_INVALID
    assert call(dtype=3) == L.ERR_INVALID
    assert call(K=32) == L.ERR_UNSUPPORTED
    assert call(dtype=0, K=128) == L.ERR_UNSUPPORTED
    assert call() == L.ERR_WORKSPACE  # no workspace given
    n = lib.gdn_state_summary_workspace_bytes(1, 64, 2, 128, 128, 1, 0)
    assert n >= lib.gdn_fwd_workspace_bytes(1, 64, 2, 128, 128, 1, 0) + 64 * 2 * 128 * 2
    assert lib.gdn_state_summary_workspace_bytes(1, 64, 2, 32, 128, 1, 0) == 0


def test_state_apply_validation_codes():
    L, lib = _lib()
    assert lib.gdn_state_apply(None, FAKE, None, FAKE, 4, 128, 128, None) == L.ERR_INVALID
    assert lib.gdn_state_apply(FAKE, None, FAKE, ctypes.c_void_p(0x900000), 4, 128, 128,
                               None) == L.ERR_INVALID  # h_in without transition
    assert lib.gdn_state_apply(FAKE, FAKE, None, FAKE, 0, 128, 128, None) == L.ERR_INVALID
    assert lib.gdn_state_apply(FAKE, FAKE, None, FAKE, 4, 512, 128, None) == L.ERR_UNSUPPORTED
    # h_out overlapping h_in
    assert lib.gdn_state_apply(FAKE, FAKE, ctypes.c_void_p(0x2000), ctypes.c_void_p(0x2100), 1,
                               16, 16, None) == L.ERR_INVALID
    assert "overlap" in L.last_error()


def test_bigdn_merged_validation_codes():
    L, lib = _lib()

    def call(**kw):
        a = dict(qkv=FAKE, qb=None, beta=FAKE, decay=FAKE, bb=None, db=None, gate=None,
                 eps_m=1e-6, out=FAKE, num=None, den=None, F=2, S=64, ws=None, ws_n=0)
        a.update(kw)
        return lib.bigdn_fwd_merged(a["qkv"], a["qb"], a["beta"], a["decay"], a["bb"], a["db"],
                                    FAKE, FAKE, FAKE, FAKE, 0.1, 1e-5, a["gate"], a["eps_m"],
                                    a["out"], a["num"], a["den"], 1, a["F"], a["S"], 2, 128,
                                    a["ws"], a["ws_n"], None)

    assert call(out=None) == L.ERR_INVALID               # nothing to write
    assert call(out=None, num=FAKE) == L.ERR_INVALID     # den missing
    assert call(out=None, num=FAKE, den=FAKE, gate=FAKE) == L.ERR_INVALID  # gate needs out
    assert call(eps_m=-1.0) == L.ERR_INVALID
    assert call(S=100) == L.ERR_UNSUPPORTED
    assert call() == L.ERR_WORKSPACE
    n0 = lib.bigdn_fwd_merged_workspace_bytes(1, 2, 64, 2, 128, 0)
    n1 = lib.bigdn_fwd_merged_workspace_bytes(1, 2, 64, 2, 128, 1)
    assert n0 == lib.bigdn_fwd_workspace_bytes(1, 2, 64, 2, 128) and n1 > n0
    # reverse-direction inputs need the larger workspace
    assert call(ws=FAKE, ws_n=n0, qb=FAKE) == L.ERR_WORKSPACE
    assert call(ws=FAKE, ws_n=n0, bb=FAKE) == L.ERR_WORKSPACE


def test_cam_validation_codes():
    L, lib = _lib()

    def prep(**kw):
        a = dict(q=FAKE, N=128, D=128, ws=None, ws_n=0, eps=1e-5)
        a.update(kw)
        return lib.cam_prep(a["q"], FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 0.1,
                            a["eps"], FAKE, FAKE, FAKE, FAKE, 1, a["N"], 2, a["D"], a["ws"],
                            a["ws_n"], None)

    assert prep(q=None) == L.ERR_INVALID
    assert prep(D=60) == L.ERR_INVALID      # D/2 not a multiple of 4
    assert prep(D=96) == L.ERR_UNSUPPORTED
    assert prep(N=6) == L.ERR_UNSUPPORTED   # N a multiple of 4
    assert prep(eps=0.0) == L.ERR_INVALID
    assert prep() == L.ERR_WORKSPACE
    assert lib.cam_prep_workspace_bytes(2, 100) == 2 * 1024

    def scan(**kw):
        a = dict(q=FAKE, rev=0, init=None, fin=None, D=128, F=3, S=64, ws=None, ws_n=0)
        a.update(kw)
        return lib.cam_scan(a["q"], FAKE, FAKE, FAKE, FAKE, a["rev"], a["init"], a["fin"], FAKE,
                            1, 2, a["D"], a["F"], a["S"], a["ws"], a["ws_n"], None)

    assert scan(q=None) == L.ERR_INVALID
    assert scan(F=0) == L.ERR_INVALID
    assert scan(rev=1, fin=FAKE) == L.ERR_UNSUPPORTED   # state in / out: forward only
    assert scan(rev=1, init=FAKE) == L.ERR_UNSUPPORTED
    assert scan(S=100) == L.ERR_UNSUPPORTED
    assert scan(D=32) == L.ERR_UNSUPPORTED
    assert scan() == L.ERR_WORKSPACE
    n = lib.cam_scan_workspace_bytes(1, 2, 128, 3)
    assert n == 2 * 3 * 128 * 128 * (2 + 4 + 2)
    assert scan(ws=FAKE, ws_n=n - 1) == L.ERR_WORKSPACE


def test_cam_bidi_validation_codes():
    L, lib = _lib()

    def call(**kw):
        a = dict(orv=FAKE, init=None, fin=None, ws=None, ws_n=0)
        a.update(kw)
        return lib.cam_scan_bidi(FAKE, FAKE, FAKE, FAKE, FAKE, None, a["init"], a["fin"], FAKE,
                                 a["orv"], 1, 2, 128, 3, 64, a["ws"], a["ws_n"], None)

    assert call(orv=None) == L.ERR_INVALID
    assert call() == L.ERR_WORKSPACE
    n1 = lib.cam_scan_workspace_bytes(1, 2, 128, 3)
    n2 = lib.cam_scan_bidi_workspace_bytes(1, 2, 128, 3)
    assert n2 == n1 + 2 * 3 * 128 * 128 * 2
    assert call(ws=FAKE, ws_n=n1) == L.ERR_WORKSPACE


def test_dhu_validation_codes():
    L, lib = _lib()

    def call(**kw):
        a = dict(q=FAKE, K=128, V=64, dt=0, T=100, gk=None)
        a.update(kw)
        return lib.gdn_bwd_dhu(a["q"], FAKE, FAKE, FAKE, FAKE, None, a["gk"], None, 1.0, None, FAKE,
                               None, 1, a["T"], 2, a["K"], a["V"], a["dt"], None)

    assert call(q=None) == L.ERR_INVALID
    assert call(T=0) == L.ERR_INVALID
    assert call(dt=5) == L.ERR_INVALID
    assert call(K=64) == L.ERR_UNSUPPORTED
    assert call(V=48) == L.ERR_UNSUPPORTED
    assert call(gk=FAKE) == L.ERR_UNSUPPORTED   # per-key gates need bf16 inputs


def test_dhu_varlen_validation_codes():
    L, lib = _lib()
    IntArr = ctypes.c_int * 4

    def call(cu, T=10, K=128, ws=None, ws_n=0):
        return lib.gdn_bwd_dhu_varlen(FAKE, FAKE, FAKE, FAKE, FAKE, None, None, None, 1.0, FAKE,
                                      IntArr(*cu), 3, None, FAKE, None, T, 2, K, 64, 0, ws, ws_n,
                                      None)

    assert call([1, 3, 6, 10]) == L.ERR_INVALID      # does not start at 0
    assert call([0, 3, 3, 10]) == L.ERR_INVALID      # empty sequence
    assert call([0, 3, 6, 9]) == L.ERR_INVALID       # last offset differs from T_total
    assert call([0, 3, 6, 10], K=64) == L.ERR_UNSUPPORTED
    assert call([0, 3, 6, 10]) == L.ERR_WORKSPACE
    assert lib.gdn_bwd_dhu_varlen_workspace_bytes(3, 3) == 256 + 256


def test_noalloc_rejects_sizes_beyond_its_scratch_before_any_launch():
    """gdn_fwd_varlen_noalloc refuses a call whose scratch would exceed the static array,
    during validation (no HIP call is made, so this runs without a GPU)."""
    L, lib = _lib()
    cu = np.array([0, 2560, 5120, 7680, 10240], np.int32)  # 4 x 40 chunks
    rc = lib.gdn_fwd_varlen_noalloc(FAKE, FAKE, FAKE, None, FAKE, FAKE, 1.0, FAKE,
                                    cu.ctypes.data_as(ctypes.c_void_p), 4, None, FAKE, None, None,
                                    None, None, None, 10240, 4, 128, 128, 1, None)
    assert rc == L.ERR_WORKSPACE
    assert "static scratch" in L.last_error()
    # malformed offsets are still INVALID
    bad = np.array([0, 5, 5], np.int32)
    rc = lib.gdn_fwd_varlen_noalloc(FAKE, FAKE, FAKE, None, None, FAKE, 1.0, FAKE,
                                    bad.ctypes.data_as(ctypes.c_void_p), 2, None, FAKE, None, None,
                                    None, None, None, 5, 4, 128, 128, 1, None)
    assert rc == L.ERR_INVALID


def test_cam_scan_bwd_validation_codes():
    L, lib = _lib()

    def call(**kw):
        a = dict(q=FAKE, dout=FAKE, rev=0, B=1, H=2, D=128, F=3, S=64, ws=None, wsn=0)
        a.update(kw)
        return lib.cam_scan_bwd(a["q"], FAKE, FAKE, FAKE, FAKE, a["dout"], a["rev"], FAKE, FAKE,
                                FAKE, FAKE, FAKE, a["B"], a["H"], a["D"], a["F"], a["S"],
                                a["ws"], a["wsn"], None)

    assert call(q=None) == L.ERR_INVALID
    assert call(dout=None) == L.ERR_INVALID
    assert call(F=0) == L.ERR_INVALID
    assert call(rev=8) == L.ERR_INVALID
    assert call(rev=-1) == L.ERR_INVALID
    assert call(D=32) == L.ERR_UNSUPPORTED
    assert call(S=100) == L.ERR_UNSUPPORTED
    assert call() == L.ERR_WORKSPACE
    assert call(rev=1 | L.BWD_ACCUMULATE) == L.ERR_WORKSPACE   # the accumulate flag is valid
    assert call(rev=1 | L.BWD_REUSE_STATS) == L.ERR_WORKSPACE  # so is the reuse flag
    assert call(rev=8) == L.ERR_INVALID
    n = lib.cam_scan_bwd_workspace_bytes(1, 2, 128, 3)
    assert n >= 1 * 2 * 3 * 128 * 128 * (4 * 4 + 4 * 2)
    assert lib.cam_scan_bwd_workspace_bytes(1, 2, 96, 3) == 0


def test_bigdn_dir_bwd_validation_codes():
    L, lib = _lib()

    def call(**kw):
        a = dict(q=FAKE, dnum=FAKE, rev=0, B=1, H=2, D=128, F=3, S=64, ws=None, wsn=0)
        a.update(kw)
        return lib.bigdn_dir_bwd(a["q"], FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, a["dnum"], FAKE,
                                 a["rev"], FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, a["B"],
                                 a["H"], a["D"], a["F"], a["S"], a["ws"], a["wsn"], None)

    assert call(q=None) == L.ERR_INVALID
    assert call(dnum=None) == L.ERR_INVALID
    assert call(rev=8) == L.ERR_INVALID
    assert call(rev=-1) == L.ERR_INVALID
    assert call(D=32) == L.ERR_UNSUPPORTED
    assert call(S=100) == L.ERR_UNSUPPORTED
    for rev in (0, 1, L.BWD_ACCUMULATE, 1 | L.BWD_ACCUMULATE, 1 | L.BWD_REUSE_STATS,
                1 | L.BWD_ACCUMULATE | L.BWD_REUSE_STATS):  # valid flags: only the workspace is missing
        assert call(rev=rev) == L.ERR_WORKSPACE


def test_bigdn_merge_bwd_validation_codes():
    L, lib = _lib()

    def call(**kw):
        a = dict(num=FAKE, gate=None, dgate=None, eps=1e-6, B=1, N=64, H=2, D=128)
        a.update(kw)
        return lib.bigdn_merge_bwd(a["num"], FAKE, a["gate"], FAKE, a["eps"], FAKE, FAKE, a["dgate"],
                                   a["B"], a["N"], a["H"], a["D"], None)

    assert call(num=None) == L.ERR_INVALID
    assert call(gate=FAKE) == L.ERR_INVALID   # gate without dgate
    assert call(dgate=FAKE) == L.ERR_INVALID  # dgate without gate
    assert call(eps=-1.0) == L.ERR_INVALID
    assert call(N=0) == L.ERR_INVALID
    assert call(D=96) == L.ERR_UNSUPPORTED
    assert call(H=64) == L.ERR_UNSUPPORTED    # H*D > 4096


def test_prep_bwd_validation_codes():
    L, lib = _lib()

    def call(**kw):
        a = dict(qkv=FAKE, ndir=2, eps=1e-5, B=1, N=64, H=2, D=128, ws=None, wsn=0)
        a.update(kw)
        return lib.gdn_prep_bwd(a["qkv"], FAKE, FAKE, FAKE, FAKE, 0.5, a["eps"], a["ndir"], FAKE,
                                FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, a["B"], a["N"], a["H"],
                                a["D"], a["ws"], a["wsn"], None)

    assert call(qkv=None) == L.ERR_INVALID
    assert call(ndir=0) == L.ERR_INVALID
    assert call(ndir=3) == L.ERR_INVALID
    assert call(eps=0.0) == L.ERR_INVALID
    assert call(D=96) == L.ERR_UNSUPPORTED
    assert call() == L.ERR_WORKSPACE
    n = lib.gdn_prep_bwd_workspace_bytes(1, 64, 2, 128)
    assert n >= 64 * 2 * 256 * 4                    # one partial pair per token group
    assert lib.gdn_prep_bwd_workspace_bytes(1, 1 << 20, 16, 128) >= 1024 * 2 * 2048 * 4
    assert call(ws=ctypes.c_void_p(0x1000 + 16), wsn=n) == L.ERR_INVALID  # misaligned


def test_cam_prep_bwd_validation_codes():
    L, lib = _lib()

    def call(**kw):
        a = dict(q=FAKE, dinfl=None, ndir=2, eps=1e-5, B=1, N=64, H=2, D=128, ws=None, wsn=0)
        a.update(kw)
        return lib.cam_prep_bwd(a["q"], FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 0.5, a["eps"],
                                a["ndir"], FAKE, FAKE, FAKE, a["dinfl"], FAKE, FAKE, FAKE, FAKE,
                                FAKE, a["B"], a["N"], a["H"], a["D"], a["ws"], a["wsn"], None)

    assert call(q=None) == L.ERR_INVALID
    assert call(ndir=0) == L.ERR_INVALID
    assert call(ndir=3) == L.ERR_INVALID
    assert call(eps=0.0) == L.ERR_INVALID
    assert call(D=36) == L.ERR_INVALID            # D/2 not a multiple of 4
    assert call(D=96) == L.ERR_UNSUPPORTED
    assert call(N=66) == L.ERR_UNSUPPORTED        # N not a multiple of 4
    assert call(H=64) == L.ERR_UNSUPPORTED        # H*D > 4096
    assert call() == L.ERR_WORKSPACE
    assert call(dinfl=FAKE) == L.ERR_WORKSPACE    # dinfl is optional
    n = lib.cam_prep_bwd_workspace_bytes(1, 64, 2, 128)
    assert n >= 64 * 4 + 64 * 2 * 256 * 4         # k inverse RMS + one partial pair per group
    assert call(ws=ctypes.c_void_p(0x1000 + 16), wsn=n) == L.ERR_INVALID  # misaligned


def test_binding_reuse_stats_needs_the_workspace():
    """Asking for reused frame statistics without the workspace that holds them is refused by
    the binding before anything is launched (CPU tensors: no launch could run here anyway)."""
    import torch

    import gated_delta_rule_29_amd as g

    B, H, D, F, S = 1, 2, 64, 2, 64
    N = F * S
    x = torch.zeros(B, H, D, N)
    beta, decay = torch.zeros(B, H, F, S), torch.zeros(B, H, F)
    with pytest.raises(ValueError, match="reuse_stats"):
        g.cam_scan_bwd(x, x, x, beta, decay, x, reverse=True, reuse_stats=True)
    t = torch.zeros(B, H, N, D, dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="reuse_stats"):
        g.bigdn_dir_bwd(t, t, t, t, t, beta, decay, torch.zeros(B, N, H, D), torch.zeros(B, H, N),
                        reverse=True, reuse_stats=True)
    with pytest.raises(ValueError, match="workspace"):
        g.cam_scan_bwd(x, x, x, beta, decay, x, reverse=True, reuse_stats=True,
                       workspace=torch.zeros(16, dtype=torch.uint8))

"""fp64 CPU oracle for the gated delta rule -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py``
may import this package.  The HIP library never imports, links or calls it, and the two
share no code: the only module both sides use is ``workloads`` (seeded random inputs,
which holds none of the method's arithmetic).

Contents
  * ``gdn_oracle.c`` (compiled to ``_build/liboracle.so`` with gcc -O2, no fast-math):
    the plain token-by-token recurrence and its transition matrix (the linear part of the
    map from initial to final state), the packed-varlen tables and driver, the BiGDN
    front end (full-channel RMSNorm, ReLU, k-scale, interleaved-pair RoPE) and the
    frame-level BiGDN scan in both directions, the camera-branch prep (UCPE 4x4 blocks and
    half-width RoPE) and its numerator-only frame scan with state in and out, the
    state-gradient pass of the chunked backward (dhu), and the backward of the BiGDN block
    (frame scan per direction, merge, front end) and of the camera branch (scan, prep).
    This is the reference every GPU result is compared with.
  * ``forms.py``: independent numpy cross-check forms (global O(T^2) solve, chunked WY
    form, BiGDN product form with flip-and-shift reverse) used only to pin the oracle.

Every function takes and returns float64 numpy arrays; inputs stored as bf16 or fp32 are
converted to float64 exactly before the call.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
# GDN_ORACLE_SRC names another copy of gdn_oracle.c to build and load (it is built next to
# that copy); tests/test_oracle_mutations.py uses it to plant mistakes in a scratch copy.
_SRC = os.environ.get("GDN_ORACLE_SRC") or os.path.join(_HERE, "gdn_oracle.c")
_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(_SRC)), "_build", "liboracle.so")
_lib = None

CHUNK = 64


def build(force: bool = False) -> str:
    """Compile the C oracle with gcc (-O2, OpenMP, no fast-math).  Returns the .so path."""
    if force or not os.path.exists(_LIB_PATH) or (
        os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC)
    ):
        os.makedirs(os.path.dirname(_LIB_PATH), exist_ok=True)
        tmp = _LIB_PATH + ".tmp%d" % os.getpid()
        cmd = ["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c99", "-Wall",
               "-Wno-unknown-pragmas", _SRC, "-o", tmp, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is None:
        build()
        lib = ctypes.CDLL(_LIB_PATH)
        P = ctypes.c_void_p
        I = ctypes.c_int
        Dd = ctypes.c_double
        lib.oracle_gdn.argtypes = [I, I, I, I, I, I, P, P, P, P, P, P, Dd, P, P, P, P, P]
        lib.oracle_gdn_varlen.argtypes = [P, I, I, I, I, I, P, P, P, P, P, P, Dd, P, P, P, P, P]
        lib.oracle_varlen_tables.argtypes = [P, I, I, P, P]
        lib.oracle_prep.argtypes = [I, I, I, I, P, P, P, P, P, Dd, Dd, P, P, P, P, P, P, P]
        lib.oracle_bigdn_dir.argtypes = [I, I, I, I, I, I, P, P, P, P, P, P, P, P, P]
        lib.oracle_bigdn.argtypes = [I, I, I, I, I, P, P, P, P, P, P, P, Dd, Dd, P, P]
        lib.oracle_gdn_transition.argtypes = [I, I, I, I, P, P, P, P, P]
        lib.oracle_cam_prep.argtypes = [I, I, I, I, P, P, P, P, P, P, P, P, P, Dd, Dd, P, P, P,
                                        P]
        lib.oracle_cam_scan.argtypes = [I, I, I, I, I, I, P, P, P, P, P, P, P, P]
        lib.oracle_gdn_dhu.argtypes = [I, I, I, I, I, I, P, P, P, P, P, P, P, P, Dd, P, P, P]
        lib.oracle_cam_scan_bwd.argtypes = [I, I, I, I, I, I, P, P, P, P, P, P, P, P, P, P, P]
        lib.oracle_gdn_bwd_prep.argtypes = [I, I, I, I, I, I, P, P, P, P, P, P, Dd, P, P]
        lib.oracle_bigdn_dir_bwd.argtypes = [I, I, I, I, I, I] + [P] * 16
        lib.oracle_prep_bwd.argtypes = [I, I, I, I, P, P, P, P, P, Dd, Dd, I] + [P] * 8
        lib.oracle_bigdn_merge_bwd.argtypes = [I, I, I, I, P, P, P, P, Dd, P, P, P]
        lib.oracle_cam_prep_bwd.argtypes = [I, I, I, I] + [P] * 8 + [Dd, Dd] + [P] * 9
        lib.oracle_set_threads.argtypes = [I]
        for name in ("oracle_gdn", "oracle_gdn_varlen", "oracle_varlen_tables", "oracle_prep",
                     "oracle_bigdn_dir", "oracle_bigdn", "oracle_max_threads",
                     "oracle_gdn_transition", "oracle_gdn_bwd_prep", "oracle_bigdn_dir_bwd",
                     "oracle_prep_bwd", "oracle_bigdn_merge_bwd", "oracle_cam_prep_bwd"):
            getattr(lib, name).restype = I
        _lib = lib
    return _lib


def _f64(x):
    if x is None:
        return None
    if hasattr(x, "detach"):  # torch tensor -> exact float64 copy on the host
        x = x.detach().to("cpu").double().numpy()
    return np.ascontiguousarray(x, dtype=np.float64)


def _p(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def max_threads() -> int:
    return _load().oracle_max_threads()


def set_threads(n: int) -> None:
    _load().oracle_set_threads(int(n))


def gdn(q, k, v, beta, g=None, gk=None, scale=1.0, h0=None, chunk=CHUNK,
        want_h=False, want_vnew=False):
    """Token recurrence over a dense batch.

    q, k [B,T,H,K]; v [B,T,H,V]; beta, g [B,T,H]; gk [B,T,H,K]; h0 [B,H,K,V].
    Returns dict with o [B,T,H,V], ht [B,H,K,V], and optionally h [B,H,NT,K,V] (state
    entering each chunk of ``chunk`` tokens) and v_new [B,T,H,V].
    """
    q, k, v, beta, g, gk, h0 = map(_f64, (q, k, v, beta, g, gk, h0))
    B, T, H, K = q.shape
    V = v.shape[-1]
    NT = (T + chunk - 1) // chunk
    o = np.empty((B, T, H, V))
    ht = np.empty((B, H, K, V))
    hch = np.empty((B, H, NT, K, V)) if want_h else None
    vn = np.empty((B, T, H, V)) if want_vnew else None
    rc = _load().oracle_gdn(B, T, H, K, V, chunk, _p(q), _p(k), _p(v), _p(g), _p(gk),
                            _p(beta), float(scale), _p(h0), _p(o), _p(ht), _p(hch), _p(vn))
    if rc != 0:
        raise RuntimeError("oracle_gdn failed")
    out = {"o": o, "ht": ht}
    if want_h:
        out["h"] = hch
    if want_vnew:
        out["v_new"] = vn
    return out


def transition(k, beta, g=None, gk=None):
    """Linear part of a fragment's state map: ht(h0) = M h0 + ht(0) per (b, h), with
    M = A_T ... A_1, A_t = (I - beta_t k_t k_t^T) diag(exp(g_t + gk_t)).
    k [B,T,H,K]; beta, g [B,T,H]; gk [B,T,H,K].  Returns M [B,H,K,K]."""
    k, beta, g, gk = map(_f64, (k, beta, g, gk))
    B, T, H, K = k.shape
    M = np.empty((B, H, K, K))
    rc = _load().oracle_gdn_transition(B, T, H, K, _p(k), _p(g), _p(gk), _p(beta), _p(M))
    if rc != 0:
        raise RuntimeError("oracle_gdn_transition failed")
    return M


def state_summary(k, v, beta, g=None, gk=None):
    """State summary of a fragment (for composing fragments run separately): state_ext =
    ht with a zero initial state [B,H,K,V], transition = M [B,H,K,K]."""
    ht = gdn(k, k, v, beta, g=g, gk=gk)["ht"]
    return {"state_ext": ht, "transition": transition(k, beta, g=g, gk=gk)}


def apply_summary(state_ext, trans, h_in=None):
    """h_out = transition h_in + state_ext per (b, h); h_in None means zero."""
    state_ext, trans, h_in = map(_f64, (state_ext, trans, h_in))
    return state_ext.copy() if h_in is None else np.matmul(trans, h_in) + state_ext


def varlen_tables(cu_seqlens, chunk=CHUNK):
    """(chunk_offsets [N+1] int32, chunk_indices [NT_total,2] int32) for a cu_seqlens array."""
    cu = np.ascontiguousarray(np.asarray(cu_seqlens), dtype=np.int32)
    N = cu.shape[0] - 1
    lib = _load()
    nt = lib.oracle_varlen_tables(_p(cu), N, chunk, None, None)
    if nt < 0:
        raise ValueError("malformed cu_seqlens")
    offs = np.empty(N + 1, np.int32)
    idx = np.empty((nt, 2), np.int32)
    lib.oracle_varlen_tables(_p(cu), N, chunk, _p(offs), _p(idx))
    return offs, idx


def gdn_varlen(cu_seqlens, q, k, v, beta, g=None, gk=None, scale=1.0, h0=None, chunk=CHUNK,
               want_h=False, want_vnew=False):
    """Packed batch of 1: q, k [1,T,H,K] ... ; h0/ht [N,H,K,V]; h [1,H,NT_total,K,V]."""
    cu = np.ascontiguousarray(np.asarray(cu_seqlens), dtype=np.int32)
    q, k, v, beta, g, gk, h0 = map(_f64, (q, k, v, beta, g, gk, h0))
    _, T, H, K = q.shape
    V = v.shape[-1]
    N = cu.shape[0] - 1
    offs, _ = varlen_tables(cu, chunk)
    NT = int(offs[-1])
    o = np.empty((1, T, H, V))
    ht = np.empty((N, H, K, V))
    hch = np.empty((1, H, NT, K, V)) if want_h else None
    vn = np.empty((1, T, H, V)) if want_vnew else None
    rc = _load().oracle_gdn_varlen(_p(cu), N, H, K, V, chunk, _p(q), _p(k), _p(v), _p(g),
                                   _p(gk), _p(beta), float(scale), _p(h0), _p(o), _p(ht),
                                   _p(hch), _p(vn))
    if rc != 0:
        raise RuntimeError("oracle_gdn_varlen failed")
    out = {"o": o, "ht": ht}
    if want_h:
        out["h"] = hch
    if want_vnew:
        out["v_new"] = vn
    return out


def prep(qkv, q_norm_w, k_norm_w, rope_cos, rope_sin, k_scale, eps=1e-5):
    """BiGDN front end.  qkv [B,N,3,H,D] -> dict of q_inv_rms, k_inv_rms [B,N] and
    q_rot, k_rot, q_pos, k_pos, v [B,H,N,D]."""
    qkv, qw, kw, cs, sn = map(_f64, (qkv, q_norm_w, k_norm_w, rope_cos, rope_sin))
    B, N, _, H, D = qkv.shape
    out = {name: np.empty((B, H, N, D)) for name in ("q_rot", "k_rot", "q_pos", "k_pos", "v")}
    out["q_inv_rms"] = np.empty((B, N))
    out["k_inv_rms"] = np.empty((B, N))
    rc = _load().oracle_prep(B, N, H, D, _p(qkv), _p(qw), _p(kw), _p(cs), _p(sn),
                             float(k_scale), float(eps), _p(out["q_inv_rms"]),
                             _p(out["k_inv_rms"]), _p(out["q_rot"]), _p(out["k_rot"]),
                             _p(out["q_pos"]), _p(out["k_pos"]), _p(out["v"]))
    if rc != 0:
        raise RuntimeError("oracle_prep failed")
    return out


def bigdn_dir(q_rot, k_rot, q_pos, k_pos, v, beta, decay, reverse):
    """One BiGDN direction on prepped [B,H,N,D] tensors; beta [B,H,F,S], decay [B,H,F].
    Returns (num [B,N,H,D], den [B,H,N])."""
    q_rot, k_rot, q_pos, k_pos, v, beta, decay = map(
        _f64, (q_rot, k_rot, q_pos, k_pos, v, beta, decay))
    B, H, N, D = q_rot.shape
    F, S = beta.shape[2], beta.shape[3]
    num = np.zeros((B, N, H, D))
    den = np.zeros((B, H, N))
    rc = _load().oracle_bigdn_dir(B, F, S, H, D, int(bool(reverse)), _p(q_rot), _p(k_rot),
                                  _p(q_pos), _p(k_pos), _p(v), _p(beta), _p(decay), _p(num),
                                  _p(den))
    if rc != 0:
        raise RuntimeError("oracle_bigdn_dir failed")
    return num, den


def bigdn_dir_bwd(q_rot, k_rot, q_pos, k_pos, v, beta, decay, dnum, dden, reverse):
    """Backward of one BiGDN direction (SANA fused_gdn.py page, "Backward / autograd
    Functions"): gradients of sum(num * dnum) + sum(den * dden) for (num, den) =
    bigdn_dir(...).  Returns dict dq_rot, dk_rot, dq_pos, dk_pos, dv [B,H,N,D], dbeta
    [B,H,F,S], ddecay [B,H,F]."""
    q_rot, k_rot, q_pos, k_pos, v, beta, decay, dnum, dden = map(
        _f64, (q_rot, k_rot, q_pos, k_pos, v, beta, decay, dnum, dden))
    B, H, N, D = q_rot.shape
    F, S = beta.shape[2], beta.shape[3]
    out = {n: np.empty((B, H, N, D)) for n in ("dq_rot", "dk_rot", "dq_pos", "dk_pos", "dv")}
    out["dbeta"] = np.empty((B, H, F, S))
    out["ddecay"] = np.empty((B, H, F))
    rc = _load().oracle_bigdn_dir_bwd(
        B, F, S, H, D, int(bool(reverse)), *(_p(x) for x in (q_rot, k_rot, q_pos, k_pos, v, beta,
                                                              decay, dnum, dden)),
        *(_p(out[n]) for n in ("dq_rot", "dk_rot", "dq_pos", "dk_pos", "dv", "dbeta", "ddecay")))
    if rc != 0:
        raise RuntimeError("oracle_bigdn_dir_bwd failed")
    return out


def bigdn(qkv, beta, decay, q_norm_w, k_norm_w, rope_cos, rope_sin, k_scale, eps=1e-5):
    """Whole BiGDN block forward: (num [B,N,H,D], den [B,H,N]) summed over both directions."""
    qkv, beta, decay, qw, kw, cs, sn = map(
        _f64, (qkv, beta, decay, q_norm_w, k_norm_w, rope_cos, rope_sin))
    B, N, _, H, D = qkv.shape
    F, S = beta.shape[2], beta.shape[3]
    num = np.empty((B, N, H, D))
    den = np.empty((B, H, N))
    rc = _load().oracle_bigdn(B, F, S, H, D, _p(qkv), _p(beta), _p(decay), _p(qw), _p(kw),
                              _p(cs), _p(sn), float(k_scale), float(eps), _p(num), _p(den))
    if rc != 0:
        raise RuntimeError("oracle_bigdn failed")
    return num, den


def bigdn_merged(qkv, beta, decay, q_norm_w, k_norm_w, rope_cos, rope_sin, k_scale, eps=1e-5,
                 beta_bwd=None, decay_bwd=None, gate=None, merge_eps=1e-6, qkv_bwd=None):
    """BiGDN block with the reverse direction's own q, k, v / beta / decay (chunk-causal
    overrides; None = the forward ones; the reverse direction's inverse RMS is that of its own
    q and k) and the merge (SANA fused_gdn.py page, fused_bigdn_func and fused_bidi_merge):
    out = (num_f + num_r) / (den_f + den_r + merge_eps) * SiLU(gate).
    Returns (out [B,N,H,D], num [B,N,H,D], den [B,H,N])."""
    def tensors(x):
        p = prep(x, q_norm_w, k_norm_w, rope_cos, rope_sin, k_scale, eps)
        return (p["q_rot"], p["k_rot"], p["q_pos"], p["k_pos"], p["v"])
    t = tensors(qkv)
    tr = t if qkv_bwd is None else tensors(qkv_bwd)
    nf, df = bigdn_dir(*t, beta, decay, reverse=False)
    nr, dr = bigdn_dir(*tr, beta if beta_bwd is None else beta_bwd,
                       decay if decay_bwd is None else decay_bwd, reverse=True)
    num, den = nf + nr, df + dr
    return bigdn_merge(num, den, gate, merge_eps), num, den


def bigdn_merge(num, den, gate=None, merge_eps=1e-6):
    """The merge of the BiGDN block (SANA fused_gdn.py page, fused_bidi_merge): out =
    num / (den + merge_eps) * SiLU(gate) (no gate: factor 1).  num, gate [B,N,H,D]; den
    [B,H,N]."""
    num, den = _f64(num), _f64(den)
    out = num / (np.transpose(den, (0, 2, 1))[..., None] + merge_eps)
    if gate is not None:
        g = _f64(gate)
        out = out * (g / (1.0 + np.exp(-g)))
    return out


def bigdn_merge_bwd(num, den, dout, gate=None, merge_eps=1e-6):
    """Backward of bigdn_merge (SANA fused_gdn.py page: the dnum / dden of
    FusedBiGDNFunction.backward, with fused_bidi_merge's gate): returns dict dnum [B,N,H,D],
    dden [B,H,N] and dgate [B,N,H,D] (None without a gate)."""
    num, den, dout, gate = map(_f64, (num, den, dout, gate))
    B, N, H, D = num.shape
    out = {"dnum": np.empty((B, N, H, D)), "dden": np.empty((B, H, N)),
           "dgate": None if gate is None else np.empty((B, N, H, D))}
    rc = _load().oracle_bigdn_merge_bwd(B, N, H, D, _p(num), _p(den), _p(gate), _p(dout),
                                        float(merge_eps), _p(out["dnum"]), _p(out["dden"]),
                                        _p(out["dgate"]))
    if rc != 0:
        raise RuntimeError("oracle_bigdn_merge_bwd failed")
    return out


def prep_bwd(qkv, q_norm_w, k_norm_w, rope_cos, rope_sin, k_scale, grads, eps=1e-5):
    """Backward of prep (SANA fused_gdn.py page, "Backward / autograd Functions": the RoPE,
    ReLU and k-scale backward of _fused_gdn_bwd_kernel and the full-channel RMSNorm backward
    of FusedBiGDNFunction.backward).  grads: dict of dq_rot, dk_rot, dq_pos, dk_pos, dv, each
    [B,H,N,D] or [ndir,B,H,N,D] (the directions are summed).  Returns dict dqkv [B,N,3,H,D],
    dq_norm_w, dk_norm_w [H*D]."""
    qkv, qw, kw, cs, sn = map(_f64, (qkv, q_norm_w, k_norm_w, rope_cos, rope_sin))
    B, N, _, H, D = qkv.shape
    names = ("dq_rot", "dk_rot", "dq_pos", "dk_pos", "dv")
    g = {n: _f64(grads[n]) for n in names}
    g = {n: (x[None] if x.ndim == 4 else x) for n, x in g.items()}
    ndir = g["dq_rot"].shape[0]
    out = {"dqkv": np.empty((B, N, 3, H, D)), "dq_norm_w": np.empty(H * D),
           "dk_norm_w": np.empty(H * D)}
    rc = _load().oracle_prep_bwd(B, N, H, D, _p(qkv), _p(qw), _p(kw), _p(cs), _p(sn),
                                 float(k_scale), float(eps), ndir, *(_p(g[n]) for n in names),
                                 _p(out["dqkv"]), _p(out["dq_norm_w"]), _p(out["dk_norm_w"]))
    if rc != 0:
        raise RuntimeError("oracle_prep_bwd failed")
    return out


def cam_prep(q, k, v, q_norm_w, k_norm_w, proj_q, proj_kv, rope_cos, rope_sin, k_scale,
             eps=1e-5):
    """Camera-branch prep (SANA fused_cam_gdn.py page, cam_prep_func): q, k, v [B,N,H,D];
    proj_q, proj_kv [B,N,4,4]; rope_cos, rope_sin [N, D/2].  Returns q_t, k_t, v_t [B,H,D,N]
    and inflation [B,H,N]."""
    q, k, v, qw, kw, pq, pkv, cs, sn = map(
        _f64, (q, k, v, q_norm_w, k_norm_w, proj_q, proj_kv, rope_cos, rope_sin))
    B, N, H, D = q.shape
    outs = [np.empty((B, H, D, N)) for _ in range(3)]
    infl = np.empty((B, H, N))
    rc = _load().oracle_cam_prep(B, N, H, D, _p(q), _p(k), _p(v), _p(qw), _p(kw), _p(pq),
                                 _p(pkv), _p(cs), _p(sn), float(k_scale), float(eps),
                                 _p(outs[0]), _p(outs[1]), _p(outs[2]), _p(infl))
    if rc != 0:
        raise RuntimeError("oracle_cam_prep failed")
    return outs[0], outs[1], outs[2], infl


def cam_prep_bwd(q, k, q_norm_w, k_norm_w, proj_q, proj_kv, rope_cos, rope_sin, k_scale, dq_t,
                 dk_t, dv_t, dinfl=None, eps=1e-5):
    """Backward of cam_prep (SANA fused_cam_gdn.py page, _cam_prep_bwd_kernel and
    _cam_prep_bwd_dispatch): from the gradients of q_t, k_t, v_t [B,H,D,N] and of the
    inflation [B,H,N] (or None), the gradients of q, k, v [B,N,H,D] and of the norm weights
    [H*D].  Returns dict dq, dk, dv, dq_norm_w, dk_norm_w."""
    q, k, qw, kw, pq, pkv, cs, sn, dq_t, dk_t, dv_t, dinfl = map(
        _f64, (q, k, q_norm_w, k_norm_w, proj_q, proj_kv, rope_cos, rope_sin, dq_t, dk_t, dv_t,
               dinfl))
    B, N, H, D = q.shape
    out = {n: np.empty((B, N, H, D)) for n in ("dq", "dk", "dv")}
    out["dq_norm_w"], out["dk_norm_w"] = np.empty(H * D), np.empty(H * D)
    rc = _load().oracle_cam_prep_bwd(B, N, H, D, _p(q), _p(k), _p(qw), _p(kw), _p(pq), _p(pkv),
                                     _p(cs), _p(sn), float(k_scale), float(eps), _p(dq_t),
                                     _p(dk_t), _p(dv_t), _p(dinfl), _p(out["dq"]), _p(out["dk"]),
                                     _p(out["dv"]), _p(out["dq_norm_w"]), _p(out["dk_norm_w"]))
    if rc != 0:
        raise RuntimeError("oracle_cam_prep_bwd failed")
    return out


def cam_scan(q, k, v, beta, decay, reverse=False, init_state=None, want_final=False):
    """Camera-branch numerator-only frame scan (SANA fused_cam_gdn.py page, cam_scan_func):
    q, k, v [B,H,D,N]; beta [B,H,F,S]; decay [B,H,F]; init_state [B*H,D,D] (forward only).
    Returns out [B,H,D,N], or (out, final [B*H,D,D]) with want_final (forward only)."""
    q, k, v, beta, decay = map(_f64, (q, k, v, beta, decay))
    B, H, D, N = q.shape
    F, S = beta.shape[2], beta.shape[3]
    if reverse and (init_state is not None or want_final):
        raise NotImplementedError("state in / out is defined for the forward scan only")
    init = None if init_state is None else _f64(init_state)
    out = np.empty((B, H, D, N))
    fin = np.empty((B * H, D, D)) if want_final else None
    rc = _load().oracle_cam_scan(B, H, D, F, S, int(bool(reverse)), _p(q), _p(k), _p(v),
                                 _p(beta), _p(decay), None if init is None else _p(init),
                                 _p(out), None if fin is None else _p(fin))
    if rc != 0:
        raise RuntimeError("oracle_cam_scan failed")
    return (out, fin) if want_final else out


def cam_scan_bwd(q, k, v, beta, decay, dout, reverse=False):
    """Backward of the camera-branch scan (no initial state), SANA fused_cam_gdn.py page,
    _cam_scan_bwd_kernel: gradients of sum(out * dout) for out = cam_scan(q, k, v, beta,
    decay, reverse).  Returns dict dq, dk, dv [B,H,D,N], dbeta [B,H,F,S], ddecay [B,H,F]."""
    q, k, v, beta, decay, dout = map(_f64, (q, k, v, beta, decay, dout))
    B, H, D, N = q.shape
    F, S = beta.shape[2], beta.shape[3]
    out = {n: np.empty((B, H, D, N)) for n in ("dq", "dk", "dv")}
    out["dbeta"] = np.empty((B, H, F, S))
    out["ddecay"] = np.empty((B, H, F))
    rc = _load().oracle_cam_scan_bwd(B, H, D, F, S, int(bool(reverse)), _p(q), _p(k), _p(v),
                                     _p(beta), _p(decay), _p(dout), _p(out["dq"]),
                                     _p(out["dk"]), _p(out["dv"]), _p(out["dbeta"]),
                                     _p(out["ddecay"]))
    if rc != 0:
        raise RuntimeError("oracle_cam_scan_bwd failed")
    return out


def gdn_dhu(q, k, w, do, dv, g=None, dht=None, scale=1.0, chunk=CHUNK, gk=None):
    """State-gradient pass of the chunked backward (dhu): q, k, w [B,T,H,K]; do, dv [B,T,H,V];
    g [B,T,H] per-token and gk [B,T,H,K] per-key log gates (the chunk-local cumsum is taken
    here); dht [B,H,K,V].  Returns dict with dh [B,H,NT,K,V] (gradient of the state entering
    each chunk), dv2 [B,T,H,V] (gradient of v_new) and dh0 [B,H,K,V]."""
    q, k, w, do, dv, g, gk, dht = map(_f64, (q, k, w, do, dv, g, gk, dht))
    B, T, H, K = q.shape
    V = do.shape[-1]
    NT = (T + chunk - 1) // chunk
    dh = np.empty((B, H, NT, K, V))
    dv2 = np.empty((B, T, H, V))
    dh0 = np.empty((B, H, K, V))
    rc = _load().oracle_gdn_dhu(B, T, H, K, V, chunk, _p(q), _p(k), _p(w), _p(g), _p(gk),
                                _p(do), _p(dv), _p(dht), float(scale), _p(dh), _p(dv2),
                                _p(dh0))
    if rc != 0:
        raise RuntimeError("oracle_gdn_dhu failed")
    return {"dh": dh, "dv2": dv2, "dh0": dh0}


def gdn_bwd_prep(q, k, beta, do, g=None, gk=None, scale=1.0, chunk=CHUNK):
    """Inputs of the state-gradient pass formed from the forward's inputs ([hyper-parallel
    "Diff Coverage" page], the chunk state pass and its dhu backward): per chunk, the WY factor
    w = (I + A)^-1 diag(beta) (e^gamma * K) and dv = P^T do, P the decayed causal Q K^T times
    scale.  q, k [B,T,H,K]; beta, g [B,T,H]; gk [B,T,H,K]; do [B,T,H,V].  Returns w, dv."""
    q, k, beta, do, g, gk = map(_f64, (q, k, beta, do, g, gk))
    B, T, H, K = q.shape
    V = do.shape[-1]
    w = np.empty((B, T, H, K))
    dv = np.empty((B, T, H, V))
    rc = _load().oracle_gdn_bwd_prep(B, T, H, K, V, chunk, _p(q), _p(k), _p(beta), _p(g), _p(gk),
                                     _p(do), float(scale), _p(w), _p(dv))
    if rc != 0:
        raise RuntimeError("oracle_gdn_bwd_prep failed")
    return w, dv


def apply_grad_summary(grad_ext, trans, grad_in=None):
    """Gradient of the state entering a fragment from the gradient of the state leaving it
    (the reverse summary of the context-parallel backward): grad_ext + M^T grad_in, with M the
    fragment's transition (h_out = M h_in + state_ext).  [B,H,K,V] and [B,H,K,K] arrays."""
    grad_ext = _f64(grad_ext)
    if grad_in is None:
        return grad_ext.copy()
    return grad_ext + np.matmul(np.swapaxes(_f64(trans), -1, -2), _f64(grad_in))

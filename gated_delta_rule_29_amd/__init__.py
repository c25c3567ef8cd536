"""MI355X (gfx950) chunkwise gated delta-rule forward.

The compute path is libgdn.so: hand-written HIP kernels behind the C ABI of include/gdn.h.
This module is its Python binding, with the same entry-point names.  It only marshals
arguments: PyTorch supplies device memory (outputs are allocated with ``torch.empty`` on the
inputs' device) and the current stream; every step of the method runs in the library.

Shapes are checked here before a pointer reaches the library, since raw pointers carry no
shape; the library itself validates sizes, dtypes and tables.
"""
from __future__ import annotations

import ctypes

import torch

from . import _lib

__all__ = ["gdn_fwd", "gdn_fwd_varlen", "gdn_prep", "bigdn_fwd", "gdn_varlen_num_chunks",
           "gdn_state_summary", "gdn_state_apply", "bigdn_fwd_merged", "cam_prep", "cam_scan",
           "cam_scan_bidi", "cam_scan_bwd", "cam_prep_bwd", "cam_bwd", "bigdn_dir_bwd",
           "bigdn_merge_bwd", "gdn_prep_bwd", "bigdn_bwd", "gdn_bwd_prep", "gdn_bwd_dhu", "gdn_bwd_dhu_varlen",
           "gdn_state_grad_summary", "gdn_state_grad_apply", "gdn_abi_version",
           "gdn_last_error", "CHUNK"]

CHUNK = 64
_DT = {torch.float32: _lib.DTYPE_F32, torch.bfloat16: _lib.DTYPE_BF16}


def gdn_abi_version() -> int:
    return _lib.load().gdn_abi_version()


def gdn_last_error() -> str:
    return _lib.last_error()


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(dev):
    return ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)


def _fwd_flags(gk, want_h, want_v_new):
    return ((_lib.FWD_PER_KEY if gk is not None else 0)
            | (_lib.FWD_SAVES if (want_h or want_v_new) else 0))


def _cu_pair(cu_seqlens, cu_seqlens_host, dev):
    """(device, host) int32 copies of the packed offsets.  A host copy given by the caller is
    used as is, so a device cu_seqlens plus its host copy costs no transfer; otherwise the
    missing side is copied (device to host waits for the device)."""
    if cu_seqlens_host is not None:
        cu_host = torch.as_tensor(cu_seqlens_host, dtype=torch.int32).contiguous()
        if cu_host.device.type != "cpu":
            raise ValueError("cu_seqlens_host must be a host tensor")
    else:
        cu_host = cu_seqlens.detach().to("cpu", torch.int32).contiguous()
    if isinstance(cu_seqlens, torch.Tensor) and cu_seqlens.device == dev and \
            cu_seqlens.dtype == torch.int32 and cu_seqlens.is_contiguous():
        cu_dev = cu_seqlens
    else:
        cu_dev = torch.as_tensor(cu_seqlens, dtype=torch.int32).to(dev).contiguous()
    if cu_dev.numel() != cu_host.numel():
        raise ValueError("cu_seqlens and cu_seqlens_host differ in length")
    return cu_dev, cu_host


def _workspace(ws, nbytes, device, required=False):
    """A caller's workspace (uint8, at least nbytes, on device, contiguous), or a new one."""
    if ws is None:
        if required:
            raise ValueError("reuse_stats needs the workspace of the call that formed them")
        return torch.empty(nbytes, dtype=torch.uint8, device=device) if nbytes else None
    if (not isinstance(ws, torch.Tensor) or ws.dtype != torch.uint8 or ws.device != device
            or not ws.is_contiguous() or ws.numel() < nbytes):
        raise ValueError("workspace must be a contiguous uint8 tensor of at least %d bytes on %s"
                         % (nbytes, device))
    return ws


def _need(t, name, shape, dtype, device):
    if t is None:
        return
    if not isinstance(t, torch.Tensor):
        raise ValueError("%s must be a torch.Tensor" % name)
    if tuple(t.shape) != tuple(shape):
        raise ValueError("%s has shape %s, expected %s" % (name, tuple(t.shape), tuple(shape)))
    if t.dtype != dtype:
        raise ValueError("%s has dtype %s, expected %s" % (name, t.dtype, dtype))
    if t.device != device:
        raise ValueError("%s is on %s, expected %s" % (name, t.device, device))
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)


def gdn_fwd(q, k, v, beta, g=None, gk=None, scale=1.0, h0=None, *, want_ht=True,
            want_h=False, want_v_new=False):
    """Dense forward.  q, k [B,T,H,K], v [B,T,H,V] (fp32 or bf16, same dtype), beta / g
    [B,T,H] fp32, gk [B,T,H,K] fp32, h0 [B,H,K,V] fp32.  Returns a dict with o [B,T,H,V]
    (input dtype), and ht [B,H,K,V] fp32, h [B,H,NT,K,V] (input dtype), v_new [B,T,H,V]
    when requested."""
    if q.dtype not in _DT:
        raise ValueError("q must be float32 or bfloat16, got %s" % q.dtype)
    B, T, H, K = q.shape
    V = v.shape[-1]
    dev, dt = q.device, q.dtype
    _need(q, "q", (B, T, H, K), dt, dev)
    _need(k, "k", (B, T, H, K), dt, dev)
    _need(v, "v", (B, T, H, V), dt, dev)
    _need(beta, "beta", (B, T, H), torch.float32, dev)
    _need(g, "g", (B, T, H), torch.float32, dev)
    _need(gk, "gk", (B, T, H, K), torch.float32, dev)
    _need(h0, "h0", (B, H, K, V), torch.float32, dev)
    NT = (T + CHUNK - 1) // CHUNK
    o = torch.empty(B, T, H, V, dtype=dt, device=dev)
    ht = torch.empty(B, H, K, V, dtype=torch.float32, device=dev) if want_ht else None
    hch = torch.empty(B, H, NT, K, V, dtype=dt, device=dev) if want_h else None
    vn = torch.empty(B, T, H, V, dtype=dt, device=dev) if want_v_new else None
    lib = _lib.load()
    ws_n = lib.gdn_fwd_workspace_bytes(B, T, H, K, V, _DT[dt], _fwd_flags(gk, want_h, want_v_new))
    ws = torch.empty(ws_n, dtype=torch.uint8, device=dev) if ws_n else None
    rc = lib.gdn_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(gk), _ptr(beta), float(scale),
                     _ptr(h0), _ptr(o), _ptr(ht), _ptr(hch), _ptr(vn), B, T, H, K, V, _DT[dt],
                     _ptr(ws), ws_n, _stream(dev))
    _lib.check(rc, "gdn_fwd")
    out = {"o": o}
    if want_ht:
        out["ht"] = ht
    if want_h:
        out["h"] = hch
    if want_v_new:
        out["v_new"] = vn
    return out


def gdn_state_summary(k, v, beta, g=None, gk=None, *, want_transition=True):
    """State summary of a fragment: (state_ext [B,H,K,V] fp32, transition [B,H,K,K] fp32 or
    None) with ht(h0) = transition @ h0 + state_ext.  k [B,T,H,K], v [B,T,H,V] (fp32 or
    bf16), beta, g [B,T,H] fp32, gk [B,T,H,K] fp32."""
    if k.dtype not in _DT:
        raise ValueError("k must be float32 or bfloat16, got %s" % k.dtype)
    B, T, H, K = k.shape
    V = v.shape[-1]
    dev, dt = k.device, k.dtype
    _need(k, "k", (B, T, H, K), dt, dev)
    _need(v, "v", (B, T, H, V), dt, dev)
    _need(beta, "beta", (B, T, H), torch.float32, dev)
    _need(g, "g", (B, T, H), torch.float32, dev)
    _need(gk, "gk", (B, T, H, K), torch.float32, dev)
    st = torch.empty(B, H, K, V, dtype=torch.float32, device=dev)
    tr = torch.empty(B, H, K, K, dtype=torch.float32, device=dev) if want_transition else None
    lib = _lib.load()
    ws_n = lib.gdn_state_summary_workspace_bytes(B, T, H, K, V, _DT[dt], _fwd_flags(gk, False, False))
    ws = torch.empty(ws_n, dtype=torch.uint8, device=dev) if ws_n else None
    rc = lib.gdn_state_summary(_ptr(k), _ptr(v), _ptr(g), _ptr(gk), _ptr(beta), _ptr(st),
                               _ptr(tr), B, T, H, K, V, _DT[dt], _ptr(ws), ws_n, _stream(dev))
    _lib.check(rc, "gdn_state_summary")
    return st, tr


def gdn_state_apply(state_ext, transition, h_in=None):
    """h_out = transition @ h_in + state_ext per (b, h) (fp32 [.., K, V]); h_in None = zero."""
    *lead, K, V = state_ext.shape
    BH = 1
    for d in lead:
        BH *= d
    dev = state_ext.device
    _need(state_ext, "state_ext", tuple(lead) + (K, V), torch.float32, dev)
    _need(transition, "transition", tuple(lead) + (K, K), torch.float32, dev)
    _need(h_in, "h_in", tuple(lead) + (K, V), torch.float32, dev)
    h_out = torch.empty_like(state_ext)
    rc = _lib.load().gdn_state_apply(_ptr(state_ext), _ptr(transition), _ptr(h_in), _ptr(h_out),
                                     BH, K, V, _stream(dev))
    _lib.check(rc, "gdn_state_apply")
    return h_out


def gdn_state_grad_apply(grad_state_ext, transition, grad_in=None):
    """grad_out = transition^T @ grad_in + grad_state_ext per (b, h) (fp32 [.., K, V]); the
    gradient of the state entering a fragment from that of the state leaving it."""
    *lead, K, V = grad_state_ext.shape
    BH = 1
    for d in lead:
        BH *= d
    dev = grad_state_ext.device
    _need(grad_state_ext, "grad_state_ext", tuple(lead) + (K, V), torch.float32, dev)
    _need(transition, "transition", tuple(lead) + (K, K), torch.float32, dev)
    _need(grad_in, "grad_in", tuple(lead) + (K, V), torch.float32, dev)
    out = torch.empty_like(grad_state_ext)
    rc = _lib.load().gdn_state_grad_apply(_ptr(grad_state_ext), _ptr(transition), _ptr(grad_in),
                                          _ptr(out), BH, K, V, _stream(dev))
    _lib.check(rc, "gdn_state_grad_apply")
    return out


def gdn_varlen_num_chunks(cu_seqlens_host) -> int:
    cu = torch.as_tensor(cu_seqlens_host, dtype=torch.int32).contiguous().cpu()
    return _lib.load().gdn_varlen_num_chunks(_ptr(cu), cu.numel() - 1)


def gdn_fwd_varlen(q, k, v, beta, cu_seqlens, g=None, gk=None, scale=1.0, h0=None, *,
                   want_ht=True, want_h=False, want_v_new=False, want_tables=True,
                   cu_seqlens_host=None, no_alloc=False):
    """Packed forward (batch 1).  cu_seqlens [N+1] int32 on the device (a device copy is made
    if it is a host tensor); cu_seqlens_host: its host copy, which the library validates and
    sizes the call from (made from cu_seqlens, with a device wait, when not given).  Returns
    o, and ht [N,H,K,V], h [1,H,NT_total,K,V], v_new, chunk_offsets [N+1] and
    chunk_indices [NT_total,2] (int32) when requested.  no_alloc: call
    gdn_fwd_varlen_noalloc, whose scratch is the library's static device array (for callers
    that cannot allocate; the call allocates nothing but its outputs here)."""
    if q.dtype not in _DT:
        raise ValueError("q must be float32 or bfloat16, got %s" % q.dtype)
    one, T, H, K = q.shape
    if one != 1:
        raise ValueError("packed input must have batch 1, got %d" % one)
    V = v.shape[-1]
    dev, dt = q.device, q.dtype
    cu_dev, cu_host = _cu_pair(cu_seqlens, cu_seqlens_host, dev)
    N = cu_host.numel() - 1
    _need(q, "q", (1, T, H, K), dt, dev)
    _need(k, "k", (1, T, H, K), dt, dev)
    _need(v, "v", (1, T, H, V), dt, dev)
    _need(beta, "beta", (1, T, H), torch.float32, dev)
    _need(g, "g", (1, T, H), torch.float32, dev)
    _need(gk, "gk", (1, T, H, K), torch.float32, dev)
    _need(h0, "h0", (N, H, K, V), torch.float32, dev)
    lib = _lib.load()
    NT = lib.gdn_varlen_num_chunks(_ptr(cu_host), N)
    if NT < 0:
        raise ValueError("malformed cu_seqlens: %s" % cu_host.tolist()[:16])
    o = torch.empty(1, T, H, V, dtype=dt, device=dev)
    ht = torch.empty(N, H, K, V, dtype=torch.float32, device=dev) if want_ht else None
    hch = torch.empty(1, H, NT, K, V, dtype=dt, device=dev) if want_h else None
    vn = torch.empty(1, T, H, V, dtype=dt, device=dev) if want_v_new else None
    offs = torch.empty(N + 1, dtype=torch.int32, device=dev) if want_tables else None
    idx = torch.empty(NT, 2, dtype=torch.int32, device=dev) if want_tables else None
    if no_alloc:
        rc = lib.gdn_fwd_varlen_noalloc(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(gk), _ptr(beta),
                                        float(scale), _ptr(cu_dev), _ptr(cu_host), N, _ptr(h0),
                                        _ptr(o), _ptr(ht), _ptr(hch), _ptr(vn), _ptr(offs),
                                        _ptr(idx), T, H, K, V, _DT[dt], _stream(dev))
        _lib.check(rc, "gdn_fwd_varlen_noalloc")
    else:
        ws_n = lib.gdn_fwd_varlen_workspace_bytes(T, N, NT, H, K, V, _DT[dt],
                                                  _fwd_flags(gk, want_h, want_v_new))
        ws = torch.empty(ws_n, dtype=torch.uint8, device=dev) if ws_n else None
        rc = lib.gdn_fwd_varlen(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(gk), _ptr(beta),
                                float(scale), _ptr(cu_dev), _ptr(cu_host), N, _ptr(h0), _ptr(o),
                                _ptr(ht), _ptr(hch), _ptr(vn), _ptr(offs), _ptr(idx), T, H, K,
                                V, _DT[dt], _ptr(ws), ws_n, _stream(dev))
        _lib.check(rc, "gdn_fwd_varlen")
    out = {"o": o}
    if want_ht:
        out["ht"] = ht
    if want_h:
        out["h"] = hch
    if want_v_new:
        out["v_new"] = vn
    if want_tables:
        out["chunk_offsets"] = offs
        out["chunk_indices"] = idx
    return out


def gdn_prep(qkv, q_norm_w, k_norm_w, rope_cos, rope_sin, k_scale, norm_eps=1e-5, *,
             outputs=("q_inv_rms", "k_inv_rms", "q_rot", "k_rot", "q_pos", "k_pos", "v")):
    """BiGDN front end.  qkv [B,N,3,H,D] bf16; weights [H*D] fp32; rope tables [N,D] fp32.
    Returns the requested outputs: q_inv_rms / k_inv_rms [B,N] fp32 and q_rot, k_rot, q_pos,
    k_pos, v [B,H,N,D] bf16."""
    B, N, three, H, D = qkv.shape
    dev = qkv.device
    if three != 3:
        raise ValueError("qkv must be [B,N,3,H,D]")
    _need(qkv, "qkv", (B, N, 3, H, D), torch.bfloat16, dev)
    _need(q_norm_w, "q_norm_w", (H * D,), torch.float32, dev)
    _need(k_norm_w, "k_norm_w", (H * D,), torch.float32, dev)
    _need(rope_cos, "rope_cos", (N, D), torch.float32, dev)
    _need(rope_sin, "rope_sin", (N, D), torch.float32, dev)
    out = {}
    for name in outputs:
        if name in ("q_inv_rms", "k_inv_rms"):
            out[name] = torch.empty(B, N, dtype=torch.float32, device=dev)
        elif name in ("q_rot", "k_rot", "q_pos", "k_pos", "v"):
            out[name] = torch.empty(B, H, N, D, dtype=torch.bfloat16, device=dev)
        else:
            raise ValueError("unknown prep output %r" % name)
    rc = _lib.load().gdn_prep(
        _ptr(qkv), _ptr(q_norm_w), _ptr(k_norm_w), _ptr(rope_cos), _ptr(rope_sin),
        float(k_scale), float(norm_eps), _ptr(out.get("q_inv_rms")), _ptr(out.get("k_inv_rms")),
        _ptr(out.get("q_rot")), _ptr(out.get("k_rot")), _ptr(out.get("q_pos")),
        _ptr(out.get("k_pos")), _ptr(out.get("v")), B, N, H, D, _stream(dev))
    _lib.check(rc, "gdn_prep")
    return out


def bigdn_fwd(qkv, beta, decay, q_norm_w, k_norm_w, rope_cos, rope_sin, k_scale,
              norm_eps=1e-5):
    """BiGDN block forward.  qkv [B,N,3,H,D] bf16, beta [B,H,F,S] fp32, decay [B,H,F] fp32.
    Returns (num [B,N,H,D] bf16, den [B,H,N] bf16), the sums over both directions."""
    B, N, three, H, D = qkv.shape
    dev = qkv.device
    F, S = beta.shape[2], beta.shape[3]
    if three != 3 or F * S != N:
        raise ValueError("qkv must be [B,N,3,H,D] with N = F*S")
    _need(qkv, "qkv", (B, N, 3, H, D), torch.bfloat16, dev)
    _need(beta, "beta", (B, H, F, S), torch.float32, dev)
    _need(decay, "decay", (B, H, F), torch.float32, dev)
    _need(q_norm_w, "q_norm_w", (H * D,), torch.float32, dev)
    _need(k_norm_w, "k_norm_w", (H * D,), torch.float32, dev)
    _need(rope_cos, "rope_cos", (N, D), torch.float32, dev)
    _need(rope_sin, "rope_sin", (N, D), torch.float32, dev)
    num = torch.empty(B, N, H, D, dtype=torch.bfloat16, device=dev)
    den = torch.empty(B, H, N, dtype=torch.bfloat16, device=dev)
    lib = _lib.load()
    ws_n = lib.bigdn_fwd_workspace_bytes(B, F, S, H, D)
    ws = torch.empty(ws_n, dtype=torch.uint8, device=dev) if ws_n else None
    rc = lib.bigdn_fwd(_ptr(qkv), _ptr(beta), _ptr(decay), _ptr(q_norm_w), _ptr(k_norm_w),
                       _ptr(rope_cos), _ptr(rope_sin), float(k_scale), float(norm_eps),
                       _ptr(num), _ptr(den), B, F, S, H, D, _ptr(ws), ws_n, _stream(dev))
    _lib.check(rc, "bigdn_fwd")
    return num, den


def bigdn_fwd_merged(qkv, beta, decay, q_norm_w, k_norm_w, rope_cos, rope_sin, k_scale,
                     norm_eps=1e-5, *, qkv_bwd=None, beta_bwd=None, decay_bwd=None, gate=None,
                     merge_eps=1e-6, want_num_den=False):
    """BiGDN block with reverse-direction overrides (qkv_bwd [B,N,3,H,D] bf16, beta_bwd
    [B,H,F,S], decay_bwd [B,H,F] fp32) and the merge epilogue out = num / (den + merge_eps) * SiLU(gate) (gate [B,N,H,D]
    bf16 or None).  Returns out [B,N,H,D] bf16, or (out, num, den) with want_num_den."""
    B, N, three, H, D = qkv.shape
    dev = qkv.device
    F, S = beta.shape[2], beta.shape[3]
    if three != 3 or F * S != N:
        raise ValueError("qkv must be [B,N,3,H,D] with N = F*S")
    _need(qkv, "qkv", (B, N, 3, H, D), torch.bfloat16, dev)
    _need(qkv_bwd, "qkv_bwd", (B, N, 3, H, D), torch.bfloat16, dev)
    _need(beta, "beta", (B, H, F, S), torch.float32, dev)
    _need(decay, "decay", (B, H, F), torch.float32, dev)
    _need(beta_bwd, "beta_bwd", (B, H, F, S), torch.float32, dev)
    _need(decay_bwd, "decay_bwd", (B, H, F), torch.float32, dev)
    _need(gate, "gate", (B, N, H, D), torch.bfloat16, dev)
    _need(q_norm_w, "q_norm_w", (H * D,), torch.float32, dev)
    _need(k_norm_w, "k_norm_w", (H * D,), torch.float32, dev)
    _need(rope_cos, "rope_cos", (N, D), torch.float32, dev)
    _need(rope_sin, "rope_sin", (N, D), torch.float32, dev)
    out = torch.empty(B, N, H, D, dtype=torch.bfloat16, device=dev)
    num = torch.empty(B, N, H, D, dtype=torch.bfloat16, device=dev) if want_num_den else None
    den = torch.empty(B, H, N, dtype=torch.bfloat16, device=dev) if want_num_den else None
    lib = _lib.load()
    rev = qkv_bwd is not None or beta_bwd is not None
    ws_n = lib.bigdn_fwd_merged_workspace_bytes(B, F, S, H, D, int(rev))
    ws = torch.empty(ws_n, dtype=torch.uint8, device=dev) if ws_n else None
    rc = lib.bigdn_fwd_merged(_ptr(qkv), _ptr(qkv_bwd), _ptr(beta), _ptr(decay), _ptr(beta_bwd),
                              _ptr(decay_bwd), _ptr(q_norm_w), _ptr(k_norm_w), _ptr(rope_cos),
                              _ptr(rope_sin), float(k_scale), float(norm_eps), _ptr(gate),
                              float(merge_eps), _ptr(out), _ptr(num), _ptr(den), B, F, S, H, D,
                              _ptr(ws), ws_n, _stream(dev))
    _lib.check(rc, "bigdn_fwd_merged")
    return (out, num, den) if want_num_den else out


def cam_prep(q, k, v, q_norm_w, k_norm_w, proj_q, proj_kv, rope_cos, rope_sin, k_scale,
             norm_eps=1e-5):
    """Camera-branch prep.  q, k, v [B,N,H,D] fp32; proj_q, proj_kv [B,N,4,4] fp32; rope_cos,
    rope_sin [N,D/2] fp32.  Returns (q_t, k_t, v_t) [B,H,D,N] fp32 and inflation [B,H,N]."""
    B, N, H, D = q.shape
    dev = q.device
    for t, name in ((q, "q"), (k, "k"), (v, "v")):
        _need(t, name, (B, N, H, D), torch.float32, dev)
    _need(q_norm_w, "q_norm_w", (H * D,), torch.float32, dev)
    _need(k_norm_w, "k_norm_w", (H * D,), torch.float32, dev)
    _need(proj_q, "proj_q", (B, N, 4, 4), torch.float32, dev)
    _need(proj_kv, "proj_kv", (B, N, 4, 4), torch.float32, dev)
    _need(rope_cos, "rope_cos", (N, D // 2), torch.float32, dev)
    _need(rope_sin, "rope_sin", (N, D // 2), torch.float32, dev)
    outs = [torch.empty(B, H, D, N, dtype=torch.float32, device=dev) for _ in range(3)]
    infl = torch.empty(B, H, N, dtype=torch.float32, device=dev)
    lib = _lib.load()
    ws_n = lib.cam_prep_workspace_bytes(B, N)
    ws = torch.empty(ws_n, dtype=torch.uint8, device=dev) if ws_n else None
    rc = lib.cam_prep(_ptr(q), _ptr(k), _ptr(v), _ptr(q_norm_w), _ptr(k_norm_w), _ptr(proj_q),
                      _ptr(proj_kv), _ptr(rope_cos), _ptr(rope_sin), float(k_scale),
                      float(norm_eps), _ptr(outs[0]), _ptr(outs[1]), _ptr(outs[2]), _ptr(infl),
                      B, N, H, D, _ptr(ws), ws_n, _stream(dev))
    _lib.check(rc, "cam_prep")
    return outs[0], outs[1], outs[2], infl


def cam_prep_bwd(q, k, q_norm_w, k_norm_w, proj_q, proj_kv, rope_cos, rope_sin, k_scale, dq_t,
                 dk_t, dv_t, dinfl=None, norm_eps=1e-5):
    """Backward of cam_prep.  q, k and the prep's parameters as given to cam_prep; dq_t, dk_t,
    dv_t the gradients of its outputs, [B,H,D,N] or [ndir,B,H,D,N] fp32 (the directions are
    summed); dinfl [B,H,N] fp32 or None.  Returns a dict with dq, dk, dv [B,N,H,D] and
    dq_norm_w, dk_norm_w [H*D] (fp32)."""
    B, N, H, D = q.shape
    dev = q.device
    _need(q, "q", (B, N, H, D), torch.float32, dev)
    _need(k, "k", (B, N, H, D), torch.float32, dev)
    _need(q_norm_w, "q_norm_w", (H * D,), torch.float32, dev)
    _need(k_norm_w, "k_norm_w", (H * D,), torch.float32, dev)
    _need(proj_q, "proj_q", (B, N, 4, 4), torch.float32, dev)
    _need(proj_kv, "proj_kv", (B, N, 4, 4), torch.float32, dev)
    _need(rope_cos, "rope_cos", (N, D // 2), torch.float32, dev)
    _need(rope_sin, "rope_sin", (N, D // 2), torch.float32, dev)
    ndir = 1 if dq_t.dim() == 4 else dq_t.shape[0]
    shape = (B, H, D, N) if dq_t.dim() == 4 else (ndir, B, H, D, N)
    for t, name in ((dq_t, "dq_t"), (dk_t, "dk_t"), (dv_t, "dv_t")):
        _need(t, name, shape, torch.float32, dev)
    _need(dinfl, "dinfl", (B, H, N), torch.float32, dev)
    out = {n: torch.empty(B, N, H, D, dtype=torch.float32, device=dev) for n in ("dq", "dk", "dv")}
    out["dq_norm_w"] = torch.empty(H * D, dtype=torch.float32, device=dev)
    out["dk_norm_w"] = torch.empty(H * D, dtype=torch.float32, device=dev)
    lib = _lib.load()
    ws_n = lib.cam_prep_bwd_workspace_bytes(B, N, H, D)
    ws = torch.empty(ws_n, dtype=torch.uint8, device=dev) if ws_n else None
    rc = lib.cam_prep_bwd(_ptr(q), _ptr(k), _ptr(q_norm_w), _ptr(k_norm_w), _ptr(proj_q),
                          _ptr(proj_kv), _ptr(rope_cos), _ptr(rope_sin), float(k_scale),
                          float(norm_eps), ndir, _ptr(dq_t), _ptr(dk_t), _ptr(dv_t), _ptr(dinfl),
                          _ptr(out["dq"]), _ptr(out["dk"]), _ptr(out["dv"]),
                          _ptr(out["dq_norm_w"]), _ptr(out["dk_norm_w"]), B, N, H, D, _ptr(ws),
                          ws_n, _stream(dev))
    _lib.check(rc, "cam_prep_bwd")
    return out


def cam_scan(q, k, v, beta, decay, *, reverse=False, init_state=None, save_final_state=False):
    """Camera-branch numerator-only frame scan.  q, k, v [B,H,D,N] fp32 (channel-major);
    beta [B,H,F,S]; decay [B,H,F]; init_state [B*H,D,D] fp32 (forward only).  Returns out
    [B,H,D,N] fp32, or (out, final_state [B*H,D,D]) with save_final_state (forward only)."""
    B, H, D, N = q.shape
    dev = q.device
    F, S = beta.shape[2], beta.shape[3]
    if F * S != N:
        raise ValueError("q must be [B,H,D,N] with N = F*S")
    for t, name in ((q, "q"), (k, "k"), (v, "v")):
        _need(t, name, (B, H, D, N), torch.float32, dev)
    _need(beta, "beta", (B, H, F, S), torch.float32, dev)
    _need(decay, "decay", (B, H, F), torch.float32, dev)
    _need(init_state, "init_state", (B * H, D, D), torch.float32, dev)
    out = torch.empty(B, H, D, N, dtype=torch.float32, device=dev)
    fin = torch.empty(B * H, D, D, dtype=torch.float32, device=dev) if save_final_state else None
    lib = _lib.load()
    ws_n = lib.cam_scan_workspace_bytes(B, H, D, F)
    ws = torch.empty(ws_n, dtype=torch.uint8, device=dev) if ws_n else None
    rc = lib.cam_scan(_ptr(q), _ptr(k), _ptr(v), _ptr(beta), _ptr(decay), int(bool(reverse)),
                      _ptr(init_state), _ptr(fin), _ptr(out), B, H, D, F, S, _ptr(ws), ws_n,
                      _stream(dev))
    _lib.check(rc, "cam_scan")
    return (out, fin) if save_final_state else out


def cam_scan_bidi(q, k, v, beta, decay, *, decay_bwd=None, init_state=None,
                  save_final_state=False):
    """Both camera-scan directions in one call (shared frame statistics).  Returns (out_fwd,
    out_rev) [B,H,D,N] fp32, plus the forward final state with save_final_state."""
    B, H, D, N = q.shape
    dev = q.device
    F, S = beta.shape[2], beta.shape[3]
    if F * S != N:
        raise ValueError("q must be [B,H,D,N] with N = F*S")
    for t, name in ((q, "q"), (k, "k"), (v, "v")):
        _need(t, name, (B, H, D, N), torch.float32, dev)
    _need(beta, "beta", (B, H, F, S), torch.float32, dev)
    _need(decay, "decay", (B, H, F), torch.float32, dev)
    _need(decay_bwd, "decay_bwd", (B, H, F), torch.float32, dev)
    _need(init_state, "init_state", (B * H, D, D), torch.float32, dev)
    of = torch.empty(B, H, D, N, dtype=torch.float32, device=dev)
    orv = torch.empty(B, H, D, N, dtype=torch.float32, device=dev)
    fin = torch.empty(B * H, D, D, dtype=torch.float32, device=dev) if save_final_state else None
    lib = _lib.load()
    ws_n = lib.cam_scan_bidi_workspace_bytes(B, H, D, F)
    ws = torch.empty(ws_n, dtype=torch.uint8, device=dev) if ws_n else None
    rc = lib.cam_scan_bidi(_ptr(q), _ptr(k), _ptr(v), _ptr(beta), _ptr(decay), _ptr(decay_bwd),
                           _ptr(init_state), _ptr(fin), _ptr(of), _ptr(orv), B, H, D, F, S,
                           _ptr(ws), ws_n, _stream(dev))
    _lib.check(rc, "cam_scan_bidi")
    return (of, orv, fin) if save_final_state else (of, orv)


def cam_scan_bwd(q, k, v, beta, decay, dout, reverse=False, *, accumulate=False, out=None,
                 workspace=None, reuse_stats=False):
    """Backward of cam_scan (one direction, no state in / out): gradients of sum(out * dout).
    q, k, v, dout [B,H,D,N] fp32; beta [B,H,F,S]; decay [B,H,F].  Returns a dict with dq,
    dk, dv [B,H,D,N], dbeta [B,H,F,S] and ddecay [B,H,F] (fp32).  out: a dict of those
    tensors to write into (contiguous; e.g. one direction's slice of [2,B,H,D,N] tensors for
    cam_prep_bwd); accumulate: add dbeta and ddecay to out's contents instead of writing
    them.  workspace: a uint8 tensor of cam_scan_bwd_workspace_bytes (else one is allocated);
    reuse_stats: it holds the frame statistics of a previous call with the same q, k, v, beta
    (the other direction's), which are then not formed again."""
    B, H, D, N = q.shape
    F, S = beta.shape[2], beta.shape[3]
    dev = q.device
    for t, name in ((q, "q"), (k, "k"), (v, "v"), (dout, "dout")):
        _need(t, name, (B, H, D, N), torch.float32, dev)
    _need(beta, "beta", (B, H, F, S), torch.float32, dev)
    _need(decay, "decay", (B, H, F), torch.float32, dev)
    if F * S != N:
        raise ValueError("beta is [B,H,F,S] with F*S = %d, but N = %d" % (F * S, N))
    shapes = dict({n: (B, H, D, N) for n in ("dq", "dk", "dv")}, dbeta=(B, H, F, S),
                  ddecay=(B, H, F))
    if out is None:
        if accumulate:
            raise ValueError("accumulate needs out (the dbeta and ddecay to add to)")
        out = {n: torch.empty(*shp, dtype=torch.float32, device=dev) for n, shp in shapes.items()}
    else:
        for n, shp in shapes.items():
            if n not in out or not isinstance(out[n], torch.Tensor):
                raise ValueError("out[%r] must be a tensor" % n)
            _need(out[n], n, shp, torch.float32, dev)
    lib = _lib.load()
    ws_n = lib.cam_scan_bwd_workspace_bytes(B, H, D, F)
    ws = _workspace(workspace, ws_n, dev, reuse_stats)
    flag = (int(bool(reverse)) | (_lib.BWD_ACCUMULATE if accumulate else 0)
            | (_lib.BWD_REUSE_STATS if reuse_stats else 0))
    rc = lib.cam_scan_bwd(_ptr(q), _ptr(k), _ptr(v), _ptr(beta), _ptr(decay), _ptr(dout),
                          flag, _ptr(out["dq"]), _ptr(out["dk"]), _ptr(out["dv"]),
                          _ptr(out["dbeta"]), _ptr(out["ddecay"]), B, H, D, F, S, _ptr(ws), ws_n,
                          _stream(dev))
    _lib.check(rc, "cam_scan_bwd")
    return out


def cam_bwd(q, k, v, q_norm_w, k_norm_w, proj_q, proj_kv, rope_cos, rope_sin, k_scale, beta,
            decay, dout_fwd, dout_rev, dinfl=None, norm_eps=1e-5, *, decay_bwd=None):
    """Backward of the camera branch: cam_prep, then cam_scan_bidi's two outputs, from their
    gradients dout_fwd, dout_rev [B,H,D,N] fp32 and (optionally) the inflation's, dinfl
    [B,H,N].  Inputs as given to cam_prep and cam_scan_bidi (decay_bwd: the reverse
    direction's decay).  The library calls, in order: cam_prep (the prepped tensors again),
    cam_scan_bwd for the forward and the reverse direction into one [2,B,H,D,N] set of
    gradients (the reverse call's dbeta added into the forward one's, and its ddecay too
    unless decay_bwd is given; it reuses the forward call's frame statistics), cam_prep_bwd
    over both directions.  Returns a dict with dq, dk, dv [B,N,H,D],
    dq_norm_w, dk_norm_w [H*D], dbeta [B,H,F,S] (both directions), ddecay [B,H,F] (both
    directions, or the forward one's with ddecay_bwd the reverse one's when decay_bwd is
    given)."""
    B, N, H, D = q.shape
    F, S = beta.shape[2], beta.shape[3]
    dev = q.device
    qt, kt, vt, _ = cam_prep(q, k, v, q_norm_w, k_norm_w, proj_q, proj_kv, rope_cos, rope_sin,
                             k_scale, norm_eps)
    grads = {n: torch.empty(2, B, H, D, N, dtype=torch.float32, device=dev)
             for n in ("dq", "dk", "dv")}
    par = {"dbeta": torch.empty(B, H, F, S, dtype=torch.float32, device=dev),
           "ddecay": torch.empty(B, H, F, dtype=torch.float32, device=dev)}
    ws = torch.empty(_lib.load().cam_scan_bwd_workspace_bytes(B, H, D, F), dtype=torch.uint8,
                     device=dev)
    cam_scan_bwd(qt, kt, vt, beta, decay, dout_fwd, reverse=False,
                 out=dict({n: grads[n][0] for n in grads}, **par), workspace=ws)
    # beta is shared by the two directions, so the reverse call always adds its dbeta; its
    # ddecay goes to a zeroed array of its own when the reverse direction has its own decay
    sep = decay_bwd is not None
    ddecay_r = torch.zeros_like(par["ddecay"]) if sep else par["ddecay"]
    cam_scan_bwd(qt, kt, vt, beta, decay if decay_bwd is None else decay_bwd, dout_rev,
                 reverse=True, accumulate=True,
                 out=dict({n: grads[n][1] for n in grads}, dbeta=par["dbeta"], ddecay=ddecay_r),
                 workspace=ws, reuse_stats=True)
    g = cam_prep_bwd(q, k, q_norm_w, k_norm_w, proj_q, proj_kv, rope_cos, rope_sin, k_scale,
                     grads["dq"], grads["dk"], grads["dv"], dinfl, norm_eps)
    res = dict(g, dbeta=par["dbeta"], ddecay=par["ddecay"])
    if sep:
        res["ddecay_bwd"] = ddecay_r
    return res


def gdn_bwd_dhu(q, k, w, do, dv, g=None, dht=None, scale=1.0, *, gk=None, want_dh=True,
                want_dh0=True):
    """State-gradient pass of the chunked backward.  q, k, w [B,T,H,K], do, dv [B,T,H,V] (fp32
    or bf16, one dtype); g [B,T,H] and gk [B,T,H,K] fp32 log gates (gk with bf16 only); dht
    [B,H,K,V] fp32.  Returns dict with dv2
    [B,T,H,V] (input dtype), dh [B,H,NT,K,V] fp32 (gradient of the state entering each
    64-token chunk) and dh0 [B,H,K,V] fp32."""
    B, T, H, K = q.shape
    V = do.shape[-1]
    dev = q.device
    dt = q.dtype
    if dt not in _DT:
        raise ValueError("q must be float32 or bfloat16")
    for t, name in ((q, "q"), (k, "k"), (w, "w")):
        _need(t, name, (B, T, H, K), dt, dev)
    _need(do, "do", (B, T, H, V), dt, dev)
    _need(dv, "dv", (B, T, H, V), dt, dev)
    _need(g, "g", (B, T, H), torch.float32, dev)
    _need(gk, "gk", (B, T, H, K), torch.float32, dev)
    _need(dht, "dht", (B, H, K, V), torch.float32, dev)
    NT = (T + CHUNK - 1) // CHUNK
    dv2 = torch.empty(B, T, H, V, dtype=dt, device=dev)
    dh = torch.empty(B, H, NT, K, V, dtype=torch.float32, device=dev) if want_dh else None
    dh0 = torch.empty(B, H, K, V, dtype=torch.float32, device=dev) if want_dh0 else None
    rc = _lib.load().gdn_bwd_dhu(_ptr(q), _ptr(k), _ptr(w), _ptr(do), _ptr(dv), _ptr(g), _ptr(gk),
                                 _ptr(dht), float(scale), _ptr(dh), _ptr(dv2), _ptr(dh0), B, T, H, K, V,
                                 _DT[dt], _stream(dev))
    _lib.check(rc, "gdn_bwd_dhu")
    return {"dv2": dv2, "dh": dh, "dh0": dh0}


def bigdn_dir_bwd(q_rot, k_rot, q_pos, k_pos, v, beta, decay, dnum, dden, reverse=False, *,
                  accumulate=False, out=None, workspace=None, reuse_stats=False):
    """Backward of one BiGDN direction on the prepped tensors (q_rot .. v [B,H,N,D] bf16, as
    gdn_prep returns them); beta [B,H,F,S], decay [B,H,F]; dnum [B,N,H,D], dden [B,H,N] fp32.
    Returns a dict with dq_rot, dk_rot, dq_pos, dk_pos, dv [B,H,N,D], dbeta [B,H,F,S] and
    ddecay [B,H,F] (fp32).  out: a dict of those tensors to write into (contiguous; e.g. one
    direction's slice of [2,B,H,N,D] tensors for gdn_prep_bwd); accumulate: add dbeta and
    ddecay to out's contents instead of writing them.  workspace: a uint8 tensor of
    bigdn_dir_bwd_workspace_bytes (else one is allocated); reuse_stats: it holds the frame
    statistics of a previous call with the same tensors, beta, dnum and dden (the other
    direction's), which are then not formed again."""
    B, H, N, D = q_rot.shape
    F, S = beta.shape[2], beta.shape[3]
    dev = q_rot.device
    for t, name in ((q_rot, "q_rot"), (k_rot, "k_rot"), (q_pos, "q_pos"), (k_pos, "k_pos"),
                    (v, "v")):
        _need(t, name, (B, H, N, D), torch.bfloat16, dev)
    _need(beta, "beta", (B, H, F, S), torch.float32, dev)
    _need(decay, "decay", (B, H, F), torch.float32, dev)
    _need(dnum, "dnum", (B, N, H, D), torch.float32, dev)
    _need(dden, "dden", (B, H, N), torch.float32, dev)
    if F * S != N:
        raise ValueError("beta is [B,H,F,S] with F*S = %d, but N = %d" % (F * S, N))
    names = ("dq_rot", "dk_rot", "dq_pos", "dk_pos", "dv")
    shapes = dict({n: (B, H, N, D) for n in names}, dbeta=(B, H, F, S), ddecay=(B, H, F))
    if out is None:
        if accumulate:
            raise ValueError("accumulate needs out (the dbeta and ddecay to add to)")
        out = {n: torch.empty(*shp, dtype=torch.float32, device=dev) for n, shp in shapes.items()}
    else:
        for n, shp in shapes.items():
            _need(out.get(n), n, shp, torch.float32, dev)
            if n not in out or not out[n].is_contiguous():
                raise ValueError("out[%r] must be a contiguous tensor" % n)
    lib = _lib.load()
    ws_n = lib.bigdn_dir_bwd_workspace_bytes(B, H, D, F)
    ws = _workspace(workspace, ws_n, dev, reuse_stats)
    flag = (int(bool(reverse)) | (_lib.BWD_ACCUMULATE if accumulate else 0)
            | (_lib.BWD_REUSE_STATS if reuse_stats else 0))
    rc = lib.bigdn_dir_bwd(*(_ptr(x) for x in (q_rot, k_rot, q_pos, k_pos, v, beta, decay, dnum,
                                               dden)), flag,
                           *(_ptr(out[n]) for n in names + ("dbeta", "ddecay")),
                           B, H, D, F, S, _ptr(ws), ws_n, _stream(dev))
    _lib.check(rc, "bigdn_dir_bwd")
    return out


def bigdn_merge_bwd(num, den, dout, gate=None, merge_eps=1e-6):
    """Backward of the block merge out = num / (den + merge_eps) * SiLU(gate): num [B,N,H,D],
    den [B,H,N], gate [B,N,H,D] (bf16, or None), dout [B,N,H,D] fp32.  Returns a dict with
    dnum [B,N,H,D], dden [B,H,N] and dgate [B,N,H,D] (None without a gate), fp32."""
    B, N, H, D = num.shape
    dev = num.device
    _need(num, "num", (B, N, H, D), torch.bfloat16, dev)
    _need(den, "den", (B, H, N), torch.bfloat16, dev)
    _need(gate, "gate", (B, N, H, D), torch.bfloat16, dev)
    _need(dout, "dout", (B, N, H, D), torch.float32, dev)
    out = {"dnum": torch.empty(B, N, H, D, dtype=torch.float32, device=dev),
           "dden": torch.empty(B, H, N, dtype=torch.float32, device=dev),
           "dgate": None if gate is None else torch.empty(B, N, H, D, dtype=torch.float32,
                                                          device=dev)}
    rc = _lib.load().bigdn_merge_bwd(_ptr(num), _ptr(den), _ptr(gate), _ptr(dout),
                                     float(merge_eps), _ptr(out["dnum"]), _ptr(out["dden"]),
                                     _ptr(out["dgate"]), B, N, H, D, _stream(dev))
    _lib.check(rc, "bigdn_merge_bwd")
    return out


def gdn_prep_bwd(qkv, q_norm_w, k_norm_w, rope_cos, rope_sin, k_scale, grads, norm_eps=1e-5):
    """Backward of gdn_prep: grads is a dict of dq_rot, dk_rot, dq_pos, dk_pos, dv, each
    [ndir,B,H,N,D] (or [B,H,N,D]) fp32, the scan directions' gradients of the prepped
    tensors (summed).  Returns a dict with dqkv [B,N,3,H,D], dq_norm_w, dk_norm_w [H*D]
    (fp32)."""
    B, N, three, H, D = qkv.shape
    dev = qkv.device
    _need(qkv, "qkv", (B, N, 3, H, D), torch.bfloat16, dev)
    _need(q_norm_w, "q_norm_w", (H * D,), torch.float32, dev)
    _need(k_norm_w, "k_norm_w", (H * D,), torch.float32, dev)
    _need(rope_cos, "rope_cos", (N, D), torch.float32, dev)
    _need(rope_sin, "rope_sin", (N, D), torch.float32, dev)
    names = ("dq_rot", "dk_rot", "dq_pos", "dk_pos", "dv")
    ndir = 1 if grads["dq_rot"].dim() == 4 else grads["dq_rot"].shape[0]
    shape = (B, H, N, D) if grads["dq_rot"].dim() == 4 else (ndir, B, H, N, D)
    for n in names:
        _need(grads[n], n, shape, torch.float32, dev)
    out = {"dqkv": torch.empty(B, N, 3, H, D, dtype=torch.float32, device=dev),
           "dq_norm_w": torch.empty(H * D, dtype=torch.float32, device=dev),
           "dk_norm_w": torch.empty(H * D, dtype=torch.float32, device=dev)}
    lib = _lib.load()
    ws_n = lib.gdn_prep_bwd_workspace_bytes(B, N, H, D)
    ws = torch.empty(ws_n, dtype=torch.uint8, device=dev) if ws_n else None
    rc = lib.gdn_prep_bwd(_ptr(qkv), _ptr(q_norm_w), _ptr(k_norm_w), _ptr(rope_cos),
                          _ptr(rope_sin), float(k_scale), float(norm_eps), ndir,
                          *(_ptr(grads[n]) for n in names), _ptr(out["dqkv"]),
                          _ptr(out["dq_norm_w"]), _ptr(out["dk_norm_w"]), B, N, H, D, _ptr(ws),
                          ws_n, _stream(dev))
    _lib.check(rc, "gdn_prep_bwd")
    return out


def bigdn_bwd(qkv, beta, decay, q_norm_w, k_norm_w, rope_cos, rope_sin, k_scale, num, den, dout,
              gate=None, merge_eps=1e-6, norm_eps=1e-5, *, beta_bwd=None, decay_bwd=None):
    """Backward of the BiGDN block out = (num_f + num_r) / (den_f + den_r + merge_eps) *
    SiLU(gate) from the upstream gradient dout [B,N,H,D] fp32, given the block's inputs (as
    passed to bigdn_fwd_merged) and its num, den sums (bf16, as it returns them).  The library
    calls, in order: gdn_prep (the prepped tensors again), bigdn_merge_bwd, bigdn_dir_bwd for
    the forward and the reverse direction (beta_bwd / decay_bwd: the reverse direction's
    overrides), gdn_prep_bwd over both directions.  Returns a dict with dqkv [B,N,3,H,D],
    dq_norm_w, dk_norm_w [H*D], dbeta [B,H,F,S], ddecay [B,H,F] (the reverse direction's are
    added in unless overridden, then dbeta_bwd / ddecay_bwd), dgate (or None)."""
    B, N, three, H, D = qkv.shape
    F, S = beta.shape[2], beta.shape[3]
    dev = qkv.device
    p = gdn_prep(qkv, q_norm_w, k_norm_w, rope_cos, rope_sin, k_scale, norm_eps,
                 outputs=("q_rot", "k_rot", "q_pos", "k_pos", "v"))
    t = (p["q_rot"], p["k_rot"], p["q_pos"], p["k_pos"], p["v"])
    m = bigdn_merge_bwd(num, den, dout, gate, merge_eps)
    names = ("dq_rot", "dk_rot", "dq_pos", "dk_pos", "dv")
    grads = {n: torch.empty(2, B, H, N, D, dtype=torch.float32, device=dev) for n in names}
    par = {"dbeta": torch.empty(B, H, F, S, dtype=torch.float32, device=dev),
           "ddecay": torch.empty(B, H, F, dtype=torch.float32, device=dev)}
    ws = torch.empty(_lib.load().bigdn_dir_bwd_workspace_bytes(B, H, D, F), dtype=torch.uint8,
                     device=dev)
    bigdn_dir_bwd(*t, beta, decay, m["dnum"], m["dden"], reverse=False,
                  out=dict({n: grads[n][0] for n in names}, **par), workspace=ws)
    sep = beta_bwd is not None or decay_bwd is not None
    par_r = ({"dbeta": torch.empty_like(par["dbeta"]), "ddecay": torch.empty_like(par["ddecay"])}
             if sep else par)
    # the frame statistics do not depend on the direction (beta does enter them)
    bigdn_dir_bwd(*t, beta if beta_bwd is None else beta_bwd,
                  decay if decay_bwd is None else decay_bwd, m["dnum"], m["dden"], reverse=True,
                  accumulate=not sep, out=dict({n: grads[n][1] for n in names}, **par_r),
                  workspace=ws, reuse_stats=beta_bwd is None)
    g = gdn_prep_bwd(qkv, q_norm_w, k_norm_w, rope_cos, rope_sin, k_scale, grads, norm_eps)
    res = dict(g, dbeta=par["dbeta"], ddecay=par["ddecay"], dgate=m["dgate"])
    if sep:
        res["dbeta_bwd"], res["ddecay_bwd"] = par_r["dbeta"], par_r["ddecay"]
    return res


def gdn_bwd_prep(q, k, beta, do, g=None, scale=1.0, *, gk=None):
    """w [B,T,H,K] and dv = P^T do [B,T,H,V] per 64-token chunk (the inputs of gdn_bwd_dhu)
    from q, k [B,T,H,K], beta, g [B,T,H] fp32 and do [B,T,H,V] (q's dtype).  Scalar gates
    only (gk is refused by the library)."""
    B, T, H, K = q.shape
    V = do.shape[-1]
    dev = q.device
    dt = q.dtype
    if dt not in _DT:
        raise ValueError("q must be float32 or bfloat16")
    _need(q, "q", (B, T, H, K), dt, dev)
    _need(k, "k", (B, T, H, K), dt, dev)
    _need(do, "do", (B, T, H, V), dt, dev)
    _need(beta, "beta", (B, T, H), torch.float32, dev)
    _need(g, "g", (B, T, H), torch.float32, dev)
    _need(gk, "gk", (B, T, H, K), torch.float32, dev)
    w = torch.empty(B, T, H, K, dtype=dt, device=dev)
    dv = torch.empty(B, T, H, V, dtype=dt, device=dev)
    rc = _lib.load().gdn_bwd_prep(_ptr(q), _ptr(k), _ptr(beta), _ptr(g), _ptr(gk), _ptr(do),
                                  float(scale), _ptr(w), _ptr(dv), B, T, H, K, V, _DT[dt],
                                  _stream(dev))
    _lib.check(rc, "gdn_bwd_prep")
    return w, dv


def gdn_state_grad_summary(q, k, w, do, dv, g=None, scale=1.0, *, gk=None):
    """Reverse (gradient) summary of a fragment: the gradient of its entering state from its
    own outputs alone, [B,H,K,V] fp32 (inputs as gdn_bwd_dhu)."""
    B, T, H, K = q.shape
    V = do.shape[-1]
    dev = q.device
    dt = q.dtype
    if dt not in _DT:
        raise ValueError("q must be float32 or bfloat16")
    for t, name in ((q, "q"), (k, "k"), (w, "w")):
        _need(t, name, (B, T, H, K), dt, dev)
    _need(do, "do", (B, T, H, V), dt, dev)
    _need(dv, "dv", (B, T, H, V), dt, dev)
    _need(g, "g", (B, T, H), torch.float32, dev)
    _need(gk, "gk", (B, T, H, K), torch.float32, dev)
    lib = _lib.load()
    ws_n = lib.gdn_state_grad_summary_workspace_bytes(B, T, H, V, _DT[dt])
    ws = torch.empty(ws_n, dtype=torch.uint8, device=dev) if ws_n else None
    out = torch.empty(B, H, K, V, dtype=torch.float32, device=dev)
    rc = lib.gdn_state_grad_summary(_ptr(q), _ptr(k), _ptr(w), _ptr(do), _ptr(dv), _ptr(g),
                                    _ptr(gk), float(scale), _ptr(out), B, T, H, K, V, _DT[dt],
                                    _ptr(ws), ws_n, _stream(dev))
    _lib.check(rc, "gdn_state_grad_summary")
    return out


def gdn_bwd_dhu_varlen(q, k, w, do, dv, cu_seqlens, g=None, dht=None, scale=1.0, *, gk=None,
                       want_dh=True, want_dh0=True):
    """gdn_bwd_dhu over packed sequences: q, k, w [1,T,H,K], do, dv [1,T,H,V]; cu_seqlens [N+1]
    int32 (any device; copied to both sides); g [1,T,H]; dht [N,H,K,V].  Returns dict with dv2,
    dh [1,H,NT_total,K,V] and dh0 [N,H,K,V]."""
    _, T, H, K = q.shape
    V = do.shape[-1]
    dev = q.device
    dt = q.dtype
    if dt not in _DT:
        raise ValueError("q must be float32 or bfloat16")
    for t, name in ((q, "q"), (k, "k"), (w, "w")):
        _need(t, name, (1, T, H, K), dt, dev)
    _need(do, "do", (1, T, H, V), dt, dev)
    _need(dv, "dv", (1, T, H, V), dt, dev)
    cu_host = cu_seqlens.detach().to("cpu", torch.int32).contiguous()
    N = cu_host.numel() - 1
    cu_dev = cu_host.to(dev)
    _need(g, "g", (1, T, H), torch.float32, dev)
    _need(gk, "gk", (1, T, H, K), torch.float32, dev)
    _need(dht, "dht", (N, H, K, V), torch.float32, dev)
    lib = _lib.load()
    nt = lib.gdn_varlen_num_chunks(ctypes.c_void_p(cu_host.data_ptr()), N)
    if nt < 0:
        raise ValueError("malformed cu_seqlens")
    dv2 = torch.empty(1, T, H, V, dtype=dt, device=dev)
    dh = torch.empty(1, H, nt, K, V, dtype=torch.float32, device=dev) if want_dh else None
    dh0 = torch.empty(N, H, K, V, dtype=torch.float32, device=dev) if want_dh0 else None
    ws_n = lib.gdn_bwd_dhu_varlen_workspace_bytes(N, max(nt, 1))
    ws = torch.empty(ws_n, dtype=torch.uint8, device=dev) if ws_n else None
    rc = lib.gdn_bwd_dhu_varlen(_ptr(q), _ptr(k), _ptr(w), _ptr(do), _ptr(dv), _ptr(g), _ptr(gk),
                                _ptr(dht), float(scale), _ptr(cu_dev), ctypes.c_void_p(cu_host.data_ptr()), N,
                                _ptr(dh), _ptr(dv2), _ptr(dh0), T, H, K, V, _DT[dt], _ptr(ws), ws_n,
                                _stream(dev))
    _lib.check(rc, "gdn_bwd_dhu_varlen")
    return {"dv2": dv2, "dh": dh, "dh0": dh0}

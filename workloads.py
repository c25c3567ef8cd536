"""Seeded synthetic inputs for the gated delta-rule workloads.

This module is shared by the tests, the benchmark and the smoke check.  It draws random
inputs and nothing else: it holds none of the method's arithmetic, and both the HIP path
and the CPU oracle consume its tensors unchanged.

Recipe (all draws on the CPU from ``torch.Generator().manual_seed(seed)``, in this order):
  lengths (packed batches only) -> q -> k -> v -> beta logits -> g logits -> gk logits.
  q and k are drawn N(0,1) in fp32 and L2-normalised per (token, head) in fp32, then cast
  (round-to-nearest-even) to the storage dtype; v ~ N(0,1) then cast; beta = sigmoid(N(0,1))
  and g = logsigmoid(N(0,1) + shift) stay fp32; gk (per-key log decay) likewise.
The BiGDN block draws qkv ~ N(0,1) (bf16), norm weights 1 + 0.1 N(0,1), beta = sigmoid(N),
decay = sigmoid(N + 3), and uses rotary angles theta[n, i] = n * 10000^(-2i/D) expanded into
the (N, D) cos / sin table format of the SANA fused_gdn.py page (prepare_rope_tables):
cos[n, 2i] = cos[n, 2i+1] = cos(theta), sin[n, 2i] = -sin(theta), sin[n, 2i+1] = +sin(theta).
"""
from __future__ import annotations

import math

import torch

DTYPES = {"f32": torch.float32, "bf16": torch.bfloat16}


def _gen(seed):
    g = torch.Generator()
    g.manual_seed(int(seed))
    return g


def _l2n(x):
    return x / x.norm(dim=-1, keepdim=True).clamp_min(1e-12)


def gdn_inputs(B, T, H, K, V, dtype="bf16", seed=0, g_shift=3.0, per_key=False,
               gk_shift=3.0, lengths=None):
    """Inputs of a dense (or packed, when ``lengths`` is given, B must be 1) GDN forward.

    Returns a dict of CPU tensors: q, k [B,T,H,K] and v [B,T,H,V] in ``dtype``; beta, g
    [B,T,H] fp32; gk [B,T,H,K] fp32 or None.
    """
    gen = _gen(seed)
    td = DTYPES[dtype]
    q = _l2n(torch.randn(B, T, H, K, generator=gen)).to(td)
    k = _l2n(torch.randn(B, T, H, K, generator=gen)).to(td)
    v = torch.randn(B, T, H, V, generator=gen).to(td)
    beta = torch.sigmoid(torch.randn(B, T, H, generator=gen))
    g = torch.nn.functional.logsigmoid(torch.randn(B, T, H, generator=gen) + g_shift)
    gk = None
    if per_key:
        gk = torch.nn.functional.logsigmoid(torch.randn(B, T, H, K, generator=gen) + gk_shift)
    return {"q": q, "k": k, "v": v, "beta": beta, "g": g, "gk": gk}


def bwd_inputs(B, T, H, K, V, dtype="bf16", seed=0, g_shift=3.0):
    """Inputs of the backward chain (gdn_bwd_prep, then gdn_bwd_dhu): gdn_inputs, then from
    seed + 7919 the output gradient do ~ N(0, 1) [B,T,H,V] in dtype and the final-state
    gradient dht ~ N(0, 1) [B,H,K,V] fp32; scale K^-1/2."""
    inp = gdn_inputs(B, T, H, K, V, dtype=dtype, seed=seed, g_shift=g_shift)
    gen = _gen(seed + 7919)
    inp["do"] = torch.randn(B, T, H, V, generator=gen).to(DTYPES[dtype])
    inp["dht"] = torch.randn(B, H, K, V, generator=gen)
    inp["scale"] = K ** -0.5
    return inp


def varlen_lengths(n_seqs, lo, hi, seed):
    """Sequence lengths uniform in [lo, hi] (inclusive), drawn first from the seed."""
    gen = _gen(seed)
    return torch.randint(lo, hi + 1, (n_seqs,), generator=gen)


def varlen_inputs(n_seqs, lo, hi, H, K, V, dtype="bf16", seed=0, g_shift=3.0):
    """Packed batch: lengths drawn first, then the tensors of gdn_inputs(B=1, T=sum)."""
    gen = _gen(seed)
    lengths = torch.randint(lo, hi + 1, (n_seqs,), generator=gen)
    cu = torch.zeros(n_seqs + 1, dtype=torch.int32)
    cu[1:] = torch.cumsum(lengths, 0).to(torch.int32)
    T = int(cu[-1])
    td = DTYPES[dtype]
    q = _l2n(torch.randn(1, T, H, K, generator=gen)).to(td)
    k = _l2n(torch.randn(1, T, H, K, generator=gen)).to(td)
    v = torch.randn(1, T, H, V, generator=gen).to(td)
    beta = torch.sigmoid(torch.randn(1, T, H, generator=gen))
    g = torch.nn.functional.logsigmoid(torch.randn(1, T, H, generator=gen) + g_shift)
    return {"q": q, "k": k, "v": v, "beta": beta, "g": g, "gk": None, "cu_seqlens": cu}


def rope_tables(N, D):
    """Expanded (N, D) fp32 cos / sin tables for theta[n, i] = n * 10000^(-2i/D)."""
    n = torch.arange(N, dtype=torch.float64)[:, None]
    i = torch.arange(D // 2, dtype=torch.float64)[None, :]
    theta = n * torch.pow(10000.0, -2.0 * i / D)
    c, s = torch.cos(theta), torch.sin(theta)
    cos_t = c.repeat_interleave(2, dim=-1)
    sin_t = torch.stack([-s, s], dim=-1).reshape(N, D)
    return cos_t.float().contiguous(), sin_t.float().contiguous()


def bigdn_inputs(B, F, S, H, D, seed=0, decay_shift=3.0):
    """BiGDN block inputs: qkv [B,N,3,H,D] bf16, beta [B,H,F,S], decay [B,H,F], norm weights
    [H*D] x2, RoPE tables [N,D] x2, k_scale = D^-1/2 * S^-1/2, eps = 1e-5."""
    gen = _gen(seed)
    N = F * S
    qkv = torch.randn(B, N, 3, H, D, generator=gen).to(torch.bfloat16)
    q_norm_w = 1.0 + 0.1 * torch.randn(H * D, generator=gen)
    k_norm_w = 1.0 + 0.1 * torch.randn(H * D, generator=gen)
    beta = torch.sigmoid(torch.randn(B, H, F, S, generator=gen))
    decay = torch.sigmoid(torch.randn(B, H, F, generator=gen) + decay_shift)
    rope_cos, rope_sin = rope_tables(N, D)
    return {"qkv": qkv, "beta": beta, "decay": decay, "q_norm_w": q_norm_w,
            "k_norm_w": k_norm_w, "rope_cos": rope_cos, "rope_sin": rope_sin,
            "k_scale": 1.0 / math.sqrt(D) / math.sqrt(S), "eps": 1e-5}


def prep_bwd_inputs(B, F, S, H, D, ndir=2, seed=0):
    """Inputs of the front-end backward: bigdn_inputs, then (from seed + 7919) the scan
    directions' gradients of the prepped tensors, dq_rot, dk_rot, dq_pos, dk_pos, dv
    [ndir,B,H,N,D] fp32 ~ N(0, 1)."""
    inp = bigdn_inputs(B, F, S, H, D, seed=seed)
    gen = _gen(seed + 7919)
    N = F * S
    inp["grads"] = {n: torch.randn(ndir, B, H, N, D, generator=gen)
                    for n in ("dq_rot", "dk_rot", "dq_pos", "dk_pos", "dv")}
    return inp


def merge_bwd_inputs(B, N, H, D, gated=True, seed=0):
    """Inputs of the merge backward: num [B,N,H,D] bf16 ~ N(0, 1), den [B,H,N] bf16 ~ U(0.5, 2)
    (the normaliser sums are positive), gate [B,N,H,D] bf16 ~ N(0, 1) (or None), dout
    [B,N,H,D] fp32 ~ N(0, 1)."""
    gen = _gen(seed)
    inp = {"num": torch.randn(B, N, H, D, generator=gen).to(torch.bfloat16),
           "den": (0.5 + 1.5 * torch.rand(B, H, N, generator=gen)).to(torch.bfloat16),
           "gate": torch.randn(B, N, H, D, generator=gen).to(torch.bfloat16) if gated else None}
    inp["dout"] = torch.randn(B, N, H, D, generator=gen)
    return inp


def bigdn_block_bwd_inputs(B, F, S, H, D, seed=0):
    """Inputs of the whole block's backward: bigdn_inputs, a gate [B,N,H,D] bf16 ~ N(0, 1) and
    (from seed + 7919) the upstream gradient dout [B,N,H,D] fp32 ~ N(0, 1)."""
    inp = bigdn_inputs(B, F, S, H, D, seed=seed)
    gen = _gen(seed + 7919)
    N = F * S
    inp["gate"] = torch.randn(B, N, H, D, generator=gen).to(torch.bfloat16)
    inp["dout"] = torch.randn(B, N, H, D, generator=gen)
    return inp


def dhu_inputs(B, T, H, K, V, dtype="bf16", seed=0, g_shift=3.0, per_key=False):
    """Inputs of the state-gradient pass: q, k L2-normalised per (token, head) and w with the
    magnitude of the WY w (a unit vector times a sigmoid), do, dv ~ N(0,1) in the given dtype;
    g = log sigmoid(N(0,1) + g_shift) [B,T,H]; dht ~ N(0,1) [B,H,K,V] fp32; scale K^-1/2;
    with per_key, gk = log sigmoid(N(0,1) + 3) [B,T,H,K] (drawn last)."""
    gen = _gen(seed)
    dt = torch.bfloat16 if dtype == "bf16" else torch.float32
    q = _l2n(torch.randn(B, T, H, K, generator=gen))
    k = _l2n(torch.randn(B, T, H, K, generator=gen))
    w = _l2n(torch.randn(B, T, H, K, generator=gen)) * torch.sigmoid(
        torch.randn(B, T, H, 1, generator=gen))
    do = torch.randn(B, T, H, V, generator=gen)
    dv = torch.randn(B, T, H, V, generator=gen)
    g = torch.nn.functional.logsigmoid(torch.randn(B, T, H, generator=gen) + g_shift)
    dht = torch.randn(B, H, K, V, generator=gen)
    gk = (torch.nn.functional.logsigmoid(torch.randn(B, T, H, K, generator=gen) + 3.0)
          if per_key else None)
    return {"q": q.to(dt), "k": k.to(dt), "w": w.to(dt), "do": do.to(dt), "dv": dv.to(dt),
            "g": g, "gk": gk, "dht": dht, "scale": K ** -0.5}


def cam_inputs(B, F, S, H, D, seed=0, decay_shift=3.0, translate=0.3):
    """Camera-branch inputs: raw q, k, v [B,N,H,D] fp32; norm weights [H*D] x2; per-token 4x4
    camera matrices proj_q = M^T and proj_kv = M^-1 [B,N,4,4] for a random rigid motion M
    (rotation from the QR factor of a Gaussian matrix, translation N(0, translate^2));
    RoPE tables [N, D/2] x2; beta [B,H,F,S]; decay [B,H,F]; k_scale = D^-1/2 * S^-1/2."""
    gen = _gen(seed)
    N = F * S
    q = torch.randn(B, N, H, D, generator=gen)
    k = torch.randn(B, N, H, D, generator=gen)
    v = torch.randn(B, N, H, D, generator=gen)
    q_norm_w = 1.0 + 0.1 * torch.randn(H * D, generator=gen)
    k_norm_w = 1.0 + 0.1 * torch.randn(H * D, generator=gen)
    a = torch.randn(B * N, 3, 3, generator=gen, dtype=torch.float64)
    rot, r = torch.linalg.qr(a)
    rot = rot * torch.sign(torch.diagonal(r, dim1=-2, dim2=-1))[:, None, :]
    m = torch.zeros(B * N, 4, 4, dtype=torch.float64)
    m[:, :3, :3] = rot
    m[:, :3, 3] = translate * torch.randn(B * N, 3, generator=gen, dtype=torch.float64)
    m[:, 3, 3] = 1.0
    proj_q = m.transpose(1, 2).reshape(B, N, 4, 4).float().contiguous()
    proj_kv = torch.linalg.inv(m).reshape(B, N, 4, 4).float().contiguous()
    beta = torch.sigmoid(torch.randn(B, H, F, S, generator=gen))
    decay = torch.sigmoid(torch.randn(B, H, F, generator=gen) + decay_shift)
    rope_cos, rope_sin = rope_tables(N, D // 2)
    return {"q": q, "k": k, "v": v, "q_norm_w": q_norm_w, "k_norm_w": k_norm_w,
            "proj_q": proj_q, "proj_kv": proj_kv, "rope_cos": rope_cos, "rope_sin": rope_sin,
            "beta": beta, "decay": decay, "k_scale": 1.0 / math.sqrt(D) / math.sqrt(S),
            "eps": 1e-5}


def cam_prep_bwd_inputs(B, F, S, H, D, ndir=2, infl=True, seed=0):
    """Inputs of the camera prep backward: cam_inputs, then (from seed + 7919) the gradients
    of the prep's outputs dq_t, dk_t, dv_t [ndir,B,H,D,N] fp32 ~ N(0, 1) and of the inflation,
    dinfl [B,H,N] ~ N(0, 1) (None without infl)."""
    inp = cam_inputs(B, F, S, H, D, seed=seed)
    gen = _gen(seed + 7919)
    N = F * S
    for n in ("dq_t", "dk_t", "dv_t"):
        inp[n] = torch.randn(ndir, B, H, D, N, generator=gen)
    inp["dinfl"] = torch.randn(B, H, N, generator=gen) if infl else None
    return inp


def cam_branch_bwd_inputs(B, F, S, H, D, seed=0):
    """Inputs of the camera branch's backward: cam_inputs, then (from seed + 7919) the
    gradients of the two scan outputs dout_fwd, dout_rev [B,H,D,N] and of the inflation, dinfl
    [B,H,N], all fp32 ~ N(0, 1)."""
    inp = cam_inputs(B, F, S, H, D, seed=seed)
    gen = _gen(seed + 7919)
    N = F * S
    inp["dout_fwd"] = torch.randn(B, H, D, N, generator=gen)
    inp["dout_rev"] = torch.randn(B, H, D, N, generator=gen)
    inp["dinfl"] = torch.randn(B, H, N, generator=gen)
    return inp


def cam_scan_inputs(B, F, S, H, D, seed=0, decay_shift=3.0):
    """Camera-scan inputs in the channel-major layout [B,H,D,N] fp32, with the magnitudes of
    prepped tensors: q, v ~ N(0, 1), k ~ N(0, k_scale^2) (k_scale = D^-1/2 * S^-1/2); beta
    [B,H,F,S]; decay [B,H,F]."""
    gen = _gen(seed)
    N = F * S
    ks = 1.0 / math.sqrt(D) / math.sqrt(S)
    q = torch.randn(B, H, D, N, generator=gen)
    k = ks * torch.randn(B, H, D, N, generator=gen)
    v = torch.randn(B, H, D, N, generator=gen)
    beta = torch.sigmoid(torch.randn(B, H, F, S, generator=gen))
    decay = torch.sigmoid(torch.randn(B, H, F, generator=gen) + decay_shift)
    return {"q": q, "k": k, "v": v, "beta": beta, "decay": decay}


def cam_scan_bwd_inputs(B, F, S, H, D, seed=0, decay_shift=3.0):
    """Inputs of the camera-scan backward: cam_scan_inputs, then the upstream gradient
    dout ~ N(0, 1) [B,H,D,N] fp32, drawn last."""
    inp = cam_scan_inputs(B, F, S, H, D, seed=seed, decay_shift=decay_shift)
    gen = _gen(seed + 7919)
    inp["dout"] = torch.randn(B, H, D, F * S, generator=gen)
    return inp


def bigdn_bwd_inputs(B, F, S, H, D, seed=0, decay_shift=3.0):
    """Inputs of the BiGDN direction backward, with the magnitudes of prepped tensors, all
    [B,H,N,D] bf16: q_rot, v ~ N(0, 1); q_pos = |N(0, 1)|; k_rot ~ N(0, k_scale^2) and
    k_pos = |N(0, 1)| k_scale (k_scale = D^-1/2 S^-1/2); beta [B,H,F,S] = sigmoid(N(0, 1));
    decay [B,H,F] = sigmoid(N(0, 1) + decay_shift); then, from seed + 7919, dnum [B,N,H,D] and
    dden [B,H,N] ~ N(0, 1) fp32."""
    gen = _gen(seed)
    N = F * S
    ks = 1.0 / math.sqrt(D) / math.sqrt(S)
    bf = torch.bfloat16
    inp = {"q_rot": torch.randn(B, H, N, D, generator=gen).to(bf),
           "k_rot": (ks * torch.randn(B, H, N, D, generator=gen)).to(bf),
           "q_pos": torch.randn(B, H, N, D, generator=gen).abs().to(bf),
           "k_pos": (ks * torch.randn(B, H, N, D, generator=gen).abs()).to(bf),
           "v": torch.randn(B, H, N, D, generator=gen).to(bf),
           "beta": torch.sigmoid(torch.randn(B, H, F, S, generator=gen)),
           "decay": torch.sigmoid(torch.randn(B, H, F, generator=gen) + decay_shift)}
    gen = _gen(seed + 7919)
    inp["dnum"] = torch.randn(B, N, H, D, generator=gen)
    inp["dden"] = torch.randn(B, H, N, generator=gen)
    return inp


# The workloads, named by what they are.
WORKLOADS = {
    "tiny_f32": dict(kind="gdn", B=1, T=256, H=2, K=64, V=64, dtype="f32", seed=0, g_shift=2.0),
    "gdn_bf16_b4h16t4096": dict(kind="gdn", B=4, T=4096, H=16, K=128, V=128, dtype="bf16",
                                seed=0, g_shift=3.0),
    "varlen_bf16_8seq": dict(kind="varlen", n_seqs=8, lo=512, hi=8192, H=16, K=128, V=128,
                             dtype="bf16", seed=0, g_shift=3.0),
    "bigdn_video_f16x1024": dict(kind="bigdn", B=1, F=16, S=1024, H=16, D=128, seed=0),
    # the whole block output of the same video block: chunk-causal reverse direction (reverse
    # decay 0 at every fourth frame) and the merge epilogue with a SiLU gate
    "bigdn_video_merged_f16x1024": dict(kind="bigdn_merged", B=1, F=16, S=1024, H=16, D=128,
                                        seed=0),
    # state-gradient pass of the backward (dhu) at the dense bf16 shape
    "dhu_bf16_b4h16t4096": dict(kind="dhu", B=4, T=4096, H=16, K=128, V=128, dtype="bf16",
                                seed=0),
    # the same pass at the long-context per-key shape
    "dhu_perkey_b2h32t32768": dict(kind="dhu", B=2, T=32768, H=32, K=128, V=128, dtype="bf16",
                                   seed=0, per_key=True),
    # the camera branch of the same video block (fp32): camera prep, then the forward and
    # the reverse numerator-only frame scans
    "cam_video_f16x1024": dict(kind="cam", B=1, F=16, S=1024, H=16, D=128, seed=0),
    # backward of the camera branch's two frame scans at the same shape (fp32 tensors with the
    # magnitudes of prepped ones, upstream gradient N(0, 1))
    "cam_bwd_video_f16x1024": dict(kind="cam_bwd", B=1, F=16, S=1024, H=16, D=128, seed=0),
    # backward of the BiGDN block's two frame-scan directions at the same shape (prepped bf16
    # tensors, fp32 upstream gradients)
    "bigdn_bwd_video_f16x1024": dict(kind="bigdn_bwd", B=1, F=16, S=1024, H=16, D=128, seed=0),
    # backward of the whole BiGDN block at the same shape, from the upstream gradient of its
    # gated output to qkv, the norm weights, beta, decay and the gate
    "bigdn_block_bwd_video_f16x1024": dict(kind="bigdn_block_bwd", B=1, F=16, S=1024, H=16, D=128,
                                           seed=0),
    # backward of the camera branch at the same shape: from the gradients of the two scan
    # outputs and of the inflation to q, k, v, the norm weights, beta and decay
    "cam_branch_bwd_video_f16x1024": dict(kind="cam_branch_bwd", B=1, F=16, S=1024, H=16,
                                          D=128, seed=0),
    "long_perkey_b2h32t32768": dict(kind="gdn", B=2, T=32768, H=32, K=128, V=128,
                                    dtype="bf16", seed=0, g_shift=3.0, per_key=True,
                                    save=True),
    # fragment state summary (transition + zero-start state) at the dense bf16 shape; the
    # gate is milder (g_shift 8) so the 4096-token transition stays inside fp32 range
    "summary_bf16_b4h16t4096": dict(kind="summary", B=4, T=4096, H=16, K=128, V=128,
                                    dtype="bf16", seed=0, g_shift=8.0),
}


def make(name):
    """Materialise a named workload's inputs (CPU tensors)."""
    w = dict(WORKLOADS[name])
    kind = w.pop("kind")
    w.pop("save", None)
    if kind in ("gdn", "summary"):
        return gdn_inputs(**w)
    if kind == "varlen":
        return varlen_inputs(**w)
    if kind == "bigdn":
        return bigdn_inputs(**w)
    if kind == "bigdn_merged":
        inp = bigdn_inputs(**w)
        gen = _gen(w["seed"] + 1)
        B, N, _, H, D = inp["qkv"].shape
        inp["decay_bwd"] = inp["decay"].clone()
        inp["decay_bwd"][:, :, ::4] = 0.0
        inp["gate"] = torch.randn(B, N, H, D, generator=gen).to(torch.bfloat16)
        return inp
    if kind == "cam":
        return cam_inputs(**w)
    if kind == "dhu":
        return dhu_inputs(**w)
    if kind == "cam_bwd":
        return cam_scan_bwd_inputs(**w)
    if kind == "bigdn_bwd":
        return bigdn_bwd_inputs(**w)
    if kind == "bigdn_block_bwd":
        return bigdn_block_bwd_inputs(**w)
    if kind == "cam_branch_bwd":
        return cam_branch_bwd_inputs(**w)
    raise KeyError(name)

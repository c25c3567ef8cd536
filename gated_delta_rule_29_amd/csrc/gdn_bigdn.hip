// gdn_bigdn.hip -- BiGDN front end (gdn_prep) and the frame-level bidirectional scan
// (bigdn_fwd) for gfx950.
//
// Front end (SANA fused_gdn.py page: _precompute_inv_rms, _fused_qk_inv_rms_kernel,
// prepare_rope_tables and the load path of _fused_gdn_kernel), per token (b, n):
//   inv_rms = 1 / sqrt(sum over all H*D channels of x^2 / (H*D) + eps)     (q and k)
//   x_pos = relu(x * inv_rms * w[h*D + d]) (times k_scale for k)
//   x_rot[d] = x_pos[d] cos[n,d] + x_pos[d^1] sin[n,d]
//
// Frame scan.  Every token of frame f reads the same decayed state (the frame loop of
// _fused_gdn_kernel), so absorbing frame f is the affine map
//   S <- d_f (S - G_f S) + U_f,   G_f = K_rot^T diag(beta) K_rot,  U_f = K_rot^T diag(beta) V
//   z <- d_f (z - Gz_f z) + uz_f, Gz_f = K_pos^T diag(beta) K_pos,  uz_f = K_pos^T beta
// (the product form state <- state W_f + U_f of _torch_cam_scan_single_chunk on the SANA
// fused_cam_gdn.py page).  The forward direction's output for frame f uses S_f (inclusive);
// the reverse direction's uses R_f, built from frames > f with R_{F-1} = 0 and
// R_f = d_{f+1}(R_{f+1} - G_{f+1} R_{f+1}) + U_{f+1} (flip-and-shift, same page).  Both
// directions share G, U, Gz, uz, and num/den only need the sums S_f + R_f, z_f + zR_f:
//   num = Q_rot (S_f + R_f),   den = Q_pos . (z_f + zR_f).
//
// Kernels: rms (inv-RMS per token; with outputs it is gdn_prep), frame_stats (G, U, Gz, uz
// per (b, h, f) from k, v with the prep applied on the fly), scan (16-column blocks of the
// state per (b, h), both directions, writes the summed states), out (num, den per 64-token
// block).  Products use fp16 operands and fp32 accumulation; the state is fp32.
#include "gdn_device.h"
#include "gdn_internal.h"

namespace gdn {

namespace {

constexpr int kPrepThreads = 256;

__device__ __forceinline__ float block_sum_256(float x, float* red) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) x += __shfl_xor(x, off, 64);
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  __syncthreads();
  if (lane == 0) red[wave] = x;
  __syncthreads();
  return red[0] + red[1] + red[2] + red[3];
}

// Loads 8 consecutive channels (16 bytes) of bf16 as floats.
__device__ __forceinline__ void load8f(const bf16* p, float* out) {
  const bf16x8 v = *reinterpret_cast<const bf16x8*>(p);
#pragma unroll
  for (int j = 0; j < 8; ++j) out[j] = (float)v[j];
}

__device__ __forceinline__ void load8f(const float* p, float* out) {
  const f32x4 a = *reinterpret_cast<const f32x4*>(p);
  const f32x4 b = *reinterpret_cast<const f32x4*>(p + 4);
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    out[j] = a[j];
    out[4 + j] = b[j];
  }
}

// Front end of 8 channels d0..d0+7 (d0 a multiple of 8, so every RoPE pair is inside).
__device__ __forceinline__ void prep8(const float* x, float inv, const float* w, const float* cs,
                                      const float* sn, float scale, float* pos, float* rot) {
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const float y = x[j] * inv * w[j];
    pos[j] = (y > 0.f ? y : 0.f) * scale;
  }
#pragma unroll
  for (int j = 0; j < 8; ++j) rot[j] = pos[j] * cs[j] + pos[j ^ 1] * sn[j];
}

__device__ __forceinline__ void store8(bf16* p, const float* x) {
  bf16x8 v;
#pragma unroll
  for (int j = 0; j < 8; ++j) v[j] = (bf16)x[j];
  *reinterpret_cast<bf16x8*>(p) = v;
}

// One workgroup per token (b, n): inverse RMS of q and k over all H*D channels, and, when
// any output pointer is set, the prepped head-major tensors.
__global__ __launch_bounds__(kPrepThreads) void rms_prep_kernel(const PrepParams p) {
  __shared__ float red[8];
  const long bn = blockIdx.x;
  const int b = bn / p.N, n = bn % p.N;
  const int C = p.H * p.D, groups = C / 8;
  const bf16* row = static_cast<const bf16*>(p.qkv) + bn * 3L * C;
  float sq = 0.f, sk = 0.f;
  for (int gi = threadIdx.x; gi < groups; gi += kPrepThreads) {
    float xq[8], xk[8];
    load8f(row + gi * 8, xq);
    load8f(row + C + gi * 8, xk);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      sq += xq[j] * xq[j];
      sk += xk[j] * xk[j];
    }
  }
  sq = block_sum_256(sq, red);
  sk = block_sum_256(sk, red + 4);
  const float iq = rsqrtf(sq / (float)C + p.eps), ik = rsqrtf(sk / (float)C + p.eps);
  if (threadIdx.x == 0) {
    if (p.q_inv_rms) p.q_inv_rms[bn] = iq;
    if (p.k_inv_rms) p.k_inv_rms[bn] = ik;
  }
  if (!(p.q_rot || p.k_rot || p.q_pos || p.k_pos || p.v_hm)) return;
  for (int gi = threadIdx.x; gi < groups; gi += kPrepThreads) {
    const int h = gi / (p.D / 8), d0 = (gi % (p.D / 8)) * 8;
    const long o = (((long)b * p.H + h) * p.N + n) * p.D + d0;
    float x[8], w[8], cs[8], sn[8], pos[8], rot[8];
    load8f(p.rope_cos + (long)n * p.D + d0, cs);
    load8f(p.rope_sin + (long)n * p.D + d0, sn);
    load8f(row + gi * 8, x);
    load8f(p.q_norm_w + gi * 8, w);
    prep8(x, iq, w, cs, sn, 1.f, pos, rot);
    if (p.q_pos) store8(static_cast<bf16*>(p.q_pos) + o, pos);
    if (p.q_rot) store8(static_cast<bf16*>(p.q_rot) + o, rot);
    load8f(row + C + gi * 8, x);
    load8f(p.k_norm_w + gi * 8, w);
    prep8(x, ik, w, cs, sn, p.k_scale, pos, rot);
    if (p.k_pos) store8(static_cast<bf16*>(p.k_pos) + o, pos);
    if (p.k_rot) store8(static_cast<bf16*>(p.k_rot) + o, rot);
    if (p.v_hm) *reinterpret_cast<uint4*>(static_cast<bf16*>(p.v_hm) + o) =
        *reinterpret_cast<const uint4*>(row + 2 * C + gi * 8);
  }
}

// ---- frame statistics -------------------------------------------------------------------
// Transposed [d][token] tiles of 64 tokens.  Token octets are XOR-swizzled with the row's
// d-octet so that the per-token stores of one wave spread over the LDS banks, while every
// 8-token run a matrix-core operand needs stays contiguous.
__device__ __forceinline__ int tr_idx(int d, int s) {
  return d * 64 + ((((s >> 3) ^ (d >> 3)) & 7) << 3) + (s & 7);
}

constexpr int kStatThreads = 256;

// part 0: G_f (fp16); part 1: U_f (fp32); part 2: Gz_f (fp16) and uz_f.  One workgroup per
// (b, h, f, part); wave w accumulates the D/2 x D/2 quadrant (w/2, w%2).
template <int D>
__global__ __launch_bounds__(kStatThreads) void frame_stats_kernel(const BigdnParams p) {
  constexpr int kT = 64;  // tokens per block
  __shared__ __attribute__((aligned(16))) f16 xa[D * kT];   // A side: x^T  (x = k_rot or k_pos)
  __shared__ __attribute__((aligned(16))) f16 xb[D * kT];   // B side: (beta x)^T or (beta v)^T
  const int part = blockIdx.y;  // 0: G, 1: U, 2: Gz
  const int bhf = blockIdx.x;
  const int f = bhf % p.F, h = (bhf / p.F) % p.H, b = bhf / (p.F * p.H);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int li = lane & 15, lq = lane >> 4;
  const int C = p.H * D;
  const bf16* qkv = static_cast<const bf16*>(p.qkv);
  const int qi = wave >> 1, qj = wave & 1;  // quadrant of D/2 x D/2
  constexpr int kQT = D / 32;                // 16x16 tiles per quadrant side
  f32x4 acc[kQT][kQT];
#pragma unroll
  for (int i = 0; i < kQT; ++i)
#pragma unroll
    for (int j = 0; j < kQT; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
  // part 2: this lane's running sum over its tokens of beta * k_pos for the d-octets its
  // wave writes (octet wave + 4i); reduced across lanes once at the end.
  float uzr[D / 32][8];
#pragma unroll
  for (int i = 0; i < D / 32; ++i)
#pragma unroll
    for (int j = 0; j < 8; ++j) uzr[i][j] = 0.f;

  for (int t0 = 0; t0 < p.S; t0 += kT) {
    __syncthreads();
    // lane -> token s = t0 + lane; wave w handles d-octets w, w+4, ... (D/8 octets)
    const int s = lane;
    const long n = (long)f * p.S + t0 + s;
    const long bn = (long)b * p.N + n;
    const float inv = p.k_inv_rms[bn];
    const float bt = p.beta[(((long)b * p.H + h) * p.F + f) * p.S + t0 + s];
    const bf16* krow = qkv + bn * 3L * C + C + (long)h * D;
    const bf16* vrow = krow + C;
#pragma unroll
    for (int oi = 0; oi < D / 32; ++oi) {
      const int oc = wave + 4 * oi;
      const int d0 = oc * 8;
      float x[8], pos[8], rot[8];
      if (part == 1) {
        float w[8], cs[8], sn[8], v[8];
        load8f(krow + d0, x);
        load8f(p.k_norm_w + h * D + d0, w);
        load8f(p.rope_cos + n * D + d0, cs);
        load8f(p.rope_sin + n * D + d0, sn);
        prep8(x, inv, w, cs, sn, p.k_scale, pos, rot);
        load8f(vrow + d0, v);
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          xa[tr_idx(d0 + j, s)] = (f16)rot[j];
          xb[tr_idx(d0 + j, s)] = (f16)(bt * v[j]);
        }
      } else {
        float w[8], cs[8], sn[8];
        load8f(krow + d0, x);
        load8f(p.k_norm_w + h * D + d0, w);
        load8f(p.rope_cos + n * D + d0, cs);
        load8f(p.rope_sin + n * D + d0, sn);
        prep8(x, inv, w, cs, sn, p.k_scale, pos, rot);
        const float* src = part == 0 ? rot : pos;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          xa[tr_idx(d0 + j, s)] = (f16)src[j];
          xb[tr_idx(d0 + j, s)] = (f16)(bt * src[j]);
          uzr[oi][j] += bt * pos[j];
        }
      }
    }
    __syncthreads();
#pragma unroll
    for (int ks = 0; ks < kT / 32; ++ks) {
      f16x8 a[kQT], bb[kQT];
#pragma unroll
      for (int i = 0; i < kQT; ++i) a[i] = lds8(&xa[tr_idx((D / 2) * qi + 16 * i + li, 32 * ks + 8 * lq)]);
#pragma unroll
      for (int j = 0; j < kQT; ++j) bb[j] = lds8(&xb[tr_idx((D / 2) * qj + 16 * j + li, 32 * ks + 8 * lq)]);
#pragma unroll
      for (int i = 0; i < kQT; ++i)
#pragma unroll
        for (int j = 0; j < kQT; ++j) acc[i][j] = mma16(a[i], bb[j], acc[i][j]);
    }
  }
  // epilogue: rows d1 = (D/2)qi + 16i + 4lq + e, columns d2 = (D/2)qj + 16j + li
  const long mat = (((long)b * p.H + h) * p.F + f) * (long)D * D;
#pragma unroll
  for (int i = 0; i < kQT; ++i)
#pragma unroll
    for (int j = 0; j < kQT; ++j)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int d1 = (D / 2) * qi + 16 * i + 4 * lq + e, d2 = (D / 2) * qj + 16 * j + li;
        const long idx = mat + (long)d1 * D + d2;
        if (part == 0) p.G[idx] = (f16)acc[i][j][e];
        else if (part == 2) p.Gz[idx] = (f16)acc[i][j][e];
        else p.U[idx] = acc[i][j][e];
      }
  if (part == 2) {
#pragma unroll
    for (int i = 0; i < D / 32; ++i)
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        float x = uzr[i][j];
#pragma unroll
        for (int off = 32; off > 0; off >>= 1) x += __shfl_xor(x, off, 64);
        if (lane == 0) p.uz[(((long)b * p.H + h) * p.F + f) * D + 8 * (wave + 4 * i) + j] = x;
      }
  }
}

// ---- scan -------------------------------------------------------------------------------
// One workgroup per (b, h, 16-column block cb) of the state; block cb == D/16 runs z.
// Wave w owns state rows 32w..32w+31 of the block.  The state lives in registers (fp32) and
// is exchanged through LDS (fp16 transposed copy) as the B operand of G S each frame.
template <int D>
__global__ __launch_bounds__(256) void scan_kernel(const BigdnParams p) {
  __shared__ __attribute__((aligned(16))) f16 st[16][D];  // state^T as fp16 operand
  __shared__ float zs[D];
  const int cb = blockIdx.x % (D / 16 + 1);
  const int bh = blockIdx.x / (D / 16 + 1);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int li = lane & 15, lq = lane >> 4;
  const int F = p.F;
  const long mat0 = (long)bh * F * D * D;
  const float* decay = p.decay + (long)bh * F;

  if (cb == D / 16) {
    // z: z <- d (z - Gz z) + uz, forward then reverse; zsum_f = z_f + zR_f.
    if (tid < D) zs[tid] = 0.f;
    __syncthreads();
    for (int f = 0; f < F; ++f) {
      float nz = 0.f;
      if (tid < D) {
        const f16* g = p.Gz + mat0 + (long)f * D * D + (long)tid * D;
        float acc = 0.f;
        for (int c = 0; c < D; ++c) acc += (float)g[c] * zs[c];
        nz = decay[f] * (zs[tid] - acc) + p.uz[((long)bh * F + f) * D + tid];
      }
      __syncthreads();
      if (tid < D) {
        zs[tid] = nz;
        p.zsum[((long)bh * F + f) * D + tid] = nz;  // forward part
      }
      __syncthreads();
    }
    if (tid < D) zs[tid] = 0.f;
    __syncthreads();
    for (int f = F - 1; f >= 0; --f) {
      if (f < F - 1) {
        float nz = 0.f;
        if (tid < D) {
          const f16* g = p.Gz + mat0 + (long)(f + 1) * D * D + (long)tid * D;
          float acc = 0.f;
          for (int c = 0; c < D; ++c) acc += (float)g[c] * zs[c];
          nz = decay[f + 1] * (zs[tid] - acc) + p.uz[((long)bh * F + f + 1) * D + tid];
        }
        __syncthreads();
        if (tid < D) zs[tid] = nz;
        __syncthreads();
      }
      if (tid < D) p.zsum[((long)bh * F + f) * D + tid] += zs[tid];
    }
    return;
  }

  constexpr int kRT = D / 64;  // 16-row tiles per wave (wave covers D/4 rows)
  const int col = cb * 16 + li;
  f32x4 s[kRT];
#pragma unroll
  for (int t = 0; t < kRT; ++t) s[t] = f32x4{0.f, 0.f, 0.f, 0.f};
  auto row_of = [&](int t, int e) { return (D / 4) * wave + 16 * t + 4 * lq + e; };
  // one step: s <- d (s - G s) + U, with G, U of frame fa
  auto step = [&](int fa) {
#pragma unroll
    for (int t = 0; t < kRT; ++t)
#pragma unroll
      for (int e = 0; e < 4; ++e) st[li][row_of(t, e)] = (f16)s[t][e];
    __syncthreads();
    const f16* G = p.G + mat0 + (long)fa * D * D;
    const float* U = p.U + mat0 + (long)fa * D * D;
    const float dcy = decay[fa];
    f32x4 gs[kRT];
#pragma unroll
    for (int t = 0; t < kRT; ++t) {
      gs[t] = f32x4{0.f, 0.f, 0.f, 0.f};
      const int r = (D / 4) * wave + 16 * t + li;
#pragma unroll
      for (int k0 = 0; k0 < D; k0 += 32)
        gs[t] = mma16(*reinterpret_cast<const f16x8*>(G + (long)r * D + k0 + 8 * lq),
                      lds8(&st[li][k0 + 8 * lq]), gs[t]);
    }
#pragma unroll
    for (int t = 0; t < kRT; ++t)
#pragma unroll
      for (int e = 0; e < 4; ++e)
        s[t][e] = dcy * (s[t][e] - gs[t][e]) + U[(long)row_of(t, e) * D + col];
    __syncthreads();
  };
  // forward: S_f after absorbing frame f; kept in fp32 in the workspace
  for (int f = 0; f < F; ++f) {
    step(f);
#pragma unroll
    for (int t = 0; t < kRT; ++t)
#pragma unroll
      for (int e = 0; e < 4; ++e) p.Sf[mat0 + (long)f * D * D + (long)row_of(t, e) * D + col] = s[t][e];
  }
  // reverse: R_{F-1} = 0, R_f from frame f+1; write (S_f + R_f)^T as fp16
#pragma unroll
  for (int t = 0; t < kRT; ++t) s[t] = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int f = F - 1; f >= 0; --f) {
    if (f < F - 1) step(f + 1);
#pragma unroll
    for (int t = 0; t < kRT; ++t)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int r = row_of(t, e);
        const float tot = s[t][e] + p.Sf[mat0 + (long)f * D * D + (long)r * D + col];
        p.SsumT[mat0 + (long)f * D * D + (long)col * D + r] = (f16)tot;
      }
  }
}

// ---- output -----------------------------------------------------------------------------
// One workgroup per (b, h, 64-token block): num = Q_rot (S + R), den = Q_pos . (z + zR).
template <int D>
__global__ __launch_bounds__(256) void out_kernel(const BigdnParams p) {
  __shared__ __attribute__((aligned(16))) f16 sT[D][D + 8];  // (S + R)^T, row = value column
  __shared__ __attribute__((aligned(16))) f16 qr[64][D + 8];  // Q_rot rows
  __shared__ float zsum[D];
  __shared__ float den_part[64][4];
  const int nblk = p.N / 64;
  const int blk = blockIdx.x % nblk;
  const int bh = blockIdx.x / nblk;
  const int b = bh / p.H, h = bh % p.H;
  const int n0 = blk * 64, f = n0 / p.S;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int li = lane & 15, lq = lane >> 4;
  const int C = p.H * D;
  const long mat = ((long)bh * p.F + f) * D * D;
  for (int e = tid; e < D * D / 8; e += 256) {
    const int r = e / (D / 8), c0 = (e % (D / 8)) * 8;
    *reinterpret_cast<uint4*>(&sT[r][c0]) = *reinterpret_cast<const uint4*>(p.SsumT + mat + (long)r * D + c0);
  }
  if (tid < D) zsum[tid] = p.zsum[((long)bh * p.F + f) * D + tid];
  __syncthreads();
  // prep of q: token t = tid / (D/8) ... 64 tokens x D/8 octets, 256 threads
  const bf16* qkv = static_cast<const bf16*>(p.qkv);
  for (int e = tid; e < 64 * (D / 8); e += 256) {
    const int t = e / (D / 8), d0 = (e % (D / 8)) * 8;
    const long n = n0 + t, bn = (long)b * p.N + n;
    float x[8], w[8], cs[8], sn[8], pos[8], rot[8];
    load8f(qkv + bn * 3L * C + (long)h * D + d0, x);
    load8f(p.q_norm_w + h * D + d0, w);
    load8f(p.rope_cos + n * D + d0, cs);
    load8f(p.rope_sin + n * D + d0, sn);
    prep8(x, p.q_inv_rms[bn], w, cs, sn, 1.f, pos, rot);
    f16x8 v;
    float dp = 0.f;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      v[j] = (f16)rot[j];
      dp += pos[j] * zsum[d0 + j];
    }
    *reinterpret_cast<f16x8*>(&qr[t][d0]) = v;
    // den partial: reduce over the D/8 octets of token t (consecutive e)
#pragma unroll
    for (int off = 1; off < D / 8; off <<= 1) dp += __shfl_xor(dp, off, 64);
    if ((e % (D / 8)) == 0) den_part[t][0] = dp;
  }
  __syncthreads();
  // num: wave w -> tokens 16w..16w+15, all D columns
  bf16* num = static_cast<bf16*>(p.num);
#pragma unroll
  for (int ct = 0; ct < D / 16; ++ct) {
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int k0 = 0; k0 < D; k0 += 32)
      acc = mma16(lds8(&qr[16 * wave + li][k0 + 8 * lq]), lds8(&sT[16 * ct + li][k0 + 8 * lq]), acc);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const long n = n0 + 16 * wave + 4 * lq + e;
      num[(((long)b * p.N + n) * p.H + h) * D + 16 * ct + li] = (bf16)acc[e];
    }
  }
  if (tid < 64) static_cast<bf16*>(p.den)[(long)bh * p.N + n0 + tid] = (bf16)den_part[tid][0];
}

}  // namespace

hipError_t launch_prep(const PrepParams& p, hipStream_t stream) {
  hipLaunchKernelGGL(rms_prep_kernel, dim3(p.B * p.N), dim3(kPrepThreads), 0, stream, p);
  return hipGetLastError();
}

hipError_t launch_bigdn(const BigdnParams& p, hipStream_t stream) {
  PrepParams pp{};
  pp.qkv = p.qkv;
  pp.q_norm_w = p.q_norm_w;
  pp.k_norm_w = p.k_norm_w;
  pp.rope_cos = p.rope_cos;
  pp.rope_sin = p.rope_sin;
  pp.k_scale = p.k_scale;
  pp.eps = p.eps;
  pp.q_inv_rms = p.q_inv_rms;
  pp.k_inv_rms = p.k_inv_rms;
  pp.B = p.B;
  pp.N = p.N;
  pp.H = p.H;
  pp.D = p.D;
  hipError_t e = launch_prep(pp, stream);
  if (e != hipSuccess) return e;
  const int nbhf = p.B * p.H * p.F;
  if (p.D == 128) {
    hipLaunchKernelGGL(frame_stats_kernel<128>, dim3(nbhf, 3), dim3(kStatThreads), 0, stream, p);
    hipLaunchKernelGGL(scan_kernel<128>, dim3(p.B * p.H * (128 / 16 + 1)), dim3(256), 0, stream, p);
    hipLaunchKernelGGL(out_kernel<128>, dim3(p.B * p.H * (p.N / 64)), dim3(256), 0, stream, p);
  } else {
    hipLaunchKernelGGL(frame_stats_kernel<64>, dim3(nbhf, 3), dim3(kStatThreads), 0, stream, p);
    hipLaunchKernelGGL(scan_kernel<64>, dim3(p.B * p.H * (64 / 16 + 1)), dim3(256), 0, stream, p);
    hipLaunchKernelGGL(out_kernel<64>, dim3(p.B * p.H * (p.N / 64)), dim3(256), 0, stream, p);
  }
  return hipGetLastError();
}

}  // namespace gdn

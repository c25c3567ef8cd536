// gdn_cam.hip -- camera branch of the SANA video block for gfx950: the camera prep and the
// numerator-only frame scan (SANA fused_cam_gdn.py page: _cam_prep_kernel, cam_prep_func,
// _cam_scan_kernel, cam_scan_func).
//
// Prep, per token n and head h (inverse RMS over all H*D channels of the token):
//   q_n = relu(q inv_q w_q),  k_n = relu(k inv_k w_k) k_scale,  v_n = v
//   channels [0, D/2): groups of four mixed by the token's 4x4 camera matrix,
//       y[4g + i] = sum_j P[i][j] x[4g + j]   (P = proj_q for q, proj_kv for k and v)
//   channels [D/2, D): interleaved-pair RoPE, y[D/2 + r] = x[D/2 + r] cos[n, r]
//       + x[D/2 + (r ^ 1)] sin[n, r]
//   inflation = max(|k_out|^2, 1e-12) / max(|k_n|^2, 1e-12)
// Outputs are channel-major, [B, H, D, N].
//
// Scan.  All tokens of frame f predict from the same decayed state, so absorbing frame f is
//   S <- d_f (S - G_f S) + U_f,   G_f = K_f diag(beta) K_f^T,  U_f = K_f diag(beta) V_f^T
// (K_f, V_f the frame's [D, S] channel-major slabs).  The forward output of frame f is
// S_f^T Q_f (after the frame's update); the reverse output reads the state built from the
// frames after f (flip-and-shift).  Kernels: stats (G_f, U_f per (b, h, f) with matrix cores:
// the channel-major slabs are already in operand order, 8 consecutive tokens of one channel
// per lane), the frame scan of gdn_bigdn.hip (one direction, no z; state in / out), out
// (S_f^T Q_f per 64-token block; Q is transposed through LDS).  Products use fp16 operands
// with fp32 accumulation (the page's scan uses TF32 dots: the same 10-bit mantissa); the
// scanned state is fp32.
#include "gdn_device.h"
#include "gdn_frame.h"
#include "gdn_internal.h"

namespace gdn {

namespace {

// ---- inverse RMS ------------------------------------------------------------------------
// One workgroup per token: 1 / sqrt(mean of x^2 over the H*D channels + eps), q and k.
__global__ __launch_bounds__(256) void cam_rms_kernel(const CamPrepParams p) {
  __shared__ float red[8];
  const long bn = blockIdx.x;
  const int C = p.H * p.D;
  const float* qr = p.q + bn * C;
  const float* kr = p.k + bn * C;
  float sq = 0.f, sk = 0.f;
  for (int i = threadIdx.x; i < C / 4; i += 256) {
    const f32x4 a = reinterpret_cast<const f32x4*>(qr)[i];
    const f32x4 b = reinterpret_cast<const f32x4*>(kr)[i];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      sq += a[j] * a[j];
      sk += b[j] * b[j];
    }
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) {
    sq += __shfl_xor(sq, off, 64);
    sk += __shfl_xor(sk, off, 64);
  }
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  if (lane == 0) {
    red[wave] = sq;
    red[4 + wave] = sk;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    p.q_inv_rms[bn] = rsqrtf((red[0] + red[1] + red[2] + red[3]) / (float)C + p.eps);
    p.k_inv_rms[bn] = rsqrtf((red[4] + red[5] + red[6] + red[7]) / (float)C + p.eps);
  }
}

// ---- prep -------------------------------------------------------------------------------
// One workgroup per (b, h, 64-token tile).  A thread takes (4-token quad, 4-channel group)
// items with a fixed group g (so its norm weights and table half are fixed); a wave's loads
// are whole 512-byte head rows of a token.  Each tensor in turn is transformed, written to an
// LDS tile [D][64] (row stride 68 floats) and stored as 256-byte runs of its [B, H, D, N] rows.
template <int D>
__global__ __launch_bounds__(256) void cam_prep_kernel(const CamPrepParams p) {
  constexpr int G = D / 4, kItems = 16 * G / 256, kRow = 68;
  __shared__ __attribute__((aligned(16))) float tile[D * kRow];
  const int nt = (p.N + 63) / 64;
  int x = blockIdx.x;
  const int tb = x % nt;
  x /= nt;
  const int h = x % p.H, b = x / p.H;
  const int n0 = tb * 64;
  const int tid = threadIdx.x, g = tid % G;
  const bool ucpe = g < G / 2;
  const long C = (long)p.H * D;
  const long out_bh = ((long)b * p.H + h) * D * p.N;
  const f32x4 wq = *reinterpret_cast<const f32x4*>(p.q_norm_w + h * D + 4 * g);
  const f32x4 wk = *reinterpret_cast<const f32x4*>(p.k_norm_w + h * D + 4 * g);
  for (int which = 0; which < 3; ++which) {
    const float* src = which == 0 ? p.q : which == 1 ? p.k : p.v;
    const float* proj = which == 0 ? p.proj_q : p.proj_kv;
    const f32x4 w = which == 0 ? wq : wk;
    const float* invp = which == 0 ? p.q_inv_rms : p.k_inv_rms;
#pragma unroll
    for (int i = 0; i < kItems; ++i) {
      const int qd = tid / G + (256 / G) * i;
      const int n = n0 + 4 * qd;  // first token of the quad (N is a multiple of 4)
      const bool live = n < p.N;
      f32x4 y[4];
      float pre[4], post[4];
      f32x4 inv = f32x4{0.f, 0.f, 0.f, 0.f};
      if (live && which < 2) inv = *reinterpret_cast<const f32x4*>(invp + (long)b * p.N + n);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        f32x4 xn = f32x4{0.f, 0.f, 0.f, 0.f};
        if (live) xn = *reinterpret_cast<const f32x4*>(src + ((long)b * p.N + n + j) * C + h * D + 4 * g);
        if (which < 2) {
#pragma unroll
          for (int c = 0; c < 4; ++c) {
            const float t = xn[c] * inv[j] * w[c];
            xn[c] = t > 0.f ? t : 0.f;
            if (which == 1) xn[c] *= p.k_scale;
          }
        }
        f32x4 o;
        if (ucpe) {
          const f32x4* pm = reinterpret_cast<const f32x4*>(proj + ((long)b * p.N + n + j) * 16);
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const f32x4 row = live ? pm[r] : f32x4{0.f, 0.f, 0.f, 0.f};
            o[r] = row[0] * xn[0] + row[1] * xn[1] + row[2] * xn[2] + row[3] * xn[3];
          }
        } else {
          f32x4 cs = f32x4{1.f, 1.f, 1.f, 1.f}, sn = f32x4{0.f, 0.f, 0.f, 0.f};
          if (live) {
            const long tr = (long)(n + j) * (D / 2) + 4 * g - D / 2;
            cs = *reinterpret_cast<const f32x4*>(p.rope_cos + tr);
            sn = *reinterpret_cast<const f32x4*>(p.rope_sin + tr);
          }
          o[0] = xn[0] * cs[0] + xn[1] * sn[0];
          o[1] = xn[1] * cs[1] + xn[0] * sn[1];
          o[2] = xn[2] * cs[2] + xn[3] * sn[2];
          o[3] = xn[3] * cs[3] + xn[2] * sn[3];
        }
        y[j] = o;
        pre[j] = xn[0] * xn[0] + xn[1] * xn[1] + xn[2] * xn[2] + xn[3] * xn[3];
        post[j] = o[0] * o[0] + o[1] * o[1] + o[2] * o[2] + o[3] * o[3];
      }
      // channel-major tile: row 4g + c holds the quad's four tokens
#pragma unroll
      for (int c = 0; c < 4; ++c)
        *reinterpret_cast<f32x4*>(&tile[(4 * g + c) * kRow + 4 * qd]) = f32x4{y[0][c], y[1][c], y[2][c], y[3][c]};
      if (which == 1) {
        // sums over the G consecutive threads of the quad
#pragma unroll
        for (int off = 1; off < G; off <<= 1)
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            pre[j] += __shfl_xor(pre[j], off, 64);
            post[j] += __shfl_xor(post[j], off, 64);
          }
        if (g == 0 && live) {
          f32x4 r;
#pragma unroll
          for (int j = 0; j < 4; ++j) r[j] = fmaxf(post[j], 1e-12f) / fmaxf(pre[j], 1e-12f);
          *reinterpret_cast<f32x4*>(p.inflation + ((long)b * p.H + h) * p.N + n) = r;
        }
      }
    }
    __syncthreads();
    float* dst = which == 0 ? p.q_out : which == 1 ? p.k_out : p.v_out;
#pragma unroll
    for (int r = 0; r < D * 16 / 256; ++r) {
      const int c = tid + 256 * r, d = c / 16, m = c % 16;
      if (n0 + 4 * m < p.N)
        *reinterpret_cast<f32x4*>(dst + out_bh + (long)d * p.N + n0 + 4 * m) =
            *reinterpret_cast<const f32x4*>(&tile[d * kRow + 4 * m]);
    }
    __syncthreads();
  }
}

// ---- frame statistics -------------------------------------------------------------------
// One workgroup of eight waves per (b, h, frame): waves 0-3 accumulate the four D/2 x D/2
// quadrants of G = K diag(beta) K^T, waves 4-7 those of U = K diag(beta) V^T, over the
// frame's tokens 64 at a time.  beta >= 0 splits as sqrt(beta) on both operands, so the LDS
// tiles hold sqrt(beta) K and sqrt(beta) V as fp16 [D][64] (row stride 72 halves: the 16
// rows of an operand read fall in distinct banks).  The tiles are double-buffered and an
// item's slab rows and betas are loaded a block ahead into registers.
template <int D>
__global__ __launch_bounds__(512) void cam_stats_kernel(const CamScanParams p) {
  constexpr int kT = 64, kRow = kT + 8, kQ = D / 2, kA = kQ / 16;
  constexpr int kItems = 2 * D * (kT / 8) / 512;  // (tensor, channel, 8-token octet) items
  __shared__ __attribute__((aligned(16))) f16 tl[2][2][D * kRow];
  const int F = p.F, S = p.S;
  const long N = (long)F * S;
  const int f = blockIdx.x % F, bh = blockIdx.x / F;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int li = lane & 15, lq = lane >> 4;
  const int m = wave >> 2, qi = (wave >> 1) & 1, qj = wave & 1;
  const int oct = tid % 8;  // fixed: 512 is a multiple of 8
  const float* kb = p.k + (long)bh * D * N + (long)f * S;
  const float* vb = p.v + (long)bh * D * N + (long)f * S;
  const float* bt = p.beta + ((long)bh * F + f) * S;
  f32x4 acc[kA][kA];
#pragma unroll
  for (int a = 0; a < kA; ++a)
#pragma unroll
    for (int c = 0; c < kA; ++c) acc[a][c] = f32x4{0.f, 0.f, 0.f, 0.f};
  f32x4 xs[kItems][2], bs[2];
  auto load_items = [&](int t0) {
#pragma unroll
    for (int i = 0; i < kItems; ++i) {
      const int it = tid + 512 * i, ten = it / (D * 8), d = (it % (D * 8)) / 8;
      const float* row = (ten ? vb : kb) + (long)d * N + t0 + 8 * oct;
      xs[i][0] = reinterpret_cast<const f32x4*>(row)[0];
      xs[i][1] = reinterpret_cast<const f32x4*>(row)[1];
    }
    bs[0] = reinterpret_cast<const f32x4*>(bt + t0 + 8 * oct)[0];
    bs[1] = reinterpret_cast<const f32x4*>(bt + t0 + 8 * oct)[1];
  };
  auto prep = [&](int buf) {
    float sb[8];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      sb[j] = sqrtf(bs[0][j]);
      sb[4 + j] = sqrtf(bs[1][j]);
    }
#pragma unroll
    for (int i = 0; i < kItems; ++i) {
      const int it = tid + 512 * i, ten = it / (D * 8), d = (it % (D * 8)) / 8;
      f16x8 r;
#pragma unroll
      for (int j = 0; j < 8; ++j) r[j] = (f16)(xs[i][j >> 2][j & 3] * sb[j]);
      *reinterpret_cast<f16x8*>(&tl[buf][ten][d * kRow + 8 * oct]) = r;
    }
  };
  auto mma_block = [&](int buf) {
    const f16* pa = tl[buf][0];
    const f16* pb = tl[buf][m];
#pragma unroll
    for (int P = 0; P < kT / 32; ++P) {
      f16x8 af[kA], bf[kA];
#pragma unroll
      for (int a = 0; a < kA; ++a) {
        af[a] = lds8(&pa[(qi * kQ + 16 * a + li) * kRow + 32 * P + 8 * lq]);
        bf[a] = lds8(&pb[(qj * kQ + 16 * a + li) * kRow + 32 * P + 8 * lq]);
      }
#pragma unroll
      for (int a = 0; a < kA; ++a)
#pragma unroll
        for (int c = 0; c < kA; ++c) acc[a][c] = mma16(af[a], bf[c], acc[a][c]);
    }
  };
  const int nb = S / kT;
  load_items(0);
  prep(0);
  if (nb > 1) load_items(kT);
  __syncthreads();
  for (int n = 0; n < nb; ++n) {
    if (n + 1 < nb) {
      prep((n + 1) & 1);
      if (n + 2 < nb) load_items((n + 2) * kT);
    }
    mma_block(n & 1);
    __syncthreads();
  }
  // lane (li, lq) of tile (a, c): row qi kQ + 16a + 4lq + e, column qj kQ + 16c + li.
  // U goes out in accumulator order (four rows e, 16 bytes); G, symmetric, transposed (its
  // four e become consecutive columns of one row, 8 bytes) -- the scan's operand layouts.
  const long mat = ((long)bh * F + f) * (long)D * D;
#pragma unroll
  for (int a = 0; a < kA; ++a)
#pragma unroll
    for (int c = 0; c < kA; ++c) {
      const int r0 = qi * kQ + 16 * a + 4 * lq, col = qj * kQ + 16 * c + li;
      if (m == 1) {
        *reinterpret_cast<f32x4*>(p.U + mat + u_lane_index<D>(r0, col)) = acc[a][c];
      } else {
        f16x4 v;
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = (f16)acc[a][c][e];
        *reinterpret_cast<f16x4*>(p.G + mat + g_lane_index<D>(col, r0)) = v;
      }
    }
}

// ---- output -----------------------------------------------------------------------------
// One workgroup per (b, h, frame f, group of grp consecutive 64-token blocks of f):
// out[:, n] = S^T q_n with S the state the scan stored for f (fp16, transposed).  Wave w
// forms value columns (D/4)w .. (D/4)w + D/4 - 1: its slice of S^T is the B operand, held in
// registers for the whole group; the A operand (tokens x keys) comes from the block's Q slab,
// converted to fp16 into LDS [D][64] and read transposed.  The accumulator of lane (li, lq)
// holds four consecutive tokens of value column li (16-byte stores).
template <int D>
__global__ __launch_bounds__(256) void cam_out_kernel(const CamScanParams p, int grp) {
  constexpr int kRow = 72, kCT = D / 64;
  __shared__ __attribute__((aligned(16))) f16 qt[D * kRow];
  const int F = p.F, S = p.S;
  const long N = (long)F * S;
  const int ngrp = (S / 64) / grp;
  int x = blockIdx.x;
  const int gi = x % ngrp;
  x /= ngrp;
  const int f = x % F, bh = x / F;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int li = lane & 15, lq = lane >> 4;
  const long bhf = (long)bh * F + f;
  f16x8 sa[kCT][D / 32];
#pragma unroll
  for (int ct = 0; ct < kCT; ++ct)
#pragma unroll
    for (int k = 0; k < D / 32; ++k)
      sa[ct][k] = *reinterpret_cast<const f16x8*>(
          p.SdT + bhf * D * D + (long)((D / 4) * wave + 16 * ct + li) * D + 32 * k + 8 * lq);
  const float* qb = p.q + (long)bh * D * N;
  float* ob = p.out + (long)bh * D * N;
  const int trj = li >> 2, trm = li & 3;  // transpose-read piece: key row offset, token quad
  for (int blk = gi * grp; blk < (gi + 1) * grp; ++blk) {
    const long n0 = (long)f * S + blk * 64;
    __syncthreads();  // the previous block's reads of qt are done
    f32x4 xq[D * 16 / 256];
#pragma unroll
    for (int r = 0; r < D * 16 / 256; ++r) {
      const int c = tid + 256 * r, d = c / 16, m4 = c % 16;
      xq[r] = *reinterpret_cast<const f32x4*>(qb + (long)d * N + n0 + 4 * m4);
    }
#pragma unroll
    for (int r = 0; r < D * 16 / 256; ++r) {
      const int c = tid + 256 * r, d = c / 16, m4 = c % 16;
      f16x4 h;
#pragma unroll
      for (int e = 0; e < 4; ++e) h[e] = (f16)xq[r][e];
      *reinterpret_cast<f16x4*>(&qt[d * kRow + 4 * m4]) = h;
    }
    __syncthreads();
#pragma unroll
    for (int tt = 0; tt < 4; ++tt) {
      f32x4 acc[kCT];
#pragma unroll
      for (int ct = 0; ct < kCT; ++ct) acc[ct] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int k = 0; k < D / 32; ++k) {
        const f16x8 aq = tr_pair(&qt[(32 * k + 8 * lq + trj) * kRow + 16 * tt + 4 * trm],
                                 &qt[(32 * k + 8 * lq + 4 + trj) * kRow + 16 * tt + 4 * trm]);
#pragma unroll
        for (int ct = 0; ct < kCT; ++ct) acc[ct] = mma16(aq, sa[ct][k], acc[ct]);
      }
#pragma unroll
      for (int ct = 0; ct < kCT; ++ct)
        *reinterpret_cast<f32x4*>(ob + (long)((D / 4) * wave + 16 * ct + li) * N + n0 + 16 * tt + 4 * lq) = acc[ct];
    }
  }
}

}  // namespace

hipError_t launch_cam_prep(const CamPrepParams& p, hipStream_t stream) {
  hipLaunchKernelGGL(cam_rms_kernel, dim3(p.B * p.N), dim3(256), 0, stream, p);
  const dim3 grid(p.B * p.H * ((p.N + 63) / 64));
  if (p.D == 128)
    hipLaunchKernelGGL(cam_prep_kernel<128>, grid, dim3(256), 0, stream, p);
  else
    hipLaunchKernelGGL(cam_prep_kernel<64>, grid, dim3(256), 0, stream, p);
  return hipGetLastError();
}

hipError_t launch_cam_scan(const CamScanParams& p, hipStream_t stream) {
  BigdnParams sp{};
  sp.decay = p.decay;
  sp.decay_bwd = p.decay;
  sp.B = p.B;
  sp.H = p.H;
  sp.F = p.F;
  sp.S = p.S;
  sp.D = p.D;
  sp.N = p.F * p.S;
  sp.G = sp.G_b = p.G;
  sp.U = sp.U_b = p.U;
  sp.SdT = p.SdT;
  sp.scan_dirs = p.reverse ? 2 : 1;
  sp.scan_z = 0;
  sp.dir_slots = 1;
  sp.s_init = p.init_state;
  sp.s_final = p.final_state;
  // 64-token blocks per output workgroup: the largest divisor of a frame's blocks up to 4
  const int nblk = p.S / 64;
  int grp = 4;
  while (nblk % grp) grp >>= 1;
  const dim3 og(p.B * p.H * p.F * (nblk / grp));
  if (p.D == 128)
    hipLaunchKernelGGL(cam_stats_kernel<128>, dim3(p.B * p.H * p.F), dim3(512), 0, stream, p);
  else
    hipLaunchKernelGGL(cam_stats_kernel<64>, dim3(p.B * p.H * p.F), dim3(512), 0, stream, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  e = launch_frame_scan(sp, stream);
  if (e != hipSuccess) return e;
  if (p.D == 128)
    hipLaunchKernelGGL(cam_out_kernel<128>, og, dim3(256), 0, stream, p, grp);
  else
    hipLaunchKernelGGL(cam_out_kernel<64>, og, dim3(256), 0, stream, p, grp);
  return hipGetLastError();
}

}  // namespace gdn

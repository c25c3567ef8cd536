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
// (S_f^T Q_f per 64-token block; Q is transposed through LDS).  The bidirectional form
// computes the statistics once, scans both directions concurrently and forms both outputs
// from one read of Q.  Products use fp16 operands
// with fp32 accumulation (the page's scan uses TF32 dots: the same 10-bit mantissa); the
// scanned state is fp32.
#include "gdn_device.h"
#include "gdn_frame.h"
#include "gdn_internal.h"

namespace gdn {

namespace {

// Workgroup ids are dealt to the eight XCDs round-robin.  When the grid is a multiple of eight,
// XCD x takes the contiguous range [x n/8, (x+1) n/8) of logical indices in order, so logical
// neighbours (which share table or state reads) run close in time on one XCD's L2.
__device__ __forceinline__ int xcd_logical(int bid, int n) {
  return n % 8 ? bid : (bid % 8) * (n / 8) + bid / 8;
}

// ---- inverse RMS ------------------------------------------------------------------------
// One wave per token (eight tokens per workgroup): 1 / sqrt(mean of x^2 over the H*D channels
// + eps) of q and k; a lane reads 16-byte pieces, so a wave's load covers 1 KB of the row.
constexpr int kRmsTokens = 8;
__global__ __launch_bounds__(256) void cam_rms_kernel(const CamPrepParams p) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int C4 = p.H * p.D / 4;
  const long total = (long)p.B * p.N;
#pragma unroll
  for (int r = 0; r < kRmsTokens / 4; ++r) {
    const long bn = (long)blockIdx.x * kRmsTokens + 4 * r + wave;
    if (bn >= total) break;
    const f32x4* qr = reinterpret_cast<const f32x4*>(p.q + bn * 4 * C4);
    const f32x4* kr = reinterpret_cast<const f32x4*>(p.k + bn * 4 * C4);
    float sq = 0.f, sk = 0.f;
#pragma unroll 8
    for (int i = lane; i < C4; i += 64) {
      const f32x4 a = qr[i], b = kr[i];
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
    if (lane == 0) {
      p.q_inv_rms[bn] = rsqrtf(sq / (float)(4 * C4) + p.eps);
      p.k_inv_rms[bn] = rsqrtf(sk / (float)(4 * C4) + p.eps);
    }
  }
}

// ---- prep -------------------------------------------------------------------------------
// One workgroup of 4D threads per (b, h, 64-token tile).  The first 2D threads (whole waves)
// take the camera-matrix half of the channels, the others the RoPE half, so neither branch
// diverges inside a wave.  A thread owns one (4-token quad, 4-channel group) item of each of
// q, k, v: all its input loads (12 pieces of 16 bytes, plus its RoPE table pieces) are issued
// at once; the tile's camera matrices and inverse RMS are staged in LDS.  Results go to LDS
// tiles [D][64] (row stride 68 floats), q and k first, then v, and leave as 256-byte runs of
// the [B, H, D, N] rows.  Tokens past N (a ragged last tile) load token N - 1 and are not
// stored.
template <int D>
__global__ __launch_bounds__(4 * D) void cam_prep_kernel(const CamPrepParams p) {
  constexpr int kThreads = 4 * D, G2 = D / 8, kRow = 68;  // G2 groups per half
  __shared__ __attribute__((aligned(16))) float tile[2][D * kRow];
  __shared__ __attribute__((aligned(16))) float pm[2][64 * 16];  // proj_q, proj_kv per token
  __shared__ __attribute__((aligned(16))) float inv[2][64];
  __shared__ float red[2][2][64];  // [half][pre, post][token]
  // logical order: head fastest, so the heads of one token tile (which read the same camera
  // matrices and RoPE rows) follow one another on one XCD
  const int nt = (p.N + 63) / 64;
  int x = xcd_logical(blockIdx.x, gridDim.x);
  const int h = x % p.H;
  x /= p.H;
  const int tb = x % nt, b = x / nt;
  const int n0 = tb * 64;
  const int tid = threadIdx.x;
  const int half = tid / (2 * D);         // 0: camera matrix, 1: RoPE (wave-uniform)
  const int gl = tid % G2, qd = (tid % (2 * D)) / G2;
  const int g = half * G2 + gl;           // channel group: channels 4g .. 4g + 3
  const long C = (long)p.H * D;
  auto tok = [&](int t) { return n0 + t < p.N ? n0 + t : p.N - 1; };
  // stage the tile's camera matrices (16-byte pieces) and inverse RMS
  for (int i = tid; i < 2 * 64 * 4; i += kThreads) {
    const int which = i / 256, t = (i % 256) / 4, r = i % 4;
    const float* src = (which ? p.proj_kv : p.proj_q) + ((long)b * p.N + tok(t)) * 16 + 4 * r;
    *reinterpret_cast<f32x4*>(&pm[which][t * 16 + 4 * r]) = *reinterpret_cast<const f32x4*>(src);
  }
  if (tid < 128) inv[tid / 64][tid % 64] = (tid < 64 ? p.q_inv_rms : p.k_inv_rms)[(long)b * p.N + tok(tid % 64)];
  // this thread's raw inputs and RoPE table pieces
  f32x4 xr[3][4], cs[4], sn[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const long row = ((long)b * p.N + tok(4 * qd + j)) * C + h * D + 4 * g;
    xr[0][j] = *reinterpret_cast<const f32x4*>(p.q + row);
    xr[1][j] = *reinterpret_cast<const f32x4*>(p.k + row);
    xr[2][j] = *reinterpret_cast<const f32x4*>(p.v + row);
    if (half) {
      const long tr = (long)tok(4 * qd + j) * (D / 2) + 4 * gl;
      cs[j] = *reinterpret_cast<const f32x4*>(p.rope_cos + tr);
      sn[j] = *reinterpret_cast<const f32x4*>(p.rope_sin + tr);
    }
  }
  const f32x4 wq = *reinterpret_cast<const f32x4*>(p.q_norm_w + h * D + 4 * g);
  const f32x4 wk = *reinterpret_cast<const f32x4*>(p.k_norm_w + h * D + 4 * g);
  __syncthreads();
  const long out_bh = ((long)b * p.H + h) * D * p.N;
  auto transform = [&](int which, int slot) {
    float pre[4], post[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int t = 4 * qd + j;
      f32x4 xn = xr[which][j];
      if (which < 2) {
        const f32x4 w = which ? wk : wq;
        const float iv = inv[which][t];
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          const float u = xn[c] * iv * w[c];
          xn[c] = (u > 0.f ? u : 0.f) * (which ? p.k_scale : 1.f);
        }
      }
      f32x4 o;
      if (half == 0) {
        const float* P = &pm[which ? 1 : 0][t * 16];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const f32x4 row = *reinterpret_cast<const f32x4*>(P + 4 * r);
          o[r] = row[0] * xn[0] + row[1] * xn[1] + row[2] * xn[2] + row[3] * xn[3];
        }
      } else {
        o[0] = xn[0] * cs[j][0] + xn[1] * sn[j][0];
        o[1] = xn[1] * cs[j][1] + xn[0] * sn[j][1];
        o[2] = xn[2] * cs[j][2] + xn[3] * sn[j][2];
        o[3] = xn[3] * cs[j][3] + xn[2] * sn[j][3];
      }
      pre[j] = xn[0] * xn[0] + xn[1] * xn[1] + xn[2] * xn[2] + xn[3] * xn[3];
      post[j] = o[0] * o[0] + o[1] * o[1] + o[2] * o[2] + o[3] * o[3];
      xr[which][j] = o;
    }
#pragma unroll
    for (int c = 0; c < 4; ++c)
      *reinterpret_cast<f32x4*>(&tile[slot][(4 * g + c) * kRow + 4 * qd]) =
          f32x4{xr[which][0][c], xr[which][1][c], xr[which][2][c], xr[which][3][c]};
    if (which == 1) {  // |k|^2 before and after, summed over the G2 threads of the half-quad
#pragma unroll
      for (int off = 1; off < G2; off <<= 1)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          pre[j] += __shfl_xor(pre[j], off, 64);
          post[j] += __shfl_xor(post[j], off, 64);
        }
      if (gl == 0)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          red[half][0][4 * qd + j] = pre[j];
          red[half][1][4 * qd + j] = post[j];
        }
    }
  };
  auto store = [&](int slot, float* dst) {
#pragma unroll
    for (int r = 0; r < D * 16 / kThreads; ++r) {
      const int c = tid + kThreads * r, d = c / 16, m = c % 16;
      if (n0 + 4 * m < p.N)
        *reinterpret_cast<f32x4*>(dst + out_bh + (long)d * p.N + n0 + 4 * m) =
            *reinterpret_cast<const f32x4*>(&tile[slot][d * kRow + 4 * m]);
    }
  };
  transform(0, 0);
  transform(1, 1);
  __syncthreads();
  store(0, p.q_out);
  store(1, p.k_out);
  if (tid < 16 && n0 + 4 * tid < p.N) {
    f32x4 r;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int t = 4 * tid + j;
      r[j] = fmaxf(red[0][1][t] + red[1][1][t], 1e-12f) / fmaxf(red[0][0][t] + red[1][0][t], 1e-12f);
    }
    *reinterpret_cast<f32x4*>(p.inflation + ((long)b * p.H + h) * p.N + n0 + 4 * tid) = r;
  }
  __syncthreads();
  transform(2, 0);
  __syncthreads();
  store(0, p.v_out);
}

// ---- frame statistics -------------------------------------------------------------------
// One workgroup of eight waves per (b, h, frame): waves 0-3 accumulate the four D/2 x D/2
// quadrants of G = K diag(beta) K^T, waves 4-7 those of U = K diag(beta) V^T, over the
// frame's tokens kT at a time (128 when S allows, so that a CU has 160 KB of loads in
// flight).  beta >= 0 splits as sqrt(beta) on both operands, so the LDS tiles hold
// sqrt(beta) K and sqrt(beta) V as fp16 [D][kT] (row stride kT + 8 halves: the 16 rows of an
// operand read fall in distinct banks).  The tiles are double-buffered and an item's slab
// rows and betas are loaded a block ahead into registers.
template <int D, int kT>
__global__ __launch_bounds__(512) void cam_stats_kernel(const CamScanParams p) {
  constexpr int kRow = kT + 8, kQ = D / 2, kA = kQ / 16;
  constexpr int kO = kT / 8;                      // 8-token octets per slab row
  constexpr int kItems = 2 * D * kO / 512;        // (tensor, channel, octet) items
  __shared__ __attribute__((aligned(16))) f16 tl[2][2][D * kRow];
  const int F = p.F, S = p.S;
  const long N = (long)F * S;
  const int f = blockIdx.x % F, bh = blockIdx.x / F;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int li = lane & 15, lq = lane >> 4;
  const int m = wave >> 2, qi = (wave >> 1) & 1, qj = wave & 1;
  const int oct = tid % kO;  // fixed: 512 is a multiple of kO
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
      const int it = tid + 512 * i, ten = it / (D * kO), d = (it % (D * kO)) / kO;
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
      const int it = tid + 512 * i, ten = it / (D * kO), d = (it % (D * kO)) / kO;
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
//
// kDirs = 2 (both directions): the two directions' states are both held as B operands and
// one Q tile serves both outputs.
template <int D, int kDirs>
__global__ __launch_bounds__(256) void cam_out_kernel(const CamScanParams p, int grp) {
  constexpr int kRow = 72, kCT = D / 64;
  __shared__ __attribute__((aligned(16))) f16 qt[D * kRow];
  const int F = p.F, S = p.S;
  const long N = (long)F * S;
  const int ngrp = (S / 64) / grp;
  // the token groups of one (b, h, frame), which read the same states, on one XCD in turn
  int x = xcd_logical(blockIdx.x, gridDim.x);
  const int gi = x % ngrp;
  x /= ngrp;
  const int f = x % F, bh = x / F;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int li = lane & 15, lq = lane >> 4;
  const long bhf = (long)bh * F + f;
  f16x8 sa[kDirs][kCT][D / 32];
  const long dir_m = (long)p.B * p.H * F * D * D;
#pragma unroll
  for (int r = 0; r < kDirs; ++r)
#pragma unroll
    for (int ct = 0; ct < kCT; ++ct)
#pragma unroll
      for (int k = 0; k < D / 32; ++k)
        sa[r][ct][k] = *reinterpret_cast<const f16x8*>(
            p.SdT + r * dir_m + bhf * D * D + (long)((D / 4) * wave + 16 * ct + li) * D + 32 * k + 8 * lq);
  const float* qb = p.q + (long)bh * D * N;
  float* ob[2] = {p.out + (long)bh * D * N, (kDirs == 2 ? p.out_rev : p.out) + (long)bh * D * N};
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
      f32x4 acc[kDirs][kCT];
#pragma unroll
      for (int r = 0; r < kDirs; ++r)
#pragma unroll
        for (int ct = 0; ct < kCT; ++ct) acc[r][ct] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int k = 0; k < D / 32; ++k) {
        const f16x8 aq = tr_pair(&qt[(32 * k + 8 * lq + trj) * kRow + 16 * tt + 4 * trm],
                                 &qt[(32 * k + 8 * lq + 4 + trj) * kRow + 16 * tt + 4 * trm]);
#pragma unroll
        for (int r = 0; r < kDirs; ++r)
#pragma unroll
          for (int ct = 0; ct < kCT; ++ct) acc[r][ct] = mma16(aq, sa[r][ct][k], acc[r][ct]);
      }
#pragma unroll
      for (int r = 0; r < kDirs; ++r)
#pragma unroll
        for (int ct = 0; ct < kCT; ++ct)
          *reinterpret_cast<f32x4*>(ob[r] + (long)((D / 4) * wave + 16 * ct + li) * N + n0 + 16 * tt + 4 * lq) = acc[r][ct];
    }
  }
}

}  // namespace

hipError_t launch_cam_prep(const CamPrepParams& p, hipStream_t stream) {
  const long ntok = (long)p.B * p.N;
  hipLaunchKernelGGL(cam_rms_kernel, dim3((ntok + kRmsTokens - 1) / kRmsTokens), dim3(256), 0,
                     stream, p);
  const dim3 grid(p.B * p.H * ((p.N + 63) / 64));
  if (p.D == 128)
    hipLaunchKernelGGL(cam_prep_kernel<128>, grid, dim3(512), 0, stream, p);
  else
    hipLaunchKernelGGL(cam_prep_kernel<64>, grid, dim3(256), 0, stream, p);
  return hipGetLastError();
}

hipError_t launch_cam_scan(const CamScanParams& p, hipStream_t stream) {
  const bool both = p.reverse == 2;
  BigdnParams sp{};
  sp.decay = p.decay;
  sp.decay_bwd = both && p.decay_bwd ? p.decay_bwd : p.decay;
  sp.B = p.B;
  sp.H = p.H;
  sp.F = p.F;
  sp.S = p.S;
  sp.D = p.D;
  sp.N = p.F * p.S;
  sp.G = sp.G_b = p.G;
  sp.U = sp.U_b = p.U;
  sp.SdT = p.SdT;
  sp.scan_dirs = both ? 3 : p.reverse ? 2 : 1;
  sp.scan_z = 0;
  sp.dir_slots = both ? 2 : 1;
  sp.s_init = p.init_state;
  sp.s_final = p.final_state;
  // 64-token blocks per output workgroup: the largest divisor of a frame's blocks up to 4
  const int nblk = p.S / 64;
  int grp = 4;
  while (nblk % grp) grp >>= 1;
  const dim3 og(p.B * p.H * p.F * (nblk / grp));
  const dim3 sg(p.B * p.H * p.F);
  const bool t128 = p.S % 128 == 0;
  if (p.D == 128 && t128) hipLaunchKernelGGL((cam_stats_kernel<128, 128>), sg, dim3(512), 0, stream, p);
  else if (p.D == 128) hipLaunchKernelGGL((cam_stats_kernel<128, 64>), sg, dim3(512), 0, stream, p);
  else if (t128) hipLaunchKernelGGL((cam_stats_kernel<64, 128>), sg, dim3(512), 0, stream, p);
  else hipLaunchKernelGGL((cam_stats_kernel<64, 64>), sg, dim3(512), 0, stream, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  e = launch_frame_scan(sp, stream);
  if (e != hipSuccess) return e;
  if (p.D == 128 && both) hipLaunchKernelGGL((cam_out_kernel<128, 2>), og, dim3(256), 0, stream, p, grp);
  else if (p.D == 128) hipLaunchKernelGGL((cam_out_kernel<128, 1>), og, dim3(256), 0, stream, p, grp);
  else if (both) hipLaunchKernelGGL((cam_out_kernel<64, 2>), og, dim3(256), 0, stream, p, grp);
  else hipLaunchKernelGGL((cam_out_kernel<64, 1>), og, dim3(256), 0, stream, p, grp);
  return hipGetLastError();
}

}  // namespace gdn

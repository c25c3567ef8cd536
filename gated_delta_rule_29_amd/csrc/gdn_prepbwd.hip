// gdn_prepbwd.hip -- backward of the BiGDN front end and of the bidirectional merge (gfx950),
// after the SANA fused_gdn.py page, "Backward / autograd Functions": the RoPE inverse, ReLU
// and k-scale backward inside _fused_gdn_bwd_kernel, the full-channel RMSNorm backward and the
// dnum / dden of FusedBiGDNFunction.backward, and the SiLU gate of fused_bidi_merge.
//
// Front end (per token, C = H*D channels, r the inverse RMS over all of them, w the norm
// weight, x_hat = x r w, x_pos = relu(x_hat) (times k_scale for k), x_rot[d] = x_pos[d] cos[d]
// + x_pos[d^1] sin[d]):
//   g_pos[d] = sum over directions of dpos[d] + drot[d] cos[d] + drot[d^1] sin[d^1]
//   g[c]     = g_pos (times k_scale for k) where x_hat > 0, else 0
//   dx[c]    = r w[c] g[c] - r^3 / C x[c] sum_c' w[c'] g[c'] x[c']
//   dw[c]    = sum over tokens of g[c] x[c] r
// The ReLU mask needs only the sign of x w (r > 0), so both sums a token needs (sum x^2 for
// r, sum w g x) come from one workgroup reduction.  A workgroup takes a contiguous group of
// tokens; thread t owns channels 8t .. 8t + 7 of each 2048-channel strip (eight consecutive
// channels lie in one head, and RoPE pairs never straddle them).  The norm weights' gradients
// are summed per workgroup in registers, written as partial sums and added in a fixed order by
// a second kernel, so the result does not depend on scheduling.
//
// Camera-branch prep (SANA fused_cam_gdn.py page: _cam_prep_bwd_kernel and
// _cam_prep_bwd_dispatch).  The forward maps x_n = relu(x r w) (times k_scale for k; v passes
// unnormed) to y = T x_n, T the token's 4x4 camera matrix P on each group of four of channels
// [0, D/2) and interleaved-pair RoPE on [D/2, D), outputs channel-major [B, H, D, N], and
// inflation = max(|y_k|^2, 1e-12) / max(|x_n,k|^2, 1e-12).  Backward:
//   d_post = dinfl [post >= 1e-12] / max(pre, 1e-12)
//   d_pre  = -dinfl max(post, 1e-12) / max(pre, 1e-12)^2 [pre >= 1e-12]
//   dx_n   = T^T (dy + 2 y d_post)  (+ 2 x_n d_pre for k)
//   T^T:  dx_n[4g + j] = sum_i P[i][j] dy[4g + i];  dx_n[D/2 + r] = dy[D/2 + r] cos[r]
//         + dy[D/2 + (r^1)] sin[r^1]
// then k_scale, the ReLU mask and the full-channel RMSNorm backward as above; dv = T^T dy_v.
// cam_prep_bwd_tile_kernel (one workgroup of 4D threads per (b, h, 64 tokens), the forward's
// layout: a thread owns 4 tokens x 4 channels, whole waves per half) reads the channel-major
// gradients as 16-byte runs of 4 tokens, so its registers hold the transposed item directly,
// and writes dv and the pre-mask gradients of q and k token-major into dv, dq, dk.
// cam_norm_bwd_kernel then applies the mask and the RMSNorm backward in place, per token.
// The inflation terms need the k inverse RMS, which cam_kinv_kernel computes first.
//
// Merge (out = num / (den + eps) * silu(gate), silu = 1 without a gate), D / 8 lanes per
// (b, n, h) row:
//   dnum = dout silu / (den + eps),  dden = -sum_d dout silu num / (den + eps)^2,
//   dgate = dout num / (den + eps) * s (1 + x (1 - s)),  s = sigmoid(gate), x = gate.
#include "gdn_bwd_params.h"
#include "gdn_device.h"

namespace gdn {
namespace {

constexpr int kStrip = 2048;  // channels per strip (256 threads x 8)

// 8 consecutive fp32 values
__device__ __forceinline__ void ld8(const float* p, float (&x)[8]) { load8f<float>(p, x); }
__device__ __forceinline__ void st8(float* p, const float (&x)[8]) {
  *reinterpret_cast<f32x4*>(p) = f32x4{x[0], x[1], x[2], x[3]};
  *reinterpret_cast<f32x4*>(p + 4) = f32x4{x[4], x[5], x[6], x[7]};
}

// x * w > 0 decided from the signs alone (the product of two fp32 values can underflow)
__device__ __forceinline__ bool pos_prod(float x, float w) {
  return x != 0.f && w != 0.f && ((x > 0.f) == (w > 0.f));
}

template <int NS>
__global__ __launch_bounds__(256) void prep_bwd_kernel(const PrepBwdParams p) {
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63;
  const int C = p.H * p.D;
  const long BN = (long)p.B * p.N;
  const long per = (BN + p.nwg - 1) / p.nwg;
  const long t0 = (long)blockIdx.x * per, t1 = min(BN, t0 + per);
  const long dir_stride = BN * C;  // elements of one direction's gradient tensor
  __shared__ float red[2][4][4];   // [token parity][wave][sum]

  float wt[2][NS][8], dw[2][NS][8];
#pragma unroll
  for (int s = 0; s < NS; ++s) {
    const int c = kStrip * s + 8 * tid;
#pragma unroll
    for (int j = 0; j < 8; ++j) dw[0][s][j] = dw[1][s][j] = 0.f;
    if (c < C) {
      ld8(p.q_norm_w + c, wt[0][s]);
      ld8(p.k_norm_w + c, wt[1][s]);
    }
  }

  for (long bn = t0; bn < t1; ++bn) {
    const long b = bn / p.N, n = bn % p.N;
    const int par = (int)(bn & 1);
    float x[2][NS][8], g[2][NS][8];
    float sum[4] = {0.f, 0.f, 0.f, 0.f};  // sum x^2 (q), sum w g x (q), the same for k
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      const int c = kStrip * s + 8 * tid;
      if (c >= C) continue;
      const int h = c / p.D, d = c % p.D;
      load8f<bf16>(p.qkv + (bn * 3 + 0) * C + c, x[0][s]);
      load8f<bf16>(p.qkv + (bn * 3 + 1) * C + c, x[1][s]);
      float cs[8], sn[8];
      ld8(p.rope_cos + n * p.D + d, cs);
      ld8(p.rope_sin + n * p.D + d, sn);
      const long o0 = ((b * p.H + h) * p.N + n) * p.D + d;
#pragma unroll
      for (int which = 0; which < 2; ++which) {
        const float* drot = which ? p.dk_rot : p.dq_rot;
        const float* dpos = which ? p.dk_pos : p.dq_pos;
        float gp[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) gp[j] = 0.f;
        for (int dir = 0; dir < p.ndir; ++dir) {
          float r8[8], p8[8];
          ld8(drot + dir * dir_stride + o0, r8);
          ld8(dpos + dir * dir_stride + o0, p8);
#pragma unroll
          for (int j = 0; j < 8; ++j) gp[j] += p8[j] + r8[j] * cs[j] + r8[j ^ 1] * sn[j ^ 1];
        }
        const float scl = which ? p.k_scale : 1.f;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const float xv = x[which][s][j], wv = wt[which][s][j];
          g[which][s][j] = pos_prod(xv, wv) ? gp[j] * scl : 0.f;
          sum[2 * which] += xv * xv;
          sum[2 * which + 1] += wv * g[which][s][j] * xv;
        }
      }
      // v passes through the front end: its gradient is the directions' sum
      float dvs[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) dvs[j] = 0.f;
      for (int dir = 0; dir < p.ndir; ++dir) {
        float v8[8];
        ld8(p.dv + dir * dir_stride + o0, v8);
#pragma unroll
        for (int j = 0; j < 8; ++j) dvs[j] += v8[j];
      }
      st8(p.dqkv + (bn * 3 + 2) * C + c, dvs);
    }
    // the token's four sums over its C channels (red is double-buffered by token parity, so
    // one barrier per token suffices)
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int off = 32; off > 0; off >>= 1) sum[i] += __shfl_xor(sum[i], off, 64);
    if (lane == 0)
#pragma unroll
      for (int i = 0; i < 4; ++i) red[par][w][i] = sum[i];
    __syncthreads();
#pragma unroll
    for (int i = 0; i < 4; ++i) sum[i] = (red[par][0][i] + red[par][1][i]) + (red[par][2][i] + red[par][3][i]);
#pragma unroll
    for (int which = 0; which < 2; ++which) {
      const float r = 1.f / sqrtf(sum[2 * which] / (float)C + p.eps);
      const float corr = r * r * r / (float)C * sum[2 * which + 1];
#pragma unroll
      for (int s = 0; s < NS; ++s) {
        const int c = kStrip * s + 8 * tid;
        if (c >= C) continue;
        float dx[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const float gv = g[which][s][j], xv = x[which][s][j];
          dx[j] = r * wt[which][s][j] * gv - corr * xv;
          dw[which][s][j] += gv * xv * r;
        }
        st8(p.dqkv + (bn * 3 + which) * C + c, dx);
      }
    }
  }
#pragma unroll
  for (int which = 0; which < 2; ++which)
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      const int c = kStrip * s + 8 * tid;
      if (c < C) st8(p.part + ((long)blockIdx.x * 2 + which) * C + c, dw[which][s]);
    }
}

// The norm weights' gradients: the workgroups' partial sums added in a fixed order.  A
// workgroup takes 64 of the 2 C (which, channel) sums; its 16 waves each add every 16th
// partial (in workgroup order), and the 16 slices are then added in order.
__global__ __launch_bounds__(1024) void prep_bwd_wsum_kernel(const float* part, int nwg, int C,
                                                             float* dq_norm_w, float* dk_norm_w) {
  const int cl = threadIdx.x & 63, sl = threadIdx.x >> 6;
  const int i = blockIdx.x * 64 + cl;  // (which, channel)
  __shared__ float red[16][64];
  float acc = 0.f;
  if (i < 2 * C) {
    const int which = i / C, c = i % C;
#pragma unroll 8
    for (int g = sl; g < nwg; g += 16) acc += part[((long)g * 2 + which) * C + c];
  }
  red[sl][cl] = acc;
  __syncthreads();
  if (sl == 0 && i < 2 * C) {
    float t = 0.f;
#pragma unroll
    for (int k = 0; k < 16; ++k) t += red[k][cl];
    (i < C ? dq_norm_w : dk_norm_w)[i % C] = t;
  }
}

// ---- camera-branch prep backward ------------------------------------------------------------

// k inverse RMS, one wave per token (four per workgroup)
__global__ __launch_bounds__(256) void cam_kinv_kernel(const CamPrepBwdParams p) {
  const int lane = threadIdx.x & 63;
  const long bn = (long)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int C4 = p.H * p.D / 4;
  if (bn >= (long)p.B * p.N) return;
  const f32x4* kr = reinterpret_cast<const f32x4*>(p.k + bn * 4 * C4);
  float s = 0.f;
#pragma unroll 8
  for (int i = lane; i < C4; i += 64) {
    const f32x4 a = kr[i];
    s += a[0] * a[0] + a[1] * a[1] + a[2] * a[2] + a[3] * a[3];
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) s += __shfl_xor(s, off, 64);
  if (lane == 0) p.k_inv_rms[bn] = 1.f / sqrtf(s / (float)(4 * C4) + p.eps);
}

template <int D>
__global__ __launch_bounds__(4 * D) void cam_prep_bwd_tile_kernel(const CamPrepBwdParams p) {
  constexpr int kThreads = 4 * D, G2 = D / 8;  // G2 groups of four channels per half
  __shared__ __attribute__((aligned(16))) float pm[2][64 * 16];  // proj_q, proj_kv per token
  __shared__ float kinv[64];
  __shared__ float red[2][2][64];  // [half][pre, post][token]
  const int nt = (p.N + 63) / 64;
  int x = xcd_logical(blockIdx.x, gridDim.x);
  const int h = x % p.H;
  x /= p.H;
  const int tb = x % nt, b = x / nt;
  const int n0 = tb * 64, tid = threadIdx.x;
  const int half = tid / (2 * D);  // 0: camera matrix, 1: RoPE (wave-uniform)
  const int gl = tid % G2, qd = (tid % (2 * D)) / G2;
  const int g = half * G2 + gl;    // channels 4g .. 4g + 3
  const long C = (long)p.H * D;
  const bool infl = p.dinfl != nullptr;
  // N is a multiple of 4, so a 4-token quad is wholly inside or wholly past the sequence; a
  // quad past it reads the last quad and stores nothing
  const bool live = n0 + 4 * qd < p.N;
  const int nq = live ? n0 + 4 * qd : p.N - 4;
  auto tok = [&](int t) { return n0 + t < p.N ? n0 + t : p.N - 1; };
  for (int i = tid; i < 2 * 64 * 4; i += kThreads) {
    const int which = i / 256, t = (i % 256) / 4, r = i % 4;
    const float* src = (which ? p.proj_kv : p.proj_q) + ((long)b * p.N + tok(t)) * 16 + 4 * r;
    *reinterpret_cast<f32x4*>(&pm[which][t * 16 + 4 * r]) = *reinterpret_cast<const f32x4*>(src);
  }
  if (infl && tid < 64) kinv[tid] = p.k_inv_rms[(long)b * p.N + tok(tid)];
  // upstream gradients: dy[which][c] holds channel 4g + c of the quad's four tokens
  const long dstride = (long)p.B * p.H * D * p.N;
  const long gbase = (((long)b * p.H + h) * D + 4 * g) * p.N + nq;
  f32x4 dy[3][4];
#pragma unroll
  for (int which = 0; which < 3; ++which) {
    const float* src = which == 0 ? p.dq_t : which == 1 ? p.dk_t : p.dv_t;
#pragma unroll
    for (int c = 0; c < 4; ++c) dy[which][c] = *reinterpret_cast<const f32x4*>(src + gbase + (long)c * p.N);
    if (p.ndir == 2)
#pragma unroll
      for (int c = 0; c < 4; ++c) dy[which][c] += *reinterpret_cast<const f32x4*>(src + dstride + gbase + (long)c * p.N);
  }
  f32x4 cs[4], sn[4], kr[4], wk;
  if (half)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const long tr = (long)(nq + j) * (D / 2) + 4 * gl;
      cs[j] = *reinterpret_cast<const f32x4*>(p.rope_cos + tr);
      sn[j] = *reinterpret_cast<const f32x4*>(p.rope_sin + tr);
    }
  if (infl) {
#pragma unroll
    for (int j = 0; j < 4; ++j)
      kr[j] = *reinterpret_cast<const f32x4*>(p.k + ((long)b * p.N + nq + j) * C + h * D + 4 * g);
    wk = *reinterpret_cast<const f32x4*>(p.k_norm_w + h * D + 4 * g);
  }
  __syncthreads();
  // forward and transposed maps of one token's four channels
  auto fwd = [&](int which, int j, const f32x4& v) {
    f32x4 o;
    if (half == 0) {
      const float* P = &pm[which][(4 * qd + j) * 16];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const f32x4 row = *reinterpret_cast<const f32x4*>(P + 4 * r);
        o[r] = row[0] * v[0] + row[1] * v[1] + row[2] * v[2] + row[3] * v[3];
      }
    } else {
#pragma unroll
      for (int c = 0; c < 4; ++c) o[c] = v[c] * cs[j][c] + v[c ^ 1] * sn[j][c];
    }
    return o;
  };
  auto bwd = [&](int which, int j, const f32x4& v) {
    f32x4 o;
    if (half == 0) {
      const float* P = &pm[which][(4 * qd + j) * 16];
      o = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const f32x4 row = *reinterpret_cast<const f32x4*>(P + 4 * r);
        o += row * v[r];
      }
    } else {
#pragma unroll
      for (int c = 0; c < 4; ++c) o[c] = v[c] * cs[j][c] + v[c ^ 1] * sn[j][c ^ 1];
    }
    return o;
  };
  auto col = [&](const f32x4 (&m)[4], int j) { return f32x4{m[0][j], m[1][j], m[2][j], m[3][j]}; };
  // the inflation's chain: k's normed vector, its output, and the two squared norms
  f32x4 xk[4], yk[4];
  float d_pre[4], d_post[4];
  if (infl) {
    float pre[4], post[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float iv = kinv[4 * qd + j];
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const float u = kr[j][c] * iv * wk[c];
        xk[j][c] = (u > 0.f ? u : 0.f) * p.k_scale;
      }
      yk[j] = fwd(1, j, xk[j]);
      pre[j] = xk[j][0] * xk[j][0] + xk[j][1] * xk[j][1] + xk[j][2] * xk[j][2] + xk[j][3] * xk[j][3];
      post[j] = yk[j][0] * yk[j][0] + yk[j][1] * yk[j][1] + yk[j][2] * yk[j][2] + yk[j][3] * yk[j][3];
    }
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
    __syncthreads();
    const f32x4 di = *reinterpret_cast<const f32x4*>(p.dinfl + ((long)b * p.H + h) * p.N + nq);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int t = 4 * qd + j;
      const float pr = red[0][0][t] + red[1][0][t], po = red[0][1][t] + red[1][1][t];
      const float prc = fmaxf(pr, 1e-12f), poc = fmaxf(po, 1e-12f);
      d_post[j] = po >= 1e-12f ? di[j] / prc : 0.f;
      d_pre[j] = pr >= 1e-12f ? -di[j] * poc / (prc * prc) : 0.f;
    }
  }
  if (!live) return;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const long o = ((long)b * p.N + nq + j) * C + h * D + 4 * g;
    f32x4 gk = col(dy[1], j);
    if (infl) gk += 2.f * d_post[j] * yk[j];
    gk = bwd(1, j, gk);
    if (infl) gk += 2.f * d_pre[j] * xk[j];
    *reinterpret_cast<f32x4*>(p.dq + o) = bwd(0, j, col(dy[0], j));
    *reinterpret_cast<f32x4*>(p.dk + o) = gk * p.k_scale;
    *reinterpret_cast<f32x4*>(p.dv + o) = bwd(1, j, col(dy[2], j));
  }
}

// The full-channel RMSNorm backward with the ReLU mask, in place on dq and dk (which hold the
// gradients of the post-ReLU values); layout as prep_bwd_kernel, fp32 raw inputs.
template <int NS>
__global__ __launch_bounds__(256) void cam_norm_bwd_kernel(const CamPrepBwdParams p) {
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63;
  const int C = p.H * p.D;
  const long BN = (long)p.B * p.N;
  const long per = (BN + p.nwg - 1) / p.nwg;
  const long t0 = (long)blockIdx.x * per, t1 = min(BN, t0 + per);
  __shared__ float red[2][4][4];  // [token parity][wave][sum]
  float wt[2][NS][8], dw[2][NS][8];
#pragma unroll
  for (int s = 0; s < NS; ++s) {
    const int c = kStrip * s + 8 * tid;
#pragma unroll
    for (int j = 0; j < 8; ++j) dw[0][s][j] = dw[1][s][j] = 0.f;
    if (c < C) {
      ld8(p.q_norm_w + c, wt[0][s]);
      ld8(p.k_norm_w + c, wt[1][s]);
    }
  }
  for (long bn = t0; bn < t1; ++bn) {
    const int par = (int)(bn & 1);
    float x[2][NS][8], g[2][NS][8];
    float sum[4] = {0.f, 0.f, 0.f, 0.f};  // sum x^2 (q), sum w g x (q), the same for k
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      const int c = kStrip * s + 8 * tid;
      if (c >= C) continue;
#pragma unroll
      for (int which = 0; which < 2; ++which) {
        ld8((which ? p.k : p.q) + bn * C + c, x[which][s]);
        ld8((which ? p.dk : p.dq) + bn * C + c, g[which][s]);
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const float xv = x[which][s][j], wv = wt[which][s][j];
          if (!pos_prod(xv, wv)) g[which][s][j] = 0.f;
          sum[2 * which] += xv * xv;
          sum[2 * which + 1] += wv * g[which][s][j] * xv;
        }
      }
    }
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int off = 32; off > 0; off >>= 1) sum[i] += __shfl_xor(sum[i], off, 64);
    if (lane == 0)
#pragma unroll
      for (int i = 0; i < 4; ++i) red[par][w][i] = sum[i];
    __syncthreads();
#pragma unroll
    for (int i = 0; i < 4; ++i) sum[i] = (red[par][0][i] + red[par][1][i]) + (red[par][2][i] + red[par][3][i]);
#pragma unroll
    for (int which = 0; which < 2; ++which) {
      const float r = 1.f / sqrtf(sum[2 * which] / (float)C + p.eps);
      const float corr = r * r * r / (float)C * sum[2 * which + 1];
#pragma unroll
      for (int s = 0; s < NS; ++s) {
        const int c = kStrip * s + 8 * tid;
        if (c >= C) continue;
        float dx[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const float gv = g[which][s][j], xv = x[which][s][j];
          dx[j] = r * wt[which][s][j] * gv - corr * xv;
          dw[which][s][j] += gv * xv * r;
        }
        st8((which ? p.dk : p.dq) + bn * C + c, dx);
      }
    }
  }
#pragma unroll
  for (int which = 0; which < 2; ++which)
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      const int c = kStrip * s + 8 * tid;
      if (c < C) st8(p.part + ((long)blockIdx.x * 2 + which) * C + c, dw[which][s]);
    }
}

// D / 8 lanes per (b, n, h) row, 8 channels each (16-byte loads), 64 / (D / 8) rows per wave.
template <int D>
__global__ __launch_bounds__(256) void merge_bwd_kernel(const MergeBwdParams p) {
  constexpr int LPR = D / 8, RPW = 64 / LPR;
  const int lane = threadIdx.x & 63, j8 = lane % LPR;
  const long row = ((long)blockIdx.x * 4 + (threadIdx.x >> 6)) * RPW + lane / LPR;  // ((b N + n) H + h)
  const long rows = (long)p.B * p.N * p.H;
  const bool on = row < rows;
  const long r = on ? row : 0;
  const long h = r % p.H, bn = r / p.H, n = bn % p.N, b = bn / p.N;
  const long di = (b * p.H + h) * p.N + n;
  const float inv = 1.f / ((float)p.den[di] + p.eps);
  const long o = r * D + 8 * j8;
  float num[8], dout[8], dnum[8], dgate[8], sl[8];
  load8f<bf16>(p.num + o, num);
  load8f<float>(p.dout + o, dout);
  float acc = 0.f;
  if (p.gate) {
    float x[8];
    load8f<bf16>(p.gate + o, x);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const float sg = 1.f / (1.f + __expf(-x[j]));
      sl[j] = x[j] * sg;
      dgate[j] = dout[j] * num[j] * inv * sg * (1.f + x[j] * (1.f - sg));
    }
  } else {
#pragma unroll
    for (int j = 0; j < 8; ++j) sl[j] = 1.f;
  }
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    dnum[j] = dout[j] * sl[j] * inv;
    acc += dout[j] * sl[j] * num[j];
  }
#pragma unroll
  for (int off = LPR / 2; off > 0; off >>= 1) acc += __shfl_xor(acc, off, 64);
  if (!on) return;
  st8(p.dnum + o, dnum);
  if (p.gate) st8(p.dgate + o, dgate);
  if (j8 == 0) p.dden[di] = -acc * inv * inv;
}

}  // namespace

hipError_t launch_prep_bwd(const PrepBwdParams& p, hipStream_t stream) {
  const int C = p.H * p.D;
  if (C <= kStrip)
    hipLaunchKernelGGL((prep_bwd_kernel<1>), dim3(p.nwg), dim3(256), 0, stream, p);
  else
    hipLaunchKernelGGL((prep_bwd_kernel<2>), dim3(p.nwg), dim3(256), 0, stream, p);
  hipLaunchKernelGGL(prep_bwd_wsum_kernel, dim3((2 * C + 63) / 64), dim3(1024), 0, stream,
                     p.part, p.nwg, C, p.dq_norm_w, p.dk_norm_w);
  return hipGetLastError();
}

hipError_t launch_cam_prep_bwd(const CamPrepBwdParams& p, hipStream_t stream) {
  const int C = p.H * p.D;
  const long ntok = (long)p.B * p.N;
  if (p.dinfl)
    hipLaunchKernelGGL(cam_kinv_kernel, dim3((unsigned)((ntok + 3) / 4)), dim3(256), 0, stream, p);
  const dim3 grid((unsigned)((long)p.B * p.H * ((p.N + 63) / 64)));
  if (p.D == 128)
    hipLaunchKernelGGL(cam_prep_bwd_tile_kernel<128>, grid, dim3(512), 0, stream, p);
  else
    hipLaunchKernelGGL(cam_prep_bwd_tile_kernel<64>, grid, dim3(256), 0, stream, p);
  if (C <= kStrip)
    hipLaunchKernelGGL((cam_norm_bwd_kernel<1>), dim3(p.nwg), dim3(256), 0, stream, p);
  else
    hipLaunchKernelGGL((cam_norm_bwd_kernel<2>), dim3(p.nwg), dim3(256), 0, stream, p);
  hipLaunchKernelGGL(prep_bwd_wsum_kernel, dim3((2 * C + 63) / 64), dim3(1024), 0, stream,
                     p.part, p.nwg, C, p.dq_norm_w, p.dk_norm_w);
  return hipGetLastError();
}

hipError_t launch_merge_bwd(const MergeBwdParams& p, hipStream_t stream) {
  const long rows = (long)p.B * p.N * p.H;
  const long rows_per_wg = 4 * (64 / (p.D / 8));
  const dim3 grid((unsigned)((rows + rows_per_wg - 1) / rows_per_wg));
  if (p.D == 128)
    hipLaunchKernelGGL((merge_bwd_kernel<128>), grid, dim3(256), 0, stream, p);
  else
    hipLaunchKernelGGL((merge_bwd_kernel<64>), grid, dim3(256), 0, stream, p);
  return hipGetLastError();
}

}  // namespace gdn

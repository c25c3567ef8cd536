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
          g[which][s][j] = xv * wv > 0.f ? gp[j] * scl : 0.f;
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
__global__ __launch_bounds__(1024) void prep_bwd_wsum_kernel(const PrepBwdParams p) {
  const int C = p.H * p.D;
  const int cl = threadIdx.x & 63, sl = threadIdx.x >> 6;
  const int i = blockIdx.x * 64 + cl;  // (which, channel)
  __shared__ float red[16][64];
  float acc = 0.f;
  if (i < 2 * C) {
    const int which = i / C, c = i % C;
#pragma unroll 8
    for (int g = sl; g < p.nwg; g += 16) acc += p.part[((long)g * 2 + which) * C + c];
  }
  red[sl][cl] = acc;
  __syncthreads();
  if (sl == 0 && i < 2 * C) {
    float t = 0.f;
#pragma unroll
    for (int k = 0; k < 16; ++k) t += red[k][cl];
    (i < C ? p.dq_norm_w : p.dk_norm_w)[i % C] = t;
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
  hipLaunchKernelGGL(prep_bwd_wsum_kernel, dim3((2 * C + 63) / 64), dim3(1024), 0, stream, p);
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

// gdn_summary.hip -- helpers of the fragment state summary (gdn_state_summary) and its
// application (gdn_state_apply), for running the fragments of a sequence separately
// (the context-parallel state summary of the MindSpore hyper-parallel page).
//
// A fragment's final state is affine in its initial state, ht(h0) = M h0 + ht(0), where M
// is the ordered product of the per-token maps A_t = (I - beta_t k_t k_t^T) diag(a_t),
// a_t = exp(g_t + gk_t).  ht(0) comes from the forward kernels.  M decays like the product
// of the a_t over the whole fragment, far below the range of the fp16 operands the chunked
// forward kernels use, so it has its own kernel: the token recurrence on M in fp32, every
// column carrying a power-of-two exponent that is renormalised once per 64 tokens (the map
// is linear and acts on each column separately, so a column may be scaled at any point).
#include <algorithm>

#include "gdn_device.h"
#include "gdn_internal.h"

namespace gdn {

namespace {

__global__ __launch_bounds__(256) void zero_kernel(uint4* p, long n16) {
  for (long i = blockIdx.x * 256L + threadIdx.x; i < n16; i += (long)gridDim.x * 256)
    p[i] = make_uint4(0u, 0u, 0u, 0u);
}

// [BH, K, K] identity matrices
__global__ __launch_bounds__(256) void identity_kernel(float* m, long BH, int K) {
  const long n = BH * K * K;
  for (long i = blockIdx.x * 256L + threadIdx.x; i < n; i += (long)gridDim.x * 256) {
    const int rc = (int)(i % ((long)K * K));
    m[i] = (rc / K == rc % K) ? 1.f : 0.f;
  }
}

// h_out = M h_in + c per (b, h): one workgroup per (bh, 16 output rows); the 16 rows of M
// are staged in LDS, each thread forms outputs (row, column) with column-contiguous loads of
// h_in.  fp32 throughout.
constexpr int kApplyRows = 16;
__global__ __launch_bounds__(256) void apply_kernel(const float* c, const float* M, const float* h_in,
                                                    float* h_out, int K, int V) {
  __shared__ float ms[kApplyRows][kApplyMaxK];
  const long bh = blockIdx.y;
  const int r0 = blockIdx.x * kApplyRows;
  const int rows = min(kApplyRows, K - r0);
  if (h_in) {
    for (int e = threadIdx.x; e < rows * K; e += 256)
      ms[e / K][e % K] = M[(bh * K + r0 + e / K) * K + e % K];
    __syncthreads();
  }
  const float* hb = h_in ? h_in + bh * K * V : nullptr;
  for (int e = threadIdx.x; e < rows * V; e += 256) {
    const int r = e / V, col = e % V;
    float acc = c[(bh * K + r0 + r) * V + col];
    if (hb)
      for (int k = 0; k < K; ++k) acc = fmaf(ms[r][k], hb[(long)k * V + col], acc);
    h_out[(bh * K + r0 + r) * V + col] = acc;
  }
}

// Sum over the 16 lanes of a DPP row, in every lane: lane pairs (xor 1), quad pairs (xor 2),
// the two quads of each half row (half-row mirror) and the two half rows (row mirror).
template <int kCtrl>
__device__ __forceinline__ float dpp_f(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), kCtrl, 0xF, 0xF, false));
}
__device__ __forceinline__ float row_sum16(float x) {
  x += dpp_f<0xB1>(x);   // quad_perm [1, 0, 3, 2]
  x += dpp_f<0x4E>(x);   // quad_perm [2, 3, 0, 1]
  x += dpp_f<0x141>(x);  // row_half_mirror
  x += dpp_f<0x140>(x);  // row_mirror
  return x;
}

// Transition M (one workgroup per (b, h, 32-column block of M)).  Lane layout: thread t owns
// columns cb*32 + 2(t/16) + {0, 1} and the K/16 consecutive rows (t%16)(K/16) + j, so the 16
// threads of a column pair are one DPP row and k^T M reduces with four DPP adds;
// two columns per thread give two independent dependency chains per token.  A chunk's keys,
// betas and decays are staged in LDS as fp32 first.  A scalar gate commutes with the rank-one
// maps, so it is not applied per token: its chunk sum goes into the column's exponent.
template <int K, bool PK, typename TI>
__global__ __launch_bounds__(256) void transition_kernel(const TI* __restrict__ k,
                                                         const float* __restrict__ g,
                                                         const float* __restrict__ gk,
                                                         const float* __restrict__ beta,
                                                         float* __restrict__ M, int T, int H) {
  constexpr int kR = K / 16;  // rows per thread
  constexpr int kC = 64;      // tokens staged at a time
  __shared__ __attribute__((aligned(16))) float ks[kC][K];
  __shared__ __attribute__((aligned(16))) float as[PK ? kC : 1][K];
  __shared__ float bs[kC], gs[kC];
  const int ncb = K / 32;
  const int cb = blockIdx.x % ncb, bh = blockIdx.x / ncb;
  const int b = bh / H, h = bh % H;
  const int tid = threadIdx.x, c0 = cb * 32 + 2 * (tid / 16), r0 = (tid % 16) * kR;
  float m[2][kR];
#pragma unroll
  for (int u = 0; u < 2; ++u)
#pragma unroll
    for (int j = 0; j < kR; ++j) m[u][j] = (r0 + j == c0 + u) ? 1.f : 0.f;
  // a column is m * 2^(ex + lg): ex from renormalisation, lg the scalar gate's log2 decay
  int ex[2] = {0, 0};
  float lg = 0.f;
  // A chunk's inputs are loaded into registers while the previous chunk's tokens are
  // processed (16-byte pieces, all issued before any is used), then written to LDS.
  constexpr int kPer = 16 / sizeof(TI);                  // key elements per 16-byte piece
  constexpr int kKP = (kC * K / kPer + 255) / 256;       // key pieces per thread
  constexpr int kAP = PK ? (kC * K / 4 + 255) / 256 : 1;  // gk pieces per thread
  typedef TI tin_v __attribute__((ext_vector_type(kPer)));
  tin_v kp[kKP];
  f32x4 gp[kAP];
  float sp = 0.f;
  auto load_chunk = [&](int t0) {
    const int n = min(kC, T - t0);
#pragma unroll
    for (int i = 0; i < kKP; ++i) {
      const int e = tid + 256 * i, t = e / (K / kPer), d = (e % (K / kPer)) * kPer;
      if (t < n) kp[i] = *reinterpret_cast<const tin_v*>(k + (((long)b * T + t0 + t) * H + h) * K + d);
    }
    if constexpr (PK) {
#pragma unroll
      for (int i = 0; i < kAP; ++i) {
        const int e = tid + 256 * i, t = e / (K / 4), d = (e % (K / 4)) * 4;
        if (t < n) gp[i] = *reinterpret_cast<const f32x4*>(gk + (((long)b * T + t0 + t) * H + h) * K + d);
      }
    }
    if (tid < 2 * kC && (tid % kC) < n) {
      const long row = ((long)b * T + t0 + tid % kC) * H + h;
      sp = tid < kC ? beta[row] : (g ? g[row] : 0.f);
    }
  };
  load_chunk(0);
  for (int t0 = 0; t0 < T; t0 += kC) {
    const int n = min(kC, T - t0);
    __syncthreads();  // the previous chunk's LDS reads are done
    if (tid < 2 * kC && (tid % kC) < n) (tid < kC ? bs : gs)[tid % kC] = tid < kC ? sp : floor_gate(sp);
    __syncthreads();
#pragma unroll
    for (int i = 0; i < kKP; ++i) {
      const int e = tid + 256 * i, t = e / (K / kPer), d = (e % (K / kPer)) * kPer;
      if (t < n)
#pragma unroll
        for (int j = 0; j < kPer; ++j) ks[t][d + j] = (float)kp[i][j];
    }
    if constexpr (PK) {
#pragma unroll
      for (int i = 0; i < kAP; ++i) {
        const int e = tid + 256 * i, t = e / (K / 4), d = (e % (K / 4)) * 4;
        if (t < n)
#pragma unroll
          for (int j = 0; j < 4; ++j) as[t][d + j] = __expf(floor_key_gate(gp[i][j] + gs[t]));
      }
    }
    __syncthreads();
    if (t0 + kC < T) load_chunk(t0 + kC);
    // token t's key rows, decays and beta are read from LDS one token ahead
    f32x4 kn[kR / 4], an[kR / 4];
    float bn = 0.f;
    auto fetch = [&](int t) {
#pragma unroll
      for (int q = 0; q < kR / 4; ++q) {
        kn[q] = *reinterpret_cast<const f32x4*>(&ks[t][r0 + 4 * q]);
        if constexpr (PK) an[q] = *reinterpret_cast<const f32x4*>(&as[t][r0 + 4 * q]);
      }
      bn = bs[t];
    };
    fetch(0);
    for (int t = 0; t < n; ++t) {
      f32x4 kc[kR / 4], ac[kR / 4];
#pragma unroll
      for (int q = 0; q < kR / 4; ++q) {
        kc[q] = kn[q];
        if constexpr (PK) ac[q] = an[q];
      }
      const float bt = bn;
      if (t + 1 < n) fetch(t + 1);
      float kr[kR], w[2][2] = {{0.f, 0.f}, {0.f, 0.f}};
#pragma unroll
      for (int j = 0; j < kR; j += 4) {
        const f32x4 kv = kc[j / 4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          kr[j + e] = kv[e];
#pragma unroll
          for (int u = 0; u < 2; ++u) {
            if constexpr (PK) m[u][j + e] *= ac[j / 4][e];
            w[u][e & 1] = fmaf(kv[e], m[u][j + e], w[u][e & 1]);
          }
        }
      }
      float bw[2];
#pragma unroll
      for (int u = 0; u < 2; ++u) bw[u] = bt * row_sum16(w[u][0] + w[u][1]);
#pragma unroll
      for (int j = 0; j < kR; ++j)
#pragma unroll
        for (int u = 0; u < 2; ++u) m[u][j] = fmaf(-bw[u], kr[j], m[u][j]);
    }
    if constexpr (!PK) {
      float gsum = 0.f;
      for (int t = 0; t < n; ++t) gsum += gs[t];
      lg += gsum * 1.4426950408889634f;
    }
    // renormalise each column to a maximum magnitude in [0.5, 1)
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      float mx = 0.f;
#pragma unroll
      for (int j = 0; j < kR; ++j) mx = fmaxf(mx, fabsf(m[u][j]));
      mx = fmaxf(mx, __shfl_xor(mx, 1, 64));
      mx = fmaxf(mx, __shfl_xor(mx, 2, 64));
      mx = fmaxf(mx, __shfl_xor(mx, 4, 64));
      mx = fmaxf(mx, __shfl_xor(mx, 8, 64));
      if (mx > 0.f) {
        int e;
        frexpf(mx, &e);
#pragma unroll
        for (int j = 0; j < kR; ++j) m[u][j] = ldexpf(m[u][j], -e);
        ex[u] += e;
      }
    }
  }
  float* out = M + (long)bh * K * K;
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const float sc = exp2f((float)ex[u] + lg);
#pragma unroll
    for (int j = 0; j < kR; ++j) out[(long)(r0 + j) * K + c0 + u] = m[u][j] * sc;
  }
}

}  // namespace

hipError_t launch_zero(void* p, size_t bytes, hipStream_t stream) {
  const long n16 = (long)(bytes / 16);
  if (n16 == 0) return hipSuccess;
  const int blocks = (int)std::min<long>((n16 + 255) / 256, 8192);
  hipLaunchKernelGGL(zero_kernel, dim3(blocks), dim3(256), 0, stream, static_cast<uint4*>(p), n16);
  return hipGetLastError();
}

hipError_t launch_identity(float* m, long BH, int K, hipStream_t stream) {
  const long n = BH * K * K;
  const int blocks = (int)std::min<long>((n + 255) / 256, 8192);
  hipLaunchKernelGGL(identity_kernel, dim3(blocks), dim3(256), 0, stream, m, BH, K);
  return hipGetLastError();
}

hipError_t launch_transition(const void* k, const float* g, const float* gk, const float* beta,
                             float* M, int B, int T, int H, int K, int dtype, hipStream_t stream) {
  const dim3 grid(B * H * (K / 32)), blk(256);
  const bool pk = gk != nullptr;
#define GDN_TRANSITION(KK, PKK, TT) \
  hipLaunchKernelGGL((transition_kernel<KK, PKK, TT>), grid, blk, 0, stream, static_cast<const TT*>(k), g, gk, beta, M, T, H)
  if (dtype == 1) {
    if (K == 128) { if (pk) GDN_TRANSITION(128, true, bf16); else GDN_TRANSITION(128, false, bf16); }
    else { if (pk) GDN_TRANSITION(64, true, bf16); else GDN_TRANSITION(64, false, bf16); }
  } else {
    if (K == 128) { if (pk) GDN_TRANSITION(128, true, float); else GDN_TRANSITION(128, false, float); }
    else { if (pk) GDN_TRANSITION(64, true, float); else GDN_TRANSITION(64, false, float); }
  }
#undef GDN_TRANSITION
  return hipGetLastError();
}

hipError_t launch_apply(const float* c, const float* M, const float* h_in, float* h_out, int BH,
                        int K, int V, hipStream_t stream) {
  hipLaunchKernelGGL(apply_kernel, dim3((K + kApplyRows - 1) / kApplyRows, BH), dim3(256), 0, stream,
                     c, M, h_in, h_out, K, V);
  return hipGetLastError();
}

}  // namespace gdn

// gdn_bwdprep.hip -- the inputs of the state-gradient pass, formed from the forward's inputs
// (hyper-parallel "Diff Coverage" page: the chunk state pass takes v_new = u - w h, and its
// dhu backward takes w and the intra-chunk gradient of v_new).  Per 64-token chunk, with
// gamma the chunk-local inclusive cumsum of the scalar log gate:
//     A_{r,s} = beta_r e^{gamma_r - gamma_s} (k_r . k_s)        (s < r)
//     w       = (I + A)^-1 diag(beta e^gamma) K
//     P_{r,s} = scale e^{gamma_r - gamma_s} (q_r . k_s)        (s <= r)
//     dv      = P^T do.
// gamma decreases along the chunk, so every factor e^{gamma_r - gamma_s} (s <= r) and e^gamma
// lies in (0, 1]; the gate is floored as everywhere else (floor_gate).
//
// One workgroup of four waves per (b, h, chunk).  Keys and queries staged as split bf16
// pairs; the Gram and Q K^T tiles on matrix cores; w by block forward substitution over the
// four 16-row blocks, W_i = D_i (diag(beta e^gamma) K_i - sum_{j<i} A_ij W_j) with
// D_i = (I + A_ii)^-1 from a 16-step substitution per column (as the fragment transition's
// chunk factor); dv = P^T do on matrix cores with do transposed into LDS.  All products take
// split bf16 operands (GDN_SPLIT), so the results are near fp32 before the output rounding.
#include "gdn_device.h"
#include "gdn_internal.h"

namespace gdn {
namespace {

typedef bf16 bf16x4 __attribute__((ext_vector_type(4)));

template <typename T>
__device__ __forceinline__ T cast_out(float x) {
  return (T)x;
}

template <int K, int V, typename TI>
__global__ __launch_bounds__(256) void bwd_prep_kernel(const BwdPrepParams p) {
  constexpr bool kSplit = !std::is_same<TI, bf16>::value;
  constexpr int kS = K + 8;   // bf16 row stride of the key / query tiles ([token][K])
  constexpr int kA = 68;      // float row stride of A and P
  constexpr int kX = 72;      // bf16 row stride of the [column][token] tiles
  constexpr int CT = K / 64;  // 16-column tiles of w per wave
  constexpr int CV = V / 64;  // 16-column tiles of dv per wave
  constexpr int kKQBytes = 4 * 64 * kS * 2, kWtBytes = 2 * K * kX * 2;
  __shared__ __attribute__((aligned(16))) unsigned char smem[kKQBytes > kWtBytes ? kKQBytes : kWtBytes];
  __shared__ __attribute__((aligned(16))) bf16 dT[2][V * kX];  // do^T hi/lo
  __shared__ __attribute__((aligned(16))) float am[64 * kA];   // A (strictly lower)
  __shared__ __attribute__((aligned(16))) float pm[64 * kA];   // P (lower incl. diagonal)
  __shared__ __attribute__((aligned(16))) float dm[64 * 20];   // D_i rows, [i][16][20]
  __shared__ float bs[64], gs[64];
  bf16* kh = reinterpret_cast<bf16*>(smem);
  bf16* kl = kh + 64 * kS;
  bf16* qh = kl + 64 * kS;
  bf16* ql = qh + 64 * kS;
  bf16* wh = reinterpret_cast<bf16*>(smem);  // W^T so far (hi/lo), once keys and queries are done
  bf16* wl = wh + K * kX;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, li = lane & 15, lq = lane >> 4;
  const int NT = (p.T + 63) / 64;
  const int n = blockIdx.x % NT;
  const long bh = blockIdx.x / NT;
  const int b = (int)(bh / p.H), h = (int)(bh % p.H);
  const int t0 = 64 * n, nt = min(64, p.T - t0);
  const TI* kin = static_cast<const TI*>(p.k);
  const TI* qin = static_cast<const TI*>(p.q);
  const TI* din = static_cast<const TI*>(p.do_);
  auto row = [&](int t) { return ((long)b * p.T + t0 + t) * p.H + h; };

  // keys and queries as split pairs ([token][K]); rows past the end are zero
  for (int e = tid; e < 64 * K / 8; e += 256) {
    const int t = e / (K / 8), d = (e % (K / 8)) * 8;
    float xk[8], xq[8];
    if (t < nt) {
      load8f(kin + row(t) * K + d, xk);
      load8f(qin + row(t) * K + d, xq);
    } else {
#pragma unroll
      for (int j = 0; j < 8; ++j) xk[j] = xq[j] = 0.f;
    }
    bf16x8 a, c, e2, f;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      GDN_SPLIT(xk[j], a[j], c[j]);
      GDN_SPLIT(xq[j], e2[j], f[j]);
    }
    *reinterpret_cast<bf16x8*>(&kh[t * kS + d]) = a;
    *reinterpret_cast<bf16x8*>(&kl[t * kS + d]) = c;
    *reinterpret_cast<bf16x8*>(&qh[t * kS + d]) = e2;
    *reinterpret_cast<bf16x8*>(&ql[t * kS + d]) = f;
  }
  // do transposed ([column][token]): lanes take consecutive tokens (conflict-free writes)
  for (int e = tid; e < 64 * V / 8; e += 256) {
    const int t = e % 64, c8 = 8 * (e / 64);
    float x[8];
    if (t < nt) {
      load8f(din + row(t) * V + c8, x);
    } else {
#pragma unroll
      for (int j = 0; j < 8; ++j) x[j] = 0.f;
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) GDN_SPLIT(x[j], dT[0][(c8 + j) * kX + t], dT[1][(c8 + j) * kX + t]);
  }
  if (tid < 64) {
    const float gv = tid < nt && p.g ? floor_gate(p.g[row(tid)]) : 0.f;
    gs[tid] = wave_incl_scan(gv, lane);
    bs[tid] = tid < nt ? p.beta[row(tid)] : 0.f;
  }
  __syncthreads();
  // lower tiles (ti >= tj) of the Gram matrix (jobs 0..9) and of Q K^T (jobs 10..19)
  for (int q = wave; q < 20; q += 4) {
    const bool isP = q >= 10;
    const int qq = isP ? q - 10 : q;
    int ti = 0;
    while (qq >= (ti + 1) * (ti + 2) / 2) ++ti;
    const int tj = qq - ti * (ti + 1) / 2;
    const bf16* ah_ = isP ? qh : kh;
    const bf16* al_ = isP ? ql : kl;
    f32x4 c = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kk = 0; kk < K / 32; ++kk) {
      const int oa = (16 * ti + li) * kS + 32 * kk + 8 * lq, ob = (16 * tj + li) * kS + 32 * kk + 8 * lq;
      c = mma3(lds8(&ah_[oa]), lds8(&al_[oa]), lds8(&kh[ob]), lds8(&kl[ob]), c);
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int r = 16 * ti + 4 * lq + e, s = 16 * tj + li;
      const float dec = __expf(gs[r] - gs[min(s, r)]);
      if (isP)
        pm[r * kA + s] = s <= r ? p.scale * dec * c[e] : 0.f;
      else
        am[r * kA + s] = s < r ? bs[r] * dec * c[e] : 0.f;
    }
  }
  // this lane's right-hand sides beta_r e^{gamma_r} k_r: rows 16 i + 4 lq + e, its columns
  float kr[4][CT][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int c = 0; c < CT; ++c)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int r = 16 * i + 4 * lq + e, o = r * kS + 16 * (CT * wave + c) + li;
        kr[i][c][e] = bs[r] * __expf(gs[r]) * ((float)kh[o] + (float)kl[o]);
      }
  __syncthreads();  // A and P complete; the key and query tiles are no longer read
  for (int e = tid; e < kWtBytes / 16; e += 256) reinterpret_cast<uint4*>(smem)[e] = make_uint4(0u, 0u, 0u, 0u);
  if (tid < 64) {
    // column c of D_i = (I + A_ii)^-1: d_r = [r == c] - sum_{s<r} A_rs d_s (d_s = 0 for s < c)
    const int i = tid >> 4, c = tid & 15;
    float d[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      float acc = r == c ? 1.f : 0.f;
#pragma unroll
      for (int s = 0; s < r; ++s) acc = fmaf(-am[(16 * i + r) * kA + 16 * i + s], d[s], acc);
      d[r] = acc;
    }
#pragma unroll
    for (int r = 0; r < 16; ++r) dm[(16 * i + r) * 20 + c] = d[r];
  }
  __syncthreads();

  // ---- w, block by block; wave `wave` owns columns 16 CT wave .. of w throughout
  TI* wout = static_cast<TI*>(p.w);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    f32x4 C[CT];
#pragma unroll
    for (int c = 0; c < CT; ++c) C[c] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < (16 * i + 31) / 32; ++ks) {
      bf16x8 ah, al;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int s = 32 * ks + 8 * lq + j;
        GDN_SPLIT(s < 16 * i ? am[(16 * i + li) * kA + s] : 0.f, ah[j], al[j]);
      }
#pragma unroll
      for (int c = 0; c < CT; ++c) {
        const int o = (16 * (CT * wave + c) + li) * kX + 32 * ks + 8 * lq;
        C[c] = mma3(ah, al, lds8(&wh[o]), lds8(&wl[o]), C[c]);
      }
    }
#pragma unroll
    for (int c = 0; c < CT; ++c) {
      const int col = 16 * (CT * wave + c) + li;
      bf16x4 xh, xl;
#pragma unroll
      for (int e = 0; e < 4; ++e) GDN_SPLIT(kr[i][c][e] - C[c][e], xh[e], xl[e]);
      *reinterpret_cast<bf16x4*>(&wh[col * kX + 16 * i + 4 * lq]) = xh;
      *reinterpret_cast<bf16x4*>(&wl[col * kX + 16 * i + 4 * lq]) = xl;
    }
    bf16x8 ah, al;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int kk = 8 * lq + j - 16 * (i % 2);
      GDN_SPLIT((kk >= 0 && kk < 16) ? dm[(16 * i + li) * 20 + (kk & 15)] : 0.f, ah[j], al[j]);
    }
#pragma unroll
    for (int c = 0; c < CT; ++c) {
      const int col = 16 * (CT * wave + c) + li;
      const int o = col * kX + 32 * (i / 2) + 8 * lq;
      const f32x4 wi = mma3(ah, al, lds8(&wh[o]), lds8(&wl[o]), f32x4{0.f, 0.f, 0.f, 0.f});
      bf16x4 xh, xl;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int r = 16 * i + 4 * lq + e;
        if (r < nt) wout[row(r) * K + col] = cast_out<TI>(wi[e]);
        GDN_SPLIT(wi[e], xh[e], xl[e]);
      }
      *reinterpret_cast<bf16x4*>(&wh[col * kX + 16 * i + 4 * lq]) = xh;
      *reinterpret_cast<bf16x4*>(&wl[col * kX + 16 * i + 4 * lq]) = xl;
    }
  }

  // ---- dv = P^T do: rows s (four 16-row blocks), wave `wave` owns columns 16 CV wave ..
  TI* dvout = static_cast<TI*>(p.dv);
#pragma unroll
  for (int js = 0; js < 4; ++js) {
    f32x4 C[CV];
#pragma unroll
    for (int c = 0; c < CV; ++c) C[c] = f32x4{0.f, 0.f, 0.f, 0.f};
    // contraction over the tokens r >= 16 js (P^T[s][r] = P[r][s])
#pragma unroll
    for (int ks = js / 2; ks < 2; ++ks) {
      bf16x8 ah, al;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int r = 32 * ks + 8 * lq + j;
        GDN_SPLIT(r >= 16 * js ? pm[r * kA + 16 * js + li] : 0.f, ah[j], al[j]);
      }
#pragma unroll
      for (int c = 0; c < CV; ++c) {
        const int o = (16 * (CV * wave + c) + li) * kX + 32 * ks + 8 * lq;
        C[c] = mma3(ah, al, lds8(&dT[0][o]), lds8(&dT[1][o]), C[c]);
      }
    }
#pragma unroll
    for (int c = 0; c < CV; ++c)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int s = 16 * js + 4 * lq + e;
        if (s < nt) dvout[row(s) * V + 16 * (CV * wave + c) + li] = cast_out<TI>(C[c][e]);
      }
  }
}

template <typename TI>
hipError_t launch_t(const BwdPrepParams& p, int K, int V, hipStream_t stream) {
  const dim3 grid(p.B * p.H * ((p.T + 63) / 64)), blk(256);
  if (K == 128) {
    if (V == 128) hipLaunchKernelGGL((bwd_prep_kernel<128, 128, TI>), grid, blk, 0, stream, p);
    else hipLaunchKernelGGL((bwd_prep_kernel<128, 64, TI>), grid, blk, 0, stream, p);
  } else {
    if (V == 128) hipLaunchKernelGGL((bwd_prep_kernel<64, 128, TI>), grid, blk, 0, stream, p);
    else hipLaunchKernelGGL((bwd_prep_kernel<64, 64, TI>), grid, blk, 0, stream, p);
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_bwd_prep(const BwdPrepParams& p, int K, int V, int dtype, hipStream_t stream) {
  return dtype == 1 ? launch_t<bf16>(p, K, V, stream) : launch_t<float>(p, K, V, stream);
}

}  // namespace gdn

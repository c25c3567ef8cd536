// gdn_bwd.hip -- state-gradient pass of the chunked backward (dhu) for gfx950.
//
// The adjoint of the chunk state pass (hyper-parallel "Diff Coverage" page, the dhu
// fragments): over chunks in reverse, with dh the gradient of the state leaving the chunk,
//   dv2_t = dv_t + e^{gamma_L - gamma_t} (K dh)_t            (gradient of v_new)
//   dh   <- e^{gamma_L} dh + scale (e^gamma Q)^T do - W^T dv2  (gradient of the state entering)
// gamma is the chunk-local inclusive cumsum of the log gate, gamma_L its value at the chunk's
// last valid token.  dh_chunks[n] receives dh after chunk n's update (the gradient of the
// saved state h[n]); dh0 the final dh.
//
// One workgroup of four waves per (chain, 32-column block of dh).  dh lives in registers as
// matrix-core accumulators (fp32) and is copied to LDS once per chunk for K dh.  Products
// use fp32 matrix-core steps (16x16x4), so fp32 inputs keep fp32 accuracy.  A chunk's K, Q,
// W, do rows and dv entries are loaded one chunk ahead into registers; the tiles sit in LDS
// in their natural [token][channel] layout with row strides chosen so every operand read of
// a wave falls in distinct banks.
#include "gdn_device.h"
#include "gdn_internal.h"

namespace gdn {

namespace {

constexpr int kC = 64;                 // chunk length
constexpr int kSK = 132, kSQ = 144;    // row strides (floats) of the K and Q / W tiles
constexpr int kSV = 48;                // row stride of the do, dv2 and dh tiles

template <typename T>
__device__ __forceinline__ void to_f32(const uint4& raw, float* out);
template <>
__device__ __forceinline__ void to_f32<float>(const uint4& raw, float* out) {
  out[0] = __uint_as_float(raw.x);
  out[1] = __uint_as_float(raw.y);
  out[2] = __uint_as_float(raw.z);
  out[3] = __uint_as_float(raw.w);
}
template <>
__device__ __forceinline__ void to_f32<bf16>(const uint4& raw, float* out) {
  const bf16x8 v = __builtin_bit_cast(bf16x8, raw);
#pragma unroll
  for (int j = 0; j < 8; ++j) out[j] = (float)v[j];
}

template <int K, typename TIn>
__global__ __launch_bounds__(256) void dhu_kernel(const DhuParams p) {
  constexpr int E = 16 / sizeof(TIn);     // elements per 16-byte piece
  constexpr int kPK = K / E;              // pieces per K row
  constexpr int kItK = kC * kPK / 256;    // pieces per thread of a K / Q / W tile
  constexpr int kPV = 32 / E;             // pieces per 32-column do row
  constexpr int kItV = kC * kPV / 256;    // pieces per thread of the do tile (1 or 2)
  __shared__ __attribute__((aligned(16))) float sk[kC * kSK];
  __shared__ __attribute__((aligned(16))) float sq[kC * kSQ];
  __shared__ __attribute__((aligned(16))) float sw[kC * kSQ];
  __shared__ __attribute__((aligned(16))) float sdo[kC * kSV];
  __shared__ __attribute__((aligned(16))) float sdv[kC * kSV];
  __shared__ __attribute__((aligned(16))) float sdh[K * kSV];
  __shared__ float gam[kC];
  static_assert(kItK * 256 == kC * kPK && kItV * 256 == kC * kPV, "tile pieces");
  // Workgroups are dealt to the eight XCDs round-robin by index; when B*H is a multiple of
  // eight, the value blocks of one chain get indices on one XCD, so its q, k, w rows come
  // from that XCD's L2 after the first read.
  const int nvb = p.V / 32;
  int vb, bh;
  if (p.B * p.H % 8 == 0) {
    const int x8 = blockIdx.x / 8;
    bh = blockIdx.x % 8 + 8 * (x8 / nvb);
    vb = x8 % nvb;
  } else {
    vb = blockIdx.x % nvb;
    bh = blockIdx.x / nvb;
  }
  const int b = bh / p.H, h = bh % p.H;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int li = lane & 15, lq = lane >> 4;
  const int T = p.T, NT = (T + kC - 1) / kC;
  const TIn* q = static_cast<const TIn*>(p.q);
  const TIn* k = static_cast<const TIn*>(p.k);
  const TIn* w = static_cast<const TIn*>(p.w);
  const TIn* dO = static_cast<const TIn*>(p.do_);
  const TIn* dV = static_cast<const TIn*>(p.dv);
  const long HK = (long)p.H * K, HV = (long)p.H * p.V;
  const int v0 = 32 * vb;
  // dh: wave w holds rows 32w + 16a + 4lq + e, columns 16ct + li
  f32x4 dh[2][2];
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int ct = 0; ct < 2; ++ct)
#pragma unroll
      for (int e = 0; e < 4; ++e)
        dh[a][ct][e] = p.dht ? p.dht[((long)bh * K + 32 * wave + 16 * a + 4 * lq + e) * p.V + v0 + 16 * ct + li] : 0.f;

  // The next chunk's inputs, loaded a chunk ahead.  Every load is unconditional, from the
  // token clamped to T - 1, and rows past T are zeroed where they are used: a load under a
  // branch makes the compiler wait for all outstanding memory right after it, which would
  // also wait for the prefetch itself.
  uint4 rk[kItK], rq[kItK], rw[kItK], rdo[kItV];
  TIn rdv[2][4];
  float rg = 0.f;
  auto tok = [&](int t) { return t < T ? t : T - 1; };
  auto load = [&](int n) {
    const int t0 = n * kC;
#pragma unroll
    for (int i = 0; i < kItK; ++i) {
      const int pc = tid + 256 * i, t = pc / kPK, j = pc % kPK;
      const long o = ((long)b * T + tok(t0 + t)) * HK + (long)h * K + j * E;
      rk[i] = *reinterpret_cast<const uint4*>(k + o);
      rq[i] = *reinterpret_cast<const uint4*>(q + o);
      rw[i] = *reinterpret_cast<const uint4*>(w + o);
    }
#pragma unroll
    for (int i = 0; i < kItV; ++i) {
      const int pc = tid + 256 * i, t = pc / kPV, j = pc % kPV;
      const long o = ((long)b * T + tok(t0 + t)) * HV + (long)h * p.V + v0 + j * E;
      rdo[i] = *reinterpret_cast<const uint4*>(dO + o);
    }
    // dv in the accumulator layout of the K dh product: tokens 16w + 4lq + e, column 16ct + li
#pragma unroll
    for (int ct = 0; ct < 2; ++ct)
#pragma unroll
      for (int e = 0; e < 4; ++e)
        rdv[ct][e] = dV[((long)b * T + tok(t0 + 16 * wave + 4 * lq + e)) * HV + (long)h * p.V + v0 + 16 * ct + li];
    if (p.g && tid < kC) rg = p.g[((long)b * T + tok(t0 + tid)) * p.H + h];
  };

  // dv2 of chunk m from its LDS tile: wave w stores the tokens 16w .. 16w + 15 it writes
  auto store_dv2 = [&](int m) {
    TIn* dst = static_cast<TIn*>(p.dv2) + (long)h * p.V + v0;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int pc = lane + 64 * i, r = pc / 8, c4 = pc % 8, t = 16 * wave + r;
      if (m * kC + t < T) {
        const f32x4 x = *reinterpret_cast<const f32x4*>(&sdv[t * kSV + 4 * c4]);
        TIn* o = dst + ((long)b * T + m * kC + t) * HV + 4 * c4;
        if constexpr (sizeof(TIn) == 4) {
          *reinterpret_cast<f32x4*>(o) = x;
        } else {
          typedef bf16 bf16x4_t __attribute__((ext_vector_type(4)));
          *reinterpret_cast<bf16x4_t*>(o) = bf16x4_t{(bf16)x[0], (bf16)x[1], (bf16)x[2], (bf16)x[3]};
        }
      }
    }
  };

  load(NT - 1);
  for (int n = NT - 1; n >= 0; --n) {
    const int t0 = n * kC;
    // chunk-local inclusive cumsum of the gate (wave 0), padded tokens add 0
    if (wave == 0) {
      float x = t0 + lane < T ? rg : 0.f;
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const float y = __shfl_up(x, off, 64);
        if (lane >= off) x += y;
      }
      gam[lane] = x;
    }
    // dh to LDS (the B operand of K dh): rows 32w + 16a + 4lq + e, column 16ct + li
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
      for (int ct = 0; ct < 2; ++ct)
#pragma unroll
        for (int e = 0; e < 4; ++e) sdh[(32 * wave + 16 * a + 4 * lq + e) * kSV + 16 * ct + li] = dh[a][ct][e];
    __syncthreads();
    const float gl = gam[kC - 1];
    // stage the tiles: K as is, Q as scale e^gamma q, W negated
#pragma unroll
    for (int i = 0; i < kItK; ++i) {
      const int pc = tid + 256 * i, t = pc / kPK, j = pc % kPK;
      float xk[E], xq[E], xw[E];
      to_f32<TIn>(rk[i], xk);
      to_f32<TIn>(rq[i], xq);
      to_f32<TIn>(rw[i], xw);
      const float live = t0 + t < T ? 1.f : 0.f;
      const float fq = live * p.scale * __expf(gam[t]);
#pragma unroll
      for (int e = 0; e < E; ++e) {
        xk[e] *= live;
        xw[e] *= live;
      }
#pragma unroll
      for (int e = 0; e < E; e += 4) {
        *reinterpret_cast<f32x4*>(&sk[t * kSK + j * E + e]) = f32x4{xk[e], xk[e + 1], xk[e + 2], xk[e + 3]};
        *reinterpret_cast<f32x4*>(&sq[t * kSQ + j * E + e]) =
            f32x4{fq * xq[e], fq * xq[e + 1], fq * xq[e + 2], fq * xq[e + 3]};
        *reinterpret_cast<f32x4*>(&sw[t * kSQ + j * E + e]) = f32x4{-xw[e], -xw[e + 1], -xw[e + 2], -xw[e + 3]};
      }
    }
#pragma unroll
    for (int i = 0; i < kItV; ++i) {
      const int pc = tid + 256 * i, t = pc / kPV, j = pc % kPV;
      float x[E];
      to_f32<TIn>(rdo[i], x);
      const float live = t0 + t < T ? 1.f : 0.f;
#pragma unroll
      for (int e = 0; e < E; ++e) x[e] *= live;
#pragma unroll
      for (int e = 0; e < E; e += 4)
        *reinterpret_cast<f32x4*>(&sdo[t * kSV + j * E + e]) = f32x4{x[e], x[e + 1], x[e + 2], x[e + 3]};
    }
    float dvc[2][4];
#pragma unroll
    for (int ct = 0; ct < 2; ++ct)
#pragma unroll
      for (int e = 0; e < 4; ++e) dvc[ct][e] = t0 + 16 * wave + 4 * lq + e < T ? (float)rdv[ct][e] : 0.f;
    __syncthreads();
    if (n > 0) load(n - 1);  // registers are free again
    // The previous chunk's results leave now, from LDS, so that their stores are in flight
    // during this chunk's products rather than in front of the next wait for loads (on this
    // GPU the wait counts stores too): dh (in sdh since the top of this step) and dv2.
    if (n + 1 < NT) {
      store_dv2(n + 1);
      if (p.dh_chunks) {
        float* dst = p.dh_chunks + ((long)bh * NT + n + 1) * K * p.V + v0;
#pragma unroll
        for (int i = 0; i < K * 8 / 256; ++i) {
          const int pc = tid + 256 * i, r = pc / 8, c4 = pc % 8;
          *reinterpret_cast<f32x4*>(dst + (long)r * p.V + 4 * c4) = *reinterpret_cast<const f32x4*>(&sdh[r * kSV + 4 * c4]);
        }
      }
    }
    // dv2 = dv + e^{gamma_L - gamma} (K dh): wave w takes tokens 16w .. 16w + 15
    // (two accumulator sets over even and odd steps, so consecutive products are independent)
    f32x4 acc[2], acc2[2];
#pragma unroll
    for (int ct = 0; ct < 2; ++ct) acc[ct] = acc2[ct] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll 4
    for (int ks = 0; ks < K / 4; ks += 2) {
      const float a0 = sk[(16 * wave + li) * kSK + 4 * ks + lq];
      const float a1 = sk[(16 * wave + li) * kSK + 4 * ks + 4 + lq];
#pragma unroll
      for (int ct = 0; ct < 2; ++ct) {
        acc[ct] = mma4(a0, sdh[(4 * ks + lq) * kSV + 16 * ct + li], acc[ct]);
        acc2[ct] = mma4(a1, sdh[(4 * ks + 4 + lq) * kSV + 16 * ct + li], acc2[ct]);
      }
    }
#pragma unroll
    for (int ct = 0; ct < 2; ++ct) acc[ct] += acc2[ct];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int t = 16 * wave + 4 * lq + e;
      const float f = __expf(gl - gam[t]);
#pragma unroll
      for (int ct = 0; ct < 2; ++ct) {
        sdv[t * kSV + 16 * ct + li] = dvc[ct][e] + f * acc[ct][e];
      }
    }
    __syncthreads();
    // dh <- e^{gamma_L} dh + (scale e^gamma Q)^T do + (-W)^T dv2: wave w takes rows 32w .. +31
    const float el = __expf(gl);
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
      for (int ct = 0; ct < 2; ++ct)
#pragma unroll
        for (int e = 0; e < 4; ++e) dh[a][ct][e] *= el;
    // the W^T dv2 products go to a second accumulator set (independent of the Q^T do ones)
    f32x4 dw[2][2];
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
      for (int ct = 0; ct < 2; ++ct) dw[a][ct] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll 4
    for (int ks = 0; ks < kC / 4; ++ks) {
      const int t = 4 * ks + lq;
      float aq[2], aw[2], bo[2], bv[2];
#pragma unroll
      for (int a = 0; a < 2; ++a) {
        aq[a] = sq[t * kSQ + 32 * wave + 16 * a + li];
        aw[a] = sw[t * kSQ + 32 * wave + 16 * a + li];
      }
#pragma unroll
      for (int ct = 0; ct < 2; ++ct) {
        bo[ct] = sdo[t * kSV + 16 * ct + li];
        bv[ct] = sdv[t * kSV + 16 * ct + li];
      }
#pragma unroll
      for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int ct = 0; ct < 2; ++ct) dh[a][ct] = mma4(aq[a], bo[ct], dh[a][ct]);
#pragma unroll
      for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int ct = 0; ct < 2; ++ct) dw[a][ct] = mma4(aw[a], bv[ct], dw[a][ct]);
    }
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
      for (int ct = 0; ct < 2; ++ct) dh[a][ct] += dw[a][ct];
    __syncthreads();  // the tiles are rewritten by the next chunk
  }
  // the last chunk's results: dv2 from LDS, dh from the accumulators
  store_dv2(0);
  if (p.dh_chunks) {
    float* dst = p.dh_chunks + (long)bh * NT * K * p.V + v0;
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
      for (int ct = 0; ct < 2; ++ct)
#pragma unroll
        for (int e = 0; e < 4; ++e) dst[(long)(32 * wave + 16 * a + 4 * lq + e) * p.V + 16 * ct + li] = dh[a][ct][e];
  }
  if (p.dh0) {
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
      for (int ct = 0; ct < 2; ++ct)
#pragma unroll
        for (int e = 0; e < 4; ++e)
          p.dh0[((long)bh * K + 32 * wave + 16 * a + 4 * lq + e) * p.V + v0 + 16 * ct + li] = dh[a][ct][e];
  }
}

}  // namespace

hipError_t launch_dhu(const DhuParams& p, int dtype, hipStream_t stream) {
  const dim3 grid(p.B * p.H * (p.V / 32));
  if (dtype == 0)
    hipLaunchKernelGGL((dhu_kernel<128, float>), grid, dim3(256), 0, stream, p);
  else
    hipLaunchKernelGGL((dhu_kernel<128, bf16>), grid, dim3(256), 0, stream, p);
  return hipGetLastError();
}

}  // namespace gdn

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
// One workgroup of eight waves per (chain, 32-column block of dh): four row groups of 32 rows
// times two 16-column halves.  dh lives in registers as
// matrix-core accumulators (fp32) and is copied to LDS once per chunk for K dh.  Products
// use fp32 matrix-core steps (16x16x4), so fp32 inputs keep fp32 accuracy.  A chunk's K, Q,
// W, do rows and dv entries are loaded one chunk ahead into registers; the tiles sit in LDS
// in their natural [token][channel] layout with row strides chosen so every operand read of
// a wave falls in distinct banks.
#include "gdn_device.h"
#include "gdn_frame.h"
#include "gdn_internal.h"

namespace gdn {

namespace {

constexpr int kC = 64;                 // chunk length
constexpr int kSK = 132, kSQ = 144;    // row strides (floats) of the K and Q / W tiles
constexpr int kSV = 48;                // row stride of the do, dv2 and dh tiles
constexpr int kThreads = 512;          // eight waves: four row groups x two column halves

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
__global__ __launch_bounds__(kThreads) void dhu_kernel(const DhuParams p) {
  constexpr int E = 16 / sizeof(TIn);     // elements per 16-byte piece
  constexpr int kPK = K / E;              // pieces per K row
  constexpr int kItK = kC * kPK / kThreads;  // pieces per thread of a K / Q / W tile
  constexpr int kPV = 32 / E;             // pieces per 32-column do row
  constexpr int kNV = kC * kPV;           // pieces of the do tile (256 or 512)
  __shared__ __attribute__((aligned(16))) float sk[kC * kSK];
  __shared__ __attribute__((aligned(16))) float sq[kC * kSQ];
  __shared__ __attribute__((aligned(16))) float sw[kC * kSQ];
  __shared__ __attribute__((aligned(16))) float sdo[kC * kSV];
  __shared__ __attribute__((aligned(16))) float sdv[kC * kSV];
  __shared__ __attribute__((aligned(16))) float sdh[K * kSV];
  __shared__ float gam[kC];
  static_assert(kItK * kThreads == kC * kPK && kNV <= kThreads, "tile pieces");
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
  const int h = bh % p.H;
  // the chain's first token, length and first dh_chunks slot (dense, or a packed sequence)
  long tb;
  int T;
  long dhc0;
  if (p.cu) {
    const int sq = bh / p.H, c0 = p.coffs[sq];
    tb = p.cu[sq];
    T = p.cu[sq + 1] - p.cu[sq];
    dhc0 = (long)h * p.nt_total + c0;
  } else {
    tb = (long)(bh / p.H) * p.T;
    T = p.T;
    dhc0 = (long)bh * ((p.T + kC - 1) / kC);
  }
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wr = wave & 3, wc = wave >> 2;  // row group and 16-column half of this wave
  const int li = lane & 15, lq = lane >> 4;
  const int NT = (T + kC - 1) / kC;
  const TIn* q = static_cast<const TIn*>(p.q);
  const TIn* k = static_cast<const TIn*>(p.k);
  const TIn* w = static_cast<const TIn*>(p.w);
  const TIn* dO = static_cast<const TIn*>(p.do_);
  const TIn* dV = static_cast<const TIn*>(p.dv);
  const long HK = (long)p.H * K, HV = (long)p.H * p.V;
  const int v0 = 32 * vb, col = 16 * wc + li;  // this lane's dh / dv2 column in the block
  auto row = [&](int a, int e) { return 32 * wr + 16 * a + 4 * lq + e; };
  // dh: wave (wr, wc) holds rows 32wr + 16a + 4lq + e of column 16wc + li
  f32x4 dh[2];
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int e = 0; e < 4; ++e)
      dh[a][e] = p.dht ? p.dht[((long)bh * K + row(a, e)) * p.V + v0 + col] : 0.f;

  // The next chunk's inputs, loaded a chunk ahead.  Every load is unconditional, from the
  // token clamped to T - 1, and rows past T are zeroed where they are used: a load under a
  // branch makes the compiler wait for all outstanding memory right after it, which would
  // also wait for the prefetch itself.
  uint4 rk[kItK], rq[kItK], rw[kItK], rdo;
  TIn rdv[4];
  float rg = 0.f;
  auto tok = [&](int t) { return t < T ? t : T - 1; };
  auto load = [&](int n) {
    const int t0 = n * kC;
#pragma unroll
    for (int i = 0; i < kItK; ++i) {
      const int pc = tid + kThreads * i, t = pc / kPK, j = pc % kPK;
      const long o = (tb + tok(t0 + t)) * HK + (long)h * K + j * E;
      rk[i] = *reinterpret_cast<const uint4*>(k + o);
      rq[i] = *reinterpret_cast<const uint4*>(q + o);
      rw[i] = *reinterpret_cast<const uint4*>(w + o);
    }
    {
      const int pc = tid < kNV ? tid : 0, t = pc / kPV, j = pc % kPV;
      rdo = *reinterpret_cast<const uint4*>(dO + (tb + tok(t0 + t)) * HV + (long)h * p.V + v0 + j * E);
    }
    // dv in the accumulator layout of the K dh product: tokens 16wr + 4lq + e, column col
#pragma unroll
    for (int e = 0; e < 4; ++e)
      rdv[e] = dV[(tb + tok(t0 + 16 * wr + 4 * lq + e)) * HV + (long)h * p.V + v0 + col];
    if (p.g && tid < kC) rg = p.g[(tb + tok(t0 + tid)) * p.H + h];
  };
  // dv2 of chunk m from its LDS tile: wave (wr, wc) stores the 16 x 16 block it writes
  auto store_dv2 = [&](int m) {
    const int r = lane >> 2, c4 = lane & 3, t = 16 * wr + r;
    if (m * kC + t < T) {
      const f32x4 x = *reinterpret_cast<const f32x4*>(&sdv[t * kSV + 16 * wc + 4 * c4]);
      TIn* o = static_cast<TIn*>(p.dv2) + (tb + m * kC + t) * HV + (long)h * p.V + v0 + 16 * wc + 4 * c4;
      if constexpr (sizeof(TIn) == 4) {
        *reinterpret_cast<f32x4*>(o) = x;
      } else {
        typedef bf16 bf16x4_t __attribute__((ext_vector_type(4)));
        *reinterpret_cast<bf16x4_t*>(o) = bf16x4_t{(bf16)x[0], (bf16)x[1], (bf16)x[2], (bf16)x[3]};
      }
    }
  };

  load(NT - 1);
  for (int n = NT - 1; n >= 0; --n) {
    const int t0 = n * kC;
    // chunk-local inclusive cumsum of the gate (wave 0), padded tokens add 0
    if (wave == 0) {
      float x = t0 + lane < T ? floor_gate(rg) : 0.f;  // floored at use: rg is a prefetch
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const float y = __shfl_up(x, off, 64);
        if (lane >= off) x += y;
      }
      gam[lane] = x;
    }
    // dh to LDS (the B operand of K dh)
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
      for (int e = 0; e < 4; ++e) sdh[row(a, e) * kSV + col] = dh[a][e];
    __syncthreads();
    const float gl = gam[kC - 1];
    // stage the tiles: K as is, Q as scale e^gamma q, W negated
#pragma unroll
    for (int i = 0; i < kItK; ++i) {
      const int pc = tid + kThreads * i, t = pc / kPK, j = pc % kPK;
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
    if (tid < kNV) {
      const int t = tid / kPV, j = tid % kPV;
      float x[E];
      to_f32<TIn>(rdo, x);
      const float live = t0 + t < T ? 1.f : 0.f;
#pragma unroll
      for (int e = 0; e < E; e += 4)
        *reinterpret_cast<f32x4*>(&sdo[t * kSV + j * E + e]) =
            f32x4{live * x[e], live * x[e + 1], live * x[e + 2], live * x[e + 3]};
    }
    float dvc[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) dvc[e] = t0 + 16 * wr + 4 * lq + e < T ? (float)rdv[e] : 0.f;
    __syncthreads();
    if (n > 0) load(n - 1);  // registers are free again
    // The previous chunk's results leave now, from LDS, so that their stores are in flight
    // during this chunk's products rather than in front of the next wait for loads (on this
    // GPU the wait counts stores too): dh (in sdh since the top of this step) and dv2.
    if (n + 1 < NT) {
      store_dv2(n + 1);
      if (p.dh_chunks) {
        float* dst = p.dh_chunks + (dhc0 + n + 1) * K * p.V + v0;
#pragma unroll
        for (int i = 0; i < K * 8 / kThreads; ++i) {
          const int pc = tid + kThreads * i, r = pc / 8, c4 = pc % 8;
          *reinterpret_cast<f32x4*>(dst + (long)r * p.V + 4 * c4) = *reinterpret_cast<const f32x4*>(&sdh[r * kSV + 4 * c4]);
        }
      }
    }
    // dv2 = dv + e^{gamma_L - gamma} (K dh): wave (wr, wc) takes tokens 16wr .. 16wr + 15 of
    // column half wc (two accumulators over even and odd steps, for independent products)
    f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f}, acc2 = acc;
#pragma unroll 4
    for (int ks = 0; ks < K / 4; ks += 2) {
      acc = mma4(sk[(16 * wr + li) * kSK + 4 * ks + lq], sdh[(4 * ks + lq) * kSV + col], acc);
      acc2 = mma4(sk[(16 * wr + li) * kSK + 4 * ks + 4 + lq], sdh[(4 * ks + 4 + lq) * kSV + col], acc2);
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int t = 16 * wr + 4 * lq + e;
      sdv[t * kSV + col] = dvc[e] + __expf(gl - gam[t]) * (acc[e] + acc2[e]);
    }
    __syncthreads();
    // dh <- e^{gamma_L} dh + (scale e^gamma Q)^T do + (-W)^T dv2: rows 32wr .. 32wr + 31
    const float el = __expf(gl);
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
      for (int e = 0; e < 4; ++e) dh[a][e] *= el;
    // the W^T dv2 products go to a second accumulator pair (independent of the Q^T do ones)
    f32x4 dw[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
#pragma unroll 4
    for (int ks = 0; ks < kC / 4; ++ks) {
      const int t = 4 * ks + lq;
      const float bo = sdo[t * kSV + col], bv = sdv[t * kSV + col];
#pragma unroll
      for (int a = 0; a < 2; ++a) {
        dh[a] = mma4(sq[t * kSQ + 32 * wr + 16 * a + li], bo, dh[a]);
        dw[a] = mma4(sw[t * kSQ + 32 * wr + 16 * a + li], bv, dw[a]);
      }
    }
#pragma unroll
    for (int a = 0; a < 2; ++a) dh[a] += dw[a];
    __syncthreads();  // the tiles are rewritten by the next chunk
  }
  // the last chunk's results: dv2 from LDS, dh from the accumulators
  store_dv2(0);
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      if (p.dh_chunks) p.dh_chunks[(dhc0 * K + row(a, e)) * p.V + v0 + col] = dh[a][e];
      if (p.dh0) p.dh0[((long)bh * K + row(a, e)) * p.V + v0 + col] = dh[a][e];
    }
}

// The bf16 form: the same pass with fp16 matrix-core operands (16x16x32).  bf16 inputs are
// exact in fp16 (within its range); dh and dv2 are rounded to fp16 as operands, with fp32
// accumulation and an fp32 dh, at the precision of the bf16 forward.  Tiles are fp16:
// K [token][channel] read by rows (K dh contracts over channels), Q, W, do and dv2
// [token][column] read transposed (ds_read_b64_tr_b16) where the products contract over
// tokens; dh goes to LDS twice, fp32 for the output and fp16 transposed as an operand.
//
// kGK (per-key gates): gamma_{t,d} = cumsum of g_t + gk_{t,d}.  Each thread takes one key and
// a quarter of the chunk's tokens, sums its quarter in registers, and the quarters are joined
// through LDS into a [token][key] tile of the per-key part; the decay factors then go into the
// staged K (e^{gamma_L,d - gamma_{t,d}}) and Q (e^{gamma_{t,d}}) and into dh's rows.
template <int K, bool kGK>
__global__ __launch_bounds__(kThreads) void dhu16_kernel(const DhuParams p) {
  constexpr int E = 8, kPK = K / E, kItK = kC * kPK / kThreads, kPV = 32 / E, kNV = kC * kPV;
  constexpr int kRK = K + 8, kRQ = K + 16, kR32 = 36, kRT = K + 8;  // fp16 row strides
  __shared__ __attribute__((aligned(16))) f16 sk[kC * kRK];
  __shared__ __attribute__((aligned(16))) f16 sq[kC * kRQ];
  __shared__ __attribute__((aligned(16))) f16 sw[kC * kRQ];
  __shared__ __attribute__((aligned(16))) f16 sdo[kC * kR32];
  __shared__ __attribute__((aligned(16))) f16 sdv[kC * kR32];
  __shared__ __attribute__((aligned(16))) f16 dht16[32 * kRT];  // dh^T, [column][row]
  __shared__ __attribute__((aligned(16))) float sdv32[kC * kSV];
  __shared__ __attribute__((aligned(16))) float sdh[K * kSV];
  __shared__ float gam[kC];
  constexpr int kRG = K + 4;
  __shared__ __attribute__((aligned(16))) float sg[kGK ? kC * kRG : 4];  // per-key cumsum part
  __shared__ float gq[kGK ? 4 * K : 4];                                 // quarter totals
  static_assert(kItK * kThreads == kC * kPK && kNV <= kThreads, "tile pieces");
  static_assert(!kGK || kThreads == 4 * K, "one thread per (key, quarter of the chunk)");
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
  const int h = bh % p.H;
  // the chain's first token, length and first dh_chunks slot (dense, or a packed sequence)
  long tb;
  int T;
  long dhc0;
  if (p.cu) {
    const int sq = bh / p.H, c0 = p.coffs[sq];
    tb = p.cu[sq];
    T = p.cu[sq + 1] - p.cu[sq];
    dhc0 = (long)h * p.nt_total + c0;
  } else {
    tb = (long)(bh / p.H) * p.T;
    T = p.T;
    dhc0 = (long)bh * ((p.T + kC - 1) / kC);
  }
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wr = wave & 3, wc = wave >> 2;
  const int li = lane & 15, lq = lane >> 4, trj = li >> 2, trm = li & 3;
  const int NT = (T + kC - 1) / kC;
  const bf16* q = static_cast<const bf16*>(p.q);
  const bf16* k = static_cast<const bf16*>(p.k);
  const bf16* w = static_cast<const bf16*>(p.w);
  const bf16* dO = static_cast<const bf16*>(p.do_);
  const bf16* dV = static_cast<const bf16*>(p.dv);
  const long HK = (long)p.H * K, HV = (long)p.H * p.V;
  const int v0 = 32 * vb, col = 16 * wc + li;
  auto row = [&](int a, int e) { return 32 * wr + 16 * a + 4 * lq + e; };
  f32x4 dh[2];
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int e = 0; e < 4; ++e)
      dh[a][e] = p.dht ? p.dht[((long)bh * K + row(a, e)) * p.V + v0 + col] : 0.f;
  // next chunk's inputs (unconditional loads from clamped tokens; see dhu_kernel)
  uint4 rk[kItK], rq[kItK], rw[kItK], rdo;
  bf16 rdv[4];
  float rg = 0.f, rgk[kGK ? 16 : 1], rgt[kGK ? 16 : 1];
  // this thread's key and token quarter (kGK); the quarter is the same for a whole wave
  // (K = 128 threads per quarter), so its gate reads are wave-uniform
  const int gkd = tid % K, gkq = __builtin_amdgcn_readfirstlane(tid / K);
  auto tok = [&](int t) { return t < T ? t : T - 1; };
  auto load = [&](int n) {
    const int t0 = n * kC;
#pragma unroll
    for (int i = 0; i < kItK; ++i) {
      const int pc = tid + kThreads * i, t = pc / kPK, j = pc % kPK;
      const long o = (tb + tok(t0 + t)) * HK + (long)h * K + j * E;
      rk[i] = *reinterpret_cast<const uint4*>(k + o);
      rq[i] = *reinterpret_cast<const uint4*>(q + o);
      rw[i] = *reinterpret_cast<const uint4*>(w + o);
    }
    {
      const int pc = tid < kNV ? tid : 0, t = pc / kPV, j = pc % kPV;
      rdo = *reinterpret_cast<const uint4*>(dO + (tb + tok(t0 + t)) * HV + (long)h * p.V + v0 + j * E);
    }
#pragma unroll
    for (int e = 0; e < 4; ++e)
      rdv[e] = dV[(tb + tok(t0 + 16 * wr + 4 * lq + e)) * HV + (long)h * p.V + v0 + col];
    if (p.g && tid < kC) rg = p.g[(tb + tok(t0 + tid)) * p.H + h];
    if constexpr (kGK) {
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const long ti = tb + tok(t0 + 16 * gkq + i);
        rgt[i] = p.g ? p.g[ti * p.H + h] : 0.f;
        rgk[i] = p.gk[ti * HK + (long)h * K + gkd];
      }
    }
  };
  auto store_dv2 = [&](int m) {
    const int r = lane >> 2, c4 = lane & 3, t = 16 * wr + r;
    if (m * kC + t < T) {
      const f32x4 x = *reinterpret_cast<const f32x4*>(&sdv32[t * kSV + 16 * wc + 4 * c4]);
      typedef bf16 bf16x4_t __attribute__((ext_vector_type(4)));
      *reinterpret_cast<bf16x4_t*>(static_cast<bf16*>(p.dv2) + (tb + m * kC + t) * HV +
                                   (long)h * p.V + v0 + 16 * wc + 4 * c4) =
          bf16x4_t{(bf16)x[0], (bf16)x[1], (bf16)x[2], (bf16)x[3]};
    }
  };
  // 8 bf16 scaled into 8 fp16
  auto cvt = [](const uint4& raw, float f) {
    const bf16x8 v = __builtin_bit_cast(bf16x8, raw);
    f16x8 r;
#pragma unroll
    for (int j = 0; j < 8; ++j) r[j] = (f16)(f * (float)v[j]);
    return r;
  };

  load(NT - 1);
  for (int n = NT - 1; n >= 0; --n) {
    const int t0 = n * kC;
    if (wave == 0) {
      float x = t0 + lane < T ? floor_gate(rg) : 0.f;  // floored at use: rg is a prefetch
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const float y = __shfl_up(x, off, 64);
        if (lane >= off) x += y;
      }
      gam[lane] = x;
    }
    float cg[kGK ? 16 : 1];
    if constexpr (kGK) {  // this quarter's running sums of gk (tokens past T add 0)
      float x = 0.f;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        // gk' = max(g + gk, floor) - g (floors applied here, not at the prefetch loads), so
        // that the two cumulative sums add up to the floored per-key decay of the forward
        const float gt = floor_gate(rgt[i]);
        x += t0 + 16 * gkq + i < T ? floor_key_gate(gt + rgk[i]) - gt : 0.f;
        cg[i] = x;
      }
      gq[gkq * K + gkd] = x;
    }
    // dh to LDS: fp32 for the output, fp16 transposed as the B operand of K dh
#pragma unroll
    for (int a = 0; a < 2; ++a) {
      f16x4 hv;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        sdh[row(a, e) * kSV + col] = dh[a][e];
        hv[e] = (f16)dh[a][e];
      }
      *reinterpret_cast<f16x4*>(&dht16[col * kRT + row(a, 0)]) = hv;
    }
    __syncthreads();
    const float gl = gam[kC - 1];
    if constexpr (kGK) {
      float off = 0.f;
      for (int r = 0; r < gkq; ++r) off += gq[r * K + gkd];
#pragma unroll
      for (int i = 0; i < 16; ++i) sg[(16 * gkq + i) * kRG + gkd] = cg[i] + off;
      __syncthreads();
    }
#pragma unroll
    for (int i = 0; i < kItK; ++i) {
      const int pc = tid + kThreads * i, t = pc / kPK, j = pc % kPK;
      const float live = t0 + t < T ? 1.f : 0.f;
      if constexpr (kGK) {
        // K~ = k e^{gamma_L,d - gamma_{t,d}}, Q~ = scale q e^{gamma_{t,d}} (scalar and per-key parts)
        const bf16x8 kv = __builtin_bit_cast(bf16x8, rk[i]), qv = __builtin_bit_cast(bf16x8, rq[i]);
        f16x8 ko, qo;
#pragma unroll
        for (int e = 0; e < E; ++e) {
          const float gt = gam[t] + sg[t * kRG + j * E + e], gL = gl + sg[(kC - 1) * kRG + j * E + e];
          ko[e] = (f16)(live * __expf(gL - gt) * (float)kv[e]);
          qo[e] = (f16)(live * p.scale * __expf(gt) * (float)qv[e]);
        }
        *reinterpret_cast<f16x8*>(&sk[t * kRK + j * E]) = ko;
        *reinterpret_cast<f16x8*>(&sq[t * kRQ + j * E]) = qo;
      } else {
        *reinterpret_cast<f16x8*>(&sk[t * kRK + j * E]) = cvt(rk[i], live);
        *reinterpret_cast<f16x8*>(&sq[t * kRQ + j * E]) = cvt(rq[i], live * p.scale * __expf(gam[t]));
      }
      *reinterpret_cast<f16x8*>(&sw[t * kRQ + j * E]) = cvt(rw[i], -live);
    }
    if (tid < kNV) {
      const int t = tid / kPV, j = tid % kPV;
      // two 8-byte halves: the 72-byte rows keep only 8-byte alignment
      const f16x8 x = cvt(rdo, t0 + t < T ? 1.f : 0.f);
      *reinterpret_cast<f16x4*>(&sdo[t * kR32 + j * E]) = f16x4{x[0], x[1], x[2], x[3]};
      *reinterpret_cast<f16x4*>(&sdo[t * kR32 + j * E + 4]) = f16x4{x[4], x[5], x[6], x[7]};
    }
    float dvc[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) dvc[e] = t0 + 16 * wr + 4 * lq + e < T ? (float)rdv[e] : 0.f;
    __syncthreads();
    if (n > 0) load(n - 1);
    if (n + 1 < NT) {
      store_dv2(n + 1);
      if (p.dh_chunks) {
        float* dst = p.dh_chunks + (dhc0 + n + 1) * K * p.V + v0;
#pragma unroll
        for (int i = 0; i < K * 8 / kThreads; ++i) {
          const int pc = tid + kThreads * i, r = pc / 8, c4 = pc % 8;
          *reinterpret_cast<f32x4*>(dst + (long)r * p.V + 4 * c4) = *reinterpret_cast<const f32x4*>(&sdh[r * kSV + 4 * c4]);
        }
      }
    }
    // dv2 = dv + e^{gamma_L - gamma} (K dh): tokens 16wr .. 16wr + 15, column half wc
    f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kk = 0; kk < K / 32; ++kk)
      acc = mma16(lds8(&sk[(16 * wr + li) * kRK + 32 * kk + 8 * lq]),
                  lds8(&dht16[col * kRT + 32 * kk + 8 * lq]), acc);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int t = 16 * wr + 4 * lq + e;
      // (with per-key gates the factor is already inside the staged K)
      const float x = dvc[e] + (kGK ? 1.f : __expf(gl - gam[t])) * acc[e];
      sdv32[t * kSV + col] = x;
      sdv[t * kR32 + col] = (f16)x;
    }
    __syncthreads();
    // dh <- e^{gamma_L} dh + (scale e^gamma Q)^T do + (-W)^T dv2: rows 32wr .. 32wr + 31
    const float el = __expf(gl);
    f32x4 dw[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
      for (int e = 0; e < 4; ++e)
        dh[a][e] *= kGK ? __expf(gl + sg[(kC - 1) * kRG + row(a, e)]) : el;
#pragma unroll
    for (int kk = 0; kk < kC / 32; ++kk) {
      const int r0 = 32 * kk + 8 * lq + trj;
      const f16x8 bo = tr_pair(&sdo[r0 * kR32 + 16 * wc + 4 * trm], &sdo[(r0 + 4) * kR32 + 16 * wc + 4 * trm]);
      const f16x8 bv = tr_pair(&sdv[r0 * kR32 + 16 * wc + 4 * trm], &sdv[(r0 + 4) * kR32 + 16 * wc + 4 * trm]);
#pragma unroll
      for (int a = 0; a < 2; ++a) {
        const int c0 = 32 * wr + 16 * a + 4 * trm;
        dh[a] = mma16(tr_pair(&sq[r0 * kRQ + c0], &sq[(r0 + 4) * kRQ + c0]), bo, dh[a]);
        dw[a] = mma16(tr_pair(&sw[r0 * kRQ + c0], &sw[(r0 + 4) * kRQ + c0]), bv, dw[a]);
      }
    }
#pragma unroll
    for (int a = 0; a < 2; ++a) dh[a] += dw[a];
    __syncthreads();
  }
  store_dv2(0);
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      if (p.dh_chunks) p.dh_chunks[(dhc0 * K + row(a, e)) * p.V + v0 + col] = dh[a][e];
      if (p.dh0) p.dh0[((long)bh * K + row(a, e)) * p.V + v0 + col] = dh[a][e];
    }
}

}  // namespace

hipError_t launch_dhu(const DhuParams& p, int dtype, hipStream_t stream) {
  const dim3 grid(p.B * p.H * (p.V / 32));
  if (dtype == 0)
    hipLaunchKernelGGL((dhu_kernel<128, float>), grid, dim3(kThreads), 0, stream, p);
  else if (p.gk)
    hipLaunchKernelGGL((dhu16_kernel<128, true>), grid, dim3(kThreads), 0, stream, p);
  else
    hipLaunchKernelGGL((dhu16_kernel<128, false>), grid, dim3(kThreads), 0, stream, p);
  return hipGetLastError();
}

}  // namespace gdn

// gdn_summary.hip -- helpers of the fragment state summary (gdn_state_summary) and its
// application (gdn_state_apply), for running the fragments of a sequence separately
// (the context-parallel state summary of the MindSpore hyper-parallel page).
//
// A fragment's final state is affine in its initial state, ht(h0) = M h0 + ht(0), where M
// is the ordered product of the per-token maps A_t = (I - beta_t k_t k_t^T) diag(a_t),
// a_t = exp(g_t + gk_t).  ht(0) comes from the forward kernels.  M decays like the product
// of the a_t over the whole fragment, far below the range of the fp16 operands the chunked
// forward kernels use, so it has kernels of its own:
//  - scalar (or no) gate: the decay factors out of M, and the rest is the product of the
//    ungated chunk maps I - K^T W, formed on matrix cores with split bf16 operands (fp32
//    exponent range);
//  - per-key gate: the token recurrence on M in fp32, every column carrying a power-of-two
//    exponent that is renormalised once per 64 tokens (the map is linear and acts on each
//    column separately, so a column may be scaled at any point).
#include <algorithm>
#include <type_traits>

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
// With TR the map is h_out = M^T h_in + c (the gradient form): the staged rows are columns of M.
constexpr int kApplyRows = 16;
template <bool TR>
__global__ __launch_bounds__(256) void apply_kernel(const float* c, const float* M, const float* h_in,
                                                    float* h_out, int K, int V) {
  __shared__ float ms[kApplyRows][kApplyMaxK];
  const long bh = blockIdx.y;
  const int r0 = blockIdx.x * kApplyRows;
  const int rows = min(kApplyRows, K - r0);
  if (h_in) {
    if (TR) {
      for (int e = threadIdx.x; e < rows * K; e += 256)
        ms[e % rows][e / rows] = M[(bh * K + e / rows) * K + r0 + e % rows];
    } else {
      for (int e = threadIdx.x; e < rows * K; e += 256)
        ms[e / K][e % K] = M[(bh * K + r0 + e / K) * K + e % K];
    }
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

// Transition M with a per-key gate, as a token recurrence (one workgroup per (b, h, 32-column
// block of M)).  Lane layout: thread t owns columns cb*32 + 2(t/16) + {0, 1} and the K/16
// consecutive rows (t%16)(K/16) + j, so the 16 threads of a column pair are one DPP row and
// k^T M reduces with four DPP adds; two columns per thread give two independent dependency
// chains per token.  A chunk's keys, betas and decays are staged in LDS as fp32 first.
template <int K, typename TI>
__global__ __launch_bounds__(256) void transition_kernel(const TI* __restrict__ k,
                                                         const float* __restrict__ g,
                                                         const float* __restrict__ gk,
                                                         const float* __restrict__ beta,
                                                         float* __restrict__ M, int T, int H) {
  constexpr int kR = K / 16;  // rows per thread
  constexpr int kC = 64;      // tokens staged at a time
  __shared__ __attribute__((aligned(16))) float ks[kC][K];
  __shared__ __attribute__((aligned(16))) float as[kC][K];
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
  // a column is m * 2^ex, ex from renormalisation
  int ex[2] = {0, 0};
  // A chunk's inputs are loaded into registers while the previous chunk's tokens are
  // processed (16-byte pieces, all issued before any is used), then written to LDS.
  constexpr int kPer = 16 / sizeof(TI);                  // key elements per 16-byte piece
  constexpr int kKP = (kC * K / kPer + 255) / 256;       // key pieces per thread
  constexpr int kAP = (kC * K / 4 + 255) / 256;  // gk pieces per thread
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
    {
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
    {
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
        an[q] = *reinterpret_cast<const f32x4*>(&as[t][r0 + 4 * q]);
      }
      bn = bs[t];
    };
    fetch(0);
    for (int t = 0; t < n; ++t) {
      f32x4 kc[kR / 4], ac[kR / 4];
#pragma unroll
      for (int q = 0; q < kR / 4; ++q) {
        kc[q] = kn[q];
        ac[q] = an[q];
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
            m[u][j + e] *= ac[j / 4][e];
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
    const float sc = exp2f((float)ex[u]);
#pragma unroll
    for (int j = 0; j < kR; ++j) out[(long)(r0 + j) * K + c0 + u] = m[u][j] * sc;
  }
}

// ---- transition with a scalar (or no) gate: chunked form on matrix cores ----------------------
// A scalar decay a_t = e^{g_t} commutes with every rank-one map, so M = e^{sum_t g_t} Mt with
// Mt = prod_n (I - K_n^T W_n) over the 64-token chunks n in order, W_n = Tm diag(beta) K_n and
// Tm = (I + strict_lower(diag(beta) K_n K_n^T))^-1 (the WY form of an ungated chunk: its
// deltas are U - W S for the state S entering it).  trans_wy_kernel forms every chunk's W_n in
// parallel; trans_chain_kernel walks a chain's chunks for 32 columns of Mt.  Products take
// split bf16 operands (GDN_SPLIT; bf16 keys are exact, lo = 0).  With unit keys and beta in
// [0, 1] every factor has spectral norm <= 1.

typedef bf16 bf16x4 __attribute__((ext_vector_type(4)));

// Workgroup ids are dealt to the eight XCDs round-robin; with a grid that is a multiple of
// eight, logical neighbours (the column blocks of one chain) land on one XCD's L2.
__device__ __forceinline__ int xcd_logical(int bid, int n) {
  return n % 8 ? bid : (bid % 8) * (n / 8) + bid / 8;
}

// Slots c = bh * NT + n (one per chunk), dealt to the workgroups in turn; each workgroup loads
// its next slot's keys while it works on the current one.  Writes W_n = Tm diag(beta) K_n as a
// hi/lo bf16 pair ([64][K] in slot c of W) and K_n^T (bf16 [K][64] in slot c of Kt; fp32 keys
// also their lo halves); the lo halves sit `lo` elements after the hi halves.  The Gram K K^T on matrix cores gives A = diag(beta) times
// its strictly lower part; then block forward substitution over the four 16-row blocks i,
//   W_i = D_i (diag(beta) K_i - sum_{j<i} A_ij W_j),   D_i = (I + A_ii)^-1,
// with D_i from a 16-step substitution per column (fp32) and both products on matrix cores.
// Wave w owns the columns 16 CT w .. 16 CT (w + 1) - 1 of W throughout, so the block steps need
// no workgroup barrier.  Rows past the end of the sequence have k = 0 and beta = 0, so their W
// rows are zero.
template <int K, typename TI>
__global__ __launch_bounds__(256) void trans_wy_kernel(const TI* __restrict__ k,
                                                       const float* __restrict__ beta,
                                                       bf16* __restrict__ W, bf16* __restrict__ Kt,
                                                       size_t lo, int T, int H, int NT,
                                                       int nslots) {
  constexpr bool kSplit = !std::is_same<TI, bf16>::value;
  constexpr int kS = K + 8;   // bf16 row stride of the key tiles ([token][K])
  constexpr int kA = 68;      // float row stride of A
  constexpr int kX = 72;      // bf16 row stride of wt ([column][token])
  constexpr int CT = K / 64;  // 16-column tiles of W per wave
  constexpr int kKeyBytes = 2 * 64 * kS * 2, kWtBytes = 2 * K * kX * 2;
  __shared__ __attribute__((aligned(16))) unsigned char smem[kKeyBytes > kWtBytes ? kKeyBytes : kWtBytes];
  __shared__ __attribute__((aligned(16))) float gm[64 * kA];
  __shared__ __attribute__((aligned(16))) float dm[64 * 20];  // D_i rows, [i][16][20]
  __shared__ float bs[64];
  bf16* kh = reinterpret_cast<bf16*>(smem);
  bf16* kl = kh + 64 * kS;
  bf16* wh = reinterpret_cast<bf16*>(smem);  // W^T so far (hi/lo), once the keys are done
  bf16* wl = wh + K * kX;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, li = lane & 15, lq = lane >> 4;
  constexpr int NKP = 64 * K / 8 / 256;  // 8-key pieces of a chunk per thread
  typedef typename std::conditional<kSplit, f32x8, bf16x8>::type kvec;
  kvec kp[NKP];
  float bp = 0.f;
  // the keys and betas of slot c into registers (rows past the end of the sequence as zero)
  auto load = [&](int c) {
    const int n = c % NT, bh = c / NT, b = bh / H, h = bh % H, t0 = 64 * n, nt = min(64, T - t0);
#pragma unroll
    for (int j = 0; j < NKP; ++j) {
      const int e = tid + 256 * j, t = e / (K / 8), d = (e % (K / 8)) * 8;
      if (t < nt) {
        const TI* src = k + (((long)b * T + t0 + t) * H + h) * K + d;
        if constexpr (kSplit) {
          const f32x4 x0 = *reinterpret_cast<const f32x4*>(src), x1 = *reinterpret_cast<const f32x4*>(src + 4);
          kp[j] = __builtin_shufflevector(x0, x1, 0, 1, 2, 3, 4, 5, 6, 7);
        } else {
          kp[j] = *reinterpret_cast<const bf16x8*>(src);
        }
      } else {
        kp[j] = kvec{};
      }
    }
    if (tid < 64) bp = tid < nt ? beta[((long)b * T + t0 + tid) * H + h] : 0.f;
  };
  load(blockIdx.x);
  for (int slot = blockIdx.x; slot < nslots; slot += gridDim.x) {
    __syncthreads();  // the previous slot is done with every LDS array
#pragma unroll
    for (int j = 0; j < NKP; ++j) {
      const int e = tid + 256 * j, t = e / (K / 8), d = (e % (K / 8)) * 8;
      bf16x8 xh, xl;
#pragma unroll
      for (int jj = 0; jj < 8; ++jj) GDN_SPLIT((float)kp[j][jj], xh[jj], xl[jj]);
      *reinterpret_cast<bf16x8*>(&kh[t * kS + d]) = xh;
      *reinterpret_cast<bf16x8*>(&kl[t * kS + d]) = xl;
    }
    if (tid < 64) bs[tid] = bp;
    if (slot + (int)gridDim.x < nslots) load(slot + gridDim.x);
    __syncthreads();
    // Gram tiles (ti, tj), tj <= ti, of the 4 x 4 grid of 16 x 16 tiles: A = beta_r (k_r . k_s), s < r
    for (int q = wave; q < 10; q += 4) {
      int ti = 0;
      while (q >= (ti + 1) * (ti + 2) / 2) ++ti;
      const int tj = q - ti * (ti + 1) / 2;
      f32x4 c = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kk = 0; kk < K / 32; ++kk) {
        const bf16x8 ah = lds8(&kh[(16 * ti + li) * kS + 32 * kk + 8 * lq]);
        const bf16x8 bh_ = lds8(&kh[(16 * tj + li) * kS + 32 * kk + 8 * lq]);
        if constexpr (kSplit) {
          const bf16x8 al = lds8(&kl[(16 * ti + li) * kS + 32 * kk + 8 * lq]);
          const bf16x8 bl = lds8(&kl[(16 * tj + li) * kS + 32 * kk + 8 * lq]);
          c = mma3(ah, al, bh_, bl, c);
        } else {
          c = mma16(ah, bh_, c);
        }
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int r = 16 * ti + 4 * lq + e, sc = 16 * tj + li;
        gm[r * kA + sc] = sc < r ? bs[r] * c[e] : 0.f;
      }
    }
    // this lane's right-hand-side keys of the block steps: rows 16 i + 4 lq + e, its columns
    float kr[4][CT][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int c = 0; c < CT; ++c)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int o = (16 * i + 4 * lq + e) * kS + 16 * (CT * wave + c) + li;
          kr[i][c][e] = (float)kh[o] + (float)kl[o];
        }
    // K^T: lanes take consecutive keys i (conflict-free LDS reads), 8 tokens each
    {
      bf16* kt = Kt + (size_t)slot * K * 64;
      for (int e = tid; e < K * 8; e += 256) {
        const int i = e % K, g8 = 8 * (e / K);
        bf16x8 vh, vl;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          vh[j] = kh[(g8 + j) * kS + i];
          vl[j] = kl[(g8 + j) * kS + i];
        }
        *reinterpret_cast<bf16x8*>(&kt[(size_t)i * 64 + g8]) = vh;
        if constexpr (kSplit) *reinterpret_cast<bf16x8*>(&kt[lo + (size_t)i * 64 + g8]) = vl;
      }
    }
    __syncthreads();  // the Gram matrix is complete and the key tiles are no longer read
    for (int e = tid; e < kWtBytes / 16; e += 256) reinterpret_cast<uint4*>(smem)[e] = make_uint4(0u, 0u, 0u, 0u);
    if (tid < 64) {
      // column c of D_i = (I + A_ii)^-1: d_r = [r == c] - sum_{s<r} A_rs d_s (d_s = 0 for s < c)
      const int i = tid >> 4, c = tid & 15;
      float d[16];
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        float acc = r == c ? 1.f : 0.f;
#pragma unroll
        for (int sc = 0; sc < r; ++sc) acc = fmaf(-gm[(16 * i + r) * kA + 16 * i + sc], d[sc], acc);
        d[r] = acc;
      }
#pragma unroll
      for (int r = 0; r < 16; ++r) dm[(16 * i + r) * 20 + c] = d[r];
    }
    __syncthreads();
    bf16* wout = W + (size_t)slot * 64 * K;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      // R_i = diag(beta) K_i - sum_{j<i} A_ij W_j (contraction over the tokens s < 16 i)
      f32x4 C[CT];
#pragma unroll
      for (int c = 0; c < CT; ++c) C[c] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < (16 * i + 31) / 32; ++ks) {
        float a[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const int sc = 32 * ks + 8 * lq + j;
          a[j] = sc < 16 * i ? gm[(16 * i + li) * kA + sc] : 0.f;
        }
        bf16x8 ah, al;
#pragma unroll
        for (int j = 0; j < 8; ++j) GDN_SPLIT(a[j], ah[j], al[j]);
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
        for (int e = 0; e < 4; ++e) {
          GDN_SPLIT(bs[16 * i + 4 * lq + e] * kr[i][c][e] - C[c][e], xh[e], xl[e]);
        }
        *reinterpret_cast<bf16x4*>(&wh[col * kX + 16 * i + 4 * lq]) = xh;
        *reinterpret_cast<bf16x4*>(&wl[col * kX + 16 * i + 4 * lq]) = xl;
      }
      // W_i = D_i R_i: D_i sits at positions 16 (i % 2) .. of the 32 tokens 32 (i / 2) ..
      {
        float a[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const int kk = 8 * lq + j - 16 * (i % 2);
          a[j] = (kk >= 0 && kk < 16) ? dm[(16 * i + li) * 20 + (kk & 15)] : 0.f;
        }
        bf16x8 ah, al;
#pragma unroll
        for (int j = 0; j < 8; ++j) GDN_SPLIT(a[j], ah[j], al[j]);
#pragma unroll
        for (int c = 0; c < CT; ++c) {
          const int col = 16 * (CT * wave + c) + li;
          const int o = col * kX + 32 * (i / 2) + 8 * lq;
          const f32x4 wi = mma3(ah, al, lds8(&wh[o]), lds8(&wl[o]), f32x4{0.f, 0.f, 0.f, 0.f});
          bf16x4 xh, xl;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            GDN_SPLIT(wi[e], xh[e], xl[e]);
            wout[(size_t)(16 * i + 4 * lq + e) * K + col] = xh[e];
            wout[lo + (size_t)(16 * i + 4 * lq + e) * K + col] = xl[e];
          }
          *reinterpret_cast<bf16x4*>(&wh[col * kX + 16 * i + 4 * lq]) = xh;
          *reinterpret_cast<bf16x4*>(&wl[col * kX + 16 * i + 4 * lq]) = xl;
        }
      }
    }
  }
}

// One workgroup per (b, h, 32 columns of Mt); wave w owns rows 16 RT w .. 16 RT (w + 1) - 1 of
// the column block in fp32 registers.  Per chunk: X = W_n Mt (wave w: tokens 16 w .. 16 w + 15;
// W rows' hi/lo pairs from memory as A operands; Mt^T's hi/lo pair in LDS), -X into LDS as
// [column][token] pairs, then Mt += K_n^T (-X) with K_n^T rows from memory as A operands.  The
// operands of chunk n + 2 are loaded while chunk n is processed.  At the end M = e^{sum g} Mt.
template <int K, typename TI>
__global__ __launch_bounds__(256) void trans_chain_kernel(const float* __restrict__ g,
                                                          const bf16* __restrict__ W,
                                                          const bf16* __restrict__ Kt,
                                                          size_t lo, float* __restrict__ M,
                                                          int T, int H, int NT) {
  constexpr bool kSplit = !std::is_same<TI, bf16>::value;
  constexpr int RT = K / 64;  // 16-row tiles of Mt per wave
  constexpr int kM = K + 8;   // bf16 row stride of ms ([32 columns][K])
  constexpr int kX = 72;      // bf16 row stride of xs ([32 columns][64 tokens])
  __shared__ __attribute__((aligned(16))) bf16 ms[2][32 * kM];
  __shared__ __attribute__((aligned(16))) bf16 xs[2][32 * kX];
  __shared__ float red[4];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, li = lane & 15, lq = lane >> 4;
  constexpr int ncb = K / 32;
  const int lg = xcd_logical(blockIdx.x, gridDim.x);
  const int cb = lg % ncb;
  const long bh = lg / ncb;
  const int b = (int)(bh / H), h = (int)(bh % H);

  float gsum = 0.f;
  if (g)
    for (int t = tid; t < T; t += 256) gsum += g[((long)b * T + t) * H + h];
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) gsum += __shfl_xor(gsum, off, 64);
  if (lane == 0) red[w] = gsum;

  f32x4 m[RT][2];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt)
#pragma unroll
    for (int c = 0; c < 2; ++c)
#pragma unroll
      for (int e = 0; e < 4; ++e)
        m[rt][c][e] = (16 * (RT * w + rt) + 4 * lq + e == 32 * cb + 16 * c + li) ? 1.f : 0.f;
  auto write_ms = [&]() {
#pragma unroll
    for (int rt = 0; rt < RT; ++rt)
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        bf16x4 xh, xl;
#pragma unroll
        for (int e = 0; e < 4; ++e) GDN_SPLIT(m[rt][c][e], xh[e], xl[e]);
        const int o = (16 * c + li) * kM + 16 * (RT * w + rt) + 4 * lq;
        *reinterpret_cast<bf16x4*>(&ms[0][o]) = xh;
        *reinterpret_cast<bf16x4*>(&ms[1][o]) = xl;
      }
  };
  struct Ahead {
    bf16x8 wh[K / 32], wl[K / 32];             // W row 16 w + li, 8 columns per k-step
    bf16x8 kh[RT][2], kl[kSplit ? RT : 1][2];  // K^T rows, 8 consecutive tokens per k-step
  };
  auto load = [&](int n, Ahead& a) {
    const bf16* wb = W + (((size_t)bh * NT + n) * 64 + 16 * w + li) * K + 8 * lq;
#pragma unroll
    for (int kk = 0; kk < K / 32; ++kk) {
      a.wh[kk] = *reinterpret_cast<const bf16x8*>(wb + 32 * kk);
      a.wl[kk] = *reinterpret_cast<const bf16x8*>(wb + lo + 32 * kk);
    }
    const bf16* kb = Kt + ((size_t)bh * NT + n) * K * 64;
#pragma unroll
    for (int rt = 0; rt < RT; ++rt)
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        const size_t o = (size_t)(16 * (RT * w + rt) + li) * 64 + 32 * ks + 8 * lq;
        a.kh[rt][ks] = *reinterpret_cast<const bf16x8*>(kb + o);
        if constexpr (kSplit) a.kl[rt][ks] = *reinterpret_cast<const bf16x8*>(kb + lo + o);
      }
  };
  auto step = [&](int n, Ahead& cur) {
    f32x4 X[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
#pragma unroll
    for (int kk = 0; kk < K / 32; ++kk)
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        const int o = (16 * c + li) * kM + 32 * kk + 8 * lq;
        X[c] = mma3(cur.wh[kk], cur.wl[kk], lds8(&ms[0][o]), lds8(&ms[1][o]), X[c]);
      }
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      bf16x4 xh, xl;
#pragma unroll
      for (int e = 0; e < 4; ++e) GDN_SPLIT(-X[c][e], xh[e], xl[e]);
      const int o = (16 * c + li) * kX + 16 * w + 4 * lq;
      *reinterpret_cast<bf16x4*>(&xs[0][o]) = xh;
      *reinterpret_cast<bf16x4*>(&xs[1][o]) = xl;
    }
    __syncthreads();  // xs written; every wave is done reading ms
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        const int ob = (16 * c + li) * kX + 32 * ks + 8 * lq;
        const bf16x8 bh_ = lds8(&xs[0][ob]), bl = lds8(&xs[1][ob]);
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) {
          if constexpr (kSplit) {
            m[rt][c] = mma3(cur.kh[rt][ks], cur.kl[rt][ks], bh_, bl, m[rt][c]);
          } else {
            m[rt][c] = mma16(cur.kh[rt][ks], bl, m[rt][c]);
            m[rt][c] = mma16(cur.kh[rt][ks], bh_, m[rt][c]);
          }
        }
      }
    if (n + 2 < NT) load(n + 2, cur);
    write_ms();
    __syncthreads();  // every wave is done reading xs; ms holds the new Mt
  };

  Ahead A0, A1;
  write_ms();
  load(0, A0);
  if (NT > 1) load(1, A1);
  __syncthreads();
  for (int n = 0; n < NT; n += 2) {
    step(n, A0);
    if (n + 1 < NT) step(n + 1, A1);
  }
  const float sc = __expf((red[0] + red[1]) + (red[2] + red[3]));
  float* out = M + (size_t)bh * K * K;
#pragma unroll
  for (int rt = 0; rt < RT; ++rt)
#pragma unroll
    for (int c = 0; c < 2; ++c)
#pragma unroll
      for (int e = 0; e < 4; ++e)
        out[(size_t)(16 * (RT * w + rt) + 4 * lq + e) * K + 32 * cb + 16 * c + li] = m[rt][c][e] * sc;
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
                             float* M, int B, int T, int H, int K, int dtype, void* wy,
                             hipStream_t stream) {
  const bool pk = gk != nullptr;
  if (!pk) {
    // scalar (or no) gate: W and K^T of every chunk, then the chain on matrix cores
    const int NT = (T + 63) / 64;
    const int slots = B * H * NT;
    const size_t lo = (size_t)slots * 64 * K;
    bf16* w = static_cast<bf16*>(wy);
    bf16* kt = w + 2 * lo;
    const int wy_grid = slots < 512 ? slots : 512;  // two resident workgroups per CU
#define GDN_CHAIN(KK, TT)                                                                             \
  do {                                                                                                \
    hipLaunchKernelGGL((trans_wy_kernel<KK, TT>), dim3(wy_grid), dim3(256), 0, stream,                \
                       static_cast<const TT*>(k), beta, w, kt, lo, T, H, NT, slots);                  \
    hipLaunchKernelGGL((trans_chain_kernel<KK, TT>), dim3(B * H * (KK / 32)), dim3(256), 0, stream,   \
                       g, w, kt, lo, M, T, H, NT);                                                    \
  } while (0)
    if (dtype == 1) {
      if (K == 128) GDN_CHAIN(128, bf16); else GDN_CHAIN(64, bf16);
    } else {
      if (K == 128) GDN_CHAIN(128, float); else GDN_CHAIN(64, float);
    }
#undef GDN_CHAIN
    return hipGetLastError();
  }
  const dim3 grid(B * H * (K / 32)), blk(256);
#define GDN_TRANSITION(KK, TT) \
  hipLaunchKernelGGL((transition_kernel<KK, TT>), grid, blk, 0, stream, static_cast<const TT*>(k), g, gk, beta, M, T, H)
  if (dtype == 1) {
    if (K == 128) GDN_TRANSITION(128, bf16); else GDN_TRANSITION(64, bf16);
  } else {
    if (K == 128) GDN_TRANSITION(128, float); else GDN_TRANSITION(64, float);
  }
#undef GDN_TRANSITION
  return hipGetLastError();
}

// bytes launch_transition needs for a scalar gate (W as a hi/lo bf16 pair and K^T bf16, with its
// lo halves for fp32 keys, per chunk); none with a per-key gate
size_t transition_ws_bytes(int B, int T, int H, int K, int dtype, bool per_key) {
  const size_t elems = (size_t)B * H * ((T + 63) / 64) * 64 * K;
  return per_key ? 0 : elems * 4 + elems * (dtype == 1 ? 2 : 4);
}

hipError_t launch_apply(const float* c, const float* M, const float* h_in, float* h_out, int BH,
                        int K, int V, hipStream_t stream) {
  hipLaunchKernelGGL(apply_kernel<false>, dim3((K + kApplyRows - 1) / kApplyRows, BH), dim3(256), 0,
                     stream, c, M, h_in, h_out, K, V);
  return hipGetLastError();
}

hipError_t launch_grad_apply(const float* grad_ext, const float* M, const float* grad_in,
                             float* grad_out, int BH, int K, int V, hipStream_t stream) {
  hipLaunchKernelGGL(apply_kernel<true>, dim3((K + kApplyRows - 1) / kApplyRows, BH), dim3(256), 0,
                     stream, grad_ext, M, grad_in, grad_out, K, V);
  return hipGetLastError();
}

}  // namespace gdn

// gdn_cambwd.hip -- backward of the camera-branch frame scan for gfx950 (SANA fused_cam_gdn.py
// page, "Backward Triton kernel": _cam_scan_bwd_kernel; the forward is cam_scan in gdn_cam.hip).
//
// Forward, per (b, h), channel-major slabs q, k, v [D, S] of frame f, one direction: step `it`
// (it = 0 .. F-1) outputs frame f(it) (it, or F-1-it in reverse) and, before that, absorbs
// frame fa(it) (f(it), or f(it)+1 in reverse; the reverse scan absorbs nothing at it = 0):
//   S_pre = g S,  S <- S_pre - G S_pre + U,  out_s = S^T q_s  (s in frame f(it)),
//   G = K diag(beta) K^T, U = K diag(beta) V^T of the absorbed frame, g = decay[fa].
// Backward (gradients of L = sum(out * dout)), with A the gradient of the state after a
// step's update, A = W_f + g' (I - G') A' where W_f = Q_f dout_f^T and the primes denote the
// next step:
//   dq_s = S dout_s                                           (tokens of the output frame)
//   r_s = v_s - S_pre^T k_s,  dd_s = A^T k_s,  dv_s = beta_s dd_s,  dbeta_s = dd_s . r_s,
//   dk_s = A (beta_s r_s) + S_pre (-beta_s dd_s)                 (tokens of the absorbed frame)
//   ddecay[fa] = sum((I - G) A * S_prev)                      (S_prev: the state before the step)
// The decays of frames that are never absorbed (frame 0 of the reverse scan) and the one
// applied to the zero initial state get 0, and never-absorbed tokens get zero k, v, beta
// gradients.
//
// Kernels:
//   stats  per (b, h, frame, matrix): G, U, W (D x D fp32) with 16x16x32 bf16 matrix products;
//          a channel-major slab row is already in operand order (consecutive tokens of one
//          channel), so the slabs go to LDS 32 tokens at a time without a transpose.
//   scan   per (b, h, 32 state columns): the forward states and then A, in fp32 (16x16x4
//          fp32 matrix products, the state in LDS); every step's state and A leave as hi/lo
//          bf16 pairs in both orientations for the token kernel, the states also in fp32 for
//          the decay gradient, whose partial sums over the block's columns go to the workspace.
//   token  per (b, h, step, 64 tokens): the five products of the per-token gradients, the
//          token slabs transposed into LDS tiles that the four waves share; wave w forms
//          output rows D/4 w .. D/4 (w+1) - 1 for all 64 tokens.
// Precision: each product splits both fp32 operands into bf16 pairs x = hi + lo (hi = bf16(x),
// lo = bf16(x - hi)) and sums hi*hi + hi*lo + lo*hi in fp32, about 16 mantissa bits per
// operand.  The page's backward takes plain bf16 operands; their rounding alone moves the
// gradients by up to 4e-2 of their RMS on the small test shapes.
#include "gdn_bwd_params.h"
#include "gdn_device.h"
#include "gdn_internal.h"

namespace gdn {
namespace {

typedef bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef bf16 bf16x4 __attribute__((ext_vector_type(4)));

// ---- stats: G_f, U_f, W_f ----------------------------------------------------------------
// blockIdx.x = (bh * F + f) * 3 + which; four waves, wave w owns rows 16 RT w .. of the D x D
// result, all columns.  Per 32-token step the two slabs go to LDS as split pairs [channel][32
// tokens] (a slab row is already token-contiguous), shared by the four waves; the next
// step's rows are loaded into registers while the current step's products run.
template <int D>
__global__ __launch_bounds__(256) void cbwd_stats_kernel(const CamBwdParams p) {
  constexpr int RT = D / 64, CT = D / 16;  // row tiles per wave, column tiles
  constexpr int kX = 40;                   // bf16 row stride of the [channel][32] tiles
  constexpr int NI = D * 4 / 256;          // (channel, token octet) items per thread per slab
  __shared__ __attribute__((aligned(16))) bf16 xt[2][D * kX];
  __shared__ __attribute__((aligned(16))) bf16 yt[2][D * kX];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, li = lane & 15, lq = lane >> 4;
  const int bid = xcd_logical(blockIdx.x, gridDim.x);
  const int which = bid % 3;
  const long bf = bid / 3;
  const int f = (int)(bf % p.F);
  const long bh = bf / p.F;
  const long N = (long)p.F * p.S;
  const float* X = which == 2 ? p.q : p.k;
  const float* Y = which == 0 ? p.k : (which == 1 ? p.v : p.dout);
  const long base = bh * D * N + (long)f * p.S;
  const float* bt = p.beta + bh * N + (long)f * p.S;
  f32x4 acc[RT][CT];
#pragma unroll
  for (int r = 0; r < RT; ++r)
#pragma unroll
    for (int c = 0; c < CT; ++c) acc[r][c] = f32x4{0.f, 0.f, 0.f, 0.f};
  // item i of this thread: channel (tid + 256 i) / 4, tokens 8 ((tid + 256 i) % 4) ..
  f32x4 xr[NI][2], yr[NI][2], br[2];
  const int oc = tid % 4;  // token octet (the same for every item)
  auto load = [&](int t0) {
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const int ch = (tid + 256 * i) / 4;
      const float* xs = X + base + (long)ch * N + t0 + 8 * oc;
      const float* ys = Y + base + (long)ch * N + t0 + 8 * oc;
      xr[i][0] = *reinterpret_cast<const f32x4*>(xs);
      xr[i][1] = *reinterpret_cast<const f32x4*>(xs + 4);
      yr[i][0] = *reinterpret_cast<const f32x4*>(ys);
      yr[i][1] = *reinterpret_cast<const f32x4*>(ys + 4);
    }
    if (which != 2) {
      br[0] = *reinterpret_cast<const f32x4*>(bt + t0 + 8 * oc);
      br[1] = *reinterpret_cast<const f32x4*>(bt + t0 + 8 * oc + 4);
    } else {
      br[0] = br[1] = f32x4{1.f, 1.f, 1.f, 1.f};
    }
  };
  load(0);
  for (int t0 = 0; t0 < p.S; t0 += 32) {
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const int ch = (tid + 256 * i) / 4, o = ch * kX + 8 * oc;
      bf16x8 xh, xl, yh, yl;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        GDN_SPLIT(xr[i][j / 4][j % 4] * br[j / 4][j % 4], xh[j], xl[j]);
        GDN_SPLIT(yr[i][j / 4][j % 4], yh[j], yl[j]);
      }
      *reinterpret_cast<bf16x8*>(&xt[0][o]) = xh;
      *reinterpret_cast<bf16x8*>(&xt[1][o]) = xl;
      *reinterpret_cast<bf16x8*>(&yt[0][o]) = yh;
      *reinterpret_cast<bf16x8*>(&yt[1][o]) = yl;
    }
    __syncthreads();
    if (t0 + 32 < p.S) load(t0 + 32);
    bf16x8 ah[RT], al[RT];
#pragma unroll
    for (int r = 0; r < RT; ++r) {
      const int o = (16 * (RT * w + r) + li) * kX + 8 * lq;
      ah[r] = lds8(&xt[0][o]);
      al[r] = lds8(&xt[1][o]);
    }
#pragma unroll
    for (int c = 0; c < CT; ++c) {
      const int o = (16 * c + li) * kX + 8 * lq;
      const bf16x8 bh_ = lds8(&yt[0][o]), bl = lds8(&yt[1][o]);
#pragma unroll
      for (int r = 0; r < RT; ++r) acc[r][c] = mma3(ah[r], al[r], bh_, bl, acc[r][c]);
    }
    __syncthreads();
  }
  float* out = (which == 0 ? p.G : (which == 1 ? p.U : p.W)) + bf * D * D;
#pragma unroll
  for (int r = 0; r < RT; ++r)
#pragma unroll
    for (int c = 0; c < CT; ++c)
#pragma unroll
      for (int e = 0; e < 4; ++e) out[(16 * (RT * w + r) + 4 * lq + e) * D + 16 * c + li] = acc[r][c][e];
}

// ---- scan: forward states, then the state gradients ---------------------------------------
// blockIdx.x = bh * (D / 32) + column block.  st[col][row] holds the block's 32 columns of the
// state (then of A), transposed so that a lane's 8 consecutive rows are one 32-byte read.
template <int D>
__global__ __launch_bounds__(256) void cbwd_scan_kernel(const CamBwdParams p) {
  constexpr int RT = D / 64;  // row tiles per wave (16 rows each)
  constexpr int kS = D + 4;   // row stride of st (floats)
  __shared__ float st[32][kS];
  __shared__ float red[4];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, li = lane & 15, lq = lane >> 4;
  const int bid = xcd_logical(blockIdx.x, gridDim.x);
  const long bh = bid / (D / 32);
  const int c0 = 32 * (bid % (D / 32));
  const int F = p.F;
  const size_t DD = (size_t)D * D;
  for (int e = threadIdx.x; e < 32 * kS; e += 256) (&st[0][0])[e] = 0.f;
  __syncthreads();
  // T = M st (rows of this wave, the block's 32 columns) with M's A operands already in
  // registers: tile (r, c) holds rows 16 (RT w + r) + 4 lq + e, column 16 c + li
  constexpr int KK = D / 32;
  struct Ops {
    f32x8 a[RT][KK];     // rows 16 (RT w + r) + li of G, columns 32 kk + 8 lq ..
    float x[RT][2][4];   // U (forward) or W (backward) at this lane's elements
    float y[RT][2][4];   // the state before the step (backward)
    float g;
  };
  auto fetch_g = [&](const float* M, Ops& o) {
#pragma unroll
    for (int r = 0; r < RT; ++r)
#pragma unroll
      for (int kk = 0; kk < KK; ++kk) o.a[r][kk] = lds8(M + (16 * (RT * w + r) + li) * D + 32 * kk + 8 * lq);
  };
  auto fetch_el = [&](const float* M, float (&x)[RT][2][4]) {
#pragma unroll
    for (int r = 0; r < RT; ++r)
#pragma unroll
      for (int c = 0; c < 2; ++c)
#pragma unroll
        for (int e = 0; e < 4; ++e)
          x[r][c][e] = M ? M[(size_t)(16 * (RT * w + r) + 4 * lq + e) * D + c0 + 16 * c + li] : 0.f;
  };
  auto prod = [&](const Ops& o, f32x4 (&T)[RT][2]) {
#pragma unroll
    for (int r = 0; r < RT; ++r)
#pragma unroll
      for (int c = 0; c < 2; ++c) T[r][c] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) {
      f32x8 b[2];
#pragma unroll
      for (int c = 0; c < 2; ++c) b[c] = lds8(&st[16 * c + li][32 * kk + 8 * lq]);
#pragma unroll
      for (int r = 0; r < RT; ++r)
#pragma unroll
        for (int c = 0; c < 2; ++c) T[r][c] = mma16(o.a[r][kk], b[c], T[r][c]);
    }
  };
  // this lane's elements: row i = 16 (RT w + r) + 4 lq + e, column j = 16 c + li of the block
  auto save = [&](int it, bool isA) {
    float* f32 = isA ? nullptr : p.Spf + ((size_t)bh * F + it) * DD;
    bf16* m = (isA ? p.Ab : p.Sp) + ((size_t)bh * F + it) * DD;
    bf16* mt = (isA ? p.AbT : p.SpT) + ((size_t)bh * F + it) * DD;
#pragma unroll
    for (int r = 0; r < RT; ++r)
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        const int j = c0 + 16 * c + li, i0 = 16 * (RT * w + r) + 4 * lq;
        bf16x4 ch, cl;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float x = st[16 * c + li][i0 + e];
          if (f32) f32[(size_t)(i0 + e) * D + j] = x;
          GDN_SPLIT(x, ch[e], cl[e]);
          m[(size_t)(i0 + e) * D + j] = ch[e];
          m[p.lo + (size_t)(i0 + e) * D + j] = cl[e];
        }
        *reinterpret_cast<bf16x4*>(&mt[(size_t)j * D + i0]) = ch;
        *reinterpret_cast<bf16x4*>(&mt[p.lo + (size_t)j * D + i0]) = cl;
      }
  };

  // ---- forward states; the operands of step it + 1 are loaded while step it runs
  auto fetch_fwd = [&](int it, Ops& o) {
    if (it >= F || (p.reverse && it == 0)) return;
    const int fa = p.reverse ? F - it : it;
    o.g = p.decay[bh * F + fa];
    fetch_g(p.G + ((size_t)bh * F + fa) * DD, o);
    fetch_el(p.U + ((size_t)bh * F + fa) * DD, o.x);
  };
  Ops cur, nxt;
  fetch_fwd(0, cur);
  for (int it = 0; it < F; ++it) {
    fetch_fwd(it + 1, nxt);
    if (!(p.reverse && it == 0)) {
      f32x4 T[RT][2];
      prod(cur, T);
      __syncthreads();  // every wave has read st
#pragma unroll
      for (int r = 0; r < RT; ++r)
#pragma unroll
        for (int c = 0; c < 2; ++c)
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int i = 16 * (RT * w + r) + 4 * lq + e, jl = 16 * c + li;
            st[jl][i] = cur.g * (st[jl][i] - T[r][c][e]) + cur.x[r][c][e];
          }
      __syncthreads();
    }
    save(it, false);
    cur = nxt;
  }
  // ---- state gradients, steps in reverse (operands of step it - 1 loaded during step it)
  auto fetch_bwd = [&](int it, Ops& o) {
    if (it < 0) return;
    const int f = p.reverse ? F - 1 - it : it;
    fetch_el(p.W + ((size_t)bh * F + f) * DD, o.x);
    if (p.reverse && it == 0) return;
    const int fa = p.reverse ? f + 1 : f;
    o.g = p.decay[bh * F + fa];
    fetch_g(p.G + ((size_t)bh * F + fa) * DD, o);
    fetch_el(it > 0 ? p.Spf + ((size_t)bh * F + it - 1) * DD : nullptr, o.y);
  };
  __syncthreads();
  for (int e = threadIdx.x; e < 32 * kS; e += 256) (&st[0][0])[e] = 0.f;
  __syncthreads();
  fetch_bwd(F - 1, cur);
  for (int it = F - 1; it >= 0; --it) {
    const int f = p.reverse ? F - 1 - it : it;
    fetch_bwd(it - 1, nxt);
#pragma unroll
    for (int r = 0; r < RT; ++r)
#pragma unroll
      for (int c = 0; c < 2; ++c)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int i = 16 * (RT * w + r) + 4 * lq + e, jl = 16 * c + li;
          st[jl][i] += cur.x[r][c][e];
        }
    __syncthreads();
    save(it, true);
    if (p.reverse && it == 0) break;
    const int fa = p.reverse ? f + 1 : f;
    f32x4 T[RT][2];
    prod(cur, T);
    __syncthreads();
    // dP = A - G A; its sum against the state before the step (zero before the first step)
    float part = 0.f;
#pragma unroll
    for (int r = 0; r < RT; ++r)
#pragma unroll
      for (int c = 0; c < 2; ++c)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int i = 16 * (RT * w + r) + 4 * lq + e, jl = 16 * c + li;
          const float dp = st[jl][i] - T[r][c][e];
          part += dp * cur.y[r][c][e];
          st[jl][i] = cur.g * dp;
        }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) part += __shfl_xor(part, off, 64);
    if (lane == 0) red[w] = part;
    __syncthreads();
    if (threadIdx.x == 0)
      p.ddecay_part[((size_t)bh * F + fa) * (D / 32) + bid % (D / 32)] = (red[0] + red[1]) + (red[2] + red[3]);
    cur = nxt;
  }
}

// ---- token gradients ---------------------------------------------------------------------
// blockIdx.x = (bh * F + it) * (S / 64) + token block: tokens 64 block .. + 63 of the frames of
// step it.  Two LDS tiles, each a hi/lo pair of bf16 [token][D], hold the token operands;
// wave w forms output rows 16 RW w .. 16 RW (w + 1) - 1.
template <int D>
__global__ __launch_bounds__(256) void cbwd_tok_kernel(const CamBwdParams p) {
  constexpr int RW = D / 64;   // 16-row output tiles per wave
  constexpr int kT = D + 8;    // LDS row stride of a [token][D] tile (elements)
  __shared__ __attribute__((aligned(16))) bf16 tl[2][2][64 * kT];  // [tile][hi, lo]
  __shared__ float red[4][64];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, li = lane & 15, lq = lane >> 4;
  const int nblk = p.S / 64;
  const int bid = xcd_logical(blockIdx.x, gridDim.x);
  const int blk = bid % nblk;
  const long sb = bid / nblk;
  const int F = p.F;
  const int it = (int)(sb % F);
  const long bh = sb / F;
  const long N = (long)F * p.S;
  const size_t DD = (size_t)D * D;
  const int s0 = 64 * blk;  // first token of this block inside its frame
  const int f = p.reverse ? F - 1 - it : it;
  const bool absorb = !(p.reverse && it == 0);
  const int fa = p.reverse ? f + 1 : f;  // used only when absorb
  const long base = bh * D * N;

  // p.acc: this direction's dbeta and ddecay are added to the arrays' contents
  if (blk == 0 && tid == 0) {
    if (absorb) {
      float s = 0.f;
      for (int cb = 0; cb < D / 32; ++cb) s += p.ddecay_part[((size_t)bh * F + fa) * (D / 32) + cb];
      p.ddecay[bh * F + fa] = (p.acc ? p.ddecay[bh * F + fa] : 0.f) + (it > 0 ? s : 0.f);
    } else if (!p.acc) {
      p.ddecay[bh * F] = 0.f;  // frame 0 of the reverse scan is never absorbed
    }
  }

  // x[:, t0 .. t0 + 63] (channel-major, [D][N] per head) into tile T as a bf16 [token][D] pair
  auto stage = [&](const float* x, long t0, int T) {
    const int t = tid & 63, cg = tid >> 6;
    bf16* H = tl[T][0];
    bf16* L = tl[T][1];
#pragma unroll 4
    for (int c = 2 * cg; c < D; c += 8) {
      bf16x2 h, l;
      GDN_SPLIT(x[base + (long)c * N + t0 + t], h[0], l[0]);
      GDN_SPLIT(x[base + (long)(c + 1) * N + t0 + t], h[1], l[1]);
      *reinterpret_cast<bf16x2*>(&H[t * kT + c]) = h;
      *reinterpret_cast<bf16x2*>(&L[t * kT + c]) = l;
    }
  };
  // four consecutive rows i0 .. i0 + 3 of token t into tile T
  auto put = [&](int T, int t, int i0, const float (&x)[4]) {
    bf16x4 h, l;
#pragma unroll
    for (int e = 0; e < 4; ++e) GDN_SPLIT(x[e], h[e], l[e]);
    *reinterpret_cast<bf16x4*>(&tl[T][0][t * kT + i0]) = h;
    *reinterpret_cast<bf16x4*>(&tl[T][1][t * kT + i0]) = l;
  };
  // C[i][t] = sum_k M[i][k] X[t][k]: M a D x D row-major hi/lo matrix pair in memory (A operand
  // rows read straight from it), X tile T; C tile (r, c): row 16 (RW w + r) + 4 lq + e, token
  // 16 c + li
  auto prod = [&](const bf16* M, int T, f32x4 (&C)[RW][4]) {
#pragma unroll
    for (int r = 0; r < RW; ++r)
#pragma unroll
      for (int c = 0; c < 4; ++c) C[r][c] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kk = 0; kk < D / 32; ++kk) {
      bf16x8 bh[4], bl[4];
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        bh[c] = lds8(&tl[T][0][(16 * c + li) * kT + 32 * kk + 8 * lq]);
        bl[c] = lds8(&tl[T][1][(16 * c + li) * kT + 32 * kk + 8 * lq]);
      }
#pragma unroll
      for (int r = 0; r < RW; ++r) {
        const size_t ro = (size_t)(16 * (RW * w + r) + li) * D + 32 * kk + 8 * lq;
        const bf16x8 ah = *reinterpret_cast<const bf16x8*>(M + ro);
        const bf16x8 al = *reinterpret_cast<const bf16x8*>(M + p.lo + ro);
#pragma unroll
        for (int c = 0; c < 4; ++c) C[r][c] = mma3(ah, al, bh[c], bl[c], C[r][c]);
      }
    }
  };
  auto row_of = [&](int r, int e) { return 16 * (RW * w + r) + 4 * lq + e; };

  // ---- dq of the output frame's tokens: dq = S dout
  stage(p.dout, (long)f * p.S + s0, 0);
  __syncthreads();
  {
    f32x4 C[RW][4];
    prod(p.Sp + ((size_t)bh * F + it) * DD, 0, C);
#pragma unroll
    for (int r = 0; r < RW; ++r)
#pragma unroll
      for (int c = 0; c < 4; ++c)
#pragma unroll
        for (int e = 0; e < 4; ++e)
          p.dq[base + (long)row_of(r, e) * N + (long)f * p.S + s0 + 16 * c + li] = C[r][c][e];
  }
  if (!absorb) {
    // frame 0 of the reverse scan: its tokens are never absorbed
#pragma unroll
    for (int r = 0; r < RW; ++r)
#pragma unroll
      for (int c = 0; c < 4; ++c)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const long o = base + (long)row_of(r, e) * N + s0 + 16 * c + li;
          p.dk[o] = 0.f;
          p.dv[o] = 0.f;
        }
    if (tid < 64 && !p.acc) p.dbeta[bh * N + s0 + tid] = 0.f;
    return;
  }
  const long ta = (long)fa * p.S + s0;  // first token of this block in the absorbed frame
  const float g = p.decay[bh * F + fa];
  float bcol[4];
#pragma unroll
  for (int c = 0; c < 4; ++c) bcol[c] = p.beta[bh * N + ta + 16 * c + li];
  __syncthreads();  // every wave is done with the dout tile
  stage(p.k, ta, 0);
  __syncthreads();

  // ---- P = S_prev^T K (S_pre = g S_prev) and dd = A^T K
  f32x4 P[RW][4], Dd[RW][4];
  if (it > 0) {
    prod(p.SpT + ((size_t)bh * F + it - 1) * DD, 0, P);
  } else {
#pragma unroll
    for (int r = 0; r < RW; ++r)
#pragma unroll
      for (int c = 0; c < 4; ++c) P[r][c] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  prod(p.AbT + ((size_t)bh * F + it) * DD, 0, Dd);
  // r = v - g P, dv = beta dd, dbeta = dd . r; the next products take beta r and -beta dd
  float db[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int r = 0; r < RW; ++r)
#pragma unroll
    for (int c = 0; c < 4; ++c)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const long o = base + (long)row_of(r, e) * N + ta + 16 * c + li;
        const float rr = p.v[o] - g * P[r][c][e];
        const float dd = Dd[r][c][e];
        p.dv[o] = bcol[c] * dd;
        db[c] += dd * rr;
        P[r][c][e] = bcol[c] * rr;
        Dd[r][c][e] = -bcol[c] * dd;
      }
  __syncthreads();  // every wave is done with the k tile
#pragma unroll
  for (int r = 0; r < RW; ++r)
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const float xr[4] = {P[r][c][0], P[r][c][1], P[r][c][2], P[r][c][3]};
      const float xd[4] = {Dd[r][c][0], Dd[r][c][1], Dd[r][c][2], Dd[r][c][3]};
      put(1, 16 * c + li, row_of(r, 0), xr);
      put(0, 16 * c + li, row_of(r, 0), xd);
    }
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    db[c] += __shfl_xor(db[c], 16, 64);
    db[c] += __shfl_xor(db[c], 32, 64);
    if (lq == 0) red[w][16 * c + li] = db[c];
  }
  __syncthreads();
  if (tid < 64)
    p.dbeta[bh * N + ta + tid] = (p.acc ? p.dbeta[bh * N + ta + tid] : 0.f) +
                                 ((red[0][tid] + red[1][tid]) + (red[2][tid] + red[3][tid]));

  // ---- dk = A (beta r) + g S_prev (-beta dd)
  f32x4 K1[RW][4];
  prod(p.Ab + ((size_t)bh * F + it) * DD, 1, K1);
  if (it > 0) {
    f32x4 K2[RW][4];
    prod(p.Sp + ((size_t)bh * F + it - 1) * DD, 0, K2);
#pragma unroll
    for (int r = 0; r < RW; ++r)
#pragma unroll
      for (int c = 0; c < 4; ++c) K1[r][c] = K1[r][c] + g * K2[r][c];
  }
#pragma unroll
  for (int r = 0; r < RW; ++r)
#pragma unroll
    for (int c = 0; c < 4; ++c)
#pragma unroll
      for (int e = 0; e < 4; ++e) p.dk[base + (long)row_of(r, e) * N + ta + 16 * c + li] = K1[r][c][e];
}

template <int D>
hipError_t launch_d(const CamBwdParams& p, hipStream_t stream) {
  const long bh = (long)p.B * p.H;
  hipLaunchKernelGGL((cbwd_stats_kernel<D>), dim3(bh * p.F * 3), dim3(256), 0, stream, p);
  hipLaunchKernelGGL((cbwd_scan_kernel<D>), dim3(bh * (D / 32)), dim3(256), 0, stream, p);
  hipLaunchKernelGGL((cbwd_tok_kernel<D>), dim3(bh * p.F * (p.S / 64)), dim3(256), 0, stream, p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_cam_scan_bwd(const CamBwdParams& p, hipStream_t stream) {
  return p.D == 128 ? launch_d<128>(p, stream) : launch_d<64>(p, stream);
}

hipError_t launch_cam_bwd_scan(const CamBwdParams& p, hipStream_t stream) {
  const long bh = (long)p.B * p.H;
  if (p.D == 128)
    hipLaunchKernelGGL((cbwd_scan_kernel<128>), dim3(bh * 4), dim3(256), 0, stream, p);
  else
    hipLaunchKernelGGL((cbwd_scan_kernel<64>), dim3(bh * 2), dim3(256), 0, stream, p);
  return hipGetLastError();
}

}  // namespace gdn

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
//   scan   per (b, h, kScanCB state columns): the forward states and then A, in fp32 with split
//          bf16 products (the state in LDS as fp32 and as a hi/lo pair, G from the statistics
//          as a hi/lo pair); every step's state and A leave as hi/lo
//          bf16 pairs in both orientations for the token kernel, the states also in fp32 for
//          the decay gradient, whose partial sums over the block's columns go to the workspace.
//   token  per (b, h, step) (or a part of the step's token blocks when there are few steps):
//          the five products of the per-token gradients; each of the D/16 waves keeps its 16
//          rows of the step's matrices in registers and forms those output rows for every
//          64-token block, whose token slabs are transposed into LDS tiles the waves share.
// Precision: each product splits both fp32 operands into bf16 pairs x = hi + lo (hi = bf16(x),
// lo = bf16(x - hi)) and sums hi*hi + hi*lo + lo*hi in fp32, about 16 mantissa bits per
// operand.  The page's backward takes plain bf16 operands; their rounding alone moves the
// gradients by up to 4e-2 of their RMS on the small test shapes.
#include "gdn_bwd_params.h"
#include "gdn_device.h"
#include "gdn_dma.h"
#include "gdn_internal.h"

namespace gdn {
namespace {

typedef bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef bf16 bf16x4 __attribute__((ext_vector_type(4)));

// ---- stats: G_f, U_f, W_f ----------------------------------------------------------------
// blockIdx.x = (bh * F + f) * 3 + which (with p.reuse, G and U are kept and blockIdx.x = bh * F
// + f forms W alone); four waves, wave w owns rows 16 RT w .. of the D x D
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
  const int nw = p.reuse ? 1 : 3;  // matrices formed: G, U, W, or W alone
  const int which = p.reuse ? 2 : bid % 3;
  const long bf = bid / nw;
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
  if (which == 0) {
    // G as a hi/lo bf16 pair (the scan's A operands): hi [D][D], then lo, in the matrix's slot
    bf16* gh = reinterpret_cast<bf16*>(p.G) + bf * 2 * D * D;
#pragma unroll
    for (int r = 0; r < RT; ++r)
#pragma unroll
      for (int c = 0; c < CT; ++c)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const size_t o = (size_t)(16 * (RT * w + r) + 4 * lq + e) * D + 16 * c + li;
          GDN_SPLIT(acc[r][c][e], gh[o], gh[D * D + o]);
        }
    return;
  }
  float* out = (which == 1 ? p.U : p.W) + bf * D * D;
#pragma unroll
  for (int r = 0; r < RT; ++r)
#pragma unroll
    for (int c = 0; c < CT; ++c)
#pragma unroll
      for (int e = 0; e < 4; ++e) out[(16 * (RT * w + r) + 4 * lq + e) * D + 16 * c + li] = acc[r][c][e];
}

// ---- scan: forward states, then the state gradients ---------------------------------------
// blockIdx.x = bh * (D / kScanCB) + column block.  st[col][row] holds the block's kScanCB
// columns of the state (then of A), transposed so that a lane's 8 consecutive rows are one
// contiguous read.
template <int D>
__global__ __launch_bounds__(256) void cbwd_scan_kernel(const CamBwdParams p) {
  constexpr int RT = D / 64;  // row tiles per wave (16 rows each)
  constexpr int kS = D + 4;   // row stride of st (floats)
  constexpr int kB = D + 8;   // row stride of the hi/lo copies (elements)
  constexpr int CB = kScanCB, NC = CB / 16;  // columns per workgroup, 16-column tiles
  __shared__ float st[CB][kS];
  __shared__ __attribute__((aligned(16))) bf16 sth[2][CB][kB];  // st as a hi/lo bf16 pair
  __shared__ float red[4];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, li = lane & 15, lq = lane >> 4;
  const int bid = xcd_logical(blockIdx.x, gridDim.x);
  const long bh = bid / (D / CB);
  const int c0 = CB * (bid % (D / CB));
  const int F = p.F;
  const size_t DD = (size_t)D * D;
  auto zero_st = [&]() {
    for (int e = threadIdx.x; e < CB * kS; e += 256) (&st[0][0])[e] = 0.f;
    for (int e = threadIdx.x; e < 2 * CB * kB; e += 256) (&sth[0][0][0])[e] = bf16{};
  };
  zero_st();
  __syncthreads();
  // st[jl][i .. i + 3] (this lane's four rows of column jl) is x; also its hi/lo copy
  auto set4 = [&](int jl, int i, const f32x4& x) {
    bf16x4 h, l;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      st[jl][i + e] = x[e];
      GDN_SPLIT(x[e], h[e], l[e]);
    }
    *reinterpret_cast<bf16x4*>(&sth[0][jl][i]) = h;
    *reinterpret_cast<bf16x4*>(&sth[1][jl][i]) = l;
  };
  // T = M st (rows of this wave, the block's CB columns) with M's A operands (hi/lo bf16)
  // already in registers: tile (r, c) holds rows 16 (RT w + r) + 4 lq + e, column 16 c + li
  constexpr int KK = D / 32;
  struct Ops {
    bf16x8 ah[RT][KK], al[RT][KK];  // rows 16 (RT w + r) + li of G, columns 32 kk + 8 lq ..
    float x[RT][NC][4];   // U (forward) or W (backward) at this lane's elements
    float y[RT][NC][4];   // the state before the step (backward)
    float g;
  };
  auto fetch_g = [&](const bf16* M, Ops& o) {
#pragma unroll
    for (int r = 0; r < RT; ++r)
#pragma unroll
      for (int kk = 0; kk < KK; ++kk) {
        const size_t ro = (size_t)(16 * (RT * w + r) + li) * D + 32 * kk + 8 * lq;
        o.ah[r][kk] = *reinterpret_cast<const bf16x8*>(M + ro);
        o.al[r][kk] = *reinterpret_cast<const bf16x8*>(M + DD + ro);
      }
  };
  auto fetch_el = [&](const float* M, float (&x)[RT][NC][4]) {
#pragma unroll
    for (int r = 0; r < RT; ++r)
#pragma unroll
      for (int c = 0; c < NC; ++c)
#pragma unroll
        for (int e = 0; e < 4; ++e)
          x[r][c][e] = M ? M[(size_t)(16 * (RT * w + r) + 4 * lq + e) * D + c0 + 16 * c + li] : 0.f;
  };
  auto prod = [&](const Ops& o, f32x4 (&T)[RT][NC]) {
#pragma unroll
    for (int r = 0; r < RT; ++r)
#pragma unroll
      for (int c = 0; c < NC; ++c) T[r][c] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) {
      bf16x8 bh[NC], bl[NC];
#pragma unroll
      for (int c = 0; c < NC; ++c) {
        bh[c] = lds8(&sth[0][16 * c + li][32 * kk + 8 * lq]);
        bl[c] = lds8(&sth[1][16 * c + li][32 * kk + 8 * lq]);
      }
#pragma unroll
      for (int r = 0; r < RT; ++r)
#pragma unroll
        for (int c = 0; c < NC; ++c) T[r][c] = mma3(o.ah[r][kk], o.al[r][kk], bh[c], bl[c], T[r][c]);
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
      for (int c = 0; c < NC; ++c) {
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
    fetch_g(reinterpret_cast<const bf16*>(p.G) + ((size_t)bh * F + fa) * 2 * DD, o);
    fetch_el(p.U + ((size_t)bh * F + fa) * DD, o.x);
  };
  Ops cur, nxt;
  fetch_fwd(0, cur);
  for (int it = 0; it < F; ++it) {
    fetch_fwd(it + 1, nxt);
    if (!(p.reverse && it == 0)) {
      f32x4 T[RT][NC];
      prod(cur, T);
      __syncthreads();  // every wave has read st
#pragma unroll
      for (int r = 0; r < RT; ++r)
#pragma unroll
        for (int c = 0; c < NC; ++c) {
          const int i = 16 * (RT * w + r) + 4 * lq, jl = 16 * c + li;
          f32x4 x;
#pragma unroll
          for (int e = 0; e < 4; ++e) x[e] = cur.g * (st[jl][i + e] - T[r][c][e]) + cur.x[r][c][e];
          set4(jl, i, x);
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
    fetch_g(reinterpret_cast<const bf16*>(p.G) + ((size_t)bh * F + fa) * 2 * DD, o);
    fetch_el(it > 0 ? p.Spf + ((size_t)bh * F + it - 1) * DD : nullptr, o.y);
  };
  __syncthreads();
  zero_st();
  __syncthreads();
  fetch_bwd(F - 1, cur);
  for (int it = F - 1; it >= 0; --it) {
    const int f = p.reverse ? F - 1 - it : it;
    fetch_bwd(it - 1, nxt);
#pragma unroll
    for (int r = 0; r < RT; ++r)
#pragma unroll
      for (int c = 0; c < NC; ++c) {
        const int i = 16 * (RT * w + r) + 4 * lq, jl = 16 * c + li;
        f32x4 x;
#pragma unroll
        for (int e = 0; e < 4; ++e) x[e] = st[jl][i + e] + cur.x[r][c][e];
        set4(jl, i, x);
      }
    __syncthreads();
    save(it, true);
    if (p.reverse && it == 0) break;
    const int fa = p.reverse ? f + 1 : f;
    f32x4 T[RT][NC];
    prod(cur, T);
    __syncthreads();
    // dP = A - G A; its sum against the state before the step (zero before the first step)
    float part = 0.f;
#pragma unroll
    for (int r = 0; r < RT; ++r)
#pragma unroll
      for (int c = 0; c < NC; ++c) {
        const int i = 16 * (RT * w + r) + 4 * lq, jl = 16 * c + li;
        f32x4 x;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float dp = st[jl][i + e] - T[r][c][e];
          part += dp * cur.y[r][c][e];
          x[e] = cur.g * dp;
        }
        set4(jl, i, x);
      }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) part += __shfl_xor(part, off, 64);
    if (lane == 0) red[w] = part;
    __syncthreads();
    if (threadIdx.x == 0)
      p.ddecay_part[((size_t)bh * F + fa) * (D / CB) + bid % (D / CB)] = (red[0] + red[1]) + (red[2] + red[3]);
    cur = nxt;
  }
}

// ---- token gradients ---------------------------------------------------------------------
// One workgroup of D/16 waves per (b, h, step, part of the frame's 64-token blocks); wave w
// owns output rows 16 w .. 16 w + 15 and keeps its rows of the step's D x D matrices (hi/lo
// A-operand fragments) in registers for all of its token blocks, so each matrix is read once
// per workgroup: S in a first pass over the blocks (dq), then S_prev^T, A^T, A and S_prev in a
// second (dv, dbeta, dk; all five at once would not fit the register file).  A block's
// channel-major slabs (dout in the first pass; k and v in the second) arrive in LDS as raw fp32
// rows by direct buffer-to-LDS loads issued one block ahead, under the current block's
// products; at the block's start they are split into hi/lo bf16 [token][D] tiles.  Two tiles:
// dout (or k), then beta r and -beta dd.
template <int D>
__global__ __launch_bounds__(D * 4) void cbwd_tok_kernel(const CamBwdParams p, int nsplit) {
  constexpr int NW = D / 16, KK = D / 32;  // waves (16 output rows each), contraction steps
  constexpr int kT = D + 8;                // LDS row stride of a [token][D] tile (elements)
  constexpr int kR = 64;                   // LDS row stride of a raw [D][64] fp32 slab (floats)
  __shared__ __attribute__((aligned(16))) bf16 tl[2][2][64 * kT];  // [tile][hi, lo]
  __shared__ __attribute__((aligned(16))) float raw[2][D * kR];    // k (or dout), v
  __shared__ float red[NW][64];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, li = lane & 15, lq = lane >> 4;
  const int nblk = p.S / 64;
  const int bid = xcd_logical(blockIdx.x, gridDim.x);
  const int part = bid % nsplit;
  const long sb = bid / nsplit;
  const int F = p.F;
  const int it = (int)(sb % F);
  const long bh = sb / F;
  const long N = (long)F * p.S;
  const int Ni = (int)N;
  const size_t DD = (size_t)D * D;
  const int b0 = part * nblk / nsplit, b1 = (part + 1) * nblk / nsplit;
  const int f = p.reverse ? F - 1 - it : it;
  const bool absorb = !(p.reverse && it == 0);
  const int fa = p.reverse ? f + 1 : f;  // used only when absorb
  const long base = bh * D * N;
  // this head's [D][N] slabs; element offsets within a slab fit 32 bits (D N < 2^29)
  float* const dqh = p.dq + base;
  float* const dkh = p.dk + base;
  float* const dvh = p.dv + base;

  // p.acc: this direction's dbeta and ddecay are added to the arrays' contents
  if (part == 0 && tid == 0) {
    if (absorb) {
      float s = 0.f;
      for (int cb = 0; cb < D / kScanCB; ++cb) s += p.ddecay_part[((size_t)bh * F + fa) * (D / kScanCB) + cb];
      p.ddecay[bh * F + fa] = (p.acc ? p.ddecay[bh * F + fa] : 0.f) + (it > 0 ? s : 0.f);
    } else if (!p.acc) {
      p.ddecay[bh * F] = 0.f;  // frame 0 of the reverse scan is never absorbed
    }
  }

  // this wave's rows of a matrix pair (row-major hi, then lo p.lo elements later)
  typedef bf16x8 Frag[KK][2];
  auto load_a = [&](const bf16* M, Frag& a) {
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) {
      const size_t ro = (size_t)(16 * w + li) * D + 32 * kk + 8 * lq;
      a[kk][0] = *reinterpret_cast<const bf16x8*>(M + ro);
      a[kk][1] = *reinterpret_cast<const bf16x8*>(M + p.lo + ro);
    }
  };
  const bool prev = it > 0;  // a state before this step exists (else S_prev = 0)
  const float g = absorb ? p.decay[bh * F + fa] : 0.f;

  // tokens t0 .. t0 + 63 of every channel row of a [D][N] slab into raw slab R (fp32 [D][64],
  // rows contiguous): an instruction moves four rows (16 lanes of 16 bytes each), wave w the
  // rows 4 w + 4 NW i .. + 3
  auto fetch = [&](const float* x, int t0, int R) {
    const dma::i32x4 rs = dma::make_rsrc(x + base + t0, (uint32_t)(((D - 1) * N + 64) * 4));
    const int wu = __builtin_amdgcn_readfirstlane(w);  // the wave index, as a scalar
#pragma unroll
    for (int i = 0; i < D / (4 * NW); ++i) {
      const int c0 = 4 * wu + 4 * NW * i;
      dma::dma16(rs, (uint32_t)(((c0 + (lane >> 4)) * Ni + 4 * (lane & 15)) * 4), 0,
                 dma::lds_addr(&raw[R][c0 * kR]));
    }
  };
  // raw slab R into tile T as hi/lo bf16 [token][D]
  auto split = [&](int R, int T) {
    const int t = tid & 63, cg = tid >> 6;
#pragma unroll 4
    for (int c = 2 * cg; c < D; c += 2 * NW) {
      bf16x2 h, l;
      GDN_SPLIT(raw[R][c * kR + t], h[0], l[0]);
      GDN_SPLIT(raw[R][(c + 1) * kR + t], h[1], l[1]);
      *reinterpret_cast<bf16x2*>(&tl[T][0][t * kT + c]) = h;
      *reinterpret_cast<bf16x2*>(&tl[T][1][t * kT + c]) = l;
    }
  };
  // C[c] (rows 16 w + 4 lq + e, tokens 16 c + li) = M X^T for the wave's fragments of M and
  // tile T, one contraction step's operand reads at a time (the scheduling barrier keeps the
  // compiler from hoisting every step's reads beside the fragments)
  auto prod = [&](const Frag& a, int T, f32x4 (&C)[4]) {
#pragma unroll
    for (int c = 0; c < 4; ++c) C[c] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) {
      bf16x8 bh[4], bl[4];
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        bh[c] = lds8(&tl[T][0][(16 * c + li) * kT + 32 * kk + 8 * lq]);
        bl[c] = lds8(&tl[T][1][(16 * c + li) * kT + 32 * kk + 8 * lq]);
      }
#pragma unroll
      for (int c = 0; c < 4; ++c) C[c] = mma3(a[kk][0], a[kk][1], bh[c], bl[c], C[c]);
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  // four consecutive rows i0 .. i0 + 3 of token t into tile T
  auto put = [&](int T, int t, int i0, const f32x4& x) {
    bf16x4 h, l;
#pragma unroll
    for (int e = 0; e < 4; ++e) GDN_SPLIT(x[e], h[e], l[e]);
    *reinterpret_cast<bf16x4*>(&tl[T][0][t * kT + i0]) = h;
    *reinterpret_cast<bf16x4*>(&tl[T][1][t * kT + i0]) = l;
  };
  const int r0 = 16 * w + 4 * lq;  // first output row of this lane

  // ---- pass 1, dq of the output frame's tokens: dq = S dout (S's fragments only)
  if (b0 < b1) fetch(p.dout, f * p.S + 64 * b0, 0);
  {
    Frag aS;
    load_a(p.Sp + ((size_t)bh * F + it) * DD, aS);
    for (int blk = b0; blk < b1; ++blk) {
      const int s0 = 64 * blk;  // first token of this block inside its frame
      dma::wait_vm0();          // this wave's slab rows have arrived
      __syncthreads();          // everyone's have, and the previous block is done with tile 0
      split(0, 0);
      __syncthreads();
      if (blk + 1 < b1) fetch(p.dout, f * p.S + s0 + 64, 0);
      else if (absorb) {        // the second pass's first block
        fetch(p.k, fa * p.S + 64 * b0, 0);
        fetch(p.v, fa * p.S + 64 * b0, 1);
      }
      f32x4 C[4];
      prod(aS, 0, C);
#pragma unroll
      for (int c = 0; c < 4; ++c)
#pragma unroll
        for (int e = 0; e < 4; ++e) dqh[(r0 + e) * Ni + f * p.S + s0 + 16 * c + li] = C[c][e];
    }
  }
  if (!absorb) {
    // frame 0 of the reverse scan: its tokens are never absorbed
    for (int blk = b0; blk < b1; ++blk) {
      const int s0 = 64 * blk;
#pragma unroll
      for (int c = 0; c < 4; ++c)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int o = (r0 + e) * Ni + s0 + 16 * c + li;
          dkh[o] = 0.f;
          dvh[o] = 0.f;
        }
      if (tid < 64 && !p.acc) p.dbeta[bh * N + s0 + tid] = 0.f;
    }
    return;
  }
  // ---- pass 2, the absorbed frame's tokens (the other four matrices' fragments)
  Frag aPT, aDT, aA, aSP;
  load_a(p.AbT + ((size_t)bh * F + it) * DD, aDT);
  load_a(p.Ab + ((size_t)bh * F + it) * DD, aA);
  if (prev) {
    load_a(p.SpT + ((size_t)bh * F + it - 1) * DD, aPT);
    load_a(p.Sp + ((size_t)bh * F + it - 1) * DD, aSP);
  }
  for (int blk = b0; blk < b1; ++blk) {
    const int s0 = 64 * blk;
    const int ta = fa * p.S + s0;  // first token of this block in the absorbed frame
    dma::wait_vm0();
    __syncthreads();  // the k and v rows are in; the previous block is done with both tiles
    split(0, 1);
    __syncthreads();
    if (blk + 1 < b1) fetch(p.k, ta + 64, 0);
    // P = S_prev^T K (S_pre = g S_prev) and dd = A^T K; r = v - g P, dv = beta dd,
    // dbeta = dd . r; the next products take beta r and -beta dd
    float bcol[4];
#pragma unroll
    for (int c = 0; c < 4; ++c) bcol[c] = p.beta[bh * N + ta + 16 * c + li];
    f32x4 P[4], Dd[4];
    if (prev) {
      prod(aPT, 1, P);
    } else {
#pragma unroll
      for (int c = 0; c < 4; ++c) P[c] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
    prod(aDT, 1, Dd);
    float db[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int c = 0; c < 4; ++c)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float rr = raw[1][(r0 + e) * kR + 16 * c + li] - g * P[c][e];
        const float dd = Dd[c][e];
        dvh[(r0 + e) * Ni + ta + 16 * c + li] = bcol[c] * dd;
        db[c] += dd * rr;
        P[c][e] = bcol[c] * rr;
        Dd[c][e] = -bcol[c] * dd;
      }
    __syncthreads();  // every wave is done with the k tile and the v rows
    if (blk + 1 < b1) fetch(p.v, ta + 64, 1);
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      put(1, 16 * c + li, r0, P[c]);
      put(0, 16 * c + li, r0, Dd[c]);
    }
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      db[c] += __shfl_xor(db[c], 16, 64);
      db[c] += __shfl_xor(db[c], 32, 64);
      if (lq == 0) red[w][16 * c + li] = db[c];
    }
    __syncthreads();
    if (tid < 64) {
      float sum = 0.f;
#pragma unroll
      for (int i = 0; i < NW; ++i) sum += red[i][tid];
      p.dbeta[bh * N + ta + tid] = (p.acc ? p.dbeta[bh * N + ta + tid] : 0.f) + sum;
    }
    // dk = A (beta r) + g S_prev (-beta dd)
    f32x4 K1[4];
    prod(aA, 1, K1);
    if (prev) {
      f32x4 K2[4];
      prod(aSP, 0, K2);
#pragma unroll
      for (int c = 0; c < 4; ++c) K1[c] = K1[c] + g * K2[c];
    }
#pragma unroll
    for (int c = 0; c < 4; ++c)
#pragma unroll
      for (int e = 0; e < 4; ++e) dkh[(r0 + e) * Ni + ta + 16 * c + li] = K1[c][e];
  }
}

// Workgroups per (b, h, step) for the token kernel: enough for about one per CU in total.
inline int tok_split(long bhf, int nblk) {
  long s = (256 + bhf - 1) / bhf;
  return (int)(s < 1 ? 1 : s > nblk ? nblk : s);
}

template <int D>
hipError_t launch_d(const CamBwdParams& p, hipStream_t stream) {
  const long bh = (long)p.B * p.H;
  hipLaunchKernelGGL((cbwd_stats_kernel<D>), dim3(bh * p.F * (p.reuse ? 1 : 3)), dim3(256), 0, stream, p);
  hipLaunchKernelGGL((cbwd_scan_kernel<D>), dim3(bh * (D / kScanCB)), dim3(256), 0, stream, p);
  const int ns = tok_split(bh * p.F, p.S / 64);
  hipLaunchKernelGGL((cbwd_tok_kernel<D>), dim3(bh * p.F * ns), dim3(D * 4), 0, stream, p, ns);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_cam_scan_bwd(const CamBwdParams& p, hipStream_t stream) {
  return p.D == 128 ? launch_d<128>(p, stream) : launch_d<64>(p, stream);
}

hipError_t launch_cam_bwd_scan(const CamBwdParams& p, hipStream_t stream) {
  const long bh = (long)p.B * p.H;
  if (p.D == 128)
    hipLaunchKernelGGL((cbwd_scan_kernel<128>), dim3(bh * (128 / kScanCB)), dim3(256), 0, stream, p);
  else
    hipLaunchKernelGGL((cbwd_scan_kernel<64>), dim3(bh * (64 / kScanCB)), dim3(256), 0, stream, p);
  return hipGetLastError();
}

}  // namespace gdn

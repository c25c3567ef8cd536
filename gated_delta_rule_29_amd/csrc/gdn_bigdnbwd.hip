// gdn_bigdnbwd.hip -- backward of one BiGDN direction for gfx950 (SANA fused_gdn.py page,
// "Backward / autograd Functions": the reverse replay of the frame recurrence behind
// FusedBiGDNFunction.backward; the forward is one direction of bigdn_fwd).
//
// A direction carries the state S (D x D; keys k_rot, values v, read out by q_rot into num)
// and the normaliser z (D; keys k_pos, value 1, read out by q_pos into den).  S follows the
// camera-branch recurrence exactly, so its backward reuses the camera backward's state /
// gradient scan (gdn_cambwd.hip) on statistics formed here from the token-major prepped
// tensors; z is the same recurrence with a scalar value, scanned as vectors.  With A and a
// the gradients of S and z after a step's update, for the tokens s of the frame that a step
// absorbs (S_pre = g S_prev, z_pre = g z_prev):
//   dk_rot_s = A (beta_s r_s) - beta_s S_pre (A^T k_rot_s),  r_s = v_s - S_pre^T k_rot_s
//   dv_s = beta_s A^T k_rot_s
//   dk_pos_s = a (beta_s e_s) - beta_s (a . k_pos_s) z_pre,   e_s = 1 - k_pos_s . z_pre
//   dbeta_s = (A^T k_rot_s) . r_s + (a . k_pos_s) e_s
// and for the tokens of the frame the step outputs: dq_rot = S dnum, dq_pos = dden z.
//
// Kernels:
//   stats  per (b, h, frame, matrix): G, U, W (the S stream) and G_pos (the z stream) as
//          D x D fp32, plus the vectors u_pos = K_pos^T beta and w_z = Q_pos^T dden; token rows
//          staged in LDS 32 at a time, operands taken with transpose reads (the contraction
//          runs over tokens)
//   S scan the camera backward's scan (states and their gradients as hi/lo pairs)
//   z scan per (b, h): z after every step and a, by matrix-vector products with G_pos
//   S tok  per (b, h, step, 64 tokens): as the camera backward's token kernel, with token-
//          major tiles (no transpose) and token-major outputs
//   z tok  per (b, h, step, 64 tokens): dq_pos, dk_pos and the z part of dbeta
// Products take split bf16 operands (GDN_SPLIT); the z stream is fp32 arithmetic.
#include "gdn_bwd_params.h"
#include "gdn_device.h"
#include "gdn_dma.h"
#include "gdn_internal.h"

namespace gdn {
namespace {

typedef bf16 bf16x4 __attribute__((ext_vector_type(4)));
using namespace dma;
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

// Transpose read of 8 bytes per lane (ds_read_b64_tr_b16); the result is used only as a whole
// vector (bit casts), as element-wise casts of it have been miscompiled.
__device__ __forceinline__ u32x2 tr16(const u16* p) {
  return __builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(uintptr_t)lds_addr(p)));
}

// ---- statistics ---------------------------------------------------------------------------
// blockIdx.x = (bh * F + f) * 4 + which: 0 G (X = beta k_rot, Y = k_rot), 1 U (X = beta k_rot,
// Y = v), 2 W (X = q_rot, Y = dnum), 3 G_pos (X = beta k_pos, Y = k_pos).  Out[i][j] =
// sum_s X[s][i] Y[s][j].  Wave w owns rows 16 RT w .., all columns.  Per 32-token step the
// token rows go to LDS as split pairs [token][D] (16-byte copies of the token-major rows),
// and the operands, whose contraction runs over tokens, come out with transpose reads
// (ds_read_b64_tr_b16): in each 16-lane group, result lane n takes element j from the 8 bytes
// that lane 4j + n/4 addresses, halfword n % 4; so lane L addresses token 8 lq + L/4 (+4 for
// the second half), channels 16 tile + 4 (L % 4) .. + 3, and lane n receives channel
// 16 tile + n of those tokens.  The next step's rows are loaded while the products run.
template <int D>
__global__ __launch_bounds__(256) void bbwd_stats_kernel(const BigdnBwdParams p) {
  constexpr int RT = D / 64, CT = D / 16;
  constexpr int kR = D + 8;              // bf16 row stride of the [32 tokens][D] tiles
  constexpr int NI = 32 * D / 8 / 256;   // 8-channel items per thread per tile
  __shared__ __attribute__((aligned(16))) bf16 xt[2][32 * kR];
  __shared__ __attribute__((aligned(16))) bf16 yt[2][32 * kR];
  const CamBwdParams& c = p.cam;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, li = lane & 15, lq = lane >> 4;
  const int bid = xcd_logical(blockIdx.x, gridDim.x);
  const int which = bid % 4;
  const long bf = bid / 4;
  const int f = (int)(bf % c.F);
  const long bh = bf / c.F;
  const int b = (int)(bh / c.H), h = (int)(bh % c.H);
  const long N = (long)c.F * c.S;
  const long t0f = (long)f * c.S;  // first token of the frame
  const __bf16* X = which == 2 ? p.q_rot : (which == 3 ? p.k_pos : p.k_rot);
  const __bf16* Y = which == 0 ? p.k_rot : (which == 1 ? p.v : p.k_pos);
  const bool xbeta = which != 2;
  const float* bt = c.beta + bh * N + t0f;
  f32x4 acc[RT][CT];
#pragma unroll
  for (int r = 0; r < RT; ++r)
#pragma unroll
    for (int cc = 0; cc < CT; ++cc) acc[r][cc] = f32x4{0.f, 0.f, 0.f, 0.f};
  // item i of this thread: token (tid + 256 i) / (D / 8), channels 8 ((tid + 256 i) % (D / 8)) ..
  bf16x8 xr[NI], qr[NI];
  f32x4 yr[NI][2];
  float br[NI], dr[NI];
  // the z stream's vector (which 2: w_z = Q_pos^T dden; which 3: u_pos = K_pos^T beta), summed
  // over this thread's tokens for its 8 channels
  float vacc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  auto load = [&](int s0) {
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const int e = tid + 256 * i, t = e / (D / 8), d = 8 * (e % (D / 8));
      const long tok = t0f + s0 + t;
      xr[i] = *reinterpret_cast<const bf16x8*>(X + (bh * N + tok) * D + d);
      br[i] = xbeta ? bt[s0 + t] : 1.f;
      if (which == 2) {
        qr[i] = *reinterpret_cast<const bf16x8*>(p.q_pos + (bh * N + tok) * D + d);
        dr[i] = p.dden[bh * N + tok];
      }
      if (which == 2) {
        const float* src = p.dnum + (((long)b * N + tok) * c.H + h) * D + d;
        yr[i][0] = *reinterpret_cast<const f32x4*>(src);
        yr[i][1] = *reinterpret_cast<const f32x4*>(src + 4);
      } else {
        const bf16x8 y = *reinterpret_cast<const bf16x8*>(Y + (bh * N + tok) * D + d);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          yr[i][0][j] = (float)y[j];
          yr[i][1][j] = (float)y[4 + j];
        }
      }
    }
  };
  // two transpose reads of tile T (channels 16 tile ..): the B / A operand of 8 tokens
  const int L = lane & 15;
  auto tr8 = [&](const bf16* T, int tile) {
    const int o = (8 * lq + L / 4) * kR + 16 * tile + 4 * (L % 4);
    const u32x4 v = __builtin_shufflevector(tr16(reinterpret_cast<const u16*>(T + o)),
                                            tr16(reinterpret_cast<const u16*>(T + o + 4 * kR)),
                                            0, 1, 2, 3);
    return __builtin_bit_cast(bf16x8, v);
  };
  load(0);
  for (int s0 = 0; s0 < c.S; s0 += 32) {
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const int e = tid + 256 * i, t = e / (D / 8), d = 8 * (e % (D / 8));
      bf16x8 xh, xl, yh, yl;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        GDN_SPLIT((float)xr[i][j] * br[i], xh[j], xl[j]);
        GDN_SPLIT(yr[i][j / 4][j % 4], yh[j], yl[j]);
        if (which == 2) vacc[j] = fmaf(dr[i], (float)qr[i][j], vacc[j]);
        if (which == 3) vacc[j] = fmaf(br[i], (float)xr[i][j], vacc[j]);
      }
      *reinterpret_cast<bf16x8*>(&xt[0][t * kR + d]) = xh;
      *reinterpret_cast<bf16x8*>(&xt[1][t * kR + d]) = xl;
      *reinterpret_cast<bf16x8*>(&yt[0][t * kR + d]) = yh;
      *reinterpret_cast<bf16x8*>(&yt[1][t * kR + d]) = yl;
    }
    __syncthreads();
    if (s0 + 32 < c.S) load(s0 + 32);
    bf16x8 ah[RT], al[RT];
#pragma unroll
    for (int r = 0; r < RT; ++r) {
      ah[r] = tr8(xt[0], RT * w + r);
      al[r] = tr8(xt[1], RT * w + r);
    }
#pragma unroll
    for (int cc = 0; cc < CT; ++cc) {
      const bf16x8 bh_ = tr8(yt[0], cc), bl = tr8(yt[1], cc);
#pragma unroll
      for (int r = 0; r < RT; ++r) acc[r][cc] = mma3(ah[r], al[r], bh_, bl, acc[r][cc]);
    }
    __syncthreads();
  }
  if (which == 0) {
    // G as a hi/lo bf16 pair (the S-stream scan's A operands): hi [D][D], then lo
    bf16* gh = reinterpret_cast<bf16*>(c.G) + bf * 2 * D * D;
#pragma unroll
    for (int r = 0; r < RT; ++r)
#pragma unroll
      for (int cc = 0; cc < CT; ++cc)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const size_t o = (size_t)(16 * (RT * w + r) + 4 * lq + e) * D + 16 * cc + li;
          GDN_SPLIT(acc[r][cc][e], gh[o], gh[D * D + o]);
        }
  } else {
    float* out = (which == 1 ? c.U : (which == 2 ? c.W : p.Gpos)) + bf * D * D;
#pragma unroll
    for (int r = 0; r < RT; ++r)
#pragma unroll
      for (int cc = 0; cc < CT; ++cc)
#pragma unroll
        for (int e = 0; e < 4; ++e) out[(16 * (RT * w + r) + 4 * lq + e) * D + 16 * cc + li] = acc[r][cc][e];
  }
  // the z stream's vectors: the threads of one channel group (tid % (D / 8) equal; the item
  // offset 256 i keeps the group) add their sums through LDS
  if (which >= 2) {
    constexpr int TG = 256 / (D / 8);  // threads per channel group
    float* red = reinterpret_cast<float*>(&xt[0][0]);  // [TG][D], after the last barrier
#pragma unroll
    for (int j = 0; j < 8; ++j) red[(tid / (D / 8)) * D + 8 * (tid % (D / 8)) + j] = vacc[j];
    __syncthreads();
    if (tid < D) {
      float sum = 0.f;
      for (int q = 0; q < TG; ++q) sum += red[q * D + tid];
      (which == 2 ? p.wz : p.upos)[bf * D + tid] = sum;
    }
  }
}

// ---- z scan --------------------------------------------------------------------------------
// One workgroup of 1024 threads per (b, h).  y = G_pos x: G_pos is symmetric, so
// y[i] = sum_j G_pos[j][i] x[j]; thread (part, i) takes the rows j = part + P m (m < D / P),
// reading element i of each (consecutive lanes, consecutive elements), and the P partial sums
// meet in LDS.  The next step's elements are loaded into registers while a step runs.
template <int D>
__global__ __launch_bounds__(1024) void bbwd_zscan_kernel(const BigdnBwdParams p) {
  constexpr int P = 1024 / D, M = D / P;
  __shared__ float zv[D], xv[D], red[16], ps[P][D];
  const CamBwdParams& c = p.cam;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const long bh = blockIdx.x;
  const int F = c.F;
  const int row = tid % D, part = tid / D;
  float gc[M], gn[M];
  auto fetch = [&](int fa, float (&o)[M]) {
    const float* G = p.Gpos + (bh * F + fa) * D * D;
#pragma unroll
    for (int m = 0; m < M; ++m) o[m] = G[(size_t)(part + P * m) * D + row];
  };
  // y[row] in the threads with part == 0
  auto matvec = [&](const float* x) {
    float sum = 0.f;
#pragma unroll
    for (int m = 0; m < M; ++m) sum = fmaf(gc[m], x[part + P * m], sum);
    ps[part][row] = sum;
    __syncthreads();
    float y = 0.f;
    if (part == 0)
#pragma unroll
      for (int q = 0; q < P; ++q) y += ps[q][row];
    return y;
  };
  auto fa_of = [&](int it) { return c.reverse ? F - it : it; };  // frame absorbed at step it
  if (tid < D) zv[tid] = 0.f;
  const int first = c.reverse ? 1 : 0;  // the first step that absorbs a frame
  if (first < F) fetch(fa_of(first), gc);
  __syncthreads();
  for (int it = 0; it < F; ++it) {
    if (!(c.reverse && it == 0)) {
      const int fa = fa_of(it);
      if (it + 1 < F) fetch(fa_of(it + 1), gn);
      const float g = c.decay[bh * F + fa];
      if (tid < D) xv[tid] = g * zv[tid];  // z_pre
      __syncthreads();
      const float y = matvec(xv);
      if (part == 0) zv[row] = xv[row] - y + p.upos[(bh * F + fa) * D + row];
      __syncthreads();
#pragma unroll
      for (int m = 0; m < M; ++m) gc[m] = gn[m];
    }
    if (tid < D) p.zs[(bh * F + it) * D + tid] = zv[tid];
  }
  // gradients of z after each step's update, in reverse (zv holds a)
  __syncthreads();
  if (tid < D) zv[tid] = 0.f;
  if (!(c.reverse && F - 1 == 0)) fetch(fa_of(F - 1), gc);
  __syncthreads();
  for (int it = F - 1; it >= 0; --it) {
    const int f = c.reverse ? F - 1 - it : it;
    if (tid < D) {
      zv[tid] += p.wz[(bh * F + f) * D + tid];
      p.as[(bh * F + it) * D + tid] = zv[tid];
    }
    __syncthreads();
    if (c.reverse && it == 0) break;
    const int fa = fa_of(it);
    if (it - 1 >= 0 && !(c.reverse && it - 1 == 0)) fetch(fa_of(it - 1), gn);
    const float g = c.decay[bh * F + fa];
    const float y = matvec(zv);  // G_pos is symmetric
    float part_dd = 0.f;
    __syncthreads();  // every thread has read zv and ps
    if (part == 0) {
      const float dzp = zv[row] - y;
      if (it > 0) part_dd = dzp * p.zs[(bh * F + it - 1) * D + row];
      zv[row] = g * dzp;
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) part_dd += __shfl_xor(part_dd, off, 64);
    if (lane == 0) red[w] = part_dd;
    __syncthreads();
    if (tid == 0) {
      float sum = 0.f;
      for (int q = 0; q < 16; ++q) sum += red[q];
      p.ddz[bh * F + fa] = sum;
    }
#pragma unroll
    for (int m = 0; m < M; ++m) gc[m] = gn[m];
  }
}

// ---- S stream token gradients ---------------------------------------------------------------
// As cbwd_tok_kernel (gdn_cambwd.hip) with token-major operands: one workgroup of D/16 waves per
// (b, h, step, part of the frame's 64-token blocks); wave w owns output channels 16 w .. 16 w + 15
// and keeps its rows of the step's D x D matrices as register fragments, S in a first pass
// (dq_rot), S_prev^T, A^T, A and S_prev in a second (dv, dbeta, dk_rot).  A block's token rows
// (dnum in the first pass; k_rot and v in the second) arrive in LDS by direct buffer-to-LDS
// loads issued one block ahead; dnum is then split into a hi/lo tile, k_rot copied into the hi
// half of a tile (bf16 values are exact, so the products against it take two terms).
template <int D>
__global__ __launch_bounds__(D * 4) void bbwd_tok_kernel(const BigdnBwdParams p, int nsplit) {
  constexpr int NW = D / 16, NT = NW * 64, KK = D / 32;
  constexpr int kT = D + 8;  // LDS row stride of a [token][D] tile (elements)
  __shared__ __attribute__((aligned(16))) bf16 tl[2][2][64 * kT];  // [tile][hi, lo]
  // raw token rows: dnum fp32 [64][D] in the first pass; k_rot and v bf16 [64][D] in the second
  __shared__ __attribute__((aligned(16))) float raw[64 * D];
  __shared__ float red[NW][64];
  bf16* const rawk = reinterpret_cast<bf16*>(raw);
  bf16* const rawv = rawk + 64 * D;
  const CamBwdParams& c = p.cam;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, li = lane & 15, lq = lane >> 4;
  const int nblk = c.S / 64;
  const int bid = xcd_logical(blockIdx.x, gridDim.x);
  const int part = bid % nsplit;
  const long sb = bid / nsplit;
  const int F = c.F;
  const int it = (int)(sb % F);
  const long bh = sb / F;
  const int b = (int)(bh / c.H), h = (int)(bh % c.H);
  const long N = (long)F * c.S;
  const size_t DD = (size_t)D * D;
  const int b0 = part * nblk / nsplit, b1 = (part + 1) * nblk / nsplit;
  const int f = c.reverse ? F - 1 - it : it;
  const bool absorb = !(c.reverse && it == 0);
  const int fa = c.reverse ? f + 1 : f;  // used only when absorb

  // p.acc: this direction's dbeta and ddecay are added to the arrays' contents
  if (part == 0 && tid == 0) {
    if (absorb) {
      float s = p.ddz[bh * F + fa];
      for (int cb = 0; cb < D / kScanCB; ++cb) s += c.ddecay_part[((size_t)bh * F + fa) * (D / kScanCB) + cb];
      c.ddecay[bh * F + fa] = (p.acc ? c.ddecay[bh * F + fa] : 0.f) + (it > 0 ? s : 0.f);
    } else if (!p.acc) {
      c.ddecay[bh * F] = 0.f;
    }
  }

  typedef bf16x8 Frag[KK][2];
  auto load_a = [&](const bf16* M, Frag& a) {
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) {
      const size_t ro = (size_t)(16 * w + li) * D + 32 * kk + 8 * lq;
      a[kk][0] = *reinterpret_cast<const bf16x8*>(M + ro);
      a[kk][1] = *reinterpret_cast<const bf16x8*>(M + c.lo + ro);
    }
  };
  const bool prev = it > 0;
  const float g = absorb ? c.decay[bh * F + fa] : 0.f;
  const int wu = __builtin_amdgcn_readfirstlane(w);  // the wave index, as a scalar

  // dnum rows of tokens t0 .. t0 + 63 ([B,N,H,D]: token stride H D) into raw as fp32 [64][D]:
  // an instruction moves 1 KB (256 / D rows, 16 bytes per lane), wave w instructions w, w + NW ..
  auto fetch_dnum = [&](long t0) {
    constexpr int RPI = 256 / D;  // rows per instruction
    const float* src = p.dnum + (((long)b * N + t0) * c.H + h) * D;
    const dma::i32x4 rs = dma::make_rsrc(src, (uint32_t)((63 * (long)c.H * D + D) * 4));
#pragma unroll
    for (int i = 0; i < D / (4 * NW); ++i) {
      const int ins = wu + NW * i;
      const int row = RPI * ins + lane / (D / 4), piece = lane % (D / 4);
      dma::dma16(rs, (uint32_t)((row * c.H * D + 4 * piece) * 4), 0, dma::lds_addr(raw + 1024 / 4 * ins));
    }
  };
  // k_rot or v rows of tokens t0 .. t0 + 63 ([B,H,N,D] bf16, contiguous) into dst [64][D]
  auto fetch_rows = [&](const __bf16* x, long t0, bf16* dst) {
    const dma::i32x4 rs = dma::make_rsrc(x + (bh * N + t0) * D, 64 * D * 2);
#pragma unroll
    for (int i = 0; i < D / (8 * NW); ++i) {
      const int ins = wu + NW * i;
      dma::dma16(rs, (uint32_t)(1024 * ins + 16 * lane), 0, dma::lds_addr(dst + 512 * ins));
    }
  };
  // raw dnum into tile 0 as a hi/lo pair; raw k_rot into tile 1's hi half
  auto split_dnum = [&]() {
#pragma unroll
    for (int e = tid; e < 64 * D / 8; e += NT) {
      const int t = e / (D / 8), d = 8 * (e % (D / 8));
      const f32x4 x0 = *reinterpret_cast<const f32x4*>(raw + t * D + d);
      const f32x4 x1 = *reinterpret_cast<const f32x4*>(raw + t * D + d + 4);
      bf16x8 xh, xl;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        GDN_SPLIT(x0[j], xh[j], xl[j]);
        GDN_SPLIT(x1[j], xh[4 + j], xl[4 + j]);
      }
      *reinterpret_cast<bf16x8*>(&tl[0][0][t * kT + d]) = xh;
      *reinterpret_cast<bf16x8*>(&tl[0][1][t * kT + d]) = xl;
    }
  };
  auto copy_k = [&]() {
#pragma unroll
    for (int e = tid; e < 64 * D / 8; e += NT) {
      const int t = e / (D / 8), d = 8 * (e % (D / 8));
      *reinterpret_cast<bf16x8*>(&tl[1][0][t * kT + d]) = *reinterpret_cast<const bf16x8*>(rawk + t * D + d);
    }
  };
  // C[cc] (channels 16 w + 4 lq + e, tokens 16 cc + li) = M X^T for the wave's fragments and
  // tile T; LO: the tile's lo half is used (else the tile holds exact bf16 values)
  auto prod = [&](const Frag& a, int T, bool LO, f32x4 (&C)[4]) {
#pragma unroll
    for (int cc = 0; cc < 4; ++cc) C[cc] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) {
      bf16x8 bh_[4], bl[4];
#pragma unroll
      for (int cc = 0; cc < 4; ++cc) {
        bh_[cc] = lds8(&tl[T][0][(16 * cc + li) * kT + 32 * kk + 8 * lq]);
        if (LO) bl[cc] = lds8(&tl[T][1][(16 * cc + li) * kT + 32 * kk + 8 * lq]);
      }
#pragma unroll
      for (int cc = 0; cc < 4; ++cc) {
        if (LO) {
          C[cc] = mma3(a[kk][0], a[kk][1], bh_[cc], bl[cc], C[cc]);
        } else {
          C[cc] = mma16(a[kk][0], bh_[cc], C[cc]);
          C[cc] = mma16(a[kk][1], bh_[cc], C[cc]);
        }
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  auto put = [&](int T, int t, int i0, const f32x4& x) {
    bf16x4 xh, xl;
#pragma unroll
    for (int e = 0; e < 4; ++e) GDN_SPLIT(x[e], xh[e], xl[e]);
    *reinterpret_cast<bf16x4*>(&tl[T][0][t * kT + i0]) = xh;
    *reinterpret_cast<bf16x4*>(&tl[T][1][t * kT + i0]) = xl;
  };
  const int ch0 = 16 * w + 4 * lq;  // first of a lane's four channels
  auto store4 = [&](float* out, long t, const f32x4& x) {
    *reinterpret_cast<f32x4*>(out + (bh * N + t) * D + ch0) = x;
  };

  // ---- pass 1, dq_rot = S dnum for the output frame's tokens
  fetch_dnum((long)f * c.S + 64 * b0);
  {
    Frag aS;
    load_a(c.Sp + ((size_t)bh * F + it) * DD, aS);
    for (int blk = b0; blk < b1; ++blk) {
      const int s0 = 64 * blk;
      dma::wait_vm0();
      __syncthreads();  // the rows are in; the previous block is done with tile 0
      split_dnum();
      __syncthreads();
      if (blk + 1 < b1) {
        fetch_dnum((long)f * c.S + s0 + 64);
      } else if (absorb) {  // the second pass's first block
        fetch_rows(p.k_rot, (long)fa * c.S + 64 * b0, rawk);
        fetch_rows(p.v, (long)fa * c.S + 64 * b0, rawv);
      }
      f32x4 C[4];
      prod(aS, 0, true, C);
#pragma unroll
      for (int cc = 0; cc < 4; ++cc) store4(p.dq_rot, (long)f * c.S + s0 + 16 * cc + li, C[cc]);
    }
  }
  if (!absorb) {
    for (int blk = b0; blk < b1; ++blk) {
      const int s0 = 64 * blk;
#pragma unroll
      for (int cc = 0; cc < 4; ++cc) {
        const long t = s0 + 16 * cc + li;
        store4(p.dk_rot, t, f32x4{0.f, 0.f, 0.f, 0.f});
        store4(p.dv, t, f32x4{0.f, 0.f, 0.f, 0.f});
      }
      if (tid < 64 && !p.acc) c.dbeta[bh * N + s0 + tid] = 0.f;
    }
    return;
  }
  // ---- pass 2, the absorbed frame's tokens
  Frag aPT, aDT, aA, aSP;
  load_a(c.AbT + ((size_t)bh * F + it) * DD, aDT);
  load_a(c.Ab + ((size_t)bh * F + it) * DD, aA);
  if (prev) {
    load_a(c.SpT + ((size_t)bh * F + it - 1) * DD, aPT);
    load_a(c.Sp + ((size_t)bh * F + it - 1) * DD, aSP);
  }
  for (int blk = b0; blk < b1; ++blk) {
    const int s0 = 64 * blk;
    const long ta = (long)fa * c.S + s0;
    dma::wait_vm0();
    __syncthreads();  // k_rot and v rows are in; the previous block is done with both tiles
    copy_k();
    __syncthreads();
    if (blk + 1 < b1) fetch_rows(p.k_rot, ta + 64, rawk);
    float bcol[4];
#pragma unroll
    for (int cc = 0; cc < 4; ++cc) bcol[cc] = c.beta[bh * N + ta + 16 * cc + li];
    f32x4 P[4], Dd[4];
    if (prev) {
      prod(aPT, 1, false, P);
    } else {
#pragma unroll
      for (int cc = 0; cc < 4; ++cc) P[cc] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
    prod(aDT, 1, false, Dd);
    float db[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int cc = 0; cc < 4; ++cc) {
      const int t = 16 * cc + li;
      const bf16x4 vv = *reinterpret_cast<const bf16x4*>(rawv + t * D + ch0);
      f32x4 dvv;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float rr = (float)vv[e] - g * P[cc][e];
        const float dd = Dd[cc][e];
        dvv[e] = bcol[cc] * dd;
        db[cc] += dd * rr;
        P[cc][e] = bcol[cc] * rr;
        Dd[cc][e] = -bcol[cc] * dd;
      }
      store4(p.dv, ta + t, dvv);
    }
    __syncthreads();  // every wave is done with the k tile and the v rows
    if (blk + 1 < b1) fetch_rows(p.v, ta + 64, rawv);
#pragma unroll
    for (int cc = 0; cc < 4; ++cc) {
      put(1, 16 * cc + li, ch0, P[cc]);
      put(0, 16 * cc + li, ch0, Dd[cc]);
    }
#pragma unroll
    for (int cc = 0; cc < 4; ++cc) {
      db[cc] += __shfl_xor(db[cc], 16, 64);
      db[cc] += __shfl_xor(db[cc], 32, 64);
      if (lq == 0) red[w][16 * cc + li] = db[cc];
    }
    __syncthreads();
    if (tid < 64) {
      float sum = 0.f;
#pragma unroll
      for (int i = 0; i < NW; ++i) sum += red[i][tid];
      c.dbeta[bh * N + ta + tid] = (p.acc ? c.dbeta[bh * N + ta + tid] : 0.f) + sum;
    }
    f32x4 K1[4];
    prod(aA, 1, true, K1);
    if (prev) {
      f32x4 K2[4];
      prod(aSP, 0, true, K2);
#pragma unroll
      for (int cc = 0; cc < 4; ++cc) K1[cc] = K1[cc] + g * K2[cc];
    }
#pragma unroll
    for (int cc = 0; cc < 4; ++cc) store4(p.dk_rot, ta + 16 * cc + li, K1[cc]);
  }
}

// Workgroups per (b, h, step) for the token kernel: enough for about one per CU in total.
inline int tok_split(long bhf, int nblk) {
  long s = (256 + bhf - 1) / bhf;
  return (int)(s < 1 ? 1 : s > nblk ? nblk : s);
}

// ---- z stream token gradients ----------------------------------------------------------------
// blockIdx.x = (bh * F + it) * (S / 64) + token block; wave w takes 16 tokens.  A lane owns
// four consecutive channels, so D / 4 lanes cover a token and a wave works on 256 / D tokens at
// once (16-byte stores, 8-byte k_pos loads, reductions over the token's lanes only).  Runs
// after bbwd_tok_kernel, whose dbeta it adds to.
template <int D>
__global__ __launch_bounds__(256) void bbwd_ztok_kernel(const BigdnBwdParams p) {
  constexpr int LPT = D / 4, TPW = 64 / LPT;  // lanes per token, tokens per wave at once
  typedef bf16 bf16x4_t __attribute__((ext_vector_type(4)));
  const CamBwdParams& c = p.cam;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int tl = lane / LPT, ch = 4 * (lane % LPT);  // token slot, first channel
  const int nblk = c.S / 64;
  const int bid = xcd_logical(blockIdx.x, gridDim.x);
  const int blk = bid % nblk;
  const long sb = bid / nblk;
  const int F = c.F;
  const int it = (int)(sb % F);
  const long bh = sb / F;
  const long N = (long)F * c.S;
  const int f = c.reverse ? F - 1 - it : it;
  const bool absorb = !(c.reverse && it == 0);
  const int fa = c.reverse ? f + 1 : f;
  const int s0 = 64 * blk + 16 * w;
  const f32x4 za = *reinterpret_cast<const f32x4*>(p.zs + (bh * F + it) * D + ch);
  const f32x4 av = *reinterpret_cast<const f32x4*>(p.as + (bh * F + it) * D + ch);
  f32x4 zp = f32x4{0.f, 0.f, 0.f, 0.f};
  if (absorb && it > 0)
    zp = c.decay[bh * F + fa] * *reinterpret_cast<const f32x4*>(p.zs + (bh * F + it - 1) * D + ch);
#pragma unroll 4
  for (int i = tl; i < 16; i += TPW) {
    const long t = (long)f * c.S + s0 + i;  // output frame
    *reinterpret_cast<f32x4*>(p.dq_pos + (bh * N + t) * D + ch) = p.dden[bh * N + t] * za;
  }
  if (!absorb) {
#pragma unroll 4
    for (int i = tl; i < 16; i += TPW)
      *reinterpret_cast<f32x4*>(p.dk_pos + (bh * N + s0 + i) * D + ch) = f32x4{0.f, 0.f, 0.f, 0.f};
    return;
  }
#pragma unroll 4
  for (int i = tl; i < 16; i += TPW) {
    const long t = (long)fa * c.S + s0 + i;  // absorbed frame
    const float bt = c.beta[bh * N + t];
    const bf16x4_t kv = *reinterpret_cast<const bf16x4_t*>(p.k_pos + (bh * N + t) * D + ch);
    float zh = 0.f, ee = 0.f;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float kp = (float)kv[j];
      zh += kp * zp[j];
      ee += kp * av[j];
    }
#pragma unroll
    for (int off = LPT / 2; off > 0; off >>= 1) {
      zh += __shfl_xor(zh, off, 64);
      ee += __shfl_xor(ee, off, 64);
    }
    const float e1 = 1.f - zh;
    *reinterpret_cast<f32x4*>(p.dk_pos + (bh * N + t) * D + ch) = av * (bt * e1) - (bt * ee) * zp;
    if (lane % LPT == 0) c.dbeta[bh * N + t] += ee * e1;
  }
}

template <int D>
hipError_t launch_d(const BigdnBwdParams& p, hipStream_t stream) {
  const CamBwdParams& c = p.cam;
  const long bh = (long)c.B * c.H;
  if (!c.reuse)  // the per-frame statistics (and the z stream's vectors) of every direction
    hipLaunchKernelGGL((bbwd_stats_kernel<D>), dim3(bh * c.F * 4), dim3(256), 0, stream, p);
  hipError_t e = launch_cam_bwd_scan(c, stream);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((bbwd_zscan_kernel<D>), dim3(bh), dim3(1024), 0, stream, p);
  const int ns = tok_split(bh * c.F, c.S / 64);
  hipLaunchKernelGGL((bbwd_tok_kernel<D>), dim3(bh * c.F * ns), dim3(D * 4), 0, stream, p, ns);
  const dim3 tg(bh * c.F * (c.S / 64));
  hipLaunchKernelGGL((bbwd_ztok_kernel<D>), tg, dim3(256), 0, stream, p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_bigdn_dir_bwd(const BigdnBwdParams& p, hipStream_t stream) {
  return p.cam.D == 128 ? launch_d<128>(p, stream) : launch_d<64>(p, stream);
}

}  // namespace gdn

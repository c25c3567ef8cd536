// gdn_bigdn.hip -- BiGDN front end (gdn_prep) and the frame-level bidirectional scan
// (bigdn_fwd) for gfx950.
//
// Front end (SANA fused_gdn.py page: _precompute_inv_rms, _fused_qk_inv_rms_kernel,
// prepare_rope_tables and the load path of _fused_gdn_kernel), per token (b, n):
//   inv_rms = 1 / sqrt(sum over all H*D channels of x^2 / (H*D) + eps)     (q and k)
//   x_pos = relu(x * inv_rms * w[h*D + d]) (times k_scale for k)
//   x_rot[d] = x_pos[d] cos[n,d] + x_pos[d^1] sin[n,d]
//
// Frame scan.  Every token of frame f reads the same decayed state (the frame loop of
// _fused_gdn_kernel), so absorbing frame f is the affine map
//   S <- d_f (S - G_f S) + U_f,   G_f = K_rot^T diag(beta) K_rot,  U_f = K_rot^T diag(beta) V
//   z <- d_f (z - Gz_f z) + uz_f, Gz_f = K_pos^T diag(beta) K_pos,  uz_f = K_pos^T beta
// (the product form state <- state W_f + U_f of _torch_cam_scan_single_chunk on the SANA
// fused_cam_gdn.py page).  The forward direction's output for frame f uses S_f (inclusive);
// the reverse direction's uses R_f, built from frames > f with R_{F-1} = 0 and
// R_f = d_{f+1}(R_{f+1} - G_{f+1} R_{f+1}) + U_{f+1} (flip-and-shift, same page).  Both
// directions share G, U, Gz, uz, and num/den only need the sums S_f + R_f, z_f + zR_f:
//   num = Q_rot (S_f + R_f),   den = Q_pos . (z_f + zR_f).
//
// Kernels: rms (inv-RMS per token; with outputs it is gdn_prep), frame_stats (G, U, Gz, uz
// per (b, h, f) from k, v with the prep applied on the fly, one workgroup per frame), scan
// (32-column blocks of the state per (b, h) and direction, the two directions concurrently;
// writes every frame's state), out (num, den per 64-token blocks, adding the directions).
// Products use fp16 operands and fp32 accumulation; the scanned state is fp32.
#include "gdn_device.h"
#include "gdn_dma.h"
#include "gdn_frame.h"
#include "gdn_internal.h"
#include "gdn_tiles.h"

namespace gdn {

namespace {

constexpr int kPrepThreads = 256;

// Sums of x and y over a 256-thread workgroup (every thread gets both).
__device__ __forceinline__ void block_sum2_256(float& x, float& y, float* red) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) {
    x += __shfl_xor(x, off, 64);
    y += __shfl_xor(y, off, 64);
  }
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  if (lane == 0) {
    red[wave] = x;
    red[4 + wave] = y;
  }
  __syncthreads();
  x = red[0] + red[1] + red[2] + red[3];
  y = red[4] + red[5] + red[6] + red[7];
}

// Loads 8 consecutive channels (16 bytes) of bf16 as floats.
__device__ __forceinline__ void load8f(const bf16* p, float* out) {
  const bf16x8 v = *reinterpret_cast<const bf16x8*>(p);
#pragma unroll
  for (int j = 0; j < 8; ++j) out[j] = (float)v[j];
}

__device__ __forceinline__ void load8f(const float* p, float* out) {
  const f32x4 a = *reinterpret_cast<const f32x4*>(p);
  const f32x4 b = *reinterpret_cast<const f32x4*>(p + 4);
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    out[j] = a[j];
    out[4 + j] = b[j];
  }
}

// Front end of W channels d0..d0+W-1 (W even, d0 a multiple of W, so every RoPE pair is
// inside).
template <int W>
__device__ __forceinline__ void prep_w(const float* x, float inv, const float* w, const float* cs,
                                       const float* sn, float scale, float* pos, float* rot) {
#pragma unroll
  for (int j = 0; j < W; ++j) {
    const float y = x[j] * inv * w[j];
    pos[j] = (y > 0.f ? y : 0.f) * scale;
  }
#pragma unroll
  for (int j = 0; j < W; ++j) rot[j] = pos[j] * cs[j] + pos[j ^ 1] * sn[j];
}

__device__ __forceinline__ void prep8(const float* x, float inv, const float* w, const float* cs,
                                      const float* sn, float scale, float* pos, float* rot) {
  prep_w<8>(x, inv, w, cs, sn, scale, pos, rot);
}

__device__ __forceinline__ void store8(bf16* p, const float* x) {
  bf16x8 v;
#pragma unroll
  for (int j = 0; j < 8; ++j) v[j] = (bf16)x[j];
  *reinterpret_cast<bf16x8*>(p) = v;
}

// One workgroup per token (b, n): inverse RMS of q and k over all H*D channels, and, when
// any output pointer is set, the prepped head-major tensors.
__global__ __launch_bounds__(kPrepThreads) void rms_prep_kernel(const PrepParams p) {
  __shared__ float red[8];
  const long bn = blockIdx.x;
  const int b = bn / p.N, n = bn % p.N;
  const int C = p.H * p.D, groups = C / 8;
  const bf16* row = static_cast<const bf16*>(p.qkv) + bn * 3L * C;
  // the RoPE tables of token n as (cos, sin) fp16 pairs, 8 channels (32 bytes) per thread;
  // loaded before the reductions so the loads overlap them
  const bool tab = p.rope_h && b == 0 && threadIdx.x < p.D / 8;
  float cs[8], sn[8];
  if (tab) {
    load8f(p.rope_cos + (long)n * p.D + 8 * threadIdx.x, cs);
    load8f(p.rope_sin + (long)n * p.D + 8 * threadIdx.x, sn);
  }
  float sq = 0.f, sk = 0.f;
  for (int gi = threadIdx.x; gi < groups; gi += kPrepThreads) {
    float xq[8], xk[8];
    load8f(row + gi * 8, xq);
    load8f(row + C + gi * 8, xk);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      sq += xq[j] * xq[j];
      sk += xk[j] * xk[j];
    }
  }
  block_sum2_256(sq, sk, red);
  const float iq = rsqrtf(sq / (float)C + p.eps), ik = rsqrtf(sk / (float)C + p.eps);
  if (threadIdx.x == 0) {
    if (p.q_inv_rms) p.q_inv_rms[bn] = iq;
    if (p.k_inv_rms) p.k_inv_rms[bn] = ik;
  }
  if (tab) {
    f16x8 lo, hi;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      lo[2 * j] = (f16)cs[j];
      lo[2 * j + 1] = (f16)sn[j];
      hi[2 * j] = (f16)cs[4 + j];
      hi[2 * j + 1] = (f16)sn[4 + j];
    }
    f16x8* dst = reinterpret_cast<f16x8*>(p.rope_h + ((long)n * p.D + 8 * threadIdx.x) * 2);
    dst[0] = lo;
    dst[1] = hi;
  }
  if (!(p.q_rot || p.k_rot || p.q_pos || p.k_pos || p.v_hm)) return;
  for (int gi = threadIdx.x; gi < groups; gi += kPrepThreads) {
    const int h = gi / (p.D / 8), d0 = (gi % (p.D / 8)) * 8;
    const long o = (((long)b * p.H + h) * p.N + n) * p.D + d0;
    float x[8], w[8], cs[8], sn[8], pos[8], rot[8];
    load8f(p.rope_cos + (long)n * p.D + d0, cs);
    load8f(p.rope_sin + (long)n * p.D + d0, sn);
    load8f(row + gi * 8, x);
    load8f(p.q_norm_w + gi * 8, w);
    prep8(x, iq, w, cs, sn, 1.f, pos, rot);
    if (p.q_pos) store8(static_cast<bf16*>(p.q_pos) + o, pos);
    if (p.q_rot) store8(static_cast<bf16*>(p.q_rot) + o, rot);
    load8f(row + C + gi * 8, x);
    load8f(p.k_norm_w + gi * 8, w);
    prep8(x, ik, w, cs, sn, p.k_scale, pos, rot);
    if (p.k_pos) store8(static_cast<bf16*>(p.k_pos) + o, pos);
    if (p.k_rot) store8(static_cast<bf16*>(p.k_rot) + o, rot);
    if (p.v_hm) *reinterpret_cast<uint4*>(static_cast<bf16*>(p.v_hm) + o) =
        *reinterpret_cast<const uint4*>(row + 2 * C + gi * 8);
  }
}

// ---- frame statistics -------------------------------------------------------------------
// One workgroup of twelve waves per (b, h, frame) computes all three statistics over the
// frame's tokens, 64 at a time:
//   G = K_rot^T diag(beta) K_rot,  U = K_rot^T diag(beta) V,  Gz = K_pos^T diag(beta) K_pos,
//   uz = K_pos^T beta.
// beta >= 0 splits as sqrt(beta) on both sides, so three fp16 token tiles serve all of them:
// sqrt(beta) K_rot, sqrt(beta) V and sqrt(beta) K_pos.
// Prep: every thread takes (token, 8-channel octet) items -- 16 threads per token row, so the
// qkv loads are whole 256-byte rows -- applies the front end once and writes the three rows
// into LDS with 16-byte stores.  The tiles are double-buffered: a block's prep runs while the
// previous block's products do (one barrier per block), and an item's inputs are loaded one
// block ahead of its prep (the RoPE table rows by direct-to-LDS transfers, which hold no
// registers).
// Products: wave w accumulates quadrant (w % 4) of statistic w / 4; both operands contract
// over tokens, so they come from the row-major tiles by LDS transpose reads
// (ds_read_b64_tr_b16: within a 16-lane group, lane n receives element j of the 8-byte piece
// addressed by lane 4j + n / 4, halfword n % 4).  A transpose-read operand pair for
// (32-block Gb, half t) gives lane (li, lq) channel 32Gb + 8(li >> 2) + 4t + (li & 3) at
// tokens 8lq + j; the accumulator of such a pair of operands holds row channel
// 32Gb + 8lq + 4t + e and column channel 32Gb' + 8(li >> 2) + 4t' + (li & 3).
constexpr int kStatThreads = 768;

template <int D>
__global__ __launch_bounds__(kStatThreads) void frame_stats_kernel(const BigdnParams p) {
  using namespace dma;
  constexpr int kT = 64;         // tokens per block
  constexpr int kOct = D / 8;    // octets per token row
  constexpr int kNG = D / 64;    // 32-channel blocks per quadrant side
  // Items (token, octet) of a block: this thread takes it = tid + kStatThreads i.
  constexpr int kItems = (kT * kOct + kStatThreads - 1) / kStatThreads;
  constexpr int kI1 = kT * kOct > kStatThreads ? kT * kOct - kStatThreads : 0;  // threads with a 2nd item
  // tiles: 0 sqrt(beta) K_rot, 1 sqrt(beta) V, 2 sqrt(beta) K_pos  ([64][D] fp16, tix_x64),
  // two buffers; then the RoPE table rows of the next block's items ((cos, sin) fp16 pairs,
  // 16-byte pieces j = channels 4j .. 4j + 3 of the octet) at the transferring lane's own slot
  constexpr int kTiles = 2 * 3 * kT * D * 2;
  constexpr int kTab = (2 * kStatThreads + 2 * kI1) * 16;
  __shared__ __attribute__((aligned(1024))) char smem[kTiles + kTab];
  typedef f16 tile_t[3][kT * D];
  tile_t* tl = reinterpret_cast<tile_t*>(smem);
  const int bhf = blockIdx.x;
  const int f = bhf % p.F, h = (bhf / p.F) % p.H, b = bhf / (p.F * p.H);
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int li = lane & 15, lq = lane >> 4;
  const int C = p.H * D;
  const bf16* qkv = static_cast<const bf16*>(p.qkv);
  const int m = wave >> 2, qi = (wave & 3) >> 1, qj = wave & 1;
  const int ta = m == 2 ? 2 : 0, tb = m;  // operand tiles of statistic m
  f32x4 acc[kNG][2][kNG][2];
#pragma unroll
  for (int a = 0; a < kNG; ++a)
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int c = 0; c < kNG; ++c)
#pragma unroll
        for (int u = 0; u < 2; ++u) acc[a][t][c][u] = f32x4{0.f, 0.f, 0.f, 0.f};
  // this thread's octet (fixed: kStatThreads is a multiple of kOct) and running beta k_pos
  const int oct = tid % kOct;
  float uzr[8], w8[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) uzr[j] = 0.f;
  load8f(p.k_norm_w + h * D + 8 * oct, w8);

  // An item's k, v rows, inverse RMS and beta are loaded into registers, and its RoPE table
  // rows transferred into LDS, one block ahead of its prep.
  bf16x8 kx[kItems], vx[kItems];
  float ivx[kItems], btx[kItems];
  const long frame_tok = (long)f * p.S;
  const i32x4 rtab = make_rsrc(p.rope_h + frame_tok * D * 2, (uint32_t)p.S * D * 4);
  const uint32_t tab = lds_addr(smem + kTiles);
  auto tab_off = [&](int i, int j) {  // byte offset of piece j of item i of this thread's wave
    return i == 0 ? (j * kStatThreads + 64 * wave) * 16 : (2 * kStatThreads + j * kI1 + 64 * wave) * 16;
  };
  auto load_items = [&](int t0) {
#pragma unroll
    for (int i = 0; i < kItems; ++i) {
      const int it = tid + kStatThreads * i;
      if (it < kT * kOct) {
        const int s = it / kOct;
        const long n = frame_tok + t0 + s, bn = (long)b * p.N + n;
        const bf16* krow = qkv + bn * 3L * C + C + (long)h * D + 8 * oct;
        kx[i] = *reinterpret_cast<const bf16x8*>(krow);
        vx[i] = *reinterpret_cast<const bf16x8*>(krow + C);
        ivx[i] = p.k_inv_rms[bn];
        btx[i] = p.beta[(((long)b * p.H + h) * p.F + f) * p.S + t0 + s];
        const uint32_t vo = ((t0 + s) * D + 8 * oct) * 4;
#pragma unroll
        for (int j = 0; j < 2; ++j) dma16(rtab, vo + 16 * j, 0, tab + tab_off(i, j));
      }
    }
  };
  auto prep = [&](int buf) {
#pragma unroll
    for (int i = 0; i < kItems; ++i) {
      const int it = tid + kStatThreads * i;
      if (it < kT * kOct) {
        const int s = it / kOct;
        float x[8], v[8], pos[8], rot[8], cs[8], sn[8];
        const char* tp = smem + kTiles + 16 * lane;
        const f16x8 t0 = *reinterpret_cast<const f16x8*>(tp + tab_off(i, 0));
        const f16x8 t1 = *reinterpret_cast<const f16x8*>(tp + tab_off(i, 1));
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          cs[j] = (float)t0[2 * j];
          sn[j] = (float)t0[2 * j + 1];
          cs[4 + j] = (float)t1[2 * j];
          sn[4 + j] = (float)t1[2 * j + 1];
        }
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          x[j] = (float)kx[i][j];
          v[j] = (float)vx[i][j];
        }
        prep8(x, ivx[i], w8, cs, sn, p.k_scale, pos, rot);
        const float bt = btx[i], sb = sqrtf(bt);
        f16x8 r0, r1, r2;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          r0[j] = (f16)(sb * rot[j]);
          r1[j] = (f16)(sb * v[j]);
          r2[j] = (f16)(sb * pos[j]);
          uzr[j] += bt * pos[j];
        }
        const int ix = tix_x64(s, 8 * oct);
        *reinterpret_cast<f16x8*>(&tl[buf][0][ix]) = r0;
        *reinterpret_cast<f16x8*>(&tl[buf][1][ix]) = r1;
        *reinterpret_cast<f16x8*>(&tl[buf][2][ix]) = r2;
      }
    }
  };
  auto mma_block = [&](int buf) {
    const f16* pa = tl[buf][ta];
    const f16* pb = tl[buf][tb];
    // lane-derived LDS addresses recomputed per block instead of held across the loop
    int ln = lane;
    asm volatile("" : "+v"(ln));
    const int lq = ln >> 4, trj = (ln >> 2) & 3, trc = ln & 3;
#pragma unroll
    for (int P = 0; P < kT / 32; ++P) {
      f16x8 af[kNG][2], bf[kNG][2];
#pragma unroll
      for (int g = 0; g < kNG; ++g)
#pragma unroll
        for (int t = 0; t < 2; ++t) {
          const int ca = 32 * (kNG * qi + g) + 8 * trc + 4 * t;
          const int cb = 32 * (kNG * qj + g) + 8 * trc + 4 * t;
          af[g][t] = tr_pair(&pa[tix_x64(32 * P + 8 * lq + trj, ca)], &pa[tix_x64(32 * P + 8 * lq + 4 + trj, ca)]);
          bf[g][t] = tr_pair(&pb[tix_x64(32 * P + 8 * lq + trj, cb)], &pb[tix_x64(32 * P + 8 * lq + 4 + trj, cb)]);
        }
#pragma unroll
      for (int a = 0; a < kNG; ++a)
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
          for (int c = 0; c < kNG; ++c)
#pragma unroll
            for (int u = 0; u < 2; ++u) acc[a][t][c][u] = mma16(af[a][t], bf[c][u], acc[a][t][c][u]);
    }
  };

  // Block n's products run while block n + 1 is prepped into the other tile buffer and block
  // n + 2's inputs are in flight; one barrier per block.  Everything a prep reads was issued
  // a whole block earlier, so it waits for all of this thread's loads.
  const int nb = p.S / kT;
  load_items(0);
  wait_vm0();
  prep(0);
  if (nb > 1) load_items(kT);
  __syncthreads();
  for (int n = 0; n < nb; ++n) {
    if (n + 1 < nb) {
      wait_vm0();
      prep((n + 1) & 1);
      if (n + 2 < nb) load_items((n + 2) * kT);
    }
    mma_block(n & 1);
    __syncthreads();
  }
  // epilogue: row channel 32(kNG qi + a) + 8lq + 4t + e, column 32(kNG qj + c) + 8(li >> 2) + 4u + (li & 3).
  // G, Gz and U go out in the scan's operand layouts (g_lane_index, u_lane_index): U's four
  // rows e are one 16-byte store; G and Gz, being symmetric, are stored transposed, so their
  // four e become four consecutive columns of one row (8 bytes).
  const long mat = (((long)b * p.H + h) * p.F + f) * (long)D * D;
#pragma unroll
  for (int a = 0; a < kNG; ++a)
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int c = 0; c < kNG; ++c)
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          const int d1 = 32 * (kNG * qi + a) + 8 * lq + 4 * t;
          const int d2 = 32 * (kNG * qj + c) + 8 * (li >> 2) + 4 * u + (li & 3);
          const f32x4 x = acc[a][t][c][u];
          if (m == 1) {
            *reinterpret_cast<f32x4*>(p.U + mat + u_lane_index<D>(d1, d2)) = x;
          } else {
            f16x4 v;
#pragma unroll
            for (int e = 0; e < 4; ++e) v[e] = (f16)x[e];
            *reinterpret_cast<f16x4*>((m == 0 ? p.G : p.Gz) + mat + g_lane_index<D>(d2, d1)) = v;
          }
        }
  // uz: sum of the per-thread partial sums of each channel (threads of one octet)
  __syncthreads();
  float* red = reinterpret_cast<float*>(smem);  // [kStatThreads][8]
#pragma unroll
  for (int j = 0; j < 8; ++j) red[tid * 8 + j] = uzr[j];
  __syncthreads();
  if (tid < D) {
    const int o = tid / 8, j = tid % 8;
    float x = 0.f;
    for (int t = o; t < kStatThreads; t += kOct) x += red[t * 8 + j];
    p.uz[(((long)b * p.H + h) * p.F + f) * D + tid] = x;
  }
}

// ---- scan -------------------------------------------------------------------------------
// The forward and reverse scans are independent, so they run in separate workgroups: per
// (b, h, direction), one workgroup per 32-column block cb of the state plus one (cb == D/32)
// for z, which runs as a block whose columns all hold z (A operand Gz, U the uz entries of
// each row).  The forward scan writes S_f^T after absorbing frame f; the reverse scan writes
// R_f^T, built from frames > f (R_{F-1} = 0), both fp16 (z and zR in fp32); the output
// kernel adds the two.  Wave w owns state rows (D/4)w .. (D/4)w + D/4 - 1 of the block.
// The state lives in registers (fp32) and is exchanged through LDS (fp16 transposed copy,
// double-buffered so one barrier per frame suffices) as the B operand of G S.
//
// Operands are staged per wave in a three-frame LDS ring by direct-to-LDS transfers issued
// two frames ahead; each wave reads back only what it transferred (at its own lane slots, so
// without bank conflicts), so a counted wait on its own loads is the only synchronisation.
// A ring stage holds, per wave, the lane-ordered G (or Gz) operands (kNG KB) and the U tiles
// (kRT kCT KB).  A lane holds the decays of 64 consecutive steps and reads the current one by
// lane index.
template <int D>
__global__ __launch_bounds__(256) void scan_kernel(const BigdnParams p) {
  using namespace dma;
  constexpr int kRT = D / 64;                  // 16-row tiles per wave
  constexpr int kCT = 2;                       // 16-column tiles per block
  constexpr int kNG = kRT * (D / 32);          // 1 KB G transfers per wave and frame
  constexpr int kStage = (kNG + kRT * kCT) * 1024;  // bytes per wave and ring stage
  constexpr int kLd = kNG + kRT * kCT;         // loads per frame
  // workgroups per (b, h): per direction run, one per 32-column block, plus z if it runs
  const int nb = (p.scan_dirs == 3 ? 2 : 1) * (D / 32 + p.scan_z);
  __shared__ __attribute__((aligned(1024))) char ring[4 * 3 * kStage];
  // state^T as fp16 operand, [32 columns][D rows].  For D = 128 the 16-byte chunks of a row
  // are XOR-swizzled by the column, so the 16 columns of a B-operand read hit distinct banks
  // without padding (the ring and both buffers then fill the 160 KB exactly); for D = 64 rows
  // are padded instead.
  constexpr int kSP = D == 128 ? D : D + 8;
  __shared__ __attribute__((aligned(16))) f16 st[2][32 * kSP];
  auto st_idx = [](int c, int r) {
    if constexpr (D == 128) return c * kSP + ((((r >> 3) ^ (c & 15)) << 3) | (r & 7));
    else return c * kSP + r;
  };
  // Workgroups are dealt to the eight XCDs round-robin by index; when B*H is a multiple of
  // eight, the workgroups of one (b, h) are given indices on one XCD, so a frame's G (read by
  // all of them) comes from that XCD's L2 after the first read.
  int slot, bh;
  if (p.B * p.H % 8 == 0) {
    const int s8 = blockIdx.x / 8;
    bh = blockIdx.x % 8 + 8 * (s8 / nb);
    slot = s8 % nb;
  } else {
    slot = blockIdx.x % nb;
    bh = blockIdx.x / nb;
  }
  const int rev = p.scan_dirs == 3 ? slot & 1 : p.scan_dirs == 2;
  const int cb = p.scan_dirs == 3 ? slot >> 1 : slot;
  const bool zb = cb == D / 32;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int li = lane & 15, lq = lane >> 4;
  const int F = p.F;
  const long mat0 = (long)bh * F * D * D;
  auto clampf = [&](int fa) { return fa < 0 ? 0 : (fa >= F ? F - 1 : fa); };
  auto row_of = [&](int t, int e) { return (D / 4) * wave + 16 * t + 4 * lq + e; };
  // step i absorbs frame fr(i) and gives the state of frame fr(i) (forward) or fr(i) - 1
  // (reverse)
  const int nsteps = rev ? F - 1 : F;
  auto fr = [&](int i) { return clampf(rev ? F - 1 - i : i); };

  // sources (every byte count below fits 32 bits: F <= 65535 and D <= 128)
  const _Float16* Gs = rev ? (zb ? p.Gz_b : p.G_b) : (zb ? p.Gz : p.G);
  const i32x4 rG = make_rsrc(Gs + mat0, (uint32_t)F * D * D * 2);
  const i32x4 rU = zb ? make_rsrc((rev ? p.uz_b : p.uz) + (long)bh * F * D, (uint32_t)F * D * 4)
                      : make_rsrc((rev ? p.U_b : p.U) + mat0, (uint32_t)F * D * D * 4);
  const uint32_t vU = zb ? 16 * lq : 16 * lane;
  const uint32_t ringw = lds_addr(ring) + wave * 3 * kStage;
  // transfers of frame fa into ring stage stg
  auto issue = [&](int fa, int stg) {
    const uint32_t sb = ringw + stg * kStage;
#pragma unroll
    for (int n = 0; n < kNG; ++n)
      dma16(rG, 16 * lane, (uint32_t)fa * (D * D * 2) + (wave * kNG + n) * 1024, sb + n * 1024);
#pragma unroll
    for (int t = 0; t < kRT; ++t)
#pragma unroll
      for (int ct = 0; ct < kCT; ++ct) {
        const uint32_t so = zb ? ((uint32_t)fa * D + (D / 4) * wave + 16 * t) * 4
                               : (uint32_t)fa * (D * D * 4) + cb * 128 * D + ((wave * kRT + t) * kCT + ct) * 1024;
        dma16(rU, vU, so, sb + (kNG + t * kCT + ct) * 1024);
      }
  };

  f32x4 s[kRT][kCT];
#pragma unroll
  for (int t = 0; t < kRT; ++t)
#pragma unroll
    for (int ct = 0; ct < kCT; ++ct) s[t][ct] = f32x4{0.f, 0.f, 0.f, 0.f};
  // the forward state entering frame 0 (not for z)
  const long st0 = (long)bh * D * D + cb * 32;
  if (p.s_init && !rev && !zb)
#pragma unroll
    for (int t = 0; t < kRT; ++t)
#pragma unroll
      for (int ct = 0; ct < kCT; ++ct)
#pragma unroll
        for (int e = 0; e < 4; ++e) s[t][ct][e] = p.s_init[st0 + (long)row_of(t, e) * D + 16 * ct + li];
  // s <- d (s - G s) + U with the operands of ring stage stg; writes and reads st[ph]
  auto step = [&](int stg, int ph, float dcy) {
    const char* sb = ring + (wave * 3 + stg) * kStage;
    f16x8 ga[kRT][D / 32];
    f32x4 uu[kRT][kCT];
#pragma unroll
    for (int t = 0; t < kRT; ++t) {
#pragma unroll
      for (int k = 0; k < D / 32; ++k)
        ga[t][k] = *reinterpret_cast<const f16x8*>(sb + (t * (D / 32) + k) * 1024 + 16 * lane);
#pragma unroll
      for (int ct = 0; ct < kCT; ++ct)
        uu[t][ct] = *reinterpret_cast<const f32x4*>(sb + (kNG + t * kCT + ct) * 1024 + 16 * lane);
    }
    f16* sp = st[ph];
#pragma unroll
    for (int t = 0; t < kRT; ++t)
#pragma unroll
      for (int ct = 0; ct < kCT; ++ct) {
        f16x4 v;
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = (f16)s[t][ct][e];
        *reinterpret_cast<f16x4*>(sp + st_idx(16 * ct + li, row_of(t, 0))) = v;
      }
    __syncthreads();
    f32x4 gs[kRT][kCT];
#pragma unroll
    for (int t = 0; t < kRT; ++t)
#pragma unroll
      for (int ct = 0; ct < kCT; ++ct) gs[t][ct] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int k = 0; k < D / 32; ++k)
#pragma unroll
      for (int ct = 0; ct < kCT; ++ct) {
        const f16x8 bq = lds8(sp + st_idx(16 * ct + li, 32 * k + 8 * lq));
#pragma unroll
        for (int t = 0; t < kRT; ++t) gs[t][ct] = mma16(ga[t][k], bq, gs[t][ct]);
      }
#pragma unroll
    for (int t = 0; t < kRT; ++t)
#pragma unroll
      for (int ct = 0; ct < kCT; ++ct)
#pragma unroll
        for (int e = 0; e < 4; ++e) s[t][ct][e] = dcy * (s[t][ct][e] - gs[t][ct][e]) + uu[t][ct][e];
  };
  // the state of frame fa: fp16 transposed (four consecutive rows of one column per lane,
  // 8 bytes) or, for z, fp32 entries of column 0
  _Float16* sdt = p.SdT + (p.dir_slots == 2 ? (long)rev * p.B * p.H * F * D * D : 0L) + mat0;
  float* zd = p.zd + ((long)rev * p.B * p.H + bh) * F * D;
  auto store_state = [&](int fa) {
#pragma unroll
    for (int t = 0; t < kRT; ++t) {
      if (zb) {
        if (li == 0) *reinterpret_cast<f32x4*>(zd + (long)fa * D + row_of(t, 0)) = s[t][0];
      } else {
#pragma unroll
        for (int ct = 0; ct < kCT; ++ct) {
          f16x4 h;
#pragma unroll
          for (int e = 0; e < 4; ++e) h[e] = (f16)s[t][ct][e];
          *reinterpret_cast<f16x4*>(sdt + (long)fa * D * D + (long)(cb * 32 + 16 * ct + li) * D + row_of(t, 0)) = h;
        }
      }
    }
  };

  if (rev) store_state(F - 1);  // R_{F-1} = 0
  issue(fr(0), 0);
  issue(fr(1), 1);
  float dv = 0.f;  // lane j: the decay of step (i & ~63) + j
  for (int i = 0; i < nsteps; ++i) {
    if ((i & 63) == 0) dv = (rev ? p.decay_bwd : p.decay)[(long)bh * F + fr(i + lane)];
    issue(fr(i + 2), (i + 2) % 3);
    wait_vm<2 * kLd>();  // step i's loads are done once only those of steps i+1, i+2 may be pending
    const float dcy = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(dv), i & 63));
    step(i % 3, i & 1, dcy);
    store_state(rev ? F - 2 - i : i);
  }
  if (p.s_final && !rev && !zb)
#pragma unroll
    for (int t = 0; t < kRT; ++t)
#pragma unroll
      for (int ct = 0; ct < kCT; ++ct)
#pragma unroll
        for (int e = 0; e < 4; ++e) p.s_final[st0 + (long)row_of(t, e) * D + 16 * ct + li] = s[t][ct][e];
  // no transfer may still be writing the ring when the workgroup ends
  wait_vm0();
}

// ---- output -----------------------------------------------------------------------------
// One workgroup per (b, group of kHW heads, frame f, group of grp consecutive 64-token blocks
// of f): num = Q_rot (S + R), den = Q_pos . (z + zR).  Wave w forms value columns
// (D/4)w .. (D/4)w + D/4 - 1 of every token: its slice of each head's (S + R)^T is the A
// operand, summed from the two directions' fp16 states into registers once per workgroup; the prepped Q_rot rows are the B operand,
// from LDS.  The accumulator of lane (li, lq) holds four consecutive value columns of token li
// (8-byte stores).  A thread's (token, octet) items keep one octet, so its norm weights load
// once, and the RoPE tables and inverse RMS of an item load once for all kHW heads.
// (Measured on the 16-frame video block: two heads and four blocks per workgroup beat one
// head or other block counts; issuing the next block's loads before the products, or using
// 4-channel items, did not help.)
//
// kTwoQ (the reverse direction reads its own q, k, v): the two slots are the forward and the
// reverse direction of one head, each with its own state and its own prepped Q rows, and their
// products accumulate into one output, num = Q_f S_f + Q_r R_f, den = q_f z_f + q_r zR_f.
template <int D, int kHW, bool kMerge, bool kTwoQ>
__global__ __launch_bounds__(256) void out_kernel(const BigdnParams p, int grp) {
  static_assert(!kTwoQ || kHW == 2, "the two-Q form has one slot per direction");
  constexpr int kHeads = kTwoQ ? 1 : kHW;  // heads per workgroup
  typedef bf16 bf16x4_t __attribute__((ext_vector_type(4)));
  constexpr int kOct = D / 8, kItems = 64 * kOct / 256, kCT = D / 64, kSP = D + 8;
  __shared__ __attribute__((aligned(16))) f16 qr[kHW][64 * kSP];  // Q_rot rows, padded
  __shared__ float zsum[kHW][D];
  __shared__ float den_part[kHW][64];
  // Logical order: head group fastest, then token group, frame and batch; when the grid is a
  // multiple of eight, XCD x takes the contiguous range [x n/8, (x+1) n/8) of it, so the head
  // groups of one token block (same RoPE rows) and the token groups of one (head, frame)
  // (same states) run close in time on one XCD's L2.
  const int ngrp = (p.S / 64) / grp, nhg = p.H / kHeads, nwg = gridDim.x;
  int x = nwg % 8 ? (int)blockIdx.x : (blockIdx.x % 8) * (nwg / 8) + blockIdx.x / 8;
  const int h0 = (x % nhg) * kHeads;
  x /= nhg;
  const int g = x % ngrp;
  x /= ngrp;
  const int f = x % p.F, b = x / p.F;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int li = lane & 15, lq = lane >> 4;
  const int C = p.H * D, o = tid % kOct;
  const bf16* qkv = static_cast<const bf16*>(p.qkv);
  bf16* num = static_cast<bf16*>(p.num);
  f16x8 sa[kHW][kCT][D / 32];
  float w[kHW][8];
  const long dir_m = (long)p.B * p.H * p.F * D * D, dir_v = (long)p.B * p.H * p.F * D;
#pragma unroll
  for (int hh = 0; hh < kHW; ++hh) {
    const int hd = kTwoQ ? h0 : h0 + hh;
    const long bhf = ((long)b * p.H + hd) * p.F + f;
#pragma unroll
    for (int ct = 0; ct < kCT; ++ct)
#pragma unroll
      for (int k = 0; k < D / 32; ++k) {
        const long e = bhf * D * D + (long)((D / 4) * wave + 16 * ct + li) * D + 32 * k + 8 * lq;
        if constexpr (kTwoQ) {
          sa[hh][ct][k] = *reinterpret_cast<const f16x8*>(p.SdT + hh * dir_m + e);
        } else {
          const f16x8 sf = *reinterpret_cast<const f16x8*>(p.SdT + e);
          const f16x8 sr = *reinterpret_cast<const f16x8*>(p.SdT + dir_m + e);
#pragma unroll
          for (int j = 0; j < 8; ++j) sa[hh][ct][k][j] = (f16)((float)sf[j] + (float)sr[j]);
        }
      }
    if (tid < D)
      zsum[hh][tid] = kTwoQ ? p.zd[hh * dir_v + bhf * D + tid]
                            : p.zd[bhf * D + tid] + p.zd[dir_v + bhf * D + tid];
    load8f(p.q_norm_w + hd * D + 8 * o, w[hh]);
  }
  for (int blk = g * grp; blk < (g + 1) * grp; ++blk) {
    const int n0 = f * p.S + blk * 64;
    __syncthreads();  // the previous block's qr and den_part reads are done
    // every load of this thread's items is issued before any of them is used
    float inv[kItems][kTwoQ ? 2 : 1];
    f16x8 tab[kItems][2];  // (cos, sin) pairs of the item's 8 channels
    bf16x8 qx[kItems][kHW];
#pragma unroll
    for (int i = 0; i < kItems; ++i) {
      const int t = tid / kOct + (256 / kOct) * i;
      const long n = n0 + t, bn = (long)b * p.N + n;
      const f16x8* tp = reinterpret_cast<const f16x8*>(p.rope_h + (n * D + 8 * o) * 2);
      tab[i][0] = tp[0];
      tab[i][1] = tp[1];
      inv[i][0] = p.q_inv_rms[bn];
      if constexpr (kTwoQ) inv[i][1] = p.q_inv_rms_b[bn];
#pragma unroll
      for (int hh = 0; hh < kHW; ++hh) {
        const bf16* src = kTwoQ && hh ? static_cast<const bf16*>(p.qkv_bwd) : qkv;
        const int hd = kTwoQ ? h0 : h0 + hh;
        qx[i][hh] = *reinterpret_cast<const bf16x8*>(src + bn * 3L * C + (long)hd * D + 8 * o);
      }
    }
#pragma unroll
    for (int i = 0; i < kItems; ++i) {
      const int t = tid / kOct + (256 / kOct) * i;
      float cs[8], sn[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        cs[j] = (float)tab[i][j >> 2][2 * (j & 3)];
        sn[j] = (float)tab[i][j >> 2][2 * (j & 3) + 1];
      }
#pragma unroll
      for (int hh = 0; hh < kHW; ++hh) {
        float xq[8], pos[8], rot[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) xq[j] = (float)qx[i][hh][j];
        prep8(xq, inv[i][kTwoQ ? hh : 0], w[hh], cs, sn, 1.f, pos, rot);
        f16x8 v;
        float dp = 0.f;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          v[j] = (f16)rot[j];
          dp += pos[j] * zsum[hh][8 * o + j];
        }
        *reinterpret_cast<f16x8*>(&qr[hh][t * kSP + 8 * o]) = v;
        // den: reduce over the kOct consecutive threads of token t
#pragma unroll
        for (int off = 1; off < kOct; off <<= 1) dp += __shfl_xor(dp, off, 64);
        if (o == 0) den_part[hh][t] = dp;
      }
    }
    __syncthreads();
    bf16x4_t gv[4][kCT];
    f32x4 acc[4][kCT];
#pragma unroll
    for (int hh = 0; hh < kHW; ++hh) {
      const int hs = kTwoQ ? 0 : hh;  // output head slot
      // lane (li, lq): token n0 + 16 tt + li, value columns (D/4) wave + 16 ct + 4 lq + e
      auto at = [&](int tt) {
        return (((long)b * p.N + n0 + 16 * tt + li) * p.H + h0 + hs) * D + (D / 4) * wave + 4 * lq;
      };
      if (!kTwoQ || hh == 0) {
        if constexpr (kMerge) {
          if (p.gate)  // issued before the products, which hide their latency
#pragma unroll
            for (int tt = 0; tt < 4; ++tt)
#pragma unroll
              for (int ct = 0; ct < kCT; ++ct)
                gv[tt][ct] = *reinterpret_cast<const bf16x4_t*>(static_cast<const bf16*>(p.gate) + at(tt) + 16 * ct);
        }
#pragma unroll
        for (int tt = 0; tt < 4; ++tt)
#pragma unroll
          for (int ct = 0; ct < kCT; ++ct) acc[tt][ct] = f32x4{0.f, 0.f, 0.f, 0.f};
      }
#pragma unroll
      for (int tt = 0; tt < 4; ++tt)
#pragma unroll
        for (int k = 0; k < D / 32; ++k) {
          const f16x8 bq = lds8(&qr[hh][(16 * tt + li) * kSP + 32 * k + 8 * lq]);
#pragma unroll
          for (int ct = 0; ct < kCT; ++ct) acc[tt][ct] = mma16(sa[hh][ct][k], bq, acc[tt][ct]);
        }
      if (kTwoQ && hh == 0) continue;  // the reverse slot adds its products first
#pragma unroll
      for (int tt = 0; tt < 4; ++tt) {
        float rden = 0.f;
        if constexpr (kMerge) {
          const float dn = kTwoQ ? den_part[0][16 * tt + li] + den_part[1][16 * tt + li]
                                 : den_part[hh][16 * tt + li];
          rden = __builtin_amdgcn_rcpf(dn + p.merge_eps);  // 1 ulp: far below bf16 output
        }
#pragma unroll
        for (int ct = 0; ct < kCT; ++ct) {
          if (num) {
            bf16x4_t o4;
#pragma unroll
            for (int e = 0; e < 4; ++e) o4[e] = (bf16)acc[tt][ct][e];
            *reinterpret_cast<bf16x4_t*>(num + at(tt) + 16 * ct) = o4;
          }
          if constexpr (kMerge) {
            bf16x4_t o4;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              float x = acc[tt][ct][e] * rden;
              if (p.gate) {
                const float gt = (float)gv[tt][ct][e];
                // SiLU; the hardware reciprocal instead of a full-precision division (whose
                // scaling and fix-up steps doubled this epilogue's VALU work)
                x *= gt * __builtin_amdgcn_rcpf(1.f + __expf(-gt));
              }
              o4[e] = (bf16)x;
            }
            *reinterpret_cast<bf16x4_t*>(static_cast<bf16*>(p.out) + at(tt) + 16 * ct) = o4;
          }
        }
      }
    }
    if (p.den && tid < 64 * kHeads) {
      const int hh = tid / 64, t = tid % 64;
      const float dn = kTwoQ ? den_part[0][t] + den_part[1][t] : den_part[hh][t];
      static_cast<bf16*>(p.den)[((long)b * p.H + h0 + hh) * p.N + n0 + t] = (bf16)dn;
    }
  }
}

}  // namespace

hipError_t launch_prep(const PrepParams& p, hipStream_t stream) {
  hipLaunchKernelGGL(rms_prep_kernel, dim3(p.B * p.N), dim3(kPrepThreads), 0, stream, p);
  return hipGetLastError();
}

hipError_t launch_bigdn(const BigdnParams& p_in, hipStream_t stream) {
  BigdnParams p = p_in;
  p.scan_dirs = 3;
  p.scan_z = 1;
  p.dir_slots = 2;
  p.s_init = nullptr;
  p.s_final = nullptr;
  if (!p.decay_bwd) p.decay_bwd = p.decay;
  const bool rev_stats = p.beta_bwd || p.qkv_bwd;
  if (!rev_stats) {  // the reverse direction shares the forward statistics
    p.G_b = p.G;
    p.Gz_b = p.Gz;
    p.U_b = p.U;
    p.uz_b = p.uz;
  }
  PrepParams pp{};
  pp.qkv = p.qkv;
  pp.q_norm_w = p.q_norm_w;
  pp.k_norm_w = p.k_norm_w;
  pp.rope_cos = p.rope_cos;
  pp.rope_sin = p.rope_sin;
  pp.k_scale = p.k_scale;
  pp.eps = p.eps;
  pp.q_inv_rms = p.q_inv_rms;
  pp.k_inv_rms = p.k_inv_rms;
  pp.rope_h = p.rope_h;
  pp.B = p.B;
  pp.N = p.N;
  pp.H = p.H;
  pp.D = p.D;
  hipError_t e = launch_prep(pp, stream);
  if (e != hipSuccess) return e;
  if (p.qkv_bwd) {  // the inverse RMS of the reverse direction's q and k
    pp.qkv = p.qkv_bwd;
    pp.q_inv_rms = p.q_inv_rms_b;
    pp.k_inv_rms = p.k_inv_rms_b;
    pp.rope_h = nullptr;
    e = launch_prep(pp, stream);
    if (e != hipSuccess) return e;
  }
  const int nbhf = p.B * p.H * p.F;
  // the reverse direction's statistics, when its beta or its keys and values differ
  BigdnParams pb = p;
  if (p.qkv_bwd) {
    pb.qkv = p.qkv_bwd;
    pb.k_inv_rms = p.k_inv_rms_b;
  }
  if (p.beta_bwd) pb.beta = p.beta_bwd;
  pb.G = p.G_b;
  pb.Gz = p.Gz_b;
  pb.U = p.U_b;
  pb.uz = p.uz_b;
  // 64-token blocks per output workgroup: the largest divisor of a frame's blocks up to 4;
  // two heads per output workgroup when H is even
  const int nblk = p.S / 64;
  int grp = 4;
  while (nblk % grp) grp >>= 1;
  // (one head per workgroup when the directions read different q)
  const int hw = p.H % 2 || p.qkv_bwd ? 1 : 2;
  const dim3 og(p.B * (p.H / hw) * p.F * (nblk / grp));
  const bool merge = p.out != nullptr;
#define GDN_OUT(DD)                                                                                          \
  do {                                                                                                       \
    if (p.qkv_bwd && merge) hipLaunchKernelGGL((out_kernel<DD, 2, true, true>), og, dim3(256), 0, stream, p, grp);  \
    else if (p.qkv_bwd) hipLaunchKernelGGL((out_kernel<DD, 2, false, true>), og, dim3(256), 0, stream, p, grp);     \
    else if (hw == 2 && merge) hipLaunchKernelGGL((out_kernel<DD, 2, true, false>), og, dim3(256), 0, stream, p, grp); \
    else if (hw == 2) hipLaunchKernelGGL((out_kernel<DD, 2, false, false>), og, dim3(256), 0, stream, p, grp);   \
    else if (merge) hipLaunchKernelGGL((out_kernel<DD, 1, true, false>), og, dim3(256), 0, stream, p, grp);      \
    else hipLaunchKernelGGL((out_kernel<DD, 1, false, false>), og, dim3(256), 0, stream, p, grp);                \
  } while (0)
  if (p.D == 128) {
    hipLaunchKernelGGL(frame_stats_kernel<128>, dim3(nbhf), dim3(kStatThreads), 0, stream, p);
    if (rev_stats) hipLaunchKernelGGL(frame_stats_kernel<128>, dim3(nbhf), dim3(kStatThreads), 0, stream, pb);
    hipLaunchKernelGGL(scan_kernel<128>, dim3(p.B * p.H * 2 * (128 / 32 + 1)), dim3(256), 0, stream, p);
    GDN_OUT(128);
  } else {
    hipLaunchKernelGGL(frame_stats_kernel<64>, dim3(nbhf), dim3(kStatThreads), 0, stream, p);
    if (rev_stats) hipLaunchKernelGGL(frame_stats_kernel<64>, dim3(nbhf), dim3(kStatThreads), 0, stream, pb);
    hipLaunchKernelGGL(scan_kernel<64>, dim3(p.B * p.H * 2 * (64 / 32 + 1)), dim3(256), 0, stream, p);
    GDN_OUT(64);
  }
#undef GDN_OUT
  return hipGetLastError();
}

hipError_t launch_frame_scan(const BigdnParams& p, hipStream_t stream) {
  const int nb = (p.scan_dirs == 3 ? 2 : 1) * (p.D / 32 + p.scan_z);
  if (p.D == 128)
    hipLaunchKernelGGL(scan_kernel<128>, dim3(p.B * p.H * nb), dim3(256), 0, stream, p);
  else
    hipLaunchKernelGGL(scan_kernel<64>, dim3(p.B * p.H * nb), dim3(256), 0, stream, p);
  return hipGetLastError();
}

}  // namespace gdn

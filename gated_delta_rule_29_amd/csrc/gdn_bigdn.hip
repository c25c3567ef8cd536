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
// (16-column blocks of the state per (b, h), both directions, writes the summed states), out
// (num, den per 64-token block).  Products use fp16 operands and fp32 accumulation; the state
// is fp32.
#include "gdn_device.h"
#include "gdn_dma.h"
#include "gdn_internal.h"
#include "gdn_tiles.h"

namespace gdn {

namespace {

constexpr int kPrepThreads = 256;

__device__ __forceinline__ float block_sum_256(float x, float* red) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) x += __shfl_xor(x, off, 64);
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  __syncthreads();
  if (lane == 0) red[wave] = x;
  __syncthreads();
  return red[0] + red[1] + red[2] + red[3];
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

// Front end of 8 channels d0..d0+7 (d0 a multiple of 8, so every RoPE pair is inside).
__device__ __forceinline__ void prep8(const float* x, float inv, const float* w, const float* cs,
                                      const float* sn, float scale, float* pos, float* rot) {
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const float y = x[j] * inv * w[j];
    pos[j] = (y > 0.f ? y : 0.f) * scale;
  }
#pragma unroll
  for (int j = 0; j < 8; ++j) rot[j] = pos[j] * cs[j] + pos[j ^ 1] * sn[j];
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
  sq = block_sum_256(sq, red);
  sk = block_sum_256(sk, red + 4);
  const float iq = rsqrtf(sq / (float)C + p.eps), ik = rsqrtf(sk / (float)C + p.eps);
  if (threadIdx.x == 0) {
    if (p.q_inv_rms) p.q_inv_rms[bn] = iq;
    if (p.k_inv_rms) p.k_inv_rms[bn] = ik;
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

// Workspace layouts of G and U (written by frame_stats, read by scan), per (b, h, frame):
//   G: A-operand order, element (r, c) at ((((r / (D/4)) kRT + (r % (D/4)) / 16) (D/32)
//      + c / 32) 64 + ((c / 8) % 4) 16 + r % 16) 8 + c % 8 with kRT = D / 64, so a scan
//      lane's 16-byte operand is one load and a wave's loads are contiguous;
//   U: accumulator order, element (r, c) at (c / 16) 16D + (((r / (D/4)) kRT
//      + (r % (D/4)) / 16) 64 + ((r % 16) / 4) 16 + c % 16) 4 + r % 4.
template <int D>
__device__ __forceinline__ long g_lane_index(int r, int c) {
  constexpr int kRT = D / 64;
  return ((((long)(r / (D / 4)) * kRT + (r % (D / 4)) / 16) * (D / 32) + c / 32) * 64 +
          ((c / 8) & 3) * 16 + (r & 15)) * 8 + (c & 7);
}
template <int D>
__device__ __forceinline__ long u_lane_index(int r, int c) {
  constexpr int kRT = D / 64;
  return (long)(c >> 4) * (16 * D) +
         (((long)(r / (D / 4)) * kRT + (r % (D / 4)) / 16) * 64 + ((r & 15) >> 2) * 16 + (c & 15)) * 4 +
         (r & 3);
}

// ---- frame statistics -------------------------------------------------------------------
// One workgroup of twelve waves per (b, h, frame) computes all three statistics over the
// frame's tokens, 64 at a time:
//   G = K_rot^T diag(beta) K_rot,  U = K_rot^T diag(beta) V,  Gz = K_pos^T diag(beta) K_pos,
//   uz = K_pos^T beta.
// Prep: every thread takes (token, 8-channel octet) items -- 16 threads per token row, so the
// qkv loads are whole 256-byte rows -- applies the front end once and writes five fp16 token
// rows (K_rot, beta K_rot, beta V, K_pos, beta K_pos) into LDS with 16-byte stores.
// Products: wave w accumulates quadrant (w % 4) of statistic w / 4; both operands contract
// over tokens, so they come from the row-major tiles by LDS transpose reads
// (ds_read_b64_tr_b16: within a 16-lane group, lane n receives element j of the 8-byte piece
// addressed by lane 4j + n / 4, halfword n % 4).  A transpose-read operand pair for
// (32-block Gb, half t) gives lane (li, lq) channel 32Gb + 8(li >> 2) + 4t + (li & 3) at
// tokens 8lq + j; the accumulator of such a pair of operands holds row channel
// 32Gb + 8lq + 4t + e and column channel 32Gb' + 8(li >> 2) + 4t' + (li & 3).
constexpr int kStatThreads = 768;

typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef f16 f16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
typedef unsigned u32x2v __attribute__((ext_vector_type(2)));
typedef unsigned u32x4v __attribute__((ext_vector_type(4)));

__device__ __forceinline__ f16x8 tr_pair(const f16* p0, const f16* p1) {
  auto rd = [](const f16* p) {
    return __builtin_bit_cast(u32x2v, __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (lds_i16x4*)(uintptr_t)(const __attribute__((address_space(3))) char*)p));
  };
  const u32x4v w = __builtin_shufflevector(rd(p0), rd(p1), 0, 1, 2, 3);
  return __builtin_bit_cast(f16x8, w);
}

template <int D>
__global__ __launch_bounds__(kStatThreads) void frame_stats_kernel(const BigdnParams p) {
  constexpr int kT = 64;         // tokens per block
  constexpr int kOct = D / 8;    // octets per token row
  constexpr int kNG = D / 64;    // 32-channel blocks per quadrant side
  // tiles: 0 K_rot, 1 beta K_rot, 2 beta V, 3 K_pos, 4 beta K_pos  ([64][D] fp16, tix_x64)
  __shared__ __attribute__((aligned(16))) f16 tl[5][kT * D];
  const int bhf = blockIdx.x;
  const int f = bhf % p.F, h = (bhf / p.F) % p.H, b = bhf / (p.F * p.H);
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int li = lane & 15, lq = lane >> 4;
  const int C = p.H * D;
  const bf16* qkv = static_cast<const bf16*>(p.qkv);
  const int m = wave >> 2, qi = (wave & 3) >> 1, qj = wave & 1;
  const f16* ta = tl[m == 2 ? 3 : 0];
  const f16* tb = tl[m == 0 ? 1 : (m == 1 ? 2 : 4)];
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
  float uzr[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) uzr[j] = 0.f;

  // Items (token, octet) of a block: this thread takes it = tid + kStatThreads i.  The k, v
  // rows, inverse RMS and beta of its first item are loaded one block ahead (in flight during
  // the products of the block before); the RoPE tables, shared by every head, and a second
  // item's rows are loaded when used.
  constexpr int kItems = (kT * kOct + kStatThreads - 1) / kStatThreads;
  bf16x8 kx, vx;
  float ivx = 0.f, btx = 0.f;
  auto load_items = [&](int t0) {
    const int it = tid;
    if (it < kT * kOct && t0 < p.S) {
      const int s = it / kOct;
      const long bn = (long)b * p.N + (long)f * p.S + t0 + s;
      const bf16* krow = qkv + bn * 3L * C + C + (long)h * D + 8 * oct;
      kx = *reinterpret_cast<const bf16x8*>(krow);
      vx = *reinterpret_cast<const bf16x8*>(krow + C);
      ivx = p.k_inv_rms[bn];
      btx = p.beta[(((long)b * p.H + h) * p.F + f) * p.S + t0 + s];
    }
  };
  load_items(0);

  for (int t0 = 0; t0 < p.S; t0 += kT) {
    __syncthreads();
#pragma unroll
    for (int i = 0; i < kItems; ++i) {
      const int it = tid + kStatThreads * i;
      if (it >= kT * kOct) continue;
      const int s = it / kOct;
      const long n = (long)f * p.S + t0 + s;
      const long bn = (long)b * p.N + n;
      bf16x8 ki, vi;
      float ivi, bt;
      if (i == 0) {
        ki = kx;
        vi = vx;
        ivi = ivx;
        bt = btx;
      } else {
        const bf16* krow = qkv + bn * 3L * C + C + (long)h * D + 8 * oct;
        ki = *reinterpret_cast<const bf16x8*>(krow);
        vi = *reinterpret_cast<const bf16x8*>(krow + C);
        ivi = p.k_inv_rms[bn];
        bt = p.beta[(((long)b * p.H + h) * p.F + f) * p.S + t0 + s];
      }
      float x[8], v[8], cs[8], sn[8], pos[8], rot[8], w8[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        x[j] = (float)ki[j];
        v[j] = (float)vi[j];
      }
      load8f(p.rope_cos + n * D + 8 * oct, cs);
      load8f(p.rope_sin + n * D + 8 * oct, sn);
      load8f(p.k_norm_w + h * D + 8 * oct, w8);
      prep8(x, ivi, w8, cs, sn, p.k_scale, pos, rot);
      f16x8 r0, r1, r2, r3, r4;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        r0[j] = (f16)rot[j];
        r1[j] = (f16)(bt * rot[j]);
        r2[j] = (f16)(bt * v[j]);
        r3[j] = (f16)pos[j];
        r4[j] = (f16)(bt * pos[j]);
        uzr[j] += bt * pos[j];
      }
      const int ix = tix_x64(s, 8 * oct);
      *reinterpret_cast<f16x8*>(&tl[0][ix]) = r0;
      *reinterpret_cast<f16x8*>(&tl[1][ix]) = r1;
      *reinterpret_cast<f16x8*>(&tl[2][ix]) = r2;
      *reinterpret_cast<f16x8*>(&tl[3][ix]) = r3;
      *reinterpret_cast<f16x8*>(&tl[4][ix]) = r4;
    }
    __syncthreads();
    load_items(t0 + kT);
    // lane-derived LDS addresses recomputed per block instead of held across the loop
    int ln = lane;
    asm volatile("" : "+v"(ln));
    const int li = ln & 15, lq = ln >> 4, trj = (ln >> 2) & 3, trc = ln & 3;
#pragma unroll
    for (int P = 0; P < kT / 32; ++P) {
      f16x8 af[kNG][2], bf[kNG][2];
#pragma unroll
      for (int g = 0; g < kNG; ++g)
#pragma unroll
        for (int t = 0; t < 2; ++t) {
          const int ca = 32 * (kNG * qi + g) + 8 * trc + 4 * t;
          const int cb = 32 * (kNG * qj + g) + 8 * trc + 4 * t;
          af[g][t] = tr_pair(&ta[tix_x64(32 * P + 8 * lq + trj, ca)], &ta[tix_x64(32 * P + 8 * lq + 4 + trj, ca)]);
          bf[g][t] = tr_pair(&tb[tix_x64(32 * P + 8 * lq + trj, cb)], &tb[tix_x64(32 * P + 8 * lq + 4 + trj, cb)]);
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
  float* red = reinterpret_cast<float*>(&tl[0][0]);  // [kStatThreads][8]
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
// One workgroup per (b, h, 16-column block cb) of the state, plus one (cb == D/16) for z: z
// runs as a 16-column block whose columns all hold z (A operand Gz, U the uz entries of each
// row), so both share this code.  Wave w owns state rows (D/4)w .. (D/4)w + D/4 - 1 of the
// block.  The state lives in registers (fp32) and is exchanged through LDS (fp16 transposed
// copy, double-buffered so one barrier per frame suffices) as the B operand of G S.
//
// Operands are staged per wave in a three-frame LDS ring by direct-to-LDS transfers issued
// two frames ahead; each wave reads back only what it transferred (at its own lane slots, so
// without bank conflicts), so a counted wait on its own loads is the only synchronisation.
// A ring stage holds, per wave: the lane-ordered G (or Gz) operands (kNG KB), the U tile
// (kRT KB), in the reverse pass the forward state of the frame being written (kRT KB), and
// the frame's decay (256 B).
template <int D>
__global__ __launch_bounds__(256) void scan_kernel(const BigdnParams p) {
  using namespace dma;
  constexpr int kRT = D / 64;                            // 16-row tiles per wave
  constexpr int kNG = kRT * (D / 32);                    // 1 KB G transfers per wave and frame
  constexpr int kStage = (kNG + 2 * kRT) * 1024 + 256;   // bytes per wave and ring stage
  constexpr int kLd = kNG + kRT + 1;                     // forward loads per frame
  constexpr int kLdR = kLd + kRT;                        // reverse loads per frame (+ S_f)
  constexpr int kSP = D + 8;  // padded st row: the 16 rows of a B-operand read hit distinct banks
  __shared__ __attribute__((aligned(1024))) char ring[4 * 3 * kStage];
  __shared__ __attribute__((aligned(16))) f16 st[2][16 * kSP];  // state^T as fp16 operand
  const int cb = blockIdx.x % (D / 16 + 1);
  const int bh = blockIdx.x / (D / 16 + 1);
  const bool zb = cb == D / 16;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int li = lane & 15, lq = lane >> 4;
  const int F = p.F;
  const long mat0 = (long)bh * F * D * D;
  auto clampf = [&](int fa) { return fa < 0 ? 0 : (fa >= F ? F - 1 : fa); };
  auto row_of = [&](int t, int e) { return (D / 4) * wave + 16 * t + 4 * lq + e; };

  // sources (every byte count below fits 32 bits: F <= 65535 and D <= 128)
  const i32x4 rG = make_rsrc(zb ? p.Gz + mat0 : p.G + mat0, (uint32_t)F * D * D * 2);
  const i32x4 rU = zb ? make_rsrc(p.uz + (long)bh * F * D, (uint32_t)F * D * 4)
                      : make_rsrc(p.U + mat0, (uint32_t)F * D * D * 4);
  const long fst = zb ? 16 * D : (long)D * D;  // floats between frames of the forward states
  float* sfw = zb ? p.Zf + (long)bh * F * 16 * D : p.Sf + mat0 + cb * 16 * D;
  const i32x4 rS = make_rsrc(sfw, (uint32_t)((F - 1) * fst + 16 * D) * 4);
  const i32x4 rD = make_rsrc(p.decay + (long)bh * F, (uint32_t)F * 4);
  const uint32_t vU = zb ? 16 * lq : 16 * lane;
  const uint32_t ringw = lds_addr(ring) + wave * 3 * kStage;
  // transfers of frame fa (and, in the reverse pass, forward state fs) into ring stage stg
  auto issue = [&](int fa, int stg, bool with_sf, int fs) {
    fa = clampf(fa);
    const uint32_t sb = ringw + stg * kStage;
#pragma unroll
    for (int n = 0; n < kNG; ++n) dma16(rG, 16 * lane, (uint32_t)fa * (D * D * 2) + (wave * kNG + n) * 1024, sb + n * 1024);
#pragma unroll
    for (int t = 0; t < kRT; ++t) {
      const uint32_t so = zb ? ((uint32_t)fa * D + (D / 4) * wave + 16 * t) * 4
                             : (uint32_t)fa * (D * D * 4) + cb * 64 * D + (wave * kRT + t) * 1024;
      dma16(rU, vU, so, sb + (kNG + t) * 1024);
    }
    dma4(rD, 0, (uint32_t)fa * 4, sb + (kNG + 2 * kRT) * 1024);
    if (with_sf) {
      fs = clampf(fs);
#pragma unroll
      for (int t = 0; t < kRT; ++t)
        dma16(rS, 16 * lane, (uint32_t)(fs * fst * 4) + (wave * kRT + t) * 1024, sb + (kNG + kRT + t) * 1024);
    }
  };
  auto stage_ptr = [&](int stg) { return ring + (wave * 3 + stg) * kStage; };

  f32x4 s[kRT];
#pragma unroll
  for (int t = 0; t < kRT; ++t) s[t] = f32x4{0.f, 0.f, 0.f, 0.f};
  // s <- d (s - G s) + U with the operands of ring stage stg; writes and reads st[ph]
  auto step = [&](int stg, int ph) {
    const char* sb = stage_ptr(stg);
    f16x8 ga[kRT][D / 32];
    f32x4 uu[kRT];
#pragma unroll
    for (int t = 0; t < kRT; ++t) {
#pragma unroll
      for (int k = 0; k < D / 32; ++k)
        ga[t][k] = *reinterpret_cast<const f16x8*>(sb + (t * (D / 32) + k) * 1024 + 16 * lane);
      uu[t] = *reinterpret_cast<const f32x4*>(sb + (kNG + t) * 1024 + 16 * lane);
    }
    const float dcy = *reinterpret_cast<const float*>(sb + (kNG + 2 * kRT) * 1024 + 4 * lane);
    f16* sp = st[ph];
#pragma unroll
    for (int t = 0; t < kRT; ++t) {
      f16x4 v;
#pragma unroll
      for (int e = 0; e < 4; ++e) v[e] = (f16)s[t][e];
      *reinterpret_cast<f16x4*>(sp + li * kSP + row_of(t, 0)) = v;
    }
    __syncthreads();
    f32x4 gs[kRT];
#pragma unroll
    for (int t = 0; t < kRT; ++t) {
      gs[t] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int k = 0; k < D / 32; ++k) gs[t] = mma16(ga[t][k], lds8(sp + li * kSP + 32 * k + 8 * lq), gs[t]);
    }
#pragma unroll
    for (int t = 0; t < kRT; ++t)
#pragma unroll
      for (int e = 0; e < 4; ++e) s[t][e] = dcy * (s[t][e] - gs[t][e]) + uu[t][e];
  };
  // output of frame fa: s + add (the forward state), as fp16 (S + R)^T -- four consecutive
  // rows of one column per lane, 8 bytes -- or, for z, fp32 entries of column 0
  auto store_sum = [&](int fa, const f32x4* add) {
#pragma unroll
    for (int t = 0; t < kRT; ++t) {
      f32x4 tot;
#pragma unroll
      for (int e = 0; e < 4; ++e) tot[e] = s[t][e] + (add ? add[t][e] : 0.f);
      if (zb) {
        if (li == 0) *reinterpret_cast<f32x4*>(p.zsum + ((long)bh * F + fa) * D + row_of(t, 0)) = tot;
      } else {
        f16x4 h;
#pragma unroll
        for (int e = 0; e < 4; ++e) h[e] = (f16)tot[e];
        *reinterpret_cast<f16x4*>(p.SsumT + mat0 + (long)fa * D * D + (long)(cb * 16 + li) * D + row_of(t, 0)) = h;
      }
    }
  };

  // forward: S_f after absorbing frame f (ring stage f % 3), kept in fp32 in the workspace in
  // the per-lane tile order
  issue(0, 0, false, 0);
  issue(1, 1, false, 0);
  for (int f = 0; f < F; ++f) {
    issue(f + 2, (f + 2) % 3, false, 0);
    wait_vm<2 * kLd>();  // frame f's loads are done once only frames f+1, f+2 may be pending
    step(f % 3, f & 1);
#pragma unroll
    for (int t = 0; t < kRT; ++t)
      *reinterpret_cast<f32x4*>(sfw + (long)f * fst + (wave * kRT + t) * 256 + 4 * lane) = s[t];
  }
  // frame F-1 reads R_{F-1} = 0: its sum is the forward state itself
  store_sum(F - 1, nullptr);
  // the reverse pass reads the forward states back and restarts the st phases: every store
  // of this wave has landed and every wave is past its last forward read
  wait_vm0();
  __syncthreads();
  // reverse: step i absorbs frame F-1-i and gives R of frame F-2-i, whose forward state comes
  // in the same ring stage (i % 3)
#pragma unroll
  for (int t = 0; t < kRT; ++t) s[t] = f32x4{0.f, 0.f, 0.f, 0.f};
  issue(F - 1, 0, true, F - 2);
  issue(F - 2, 1, true, F - 3);
  for (int i = 0; i < F - 1; ++i) {
    issue(F - 3 - i, (i + 2) % 3, true, F - 4 - i);
    wait_vm<2 * kLdR>();
    step(i % 3, i & 1);
    f32x4 sf[kRT];
#pragma unroll
    for (int t = 0; t < kRT; ++t)
      sf[t] = *reinterpret_cast<const f32x4*>(stage_ptr(i % 3) + (kNG + kRT + t) * 1024 + 16 * lane);
    store_sum(F - 2 - i, sf);
  }
  // no transfer may still be writing the ring when the workgroup ends
  wait_vm0();
}

// ---- output -----------------------------------------------------------------------------
// One workgroup per (b, h, group of `grp` consecutive 64-token blocks of one frame):
// num = Q_rot (S + R), den = Q_pos . (z + zR).  The frame's (S + R)^T is loaded once per group.
// num is formed transposed (the state rows as the A operand) so a lane's accumulator holds
// four consecutive value columns of one token: 8-byte stores.
template <int D>
__global__ __launch_bounds__(256) void out_kernel(const BigdnParams p, int grp) {
  __shared__ __attribute__((aligned(16))) f16 sT[D][D + 8];  // (S + R)^T, row = value column
  __shared__ __attribute__((aligned(16))) f16 qr[64][D + 8];  // Q_rot rows
  __shared__ float zsum[D];
  __shared__ float den_part[64];
  const int nblk = p.N / 64, ngrp = nblk / grp;
  const int g = blockIdx.x % ngrp;
  const int bh = blockIdx.x / ngrp;
  const int b = bh / p.H, h = bh % p.H;
  const int f = (g * grp * 64) / p.S;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int li = lane & 15, lq = lane >> 4;
  const int C = p.H * D;
  const long mat = ((long)bh * p.F + f) * D * D;
  for (int e = tid; e < D * D / 8; e += 256) {
    const int r = e / (D / 8), c0 = (e % (D / 8)) * 8;
    *reinterpret_cast<uint4*>(&sT[r][c0]) = *reinterpret_cast<const uint4*>(p.SsumT + mat + (long)r * D + c0);
  }
  if (tid < D) zsum[tid] = p.zsum[((long)bh * p.F + f) * D + tid];
  const bf16* qkv = static_cast<const bf16*>(p.qkv);
  bf16* num = static_cast<bf16*>(p.num);
  for (int blk = g * grp; blk < (g + 1) * grp; ++blk) {
    const int n0 = blk * 64;
    __syncthreads();
    // prep of q: 64 tokens x D/8 octets over 256 threads; every load of this thread's items
    // is issued before any of them is used
    constexpr int kItems = 64 * (D / 8) / 256;
    float x[kItems][8], w[kItems][8], cs[kItems][8], sn[kItems][8], inv[kItems];
#pragma unroll
    for (int i = 0; i < kItems; ++i) {
      const int e = tid + 256 * i, t = e / (D / 8), d0 = (e % (D / 8)) * 8;
      const long n = n0 + t, bn = (long)b * p.N + n;
      load8f(qkv + bn * 3L * C + (long)h * D + d0, x[i]);
      load8f(p.q_norm_w + h * D + d0, w[i]);
      load8f(p.rope_cos + n * D + d0, cs[i]);
      load8f(p.rope_sin + n * D + d0, sn[i]);
      inv[i] = p.q_inv_rms[bn];
    }
#pragma unroll
    for (int i = 0; i < kItems; ++i) {
      const int e = tid + 256 * i, t = e / (D / 8), d0 = (e % (D / 8)) * 8;
      float pos[8], rot[8];
      prep8(x[i], inv[i], w[i], cs[i], sn[i], 1.f, pos, rot);
      f16x8 v;
      float dp = 0.f;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        v[j] = (f16)rot[j];
        dp += pos[j] * zsum[d0 + j];
      }
      *reinterpret_cast<f16x8*>(&qr[t][d0]) = v;
      // den partial: reduce over the D/8 octets of token t (consecutive e)
#pragma unroll
      for (int off = 1; off < D / 8; off <<= 1) dp += __shfl_xor(dp, off, 64);
      if ((e % (D / 8)) == 0) den_part[t] = dp;
    }
    __syncthreads();
    // num^T: wave w -> tokens 16w..16w+15 (column li of the accumulator), all D value columns
    const long n = n0 + 16 * wave + li;
    bf16* orow = num + (((long)b * p.N + n) * p.H + h) * D;
#pragma unroll
    for (int ct = 0; ct < D / 16; ++ct) {
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int k0 = 0; k0 < D; k0 += 32)
        acc = mma16(lds8(&sT[16 * ct + li][k0 + 8 * lq]), lds8(&qr[16 * wave + li][k0 + 8 * lq]), acc);
      typedef bf16 bf16x4_t __attribute__((ext_vector_type(4)));
      bf16x4_t o4;
#pragma unroll
      for (int e = 0; e < 4; ++e) o4[e] = (bf16)acc[e];
      *reinterpret_cast<bf16x4_t*>(orow + 16 * ct + 4 * lq) = o4;
    }
    if (tid < 64) static_cast<bf16*>(p.den)[(long)bh * p.N + n0 + tid] = (bf16)den_part[tid];
  }
}

}  // namespace

hipError_t launch_prep(const PrepParams& p, hipStream_t stream) {
  hipLaunchKernelGGL(rms_prep_kernel, dim3(p.B * p.N), dim3(kPrepThreads), 0, stream, p);
  return hipGetLastError();
}

hipError_t launch_bigdn(const BigdnParams& p, hipStream_t stream) {
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
  pp.B = p.B;
  pp.N = p.N;
  pp.H = p.H;
  pp.D = p.D;
  hipError_t e = launch_prep(pp, stream);
  if (e != hipSuccess) return e;
  const int nbhf = p.B * p.H * p.F;
  // 64-token blocks per output workgroup (a divisor of the blocks of a frame)
  const int grp = 1;
  if (p.D == 128) {
    hipLaunchKernelGGL(frame_stats_kernel<128>, dim3(nbhf), dim3(kStatThreads), 0, stream, p);
    hipLaunchKernelGGL(scan_kernel<128>, dim3(p.B * p.H * (128 / 16 + 1)), dim3(256), 0, stream, p);
    hipLaunchKernelGGL(out_kernel<128>, dim3(p.B * p.H * (p.N / 64 / grp)), dim3(256), 0, stream, p, grp);
  } else {
    hipLaunchKernelGGL(frame_stats_kernel<64>, dim3(nbhf), dim3(kStatThreads), 0, stream, p);
    hipLaunchKernelGGL(scan_kernel<64>, dim3(p.B * p.H * (64 / 16 + 1)), dim3(256), 0, stream, p);
    hipLaunchKernelGGL(out_kernel<64>, dim3(p.B * p.H * (p.N / 64 / grp)), dim3(256), 0, stream, p, grp);
  }
  return hipGetLastError();
}

}  // namespace gdn

// gdn_prep16.hip -- per-chunk prep of the chunkwise forward for bf16 inputs on gfx950.
//
// One workgroup per 64-token chunk computes everything that does not depend on the state
// (definitions in gdn_fwd.hip): gamma, the decays, A = strict_lower(diag(beta)(K K^T o D)),
// Tm = (I + A)^-1, P = lower(Q K^T o D), and writes them to the chunk's workspace slot as the
// exact LDS images the state scan copies (Slot16): Tm, P and K in fp16, plus the per-token /
// per-key vectors.  For a per-key gate the decay sits inside the key sum, so Q and K are
// scaled per key around the chunk's middle token (rows e^{gamma - gamma_mid}, Gram columns
// e^{gamma_mid - gamma}) and the update operand K e^{gamma_last - gamma} is produced too.
//
// q and k arrive by direct global-to-LDS transfers (one batch, one wait); rows past the end
// of the sequence read as zero through the buffer bounds.  Their LDS layout XOR-permutes the
// 16-byte octets of a row by swz64(row) (gdn_tiles.h), which makes the 16-byte operand reads of 16
// consecutive rows (one octet each) hit 16 distinct bank groups.
#include "gdn_chunk.h"
#include "gdn_dma.h"

namespace gdn {
namespace {

using namespace chunk;
using namespace dma;

constexpr int kThreads = 256;

// element index of (row r, column c) in a [64][K] q / k tile (32-column sub-tiles of 64-byte
// rows, octet o of row r stored at o ^ swz64(r))
__device__ __forceinline__ int pix(int r, int c) {
  return (c >> 5) * (kC * 32) + r * 32 + ((((c >> 3) & 3) ^ swz64(r)) << 3) + (c & 7);
}

template <int K, bool PK>
struct __attribute__((aligned(16))) Prep16Smem {
  typedef f16 TO;
  static constexpr int kTP = kC + 8;
  u16 q[kC * K];            // bf16 Q (per-key gate: fp16 Q e^{gamma - gamma_mid}, in place)
  u16 k[kC * K];            // bf16 K (per-key gate: fp16 K e^{gamma - gamma_mid}, in place)
  u16 kb[PK ? kC * K : 8];  // per-key gate: fp16 K e^{gamma_mid - gamma} (Gram columns)
  u16 kh[PK ? kC * K : 8];  // per-key gate: fp16 K e^{gamma_last - gamma}
  TO tm[kC][kTP];
  TO p[kC][kTP];
  float a[kC][kC + 4];
  float x[32][36];
  float gam[kC], beta[kC], g[kC];
};

template <int K, bool VARLEN, bool PK>
__global__ __launch_bounds__(kThreads) void prep16_kernel(const FwdParams p) {
  typedef Prep16Smem<K, PK> SM;
  typedef Slot16<K, PK> SL;
  typedef typename QKT<bf16, PK>::type TQ;  // tile element type for the products
  typedef typename Vec8<TQ>::type Q8;
  constexpr int kG = K / 32;
  constexpr int kQB = kC * K * 2 / 1024;  // 1 KiB transfer blocks per tile
  __shared__ SM s;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int li = lane & 15, lq = lane >> 4;

  // chunk -> (chain, n)
  int chain, n;
  if (VARLEN) {
    const int h = blockIdx.x / p.nt_total, cg = blockIdx.x % p.nt_total;
    int lo = 0, hi = p.nseq;  // largest i with coffs[i] <= cg
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (p.coffs[mid] <= cg) lo = mid;
      else hi = mid;
    }
    chain = lo * p.H + h;
    n = cg - p.coffs[lo];
  } else {
    const int nt = (p.T + kC - 1) / kC;
    chain = blockIdx.x / nt;
    n = blockIdx.x % nt;
  }
  const ChunkPos cp = chain_pos(p, chain, VARLEN);
  const int h = chain % p.H;
  const int t0 = n * kC, rows = min(kC, cp.len - t0);
  const long tok = cp.tok0 + t0;
  const uint32_t qk_row = (uint32_t)p.H * K * 2;

  // q, k -> LDS (this wave's blocks), bounded to the sequence's remaining rows
  {
    const uint32_t span = (uint32_t)(cp.len - t0) * qk_row;
    const i32x4 rq = make_rsrc(static_cast<const bf16*>(p.q) + (tok * p.H + h) * K, span);
    const i32x4 rk = make_rsrc(static_cast<const bf16*>(p.k) + (tok * p.H + h) * K, span);
#pragma unroll
    for (int i = 0; i < kQB / 4; ++i) {
      const int b = wave + 4 * i;
      const int r = 16 * (b & 3) + (lane >> 2), lo = (lane & 3) ^ swz64(r);
      const uint32_t voff = r * qk_row + (4 * (b >> 2) + lo) * 16;
      dma16(rq, voff, 0, lds_addr(s.q) + 1024u * b);
      dma16(rk, voff, 0, lds_addr(s.k) + 1024u * b);
    }
  }
  if (tid < kC) {
    const bool ok = tid < rows;
    const long gi = (tok + tid) * p.H + h;
    s.g[tid] = ok && p.g ? floor_gate(p.g[gi]) : 0.f;
    s.beta[tid] = ok ? p.beta[gi] : 0.f;
  }
  constexpr int kTPK = kThreads / K, kGT = kC / kTPK;
  float gkr[PK ? kGT : 1];
  if constexpr (PK) {
    const int d = tid / kTPK, part = tid % kTPK;
#pragma unroll
    for (int i = 0; i < kGT; ++i) {
      const int t = part * kGT + i;
      gkr[i] = t < rows ? p.gk[((tok + t) * p.H + h) * (long)K + d] : 0.f;
    }
  }
  // strict upper 16x16 tiles of A / Tm / P stay zero
  for (int e = tid; e < 6 * 256; e += kThreads) {
    const int t = e >> 8, r = (e >> 4) & 15, c = e & 15;
    const int I = (t >= 3) + (t >= 5);
    const int J = (t < 3) ? t + 1 : (t < 5 ? t - 1 : 3);
    s.a[16 * I + r][16 * J + c] = 0.f;
    s.tm[16 * I + r][16 * J + c] = (f16)0.f;
    s.p[16 * I + r][16 * J + c] = (f16)0.f;
  }
  wait_vm0();
  __syncthreads();

  char* slot = static_cast<char*>(p.ws) + (cp.slot0 + n) * (long)SL::kBytes;
  float* vec = reinterpret_cast<float*>(slot + SL::kVec);
  if constexpr (PK) {
    // per-key gamma; scaled Q, K in place, the Gram column operand and the update operand;
    // beta, e^{gamma_mid}, e^{gamma_last} to the slot
    const int d = tid / kTPK, part = tid % kTPK;
    float gam[kGT], gm, gL;
    key_cumsum<K, kGT>(gkr, [&](int t) { return s.g[t]; }, part, gam, gm, gL);
    const bf16* qb = reinterpret_cast<const bf16*>(s.q);
    const bf16* kbf = reinterpret_cast<const bf16*>(s.k);
#pragma unroll
    for (int i = 0; i < kGT; ++i) {
      const int t = part * kGT + i, ix = pix(t, d);
      const float up = __expf(gam[i] - gm), dn = __expf(gm - gam[i]);
      const float kk = (float)kbf[ix], qq = (float)qb[ix];
      reinterpret_cast<f16*>(s.k)[ix] = (f16)(kk * up);
      reinterpret_cast<f16*>(s.q)[ix] = (f16)(qq * up);
      reinterpret_cast<f16*>(s.kb)[ix] = (f16)(kk * dn);
      reinterpret_cast<f16*>(s.kh)[ix] = (f16)(kk * __expf(gL - gam[i]));
    }
    if (part == 0) {
      vec[SL::kEmid + d] = __expf(gm);
      vec[SL::kEglk + d] = __expf(gL);
    }
    if (tid < kC) vec[SL::kBeta + tid] = s.beta[tid];
  } else if (wave == 0) {
    const float gam = wave_incl_scan(s.g[lane], lane);
    const float gl = __shfl(gam, 63, 64);
    s.gam[lane] = gam;
    vec[SL::kEg + lane] = __expf(gam);
    vec[SL::kEl + lane] = __expf(gl - gam);
    vec[SL::kBeta + lane] = s.beta[lane];
    if (lane == 0) vec[SL::kEgl] = __expf(gl);
  }
  __syncthreads();

  // Gram (-> A) and Q K^T (-> P), lower 16x16 tiles: 20 jobs, 5 per wave
  const TQ* qt = reinterpret_cast<const TQ*>(s.q);
  const TQ* kt = reinterpret_cast<const TQ*>(s.k);
  const TQ* kbt = reinterpret_cast<const TQ*>(PK ? s.kb : s.k);
#pragma unroll
  for (int ji = 0; ji < 5; ++ji) {
    const int job = wave + 4 * ji;
    const bool is_qk = job >= 10;
    int I, J;
    tri_tile(is_qk ? job - 10 : job, I, J);
    const TQ* at = is_qk ? qt : kt;
    Q8 av[kG], bv[kG];
#pragma unroll
    for (int kk = 0; kk < kG; ++kk) {
      av[kk] = lds8(at + pix(16 * I + li, 32 * kk + 8 * lq));
      bv[kk] = lds8(kbt + pix(16 * J + li, 32 * kk + 8 * lq));
    }
    const int sc = 16 * J + li;
    float gr[4], br[4];
    const float gs = PK ? 0.f : s.gam[sc];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      gr[e] = PK ? 0.f : s.gam[16 * I + 4 * lq + e];
      br[e] = s.beta[16 * I + 4 * lq + e];
    }
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kk = 0; kk < kG; ++kk) acc = mma16(av[kk], bv[kk], acc);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int r = 16 * I + 4 * lq + e;
      const float dd = PK ? 1.f : __expf(gr[e] - gs);
      if (is_qk) s.p[r][sc] = (f16)(sc <= r ? dd * acc[e] : 0.f);
      else s.a[r][sc] = sc < r ? br[e] * dd * acc[e] : 0.f;
    }
  }
  __syncthreads();
  solve_unit_lower(s, wave, lane);

  // Tm, P -> slot, 16-byte pieces in the scan's column-split layout
  for (int c = tid; c < 2 * kC * kC / 8; c += kThreads) {
    const int which = c / (kC * kC / 8), cc = c % (kC * kC / 8);
    const int r = cc / (kC / 8), c0 = (cc % (kC / 8)) * 8;
    const f16* src = which ? &s.p[r][c0] : &s.tm[r][c0];
    *reinterpret_cast<u32x4*>(slot + (which ? SL::kP : SL::kTm) + 2 * tix_s32<kC>(r, c0)) =
        *reinterpret_cast<const u32x4*>(src);
  }
  if constexpr (PK) {
    // scaled Q, K and the update operand (already fp16)
    constexpr int kPieces = kC * K / 8;
    for (int c = tid; c < 3 * kPieces; c += kThreads) {
      const int which = c / kPieces, cc = c % kPieces;
      const int r = cc / (K / 8), c0 = (cc % (K / 8)) * 8;
      const u16* src = which == 0 ? s.q : (which == 1 ? s.k : s.kh);
      const size_t base = which == 0 ? SL::kQ : (which == 1 ? SL::kK : SL::kKh);
      *reinterpret_cast<u32x4*>(slot + base + 2 * tix_s32<kC>(r, c0)) =
          *reinterpret_cast<const u32x4*>(&src[pix(r, c0)]);
    }
  } else {
    // K as fp16 (exact for bf16 values in fp16's normal range)
    for (int c = tid; c < kC * K / 8; c += kThreads) {
      const int r = c / (K / 8), c0 = (c % (K / 8)) * 8;
      const u32x4 x = *reinterpret_cast<const u32x4*>(&s.k[pix(r, c0)]);
      u32x4 y;
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const float lo = __uint_as_float(x[w] << 16), hi = __uint_as_float(x[w] & 0xffff0000u);
        y[w] = __builtin_bit_cast(unsigned, __builtin_amdgcn_cvt_pkrtz(lo, hi));
      }
      *reinterpret_cast<u32x4*>(slot + SL::kK + 2 * tix_s32<kC>(r, c0)) = y;
    }
  }
}

// ---------------------------------------------------------------------------------------
// Per-key gate.  Thread (octet o, part) loads keys 8o .. 8o+7 of q, k and gk for kTP
// consecutive tokens, so the per-key cumulative decay is a running sum over its tokens plus a
// prefix over the parts (lanes of one wave).
//
// The decay of a Gram / Q K^T entry sits inside the key sum, sum_d x_{r,d} k_{s,d}
// e^{gamma_{r,d} - gamma_{s,d}} (s <= r), so it is factored around a reference token m as
// (x_r e^{gamma_r - gamma_m}) . (k_s e^{gamma_m - gamma_s}).  Each 16x16 tile takes its own
// reference, chosen so that the factors stay in range for any decay:
//  - off-diagonal tile (I, J < I): m = 16I, the first row of block I.  Both factors are then
//    at most 1 (gamma only decreases), so the tiles take fp16 operands; a factor that
//    underflows belongs to a product that is smaller still.
//  - diagonal tile (I, I): m = 16I + 8.  The factors span e^{+-8 lambda_max}; with the per-key
//    log decay floored at kKeyGateFloor (-10) they stay within e^{+-80}, inside the bf16
//    exponent range.  The Gram tile takes bf16 operands; the Q K^T tile (the intra-chunk part
//    of the output) needs more than bf16's 8-bit significand, so both of its operands are
//    split into a bf16 value and a bf16 remainder and three products are summed.
// The operand tiles of the four phases (off-diagonal K rows, off-diagonal Q rows, diagonal
// tiles of blocks 0-1, of blocks 2-3) share one LDS region with the solve's work arrays,
// which keeps the kernel at 2 workgroups per CU.
//
// The scan's operands go straight to the slot in fp16: Q e^{gamma}, K e^{gamma} and
// K e^{gamma_last - gamma}, all at most |x| (the per-key reference of the scan is 1).
// ---------------------------------------------------------------------------------------
template <int K>
struct __attribute__((aligned(16))) PrepPkSmem {
  typedef f16 TO;
  static constexpr int kTP = kC + 8;
  static constexpr int kBlk = 16 * K;  // elements of one 16-row operand block
  union {
    struct {                   // off-diagonal tiles (fp16)
      u16 row[kC * K];         // K (then Q) times e^{gamma - gamma_{16b}}, b the row's block (pix)
      u16 col[6 * kBlk];       // K times e^{gamma_{16I} - gamma} on the rows of block J < I,
                               // pair (I, J) at block I (I - 1) / 2 + J (tix_s32<16>)
    };
    struct {                   // diagonal tiles of two blocks (bf16, tix_s32<32>)
      u16 dqh[2 * kBlk], dql[2 * kBlk];  // Q e^{gamma - gamma_mid}: value and remainder
      u16 dk[2 * kBlk];                  // K e^{gamma - gamma_mid}
      u16 dch[2 * kBlk], dcl[2 * kBlk];  // K e^{gamma_mid - gamma}: value and remainder
    };
    struct {                   // solve work arrays, used once the products are done
      float x[32][36];
      TO tm[kC][kTP];
    };
  };
  float a[kC][kC + 4];
  TO p[kC][kTP];
  float beta[kC];
  float gx[2][4][K];  // per 16-token block and key: the block's decay sum and the decay of
                      // its first token
};

template <int K, bool VARLEN>
__global__ __launch_bounds__(kThreads, 2) void prep16pk_kernel(const FwdParams p) {
  typedef PrepPkSmem<K> SM;
  typedef Slot16<K, true> SL;
  constexpr int kG = K / 32;
  constexpr int kOct = K / 8;              // 16-byte octets per row
  constexpr int kParts = kThreads / kOct;  // token parts of kTP tokens each
  constexpr int kTP = kC / kParts;         // tokens per thread
  static_assert(kParts <= 64 && kC % kParts == 0 && (kC / 2) % kTP == 0, "thread layout");
  __shared__ SM s;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int li = lane & 15, lq = lane >> 4;

  // chunk -> (chain, n)
  int chain, n;
  if (VARLEN) {
    const int hh = blockIdx.x / p.nt_total, cg = blockIdx.x % p.nt_total;
    int lo = 0, hi = p.nseq;  // largest i with coffs[i] <= cg
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (p.coffs[mid] <= cg) lo = mid;
      else hi = mid;
    }
    chain = lo * p.H + hh;
    n = cg - p.coffs[lo];
  } else {
    const int nt = (p.T + kC - 1) / kC;
    chain = blockIdx.x / nt;
    n = blockIdx.x % nt;
  }
  const ChunkPos cp = chain_pos(p, chain, VARLEN);
  const int h = chain % p.H;
  const int t0 = n * kC;
  const uint32_t rows = (uint32_t)min(kC, cp.len - t0);
  const long tok = cp.tok0 + t0;
  char* slot = static_cast<char*>(p.ws) + (cp.slot0 + n) * (long)SL::kBytes;
  float* vec = reinterpret_cast<float*>(slot + SL::kVec);

  // ---- thread layout: wave w holds the 16-token block w, lane = o kPB + pb (octet o of the
  // keys, part pb of the block's tokens), so every branch on the block is wave-uniform
  constexpr int kPB = 16 / kTP;  // parts per 16-token block
  static_assert(kOct * kPB == 64, "one 16-token block per wave");
  const int blk = wave;
  const int pb = lane % kPB, o = lane / kPB;
  const int part = blk * kPB + pb;

  // ---- loads: q, k (bf16) and gk (fp32) of this thread's keys and tokens, g and beta per
  // token; rows past the end of the sequence read as zero through the buffer bounds
  const uint32_t qk_row = (uint32_t)p.H * K * 2, gk_row = (uint32_t)p.H * K * 4;
  const __amdgpu_buffer_rsrc_t rq = store_rsrc(const_cast<bf16*>(static_cast<const bf16*>(p.q)) + (tok * p.H + h) * K, rows * qk_row);
  const __amdgpu_buffer_rsrc_t rk = store_rsrc(const_cast<bf16*>(static_cast<const bf16*>(p.k)) + (tok * p.H + h) * K, rows * qk_row);
  const __amdgpu_buffer_rsrc_t rg = store_rsrc(const_cast<float*>(p.gk) + (tok * p.H + h) * (long)K, rows * gk_row);
  u32x4 qv[kTP], kv[kTP];
  f32x4 gk0[kTP], gk1[kTP];
  float gt[kTP];
#pragma unroll
  for (int i = 0; i < kTP; ++i) {
    const int t = part * kTP + i;
    qv[i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rq, t * qk_row + 16 * o, 0, 0));
    kv[i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rk, t * qk_row + 16 * o, 0, 0));
    gk0[i] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(rg, t * gk_row + 32 * o, 0, 0));
    gk1[i] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(rg, t * gk_row + 32 * o + 16, 0, 0));
    gt[i] = (p.g && (uint32_t)t < rows) ? floor_gate(p.g[(tok + t) * p.H + h]) : 0.f;
  }
  if (tid < kC) s.beta[tid] = (uint32_t)tid < rows ? p.beta[(tok + tid) * p.H + h] : 0.f;

  // ---- per-key cumulative decay gamma[t][8o + j] of lambda = max(g + gk, kKeyGateFloor):
  // running sum over this thread's tokens, the inclusive prefix over the block's parts (lane
  // shuffles), then the sums of the blocks before it (through LDS).  Rows past the end carry
  // lambda = 0.
  float gam[kTP][8], tot[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    float run = 0.f;
#pragma unroll
    for (int i = 0; i < kTP; ++i) {
      run += floor_key_gate(gt[i] + (j < 4 ? gk0[i][j] : gk1[i][j - 4]));
      gam[i][j] = run;
    }
    tot[j] = run;
  }
  float incl[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) incl[j] = tot[j];
#pragma unroll
  for (int sh = 1; sh < kPB; sh <<= 1) {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const float u = __shfl_up(incl[j], sh, kPB);
      incl[j] += pb >= sh ? u : 0.f;
    }
  }
  if (pb == kPB - 1) {
#pragma unroll
    for (int j = 0; j < 8; ++j) s.gx[0][blk][8 * o + j] = incl[j];
  }
  if (pb == 0) {
#pragma unroll
    for (int j = 0; j < 8; ++j) s.gx[1][blk][8 * o + j] = gam[0][j];
  }
  __syncthreads();
  // gs[I]: gamma at the first token of block I (used for the blocks after this one); gl:
  // gamma at token 63
  float gs[4][8], gl[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    float run = 0.f, off = 0.f;
#pragma unroll
    for (int I = 0; I < 4; ++I) {
      off = I == blk ? run : off;
      gs[I][j] = run + s.gx[1][I][8 * o + j];
      run += s.gx[0][I][8 * o + j];
    }
    gl[j] = run;
    const float ex = off + incl[j] - tot[j];
#pragma unroll
    for (int i = 0; i < kTP; ++i) gam[i][j] += ex;
  }
  // gamma at the first and the middle token of this block (element 0 of a part, since kTP
  // divides 8)
  float gsb[8], gmb[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    gsb[j] = __shfl(gam[0][j], o * kPB, 64);
    gmb[j] = __shfl(gam[0][j], o * kPB + 8 / kTP, 64);
  }
  if (blk == 0 && pb == 0) {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      vec[SL::kEmid + 8 * o + j] = 1.f;  // the scan's operands carry e^{gamma} themselves
      vec[SL::kEglk + 8 * o + j] = __expf(gl[j]);
    }
  }

  // bf16 raw -> fp32
  auto unpack = [](const u32x4& w, f32x4& lo4, f32x4& hi4) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const unsigned x0 = w[j >> 1], x1 = w[2 + (j >> 1)];
      lo4[j] = (j & 1) ? __uint_as_float(x0 & 0xffff0000u) : __uint_as_float(x0 << 16);
      hi4[j] = (j & 1) ? __uint_as_float(x1 & 0xffff0000u) : __uint_as_float(x1 << 16);
    }
  };
  // x (8 keys) times e^{e[j]} into 8 16-bit values of type T
  auto scaled = [](const f32x4& x0, const f32x4& x1, const float* e, auto tag) {
    typedef decltype(tag) T;
    f32x4 y0, y1;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      y0[j] = x0[j] * __expf(e[j]);
      y1[j] = x1[j] * __expf(e[4 + j]);
    }
    return __builtin_bit_cast(u32x4, pack8<T>(y0, y1));
  };
  // bf16 value and bf16 remainder of x (8 keys) times e^{e[j]}
  auto split = [](const f32x4& x0, const f32x4& x1, const float* e, u32x4& hi, u32x4& lo) {
    f32x4 y0, y1, r0, r1;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      y0[j] = x0[j] * __expf(e[j]);
      y1[j] = x1[j] * __expf(e[4 + j]);
    }
    const bf16x8 h = pack8<bf16>(y0, y1);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      r0[j] = y0[j] - (float)h[j];
      r1[j] = y1[j] - (float)h[4 + j];
    }
    hi = __builtin_bit_cast(u32x4, h);
    lo = __builtin_bit_cast(u32x4, pack8<bf16>(r0, r1));
  };

  // x (8 keys) times m[j] into 8 16-bit values of type T
  auto scaledm = [](const f32x4& x0, const f32x4& x1, const float* m, auto tag) {
    typedef decltype(tag) T;
    f32x4 y0, y1;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      y0[j] = x0[j] * m[j];
      y1[j] = x1[j] * m[4 + j];
    }
    return __builtin_bit_cast(u32x4, pack8<T>(y0, y1));
  };

  // ---- the scan's operands, straight to the slot: Q e^{gamma}, K e^{gamma} and
  // K e^{gamma_last - gamma} (fp16); and the column operands of the off-diagonal tiles,
  // K e^{gamma_16I - gamma} on this block's rows for every row block I after it.  The last
  // two are e^{gamma_mid - gamma} (at most e^{70} inside the block, by the floor) times a
  // per-key factor of the block that is at most 1, so one exponential per element serves
  // all four; a factor that underflows leaves products below fp16's subnormal range.
  float ckh[8], ccol[4][8];
#pragma unroll
  for (int j = 0; j < 8; ++j) ckh[j] = __expf(gl[j] - gmb[j]);
#pragma unroll
  for (int I = 1; I < 4; ++I) {
    if (I <= blk) continue;
#pragma unroll
    for (int j = 0; j < 8; ++j) ccol[I][j] = __expf(gs[I][j] - gmb[j]);
  }
  f32x4 qf0[kTP], qf1[kTP], kf0[kTP], kf1[kTP];
#pragma unroll
  for (int i = 0; i < kTP; ++i) {
    const int t = part * kTP + i;
    unpack(qv[i], qf0[i], qf1[i]);
    unpack(kv[i], kf0[i], kf1[i]);
    float eg[8], ed[8], m[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      eg[j] = __expf(gam[i][j]);
      ed[j] = __expf(gmb[j] - gam[i][j]);
      m[j] = ed[j] * ckh[j];
    }
    const int sx = 2 * tix_s32<kC>(t, 8 * o);
    *reinterpret_cast<u32x4*>(slot + SL::kQ + sx) = scaledm(qf0[i], qf1[i], eg, f16{});
    *reinterpret_cast<u32x4*>(slot + SL::kK + sx) = scaledm(kf0[i], kf1[i], eg, f16{});
    *reinterpret_cast<u32x4*>(slot + SL::kKh + sx) = scaledm(kf0[i], kf1[i], m, f16{});
#pragma unroll
    for (int I = 1; I < 4; ++I) {
      if (I <= blk) continue;
#pragma unroll
      for (int j = 0; j < 8; ++j) m[j] = ed[j] * ccol[I][j];
      const int c = I * (I - 1) / 2 + blk;
      *reinterpret_cast<u32x4*>(&s.col[c * SM::kBlk + tix_s32<16>(t - 16 * blk, 8 * o)]) =
          scaledm(kf0[i], kf1[i], m, f16{});
    }
  }
  // strict upper 16x16 tiles of A and P stay zero
  for (int e = tid; e < 6 * 256; e += kThreads) {
    const int t = e >> 8, r = (e >> 4) & 15, c = e & 15;
    const int I = (t >= 3) + (t >= 5);
    const int J = (t < 3) ? t + 1 : (t < 5 ? t - 1 : 3);
    s.a[16 * I + r][16 * J + c] = 0.f;
    s.p[16 * I + r][16 * J + c] = (f16)0.f;
  }

  // One 16x16 product tile: rows 16 RI + li of tile `at`, rows 16 RJ + li of tile `bt` (both
  // R-row column-split tiles), contraction over the K keys.
  auto tile = [&](auto ra_c, const u16* at, int RI, auto rb_c, const u16* bt, int RJ, auto elt,
                  f32x4 acc) {
    constexpr int RA = decltype(ra_c)::value, RB = decltype(rb_c)::value;
    typedef decltype(elt) T;
    typedef typename Vec8<T>::type T8;
    const T* a = reinterpret_cast<const T*>(at);
    const T* b = reinterpret_cast<const T*>(bt);
    T8 av[kG], bv[kG];
#pragma unroll
    for (int kk = 0; kk < kG; ++kk) {
      av[kk] = *reinterpret_cast<const T8*>(a + tix_s32<RA>(16 * RI + li, 32 * kk + 8 * lq));
      bv[kk] = *reinterpret_cast<const T8*>(b + tix_s32<RB>(16 * RJ + li, 32 * kk + 8 * lq));
    }
#pragma unroll
    for (int kk = 0; kk < kG; ++kk) acc = mma16(av[kk], bv[kk], acc);
    return acc;
  };
  // stores of a tile's accumulator: lane holds column 16 J + li, rows 16 I + 4 lq + e
  auto store_a = [&](int I, int J, const f32x4& acc) {
    const int sc = 16 * J + li;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int r = 16 * I + 4 * lq + e;
      s.a[r][sc] = sc < r ? s.beta[r] * acc[e] : 0.f;
    }
  };
  auto store_p = [&](int I, int J, const f32x4& acc) {
    const int sc = 16 * J + li;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int r = 16 * I + 4 * lq + e;
      s.p[r][sc] = (f16)(sc <= r ? acc[e] : 0.f);
    }
  };
  const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
  constexpr auto R16 = std::integral_constant<int, 16>{};
  constexpr auto R32 = std::integral_constant<int, 32>{};
  constexpr auto R64 = std::integral_constant<int, kC>{};

  // ---- off-diagonal tiles, reference = first row of the row block (fp16 operands); the
  // column operands are in place.
  // phase 1a: K rows; Gram tiles (I, J < I)
  auto rows_off = [&](const f32x4* x0, const f32x4* x1) {
#pragma unroll
    for (int i = 0; i < kTP; ++i) {
      const int t = part * kTP + i;
      float e[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) e[j] = gam[i][j] - gsb[j];
      *reinterpret_cast<u32x4*>(&s.row[pix(t, 8 * o)]) = scaled(x0[i], x1[i], e, f16{});
    }
  };
  rows_off(kf0, kf1);
  __syncthreads();
  // six tiles (1,0) (2,0) (2,1) (3,0) (3,1) (3,2); waves 0, 1 take two, waves 2, 3 one
  for (int jb = wave; jb < 6; jb += 4) {
    const int I = jb < 1 ? 1 : (jb < 3 ? 2 : 3), J = jb - I * (I - 1) / 2;
    const f32x4 acc = tile(R64, s.row, I, R16, s.col + (I * (I - 1) / 2 + J) * SM::kBlk, 0, f16{}, zero);
    store_a(I, J, acc);
  }
  __syncthreads();
  // phase 1b: Q rows; Q K^T tiles (I, J < I)
  rows_off(qf0, qf1);
  __syncthreads();
  for (int jb = wave; jb < 6; jb += 4) {
    const int I = jb < 1 ? 1 : (jb < 3 ? 2 : 3), J = jb - I * (I - 1) / 2;
    const f32x4 acc = tile(R64, s.row, I, R16, s.col + (I * (I - 1) / 2 + J) * SM::kBlk, 0, f16{}, zero);
    store_p(I, J, acc);
  }
  // ---- diagonal tiles, reference = middle row of the block (bf16 operands), two blocks per
  // phase: waves 0, 1 the Gram tiles, waves 2, 3 the Q K^T tiles (split operands)
#pragma unroll
  for (int ph = 0; ph < 2; ++ph) {
    __syncthreads();  // the previous phase's operand reads are done
    if ((blk >> 1) == ph) {
#pragma unroll
      for (int i = 0; i < kTP; ++i) {
        const int t = part * kTP + i, rr = t - 32 * ph;
        float eu[8], ed[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          eu[j] = gam[i][j] - gmb[j];
          ed[j] = -eu[j];
        }
        const int ix = tix_s32<32>(rr, 8 * o);
        u32x4 hi, lo;
        split(qf0[i], qf1[i], eu, hi, lo);
        *reinterpret_cast<u32x4*>(&s.dqh[ix]) = hi;
        *reinterpret_cast<u32x4*>(&s.dql[ix]) = lo;
        *reinterpret_cast<u32x4*>(&s.dk[ix]) = scaled(kf0[i], kf1[i], eu, bf16{});
        split(kf0[i], kf1[i], ed, hi, lo);
        *reinterpret_cast<u32x4*>(&s.dch[ix]) = hi;
        *reinterpret_cast<u32x4*>(&s.dcl[ix]) = lo;
      }
    }
    __syncthreads();
    const int u = wave & 1, I = 2 * ph + u;
    if (wave < 2) {
      store_a(I, I, tile(R32, s.dk, u, R32, s.dch, u, bf16{}, zero));
    } else {
      f32x4 acc = tile(R32, s.dqh, u, R32, s.dch, u, bf16{}, zero);
      acc = tile(R32, s.dqh, u, R32, s.dcl, u, bf16{}, acc);
      acc = tile(R32, s.dql, u, R32, s.dch, u, bf16{}, acc);
      store_p(I, I, acc);
    }
  }
  if (tid < kC) vec[SL::kBeta + tid] = s.beta[tid];
  __syncthreads();  // the operand tiles are dead from here: x and tm reuse their space
  // strict upper 16x16 tiles of Tm stay zero
  for (int e = tid; e < 6 * 256; e += kThreads) {
    const int t = e >> 8, r = (e >> 4) & 15, c = e & 15;
    const int I = (t >= 3) + (t >= 5);
    const int J = (t < 3) ? t + 1 : (t < 5 ? t - 1 : 3);
    s.tm[16 * I + r][16 * J + c] = (f16)0.f;
  }
  solve_unit_lower(s, wave, lane);

  // Tm, P -> slot, 16-byte pieces in the scan's column-split layout
  for (int c = tid; c < 2 * kC * kC / 8; c += kThreads) {
    const int which = c / (kC * kC / 8), cc = c % (kC * kC / 8);
    const int r = cc / (kC / 8), c0 = (cc % (kC / 8)) * 8;
    const f16* src = which ? &s.p[r][c0] : &s.tm[r][c0];
    *reinterpret_cast<u32x4*>(slot + (which ? SL::kP : SL::kTm) + 2 * tix_s32<kC>(r, c0)) =
        *reinterpret_cast<const u32x4*>(src);
  }
}

template <int K, bool VL, bool PK>
hipError_t launch_k(const FwdParams& p, long nslots, hipStream_t stream) {
  if constexpr (PK) hipLaunchKernelGGL((prep16pk_kernel<K, VL>), dim3(nslots), dim3(kThreads), 0, stream, p);
  else hipLaunchKernelGGL((prep16_kernel<K, VL, PK>), dim3(nslots), dim3(kThreads), 0, stream, p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_prep16(const FwdParams& p, int K, bool varlen, bool pk, long nslots,
                         hipStream_t stream) {
  if (K == 128) {
    if (pk) return varlen ? launch_k<128, true, true>(p, nslots, stream) : launch_k<128, false, true>(p, nslots, stream);
    return varlen ? launch_k<128, true, false>(p, nslots, stream) : launch_k<128, false, false>(p, nslots, stream);
  }
  if (pk) return varlen ? launch_k<64, true, true>(p, nslots, stream) : launch_k<64, false, true>(p, nslots, stream);
  return varlen ? launch_k<64, true, false>(p, nslots, stream) : launch_k<64, false, false>(p, nslots, stream);
}

}  // namespace gdn

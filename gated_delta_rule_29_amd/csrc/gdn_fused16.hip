// gdn_fused16.hip -- single-kernel chunkwise gated delta-rule forward for bf16 inputs with a
// scalar gate (gfx950).
//
// The state pass over the chunks of a chain is sequential; everything a chunk needs that does
// not depend on the state (gamma, the decays, A = strict_lower(diag(beta)(K K^T o D)),
// Tm = (I + A)^-1 and P = lower(Q K^T o D); definitions in gdn_fwd.hip) is not.  This kernel
// overlaps the two inside one workgroup per (chain, 32-column value block), eight waves (wave
// w and w + 4 share a SIMD):
//
//   waves 0, 1     state scan of chunk n for 16 value columns each (h in registers, fp32):
//                    X_K = K h, Y = V - diag(e^gamma) X_K, v_new = (Tm diag(beta)) Y,
//                    o = scale (diag(e^gamma) Q h + P v_new),
//                    h <- e^gl h + K^T diag(e^{gl-gamma}) v_new
//   waves 2, 3     Gram tiles of the diagonal 16x16 blocks of chunk n+1 and their inverses;
//                    then the off-diagonal block columns of Tm
//   wave 6         off-diagonal Gram tiles of chunk n+1 -> A
//   wave 7         Q K^T tiles of chunk n+1 -> P
//   waves 4, 5     transfers: q, k of chunk n+2 and v of chunk n+1 straight from HBM into
//                    LDS (buffer loads with the LDS destination); g, beta of chunk n+3 into
//                    registers; the gate quantities of chunk n+2 (gamma and its exponentials).
//
// One workgroup barrier per chunk hands every stage on.  q / k tiles and the gate quantities
// sit in rings of three LDS slots (scan reads n, prep reads n+1, transfers fill n+2); v, Tm
// and P in rings of two.  Waves 2, 3 and 6 meet once more inside a step through a counter in
// LDS (solve_bar).  Nothing per chunk goes through HBM: q, k, v are read once per workgroup
// (the value blocks of a chain share them in L2) and o is written once.
//
// Decays.  The Gram and Q K^T epilogues need e^{gamma_r - gamma_s} for s <= r.  When the
// chunk's total decay gamma_0 - gamma_63 is below 80 it is formed as the product of per-token
// factors around the middle token, e^{gamma_r - gamma_31} e^{gamma_31 - gamma_s}, which cannot
// overflow; otherwise every element takes its own exponential.
//
// The solve.  A diagonal block L (strictly lower, L^16 = 0) is inverted as
// (I + L)^-1 = (I - L)(I + L^2)(I + L^4)(I + L^8); the off-diagonal blocks follow block
// column by block column, T_ij = -T_ii sum_{j<=k<i} A_ik T_kj.  Both use 16x16x16 fp16
// matrix products with fp32 accumulation; every matrix is kept in the two register layouts
// the products need (a product's accumulator is the B operand of the next one, and the
// accumulator of the transposed product is its A operand), so the chains never go through LDS.
//
// Operand precision: K h, Q h and the Gram / Q K^T products take bf16 operands (the inputs are
// bf16; h is rounded to bf16); Tm Y and P v_new take fp16 (bounded factors, 11-bit
// significands); the state update K^T v_new takes K exactly in bf16 against v_new e^{gl-gamma}
// split into a bf16 high part and a bf16 remainder (two products).
//
// LDS tiles: column-split [64][W] layout (32-column sub-tiles of 64-byte rows) whose 16-byte
// octets are XOR-permuted by swz64(r) (gdn_tiles.h): the reads of one octet from 16 rows in
// both row orders the kernel uses -- 16 consecutive rows (Gram tiles) and the pair rows
// 32G + 8i + 4t + j (scan products) -- and the transposed reads of the v tile are then free of
// LDS bank conflicts on gfx950.
#include "gdn_chunk.h"
#include "gdn_dma.h"

namespace gdn {
namespace {

using namespace chunk;
using namespace dma;

typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

constexpr int kBV = 32;    // value columns per workgroup (16 per scan wave)
constexpr int kThr = 512;  // 8 waves

// element index of (r, c) in a [64][W] tile (W a multiple of 32)
__device__ __forceinline__ int tix(int r, int c) {
  return (c >> 5) * (kC * 32) + r * 32 + ((((c >> 3) & 3) ^ swz64(r)) << 3) + (c & 7);
}
// logical octet a lane must fetch so that a linear 16-byte-per-lane LDS write lands it at
// physical octet (lane & 3) of row r
__device__ __forceinline__ int src_octet(int r, int lane) { return (lane & 3) ^ swz64(r); }

// Gate slot of one chunk (floats): e^gamma [0, 64), e^{gl - gamma} [64, 128), beta [128, 192),
// e^gl at 192; factors beta e^{gamma - gamma_31} [256, 320), e^{gamma - gamma_31} [320, 384),
// e^{gamma_31 - gamma} [384, 448); gamma [448, 512); at 512 a flag: the factors are usable.
constexpr int kEg = 0, kEl = 64, kBeta = 128, kEgl = 192, kFrk = 256, kFrq = 320, kFc = 384,
              kGam = 448, kFast = 512, kGateF = 516;

template <int K>
struct __attribute__((aligned(16))) FusedSmem {
  struct QK {
    u16 q[kC * K];
    u16 k[kC * K];
  } qk[3];
  u16 v[2][kC * kBV];
  struct TP {
    u16 tm[kC * kC];  // fp16 Tm
    u16 p[kC * kC];   // fp16 P
  } tp[2];
  float gate[3][kGateF];
  u16 af[kC * kC];      // fp16 rows of the off-diagonal blocks of A (tix layout)
  unsigned pbar;        // prep-wave pair barrier counter
  unsigned sink[64];    // destination of the L2 prefetch loads (never read)
};

// L2 prefetch distance: while chunk n is scanned, transfer wave 1 touches the lines of chunk
// n + 2 + kPF, whose q / k transfers are issued kPF steps later.
constexpr int kPF = 2;

// LDS base addresses the optimiser cannot relate to one another: each tile read is then
// issued as its own base plus an instruction immediate (the compiler would otherwise derive
// many addresses from one register with a separate add each).
typedef __attribute__((address_space(3))) const u16 lds_u16;
__device__ __forceinline__ lds_u16* lds_base(const u16* p) {
  lds_u16* b = (lds_u16*)(uintptr_t)lds_addr(p);
  asm volatile("" : "+v"(b));
  return b;
}
template <typename V>
__device__ __forceinline__ V lds_at(lds_u16* b, int off) {
  return *(const __attribute__((address_space(3))) V*)(b + off);
}
__device__ __forceinline__ u32x2 tr16_at(lds_u16* b, int off) {
  return __builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(b + off)));
}

__device__ __forceinline__ float bf_lo(unsigned w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf_hi(unsigned w) { return __uint_as_float(w & 0xffff0000u); }
__device__ __forceinline__ float bf_at(const u32x2& v, int e) {
  return (e & 1) ? bf_hi(v[e >> 1]) : bf_lo(v[e >> 1]);
}

__device__ __forceinline__ u32x2 pack_bf16x4(float a, float b, float c, float d) {
  // built as one vector so that the conversions pair up into packed converts
  bf16x4 v;
  v[0] = (bf16)a;
  v[1] = (bf16)b;
  v[2] = (bf16)c;
  v[3] = (bf16)d;
  return __builtin_bit_cast(u32x2, v);
}

typedef f16 f16x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ f16x4 cvt_f16x4(const f32x4& x) {
  return f16x4{(f16)x[0], (f16)x[1], (f16)x[2], (f16)x[3]};
}

// 16x16 output, contraction 16: lane (li, lq) supplies A[li][4lq + j] and B[4lq + j][li]
// (j = 0..3) and holds C[4lq + e][li], so an accumulator can feed the next product as B.
__device__ __forceinline__ f32x4 mma16x16x16(const f16x4& a, const f16x4& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x16f16(a, b, c, 0, 0, 0);
}

// The lane index, opaque to the optimiser: addresses derived from it are recomputed where
// they are used instead of being kept in registers from an earlier computation.
__device__ __forceinline__ int opaque_lane() {
  int l = __lane_id();
  asm volatile("" : "+v"(l));
  return l;
}

// Barrier of the prep waves that build Tm (three of them).  Each wave's earlier LDS accesses
// complete before its increment (lgkmcnt(0)); LDS is coherent within the workgroup, so after
// the wait the other waves' writes are visible.  Each of them calls it once per step.
__device__ __forceinline__ void solve_bar(unsigned* ctr, unsigned& target) {
  target += 3;
  asm volatile("s_waitcnt lgkmcnt(0)" : : : "memory");
  if ((threadIdx.x & 63) == 0) __hip_atomic_fetch_add(ctr, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
  while (__hip_atomic_load(ctr, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP) < target)
    __builtin_amdgcn_s_sleep(1);
  asm volatile("" : : : "memory");
}

// Stores of 16x16 accumulator rows into a [64][64] fp16 tile: element
// tix(16I + li, 16J + 4lq) = tix(li, 16(J & 1) + 4lq) + 2048 (J >> 1) + 512 I (the octet
// permutation sees only li), so two per-lane bases (J even, J odd) plus instruction immediates
// address every tile.
typedef __attribute__((address_space(3))) u16 lds_u16w;
__device__ __forceinline__ lds_u16w* lds_wbase(u16* p) {
  lds_u16w* b = (lds_u16w*)(uintptr_t)lds_addr(p);
  asm volatile("" : "+v"(b));
  return b;
}
__device__ __forceinline__ void put_f16x4(lds_u16w* b, int off, const f16x4& v) {
  *(__attribute__((address_space(3))) f16x4*)(b + off) = v;
}

// Lower 16x16 tiles (I, J) of the Gram K K^T (ISQ false: A, strictly lower, rows scaled by
// beta) or of Q K^T (ISQ true: P, with the output scale), those selected by MASK (bit
// I(I+1)/2 + J), decay-weighted and stored as fp16 rows of dst.  The products take the rows of
// their second factor as the A operand, so a lane's accumulator of tile (I, J) holds columns
// s = 16J + 4lq + e of row r = 16I + li.  decay(r, s) = e^{gamma_r - gamma_s} comes from the
// per-token factors of the gate slot (FAST) or, when the chunk decays too fast for them, from
// gamma itself.
template <int K, bool ISQ, unsigned MASK, bool FAST>
__device__ __forceinline__ void prod_tiles(const bf16* qt, const bf16* kt, const float* G,
                                           u16* dst, float scale) {
  constexpr int kG = K / 32;
  const int lane = __lane_id(), li = lane & 15, lq = lane >> 4;
  constexpr auto tile_on = [](int I, int J) { return ((MASK >> (I * (I + 1) / 2 + J)) & 1u) != 0; };
  constexpr auto row_on = [](int I) {
    for (int J = 0; J <= I; ++J)
      if (((MASK >> (I * (I + 1) / 2 + J)) & 1u) != 0) return true;
    return false;
  };
  constexpr auto col_on = [](int J) {
    for (int I = J; I < 4; ++I)
      if (((MASK >> (I * (I + 1) / 2 + J)) & 1u) != 0) return true;
    return false;
  };
  bf16x8 af[4][kG], bf[4][kG];
#pragma unroll
  for (int kk = 0; kk < kG; ++kk)
#pragma unroll
    for (int I = 0; I < 4; ++I) {
      if (col_on(I) || (!ISQ && row_on(I))) bf[I][kk] = lds8(kt + tix(16 * I + li, 32 * kk + 8 * lq));
      if (ISQ && row_on(I)) af[I][kk] = lds8(qt + tix(16 * I + li, 32 * kk + 8 * lq));
    }
  __builtin_amdgcn_sched_barrier(0);
  f32x4 acc[10];
#pragma unroll
  for (int t = 0; t < 10; ++t) acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int kk = 0; kk < kG; ++kk) {
#pragma unroll
    for (int I = 0, t = 0; I < 4; ++I)
#pragma unroll
      for (int J = 0; J <= I; ++J, ++t)
        if (tile_on(I, J)) acc[t] = mma16(bf[J][kk], ISQ ? af[I][kk] : bf[I][kk], acc[t]);
    __builtin_amdgcn_sched_barrier(0);
  }
  lds_u16w* sb[2] = {lds_wbase(dst + tix(li, 4 * lq)), lds_wbase(dst + tix(li, 16 + 4 * lq))};
  f32x4 cv[4];
#pragma unroll
  for (int J = 0; J < 4; ++J)
    if (col_on(J)) cv[J] = *reinterpret_cast<const f32x4*>(&G[(FAST ? kFc : kGam) + 16 * J + 4 * lq]);
#pragma unroll
  for (int I = 0, t = 0; I < 4; ++I) {
    if (!row_on(I)) {
      t += I + 1;
      continue;
    }
    const int r = 16 * I + li;
    // P carries the output scale: one factor per row here instead of one per output element
    // in the scan
    float rv, be_r;
    if constexpr (FAST) {
      rv = G[(ISQ ? kFrq : kFrk) + r] * (ISQ ? scale : 1.f);
      be_r = 1.f;
    } else {
      rv = G[kGam + r];
      be_r = ISQ ? scale : G[kBeta + r];
    }
#pragma unroll
    for (int J = 0; J <= I; ++J, ++t) {
      if (!tile_on(I, J)) continue;
      f32x4 val;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float d = FAST ? rv * cv[J][e] : be_r * __expf(rv - cv[J][e]);
        val[e] = d * acc[t][e];
        if (J == I) val[e] = (4 * lq + e <= li) ? val[e] : 0.f;
      }
      put_f16x4(sb[J & 1], 2048 * (J >> 1) + 512 * I, cvt_f16x4(val));
    }
  }
}

// OUT false: the state pass alone (o is not formed): no q transfers, no Q K^T role, and the
// scan waves skip Q h, P v_new and the output stores (the fragment state summary's use).
template <int K, bool VARLEN, bool OUT>
__global__ __launch_bounds__(kThr) void fused16_kernel(const FwdParams p) {
  typedef FusedSmem<K> SM;
  constexpr int kG = K / 32;
  __shared__ SM s;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);

  // Workgroup -> (chain, value block); the value blocks of a chain stay on one XCD.
  // Consecutive workgroup ids go round-robin to the 8 XCDs, and each XCD starts its
  // workgroups in id order.  Dense batches: XCD x takes a contiguous range of chains.  Packed
  // batches: chains start longest first (sequences ranked by length, heads of one sequence
  // consecutive) and are dealt to the XCDs in turn, so that the long chains start at once and
  // the short ones fill in behind them.
  const int nwg = gridDim.x, bid = blockIdx.x, nch = nwg / p.nvb;
  int chain, vb;
  if (VARLEN && p.order) {
    int j;
    if ((nch & 7) == 0) {
      const int sl = bid >> 3;
      j = 8 * (sl / p.nvb) + (bid & 7);
      vb = sl % p.nvb;
    } else {
      j = bid / p.nvb;
      vb = bid % p.nvb;
    }
    chain = p.order[j / p.H] * p.H + j % p.H;
  } else {
    int logical = bid;
    if ((nwg & 7) == 0) logical = (bid & 7) * (nwg >> 3) + (bid >> 3);
    chain = logical / p.nvb;
    vb = logical % p.nvb;
  }
  const int v0 = vb * kBV;
  const int h = chain % p.H, bs = chain / p.H;
  long tok0;
  int len;
  if (VARLEN) {
    tok0 = p.cu[bs];
    len = p.cu[bs + 1] - p.cu[bs];
  } else {
    tok0 = (long)bs * p.T;
    len = p.T;
  }
  const int nchunks = (len + kC - 1) / kC;
  const uint32_t qk_row = (uint32_t)p.H * K * 2, v_row = (uint32_t)p.H * p.V * 2;

  if (wave == 4 || wave == 5) {
    // =============================== transfer waves ===============================
    const int tw = wave - 4;  // 0: q, g, beta and the gate slots; 1: k and v
    // per-lane source offsets of the 1 KiB transfer blocks: block b holds rows 16 (b & 3) ..
    // +15 of sub-tile b >> 2; lane L writes physical octet L & 3 of row 16 (b & 3) + L / 4
    uint32_t off_qk[4], off_v[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int r = 16 * j + (lane >> 2), o = src_octet(r, lane);
      off_qk[j] = r * qk_row + o * 16;
      off_v[j] = r * v_row + o * 16;
    }
    const bf16* qg = static_cast<const bf16*>(p.q);
    const bf16* kg = static_cast<const bf16*>(p.k);
    const bf16* vg = static_cast<const bf16*>(p.v);
    auto rows_of = [&](int c) { return (uint32_t)min(kC, len - c * kC); };
    auto issue_qk = [&](int c) {  // q (wave 4) or k (wave 5) of chunk c into ring slot c % 3
      if (c >= nchunks || (!OUT && tw == 0)) return;
      const long tok = tok0 + (long)c * kC;
      const i32x4 r = make_rsrc((tw ? kg : qg) + (tok * p.H + h) * K, rows_of(c) * qk_row);
      u16* dst = tw ? s.qk[c % 3].k : s.qk[c % 3].q;
#pragma unroll
      for (int b = 0; b < 4 * kG; ++b) dma16(r, off_qk[b & 3] + (b >> 2) * 64, 0, lds_addr(dst) + 1024u * b);
    };
    auto issue_v = [&](int c) {  // v of chunk c (this workgroup's 32 columns, four blocks)
      if (c >= nchunks) return;
      const long tok = tok0 + (long)c * kC;
      const i32x4 r = make_rsrc(vg + (tok * p.H + h) * p.V + v0, rows_of(c) * v_row);
#pragma unroll
      for (int b = 0; b < 4; ++b) dma16(r, off_v[b], 0, lds_addr(s.v[c & 1]) + 1024u * b);
    };
    auto load_gb = [&](int c, float& gv, float& bv) {  // lane = token of chunk c
      const int t = c * kC + lane;
      const bool ok = c < nchunks && t < len;
      const long gi = (tok0 + t) * p.H + h;
      gv = ok && p.g ? p.g[gi] : 0.f;
      bv = ok ? p.beta[gi] : 0.f;
    };
    // gate slot of chunk c from its g, beta (rows past the end carry g = 0, beta = 0)
    auto gates = [&](int c, float gv, float bv) {
      if (c >= nchunks) return;
      float* G = s.gate[c % 3];
      // floored here, where it is used, not at the load (which is a prefetch)
      const float gam = wave_incl_scan(floor_gate(gv), lane);
      const float gl = __shfl(gam, 63, 64), gref = __shfl(gam, 31, 64), g0 = __shfl(gam, 0, 64);
      G[kEg + lane] = __expf(gam);
      G[kEl + lane] = __expf(gl - gam);
      G[kBeta + lane] = bv;
      const float up = __expf(gam - gref);
      G[kFrk + lane] = bv * up;
      G[kFrq + lane] = up;
      G[kFc + lane] = __expf(gref - gam);
      G[kGam + lane] = gam;
      if (lane == 0) {
        G[kEgl] = __expf(gl);
        G[kFast] = (g0 - gl < 80.f) ? 1.f : 0.f;
      }
    };
    // L2 prefetch of chunk c (wave 1 only: its loads are all direct-to-LDS, so no register
    // load of this wave makes the compiler wait for them): one-dword loads into a dummy LDS
    // area, one per 128-byte line.  The value blocks of a chain split the q and k lines between
    // them (lane L < 32: q, else k; rows 16 vb + (L & 15), line (L >> 4) & 1 of the row);
    // each workgroup touches its own v rows.  Rows past the chain read nothing.
    const uint32_t sink = lds_addr(s.sink);
    const int nvb = p.nvb;
    auto touch = [&](int c) {
      const long tok = tok0 + (long)c * kC;
      const uint32_t rows = (uint32_t)max(0, min(kC, len - c * kC));
      const int r = (16 * vb + (lane & 15)) % kC;  // nvb <= 4 value blocks cover rows 0..63
      const i32x4 rqk = make_rsrc((lane < 32 ? qg : kg) + (tok * p.H + h) * K, rows * qk_row);
      dma4(rqk, (uint32_t)r * qk_row + 128u * ((lane >> 4) & 1), 0, sink);
      const i32x4 rv = make_rsrc(vg + (tok * p.H + h) * p.V + v0, rows * v_row);
      dma4(rv, (uint32_t)lane * v_row, 0, sink);
      (void)nvb;
    };
    bool touched = false;  // wave 1 issued two prefetch loads after its transfers
    float g1 = 0.f, b1 = 0.f, g2 = 0.f, b2 = 0.f;
    issue_qk(0);
    if (tw == 0) {
      float g0v, b0v;
      load_gb(0, g0v, b0v);
      load_gb(1, g1, b1);
      wait_vm0();
      gates(0, g0v, b0v);
    } else {
      wait_vm0();
    }
    __syncthreads();
    for (int n = -1; n < nchunks; ++n) {
      issue_qk(n + 2);
      if (tw == 1) {
        issue_v(n + 1);
        touched = n + 2 + kPF < nchunks;
        if (touched) touch(n + 2 + kPF);
      } else {
        load_gb(n + 3, g2, b2);
        gates(n + 2, g1, b1);
      }
      // this wave's transfers have landed in LDS (loads complete in issue order; only the
      // two prefetch loads issued after them may still be pending)
      if (touched) wait_vm<2>();
      else wait_vm0();
      g1 = g2;
      b1 = b2;
      __syncthreads();
    }
    wait_vm0();
    return;
  }

  if (wave >= 2) {
    // =============================== prep waves ===============================
    // Four waves; waves 2 and 6 share a SIMD, as do 3 and 7.
    //   pq 0 (wave 2), pq 1 (wave 3): Gram tiles (b, b) and the inverses T_bb of the
    //     diagonal blocks b = 2pq, 2pq + 1; then the off-diagonal block columns of Tm
    //     (pq 0: column 0; pq 1: columns 1, 2)
    //   pq 2 (wave 6): off-diagonal Gram tiles -> A (fp16 rows)
    //   pq 3 (wave 7): Q K^T tiles -> P
    // Each role runs its own loop (the lambda is instantiated per role), so that the
    // lane-derived LDS addresses of a role stay in registers across the steps.
    auto prep_role = [&](auto pq_c) {
      constexpr int pq = decltype(pq_c)::value;
      unsigned pbt = 0;
      if (pq == 0 && lane == 0) s.pbar = 0u;
      // upper 16x16 tiles (0,1) and (2,3) of Tm and P stay zero in both slots
      for (int e = 64 * pq + lane; e < 2 * 2 * 2 * 256; e += 256) {
        const int slot = e >> 10, which = (e >> 9) & 1, t = (e >> 8) & 1, rr = (e >> 4) & 15, cc = e & 15;
        u16* tile = which ? s.tp[slot].p : s.tp[slot].tm;
        tile[tix(32 * t + rr, 32 * t + 16 + cc)] = 0;
      }
      __syncthreads();

      for (int n = -1; n < nchunks; ++n) {
        const int m = n + 1;  // chunk prepared in this step
        if (m < nchunks) {
          const int lane = __lane_id(), li = lane & 15, lq = lane >> 4;
          typename SM::TP& T = s.tp[m & 1];
          const typename SM::QK& Q = s.qk[m % 3];
          const float* G = s.gate[m % 3];
          const bf16* qt = reinterpret_cast<const bf16*>(Q.q);
          const bf16* kt = reinterpret_cast<const bf16*>(Q.k);
          f16* tmt = reinterpret_cast<f16*>(T.tm);
          f16* aft = reinterpret_cast<f16*>(s.af);
          const bool fast = __builtin_amdgcn_readfirstlane(__float_as_int(G[kFast])) != 0;
          f16x4 tc0;  // C-form (accumulator layout) of this wave's first diagonal block of Tm

          // The products below take the rows of their second factor as the A operand, so a
          // lane's accumulator of tile (I, J) holds columns s = 16J + 4lq + e of row
          // r = 16I + li ("row form", the A-operand layout of the product); the Gram tile is
          // symmetric, so the same accumulator also gives the C form r = 16I + 4lq + e,
          // s = 16I + li of a diagonal block.  decay(r, s) = e^{gamma_r - gamma_s} (times
          // beta_r unless the Q K^T tile is meant), from per-token factors or, when the chunk
          // decays too fast for them, from gamma itself.
          auto body = [&](auto fast_c) {
            constexpr bool kFastDecay = decltype(fast_c)::value;
            auto rowv = [&](int r, bool qk) -> float {
              return kFastDecay ? G[(qk ? kFrq : kFrk) + r] : G[kGam + r];
            };
            auto colv = [&](int c) -> float { return kFastDecay ? G[kFc + c] : G[kGam + c]; };
            auto rows4 = [&](int r0, bool qk) -> f32x4 {
              return *reinterpret_cast<const f32x4*>(&G[(kFastDecay ? (qk ? kFrq : kFrk) : kGam) + r0]);
            };
            auto cols4 = [&](int c0) -> f32x4 {
              return *reinterpret_cast<const f32x4*>(&G[(kFastDecay ? kFc : kGam) + c0]);
            };
            auto dec = [&](float rv, float cv, float beta_r) -> float {
              if constexpr (kFastDecay) return rv * cv;
              else return beta_r * __expf(rv - cv);
            };

            if (pq < 2) {
              // ---- diagonal blocks b = 2pq, 2pq + 1: Gram tile, then (I + L)^-1 as
              // (I - L)(I + L^2)(I + L^4)(I + L^8) (L strictly lower, L^16 = 0) on fp16 operands
              bf16x8 kf[2][kG];
#pragma unroll
              for (int kk = 0; kk < kG; ++kk)
#pragma unroll
                for (int u = 0; u < 2; ++u) kf[u][kk] = lds8(kt + tix(16 * (2 * pq + u) + li, 32 * kk + 8 * lq));
              __builtin_amdgcn_sched_barrier(0);
              f32x4 g[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
#pragma unroll
              for (int kk = 0; kk < kG; ++kk)
#pragma unroll
                for (int u = 0; u < 2; ++u) g[u] = mma16(kf[u][kk], kf[u][kk], g[u]);
              f16x4 la[2], lc[2];
              f32x4 x0a[2], x0c[2];
#pragma unroll
              for (int u = 0; u < 2; ++u) {
                const int b0 = 16 * (2 * pq + u);
                const float r_li = rowv(b0 + li, false), c_li = colv(b0 + li);
                const float be_li = kFastDecay ? 1.f : G[kBeta + b0 + li];
                const f32x4 r_q = rows4(b0 + 4 * lq, false), c_q = cols4(b0 + 4 * lq);
                f32x4 be_q = {1.f, 1.f, 1.f, 1.f};
                if constexpr (!kFastDecay) be_q = *reinterpret_cast<const f32x4*>(&G[kBeta + b0 + 4 * lq]);
                f32x4 va, vc;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                  const int c = 4 * lq + e;
                  va[e] = (c < li) ? dec(r_li, c_q[e], be_li) * g[u][e] : 0.f;   // L[li][c]
                  vc[e] = (li < c) ? dec(r_q[e], c_li, be_q[e]) * g[u][e] : 0.f;  // L[c][li]
                  x0a[u][e] = (c == li ? 1.f : 0.f) - va[e];
                  x0c[u][e] = (c == li ? 1.f : 0.f) - vc[e];
                }
                la[u] = cvt_f16x4(va);
                lc[u] = cvt_f16x4(vc);
              }
              f16x4 p2a[2], p2c[2], p4a[2], p4c[2], p8c[2];
#pragma unroll
              for (int u = 0; u < 2; ++u) {
                p2c[u] = cvt_f16x4(mma16x16x16(la[u], lc[u], f32x4{0.f, 0.f, 0.f, 0.f}));
                p2a[u] = cvt_f16x4(mma16x16x16(lc[u], la[u], f32x4{0.f, 0.f, 0.f, 0.f}));
              }
#pragma unroll
              for (int u = 0; u < 2; ++u) {
                p4c[u] = cvt_f16x4(mma16x16x16(p2a[u], p2c[u], f32x4{0.f, 0.f, 0.f, 0.f}));
                p4a[u] = cvt_f16x4(mma16x16x16(p2c[u], p2a[u], f32x4{0.f, 0.f, 0.f, 0.f}));
              }
#pragma unroll
              for (int u = 0; u < 2; ++u) p8c[u] = cvt_f16x4(mma16x16x16(p4a[u], p4c[u], f32x4{0.f, 0.f, 0.f, 0.f}));
              // X_{k+1} = X_k + X_k L^(2^k) in both forms (the row form of X is the C form of X^T).
              // The scan forms v_new = (Tm diag(beta)) (V - diag(e^gamma) K h), so the Tm it reads
              // carries beta on its columns; the unscaled T_bb, the left factor of the block-column
              // chains below, goes into the diagonal block of the A tile, which A leaves unused.
              f32x4 xa[2], xc[2];
#pragma unroll
              for (int u = 0; u < 2; ++u) {
                const f16x4 x0a16 = cvt_f16x4(x0a[u]);
                xc[u] = mma16x16x16(x0a16, p2c[u], x0c[u]);
                xa[u] = mma16x16x16(p2c[u], x0a16, x0a[u]);
              }
#pragma unroll
              for (int u = 0; u < 2; ++u) {
                const f16x4 x1a16 = cvt_f16x4(xa[u]);
                xc[u] = mma16x16x16(x1a16, p4c[u], xc[u]);
                xa[u] = mma16x16x16(p4c[u], x1a16, xa[u]);
              }
#pragma unroll
              for (int u = 0; u < 2; ++u) {
                const f16x4 x2a16 = cvt_f16x4(xa[u]);
                xc[u] = mma16x16x16(x2a16, p8c[u], xc[u]);
                xa[u] = mma16x16x16(p8c[u], x2a16, xa[u]);
                const int b0 = 16 * (2 * pq + u);
                const f32x4 bc = *reinterpret_cast<const f32x4*>(&G[kBeta + b0 + 4 * lq]);
                *reinterpret_cast<f16x4*>(&aft[tix(b0 + li, b0 + 4 * lq)]) = cvt_f16x4(xa[u]);
                *reinterpret_cast<f16x4*>(&tmt[tix(b0 + li, b0 + 4 * lq)]) = cvt_f16x4(xa[u] * bc);
              }
              tc0 = cvt_f16x4(xc[0] * G[kBeta + 32 * pq + li]);
              // the C form of the scaled T_11 for the other solve wave's block-column chain,
              // parked in the (unused) upper tile (0, 1) of the A tile
              if (pq == 0) *reinterpret_cast<f16x4*>(&aft[tix(li, 16 + 4 * lq)]) = cvt_f16x4(xc[1] * G[kBeta + 16 + li]);
            } else if (pq == 2) {
              // ---- off-diagonal Gram tiles -> A rows (fp16)
              prod_tiles<K, false, 0x1dau, kFastDecay>(qt, kt, G, s.af, p.scale);
            } else if constexpr (OUT) {
              // ---- Q K^T tiles -> P rows (fp16)
              prod_tiles<K, true, 0x3ffu, kFastDecay>(qt, kt, G, T.p, p.scale);
            }
          };
          if (fast) body(std::true_type{});
          else body(std::false_type{});

          if (pq < 3) solve_bar(&s.pbar, pbt);  // A rows (pq 2) and T_bb (pq 0, 1) are in LDS
          // Off-diagonal 16x16 blocks, one block column per chain of products (fp16 operands,
          // fp32 accumulation):  T_ij = -T_ii sum_{j<=k<i} A_ik T_kj, with A_ik and T_ii as
          // row-form A operands from LDS and T_kj in C form (the B-operand layout) in registers.
          // Scaling column block j by beta commutes with the chain, so seeding it with the
          // scaled T_jj yields the scaled T_ij.
          // pq 0 takes column 0, pq 1 columns 1 and 2.
          if (pq < 2) {
            auto chain = [&](int j, f16x4 tjj) {
              f16x4 bt[4];
              bt[j] = tjj;
#pragma unroll
              for (int i = 1; i < 4; ++i) {
                if (i <= j) continue;
                f32x4 sacc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int k = 0; k < i; ++k)
                  if (k >= j)
                    sacc = mma16x16x16(*reinterpret_cast<const f16x4*>(&aft[tix(16 * i + li, 16 * k + 4 * lq)]), bt[k], sacc);
                const f16x4 tii = *reinterpret_cast<const f16x4*>(&aft[tix(16 * i + li, 16 * i + 4 * lq)]);
                const f16x4 s16 = cvt_f16x4(sacc);
                const f32x4 t = mma16x16x16(tii, s16, f32x4{0.f, 0.f, 0.f, 0.f});
                bt[i] = cvt_f16x4(-t);
                // the row form of T_ij for the store: (T_ii S)^T = S^T T_ii^T
                const f32x4 tr = mma16x16x16(s16, tii, f32x4{0.f, 0.f, 0.f, 0.f});
                *reinterpret_cast<f16x4*>(&tmt[tix(16 * i + li, 16 * j + 4 * lq)]) = cvt_f16x4(-tr);
              }
            };
            if (pq == 0) {
              chain(0, tc0);
            } else {
              // T_11 in C form, parked by the other solve wave
              const f16x4 t11 = *reinterpret_cast<const f16x4*>(&aft[tix(li, 16 + 4 * lq)]);
              chain(1, t11);
              chain(2, tc0);
            }
          }
        }
        __syncthreads();
      }
    };
    if (wave == 2) prep_role(std::integral_constant<int, 0>{});
    else if (wave == 3) prep_role(std::integral_constant<int, 1>{});
    else if (wave == 6) prep_role(std::integral_constant<int, 2>{});
    else prep_role(std::integral_constant<int, 3>{});
    return;
  }

  // =============================== scan waves ===============================
  // hs[G][t] holds keys 32G + 8lq + 4t + e (e = 0..3) of value column v0 + 16 wave + li.
  f32x4 hs[kG][2];
  const int li = lane & 15, lq = lane >> 4;
#pragma unroll
  for (int G = 0; G < kG; ++G)
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int e = 0; e < 4; ++e)
        hs[G][t][e] = p.h0 ? p.h0[((long)chain * K + 32 * G + 8 * lq + 4 * t + e) * p.V + v0 + 16 * wave + li] : 0.f;
  bf16* og = static_cast<bf16*>(p.o);
  // K and Q rows of a chunk (pair-row order).  The first contraction half of K is read during
  // the step before the one that uses it (a chunk's q / k tiles are in LDS from the end of
  // the step two before its own); the rest is read under the K h products.
  bf16x8 kfr[2][2][kG], qfr[2][2][kG];
  // Tile reads go through a few per-lane element offsets taken once per step: the swizzle
  // does not see row bit 5 or the column sub-tile, so rows 32P and sub-tiles 32G add the
  // constants 1024 P and 2048 G (instruction immediates).  ob[t]: the pair rows
  // pair_row(0, t, li) at octet lq; ot[h]: rows 8lq + 4h + trj at octet trc (transposed reads).
  auto read_k = [&](int c, const int* ob, int g0, int g1) {
    lds_u16* kb[2] = {lds_base(s.qk[c % 3].k + ob[0]), lds_base(s.qk[c % 3].k + ob[1])};
#pragma unroll
    for (int G = 0; G < kG; ++G)
#pragma unroll
      for (int P = 0; P < 2; ++P)
#pragma unroll
        for (int t = 0; t < 2; ++t)
          if (G >= g0 && G < g1) kfr[P][t][G] = lds_at<bf16x8>(kb[t], 1024 * P + 2048 * G);
  };
  auto read_q = [&](int c, const int* ob) {
    lds_u16* qb[2] = {lds_base(s.qk[c % 3].q + ob[0]), lds_base(s.qk[c % 3].q + ob[1])};
#pragma unroll
    for (int Gk = 0; Gk < kG; ++Gk)
#pragma unroll
      for (int G = 0; G < 2; ++G)
#pragma unroll
        for (int t = 0; t < 2; ++t) qfr[G][t][Gk] = lds_at<bf16x8>(qb[t], 1024 * G + 2048 * Gk);
  };
  __syncthreads();
  // Step -1 (the other roles' first step): the first half of chunk 0's K rows.  It is peeled
  // off the loop so that the loop body has one path: a loop whose body merges two paths makes
  // the compiler copy every loop-carried register (state and prefetched K rows) at the end of
  // each step.
  {
    const int lane = __lane_id(), li = lane & 15, lq = lane >> 4;
    const int ob[2] = {tix(pair_row(0, 0, li), 8 * lq), tix(pair_row(0, 1, li), 8 * lq)};
    read_k(0, ob, 0, kG / 2);  // chunk 0's slot (stale and unused when there are no chunks)
  }
  __syncthreads();

  for (int n = 0; n < nchunks; ++n) {
    const int lane = __lane_id(), li = lane & 15, lq = lane >> 4;
    const int trj = (lane >> 2) & 3, trc = lane & 3;
    const int ob[2] = {tix(pair_row(0, 0, li), 8 * lq), tix(pair_row(0, 1, li), 8 * lq)};
    const int ot[2] = {tix(8 * lq + trj, 8 * trc), tix(8 * lq + 4 + trj, 8 * trc)};
    {
      const typename SM::QK& Q = s.qk[n % 3];
      const u16* vt = s.v[n & 1];
      const typename SM::TP& T = s.tp[n & 1];
      const float* vec = s.gate[n % 3];
      const long tok = tok0 + (long)n * kC;
      const uint32_t rows = (uint32_t)min(kC, len - n * kC);

      // The step is software-pipelined in stages: each stage issues the LDS reads of a later
      // stage (or of the next chunk) before its own products, and scheduling barriers keep
      // the compiler from sinking those reads next to their uses, so LDS latency overlaps
      // matrix work.  Dependent chain: K h -> Y -> Tm Y -> update (-> next chunk); Q h and
      // P v_new are off it and fill the matrix pipe while the chain waits on vector work.

      // ---- stage 1: X_K = K h (tokens 32P + 8lq + 4t + e of this lane's column), a
      // contraction round at a time; under it, reads of the rest of K, of V, the Y gates and
      // the Q rows
      read_k(n, ob, kG / 2, kG);
      bf16x8 bh[kG];
#pragma unroll
      for (int G = 0; G < kG; ++G) bh[G] = pack8<bf16>(hs[G][0], hs[G][1]);
      __builtin_amdgcn_sched_barrier(0);
      u32x2 vv[2][2];
      lds_u16* vb[2] = {lds_base(vt + tix(8 * lq + trj, 16 * wave + 4 * trc)),
                        lds_base(vt + tix(8 * lq + 4 + trj, 16 * wave + 4 * trc))};
      // gate vectors through two per-lane bases (the ring sits beyond the 64 KB reach of an
      // instruction offset from address 0): rows 8lq + c and pair rows pair_row(0, 0, li) + c
      lds_u16* gq = lds_base(reinterpret_cast<const u16*>(vec + 8 * lq));
      lds_u16* gp = lds_base(reinterpret_cast<const u16*>(vec + pair_row(0, 0, li)));
      f32x4 eg[2][2];
      f32x4 xk[2][2];
#pragma unroll
      for (int P = 0; P < 2; ++P)
#pragma unroll
        for (int t = 0; t < 2; ++t) xk[P][t] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int G = 0; G < kG; ++G) {
#pragma unroll
        for (int P = 0; P < 2; ++P)
#pragma unroll
          for (int t = 0; t < 2; ++t) xk[P][t] = mma16(kfr[P][t][G], bh[G], xk[P][t]);
        if (G == kG / 2 - 1) {
#pragma unroll
          for (int P = 0; P < 2; ++P)
#pragma unroll
            for (int t = 0; t < 2; ++t) {
              const int r0 = 32 * P + 8 * lq + 4 * t;
              vv[P][t] = tr16_at(vb[t], 1024 * P);
              eg[P][t] = lds_at<f32x4>(gq, 2 * (kEg + r0 - 8 * lq));
            }
        }
        if (OUT && G == kG - 1) read_q(n, ob);
        __builtin_amdgcn_sched_barrier(0);
      }

      // ---- stage 2: reads of Tm rows; Y = V - diag(e^gamma) X_K (fp16 B operand; beta is on
      // the columns of the stored Tm); the Q h part
      // of o (value columns 4lq..4lq+3 of token pair_row(G, t, li), the state as the A
      // operand), which fills the matrix pipe while Y is formed
      f16x8 tmf[2][2][2];
      lds_u16* tb[2] = {lds_base(T.tm + ob[0]), lds_base(T.tm + ob[1])};
#pragma unroll
      for (int P = 0; P < 2; ++P)
#pragma unroll
        for (int G = P; G < 2; ++G)
#pragma unroll
          for (int t = 0; t < 2; ++t) tmf[G][t][P] = lds_at<f16x8>(tb[t], 1024 * G + 2048 * P);
      f32x4 oacc[2][2];
#pragma unroll
      for (int G = 0; G < 2; ++G)
#pragma unroll
        for (int t = 0; t < 2; ++t) oacc[G][t] = f32x4{0.f, 0.f, 0.f, 0.f};
      f16x8 by[2];
      // K^T (the update's A operand, transpose reads), one contraction round per Q h round:
      // the round's K^T fragments take the registers its Q rows free
      bf16x8 ktf[kG][2][2];
      lds_u16* ktb[2] = {lds_base(Q.k + ot[0]), lds_base(Q.k + ot[1])};
#pragma unroll
      for (int Gk = 0; Gk < kG; ++Gk) {
        if constexpr (OUT)
#pragma unroll
          for (int G = 0; G < 2; ++G)
#pragma unroll
            for (int t = 0; t < 2; ++t) oacc[G][t] = mma16(bh[Gk], qfr[G][t][Gk], oacc[G][t]);
#pragma unroll
        for (int P = 0; P < 2; ++P)
#pragma unroll
          for (int t = 0; t < 2; ++t)
            ktf[Gk][t][P] = __builtin_bit_cast(bf16x8, __builtin_shufflevector(tr16_at(ktb[0], 1024 * P + 2048 * Gk + 4 * t),
                                                                               tr16_at(ktb[1], 1024 * P + 2048 * Gk + 4 * t), 0, 1, 2, 3));
        if (Gk == 0) {
#pragma unroll
          for (int P = 0; P < 2; ++P)
#pragma unroll
            for (int t = 0; t < 2; ++t)
#pragma unroll
              for (int e = 0; e < 4; ++e)
                by[P][4 * t + e] = (f16)(bf_at(vv[P][t], e) - eg[P][t][e] * xk[P][t][e]);
        }
        __builtin_amdgcn_sched_barrier(0);
      }

      // ---- stage 3: reads of the update gates, P rows and the o gates; v_new = Tm Y (token
      // group P feeds groups G >= P)
      f32x4 l0[2], l1[2];
#pragma unroll
      for (int P = 0; P < 2; ++P) {
        l0[P] = lds_at<f32x4>(gq, 2 * (kEl + 32 * P));
        l1[P] = lds_at<f32x4>(gq, 2 * (kEl + 32 * P + 4));
      }
      const float egl = vec[kEgl];
      f16x8 pfr[2][2][2];
      lds_u16* pb[2] = {lds_base(T.p + ob[0]), lds_base(T.p + ob[1])};
      float ego[2][2];
      if constexpr (OUT)
#pragma unroll
        for (int G = 0; G < 2; ++G)
#pragma unroll
          for (int t = 0; t < 2; ++t) {
            const int r = pair_row(G, t, li);
#pragma unroll
            for (int P = 0; P <= G; ++P) pfr[G][t][P] = lds_at<f16x8>(pb[t], 1024 * G + 2048 * P);
            ego[G][t] = lds_at<float>(gp, 2 * (kEg + r - pair_row(0, 0, li))) * p.scale;
          }
      f32x4 vn[2][2];
#pragma unroll
      for (int G = 0; G < 2; ++G)
#pragma unroll
        for (int t = 0; t < 2; ++t) vn[G][t] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int P = 0; P < 2; ++P) {
#pragma unroll
        for (int G = P; G < 2; ++G)
#pragma unroll
          for (int t = 0; t < 2; ++t) vn[G][t] = mma16(tmf[G][t][P], by[P], vn[G][t]);
        __builtin_amdgcn_sched_barrier(0);
      }

      // ---- stage 4: bv = v_new (fp16) for P v_new; v_new e^{gl - gamma} as two bf16 parts;
      // h <- e^gl h + K^T diag(e^{gl - gamma}) v_new, a round (token half, part) at a time
      // token half 1's operands are formed while half 0's products run
      f16x8 bv[2];
      bf16x8 buh[2], bul[2];
      auto operands = [&](int P) {
        bv[P] = pack8<f16>(vn[P][0], vn[P][1]);
        const f32x4 u0 = vn[P][0] * l0[P], u1 = vn[P][1] * l1[P];
        buh[P] = pack8<bf16>(u0, u1);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          bul[P][j] = (bf16)(u0[j] - (float)buh[P][j]);
          bul[P][4 + j] = (bf16)(u1[j] - (float)buh[P][4 + j]);
        }
      };
      operands(0);
#pragma unroll
      for (int G = 0; G < kG; ++G)
#pragma unroll
        for (int t = 0; t < 2; ++t) hs[G][t] = mma16(ktf[G][t][0], buh[0], hs[G][t] * egl);
      __builtin_amdgcn_sched_barrier(0);
      operands(1);
#pragma unroll
      for (int G = 0; G < kG; ++G)
#pragma unroll
        for (int t = 0; t < 2; ++t) hs[G][t] = mma16(ktf[G][t][0], bul[0], hs[G][t]);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int part = 0; part < 2; ++part) {
#pragma unroll
        for (int G = 0; G < kG; ++G)
#pragma unroll
          for (int t = 0; t < 2; ++t) hs[G][t] = mma16(ktf[G][t][1], part ? bul[1] : buh[1], hs[G][t]);
        __builtin_amdgcn_sched_barrier(0);
      }

      // ---- stage 5: o^T = (Q h)^T diag(scale e^gamma) + (scale P v_new)^T (P carries the
      // scale), 8-byte row stores;
      // reads of the first half of the next chunk's K rows (after the last chunk they read a
      // stale ring slot and go unused: reading unconditionally keeps the registers in place
      // instead of copying the old values on the path that skips the read)
      read_k(n + 1, ob, 0, kG / 2);
      if constexpr (OUT) {
        const __amdgpu_buffer_rsrc_t ro = store_rsrc(og + (tok * p.H + h) * p.V + v0, rows * v_row);
#pragma unroll
        for (int G = 0; G < 2; ++G)
#pragma unroll
          for (int t = 0; t < 2; ++t) {
            f32x4 acc = oacc[G][t] * ego[G][t];
#pragma unroll
            for (int P = 0; P <= G; ++P) acc = mma16(bv[P], pfr[G][t][P], acc);
            __builtin_amdgcn_raw_buffer_store_b64(pack_bf16x4(acc[0], acc[1], acc[2], acc[3]), ro,
                                                  pair_row(G, t, li) * v_row + (16 * wave + 4 * lq) * 2, 0, 0);
          }
      }
    }
    __syncthreads();
  }

  if (p.ht) {
    // lane-derived offsets recomputed here rather than kept live across the loop
    const int ln = opaque_lane();
    float* ht = p.ht + (long)chain * K * p.V + v0 + 16 * wave + (ln & 15);
#pragma unroll
    for (int G = 0; G < kG; ++G)
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int e = 0; e < 4; ++e) ht[(long)(32 * G + 8 * (ln >> 4) + 4 * t + e) * p.V] = hs[G][t][e];
  }
}

// Packed batches: order[r] = the sequence of rank r by chunk count, longest first, ties by
// index (rank of i = number of longer sequences + number of equally long ones before it).
// One workgroup; up to kMaxRank sequences, beyond that the identity order.
constexpr int kMaxRank = 4096;
__global__ __launch_bounds__(1024) void rank_kernel(const int* cu, int N, int* order) {
  __shared__ int nc[kMaxRank];
  if (N > kMaxRank) {
    for (int i = threadIdx.x; i < N; i += 1024) order[i] = i;
    return;
  }
  for (int i = threadIdx.x; i < N; i += 1024) nc[i] = (cu[i + 1] - cu[i] + kC - 1) / kC;
  __syncthreads();
  for (int i = threadIdx.x; i < N; i += 1024) {
    const int ci = nc[i];
    int r = 0;
    for (int j = 0; j < N; ++j) {
      const int cj = nc[j];
      r += (cj > ci) || (cj == ci && j < i);
    }
    order[r] = i;
  }
}

template <int K, bool VL, bool OUT>
hipError_t launch_k(const FwdParams& p0, int nchains, hipStream_t stream) {
  FwdParams p = p0;
  p.nvb = p.V / kBV;
  p.order = nullptr;
  if (VL) {
    // the order table sits at the start of the workspace (unused by this path otherwise)
    int* order = static_cast<int*>(p.ws);
    hipLaunchKernelGGL(rank_kernel, dim3(1), dim3(1024), 0, stream, p.cu, p.nseq, order);
    p.order = order;
  }
  hipLaunchKernelGGL((fused16_kernel<K, VL, OUT>), dim3(nchains * p.nvb), dim3(kThr), 0, stream, p);
  return hipGetLastError();
}

}  // namespace

// o == nullptr (dense batches): the state pass alone
hipError_t launch_fused16(const FwdParams& p, int K, bool varlen, int nchains, hipStream_t stream) {
  if (!p.o && !varlen)
    return K == 128 ? launch_k<128, false, false>(p, nchains, stream) : launch_k<64, false, false>(p, nchains, stream);
  if (K == 128)
    return varlen ? launch_k<128, true, true>(p, nchains, stream) : launch_k<128, false, true>(p, nchains, stream);
  return varlen ? launch_k<64, true, true>(p, nchains, stream) : launch_k<64, false, true>(p, nchains, stream);
}

}  // namespace gdn

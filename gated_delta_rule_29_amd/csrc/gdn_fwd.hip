// gdn_fwd.hip -- chunkwise gated delta-rule forward for gfx950: a chunk-parallel prep kernel
// and a sequential state-pass kernel.
//
// For chunk n of a chain (64 tokens, h = state entering the chunk):
//   gamma_r = sum_{i<=r} g_i (chunk-local inclusive cumsum),  gl = gamma of the last row
//   A   = strict_lower( diag(beta) (K K^T o D) ),  D[r,s] = exp(gamma_r - gamma_s)
//   Tm  = (I + A)^-1                                   (unit lower triangular, fp32 solve)
//   P   = lower( Q K^T o D )
//   X_K = diag(e^gamma) K h,    X_Q = diag(e^gamma) Q h
//   v_new = Tm ( diag(beta) (V - X_K) )        ( = u - w h of the WY form )
//   o   = scale (X_Q + P v_new)
//   h  <- e^gl h + K^T diag(e^{gl - gamma}) v_new
// This is the WY/chunkwise form of the recurrence: the state-pass lines are the ones in the
// chunk_gated_delta_rule_fwd_h fragments on the hyper-parallel "Diff Coverage" page (v_new =
// u - w h, decay by the last gate, state += K^T (v_new * e^{g_last - g})); the intra-chunk
// solve and the masked output follow from unrolling the recurrence over one chunk.  w h is
// evaluated as Tm (diag(beta e^gamma) K h), so w and u are never formed.
//
// Everything that does not depend on the state (gamma, A, the solve, P) is computed by
// chunk_prep_kernel, one workgroup per chunk across the whole GPU, into a workspace slot per
// chunk (Tm and P in the operand type, e^gamma, e^{gl-gamma}, e^gl).  scan_kernel then walks
// each chain's chunks in order doing only the state-dependent products, with the next chunk's
// operands staged into the other half of a double-buffered LDS while the current one is used.
//
// Per-key gates (gk, added to g in log space) put the decay inside the key sum; the Gram /
// Q K^T operands are then scaled per key around the chunk's middle token (rows
// e^{gamma - gamma_mid}, columns e^{gamma_mid - gamma}); K h / Q h use the state rows scaled
// by e^{gamma_mid}; the state decays row by row with e^{gamma_last}; K^T in the update carries
// e^{gamma_last - gamma}.  The per-key gamma is a column cumsum done by 2 (K = 128) or 4
// (K = 64) adjacent lanes per key, combined with shuffles.
//
// State layout in scan_kernel's registers.  Wave w owns value columns 16w..16w+15 of the
// block and every key row.  Keys are grouped by 32; for group G a lane holds keys 32G+8lq+j,
// j=0..7, of its column li, split over two 16x16 accumulators (j<4 and j>=4).  The MFMA tiles
// that produce the state pick A-operand rows so that this holds (row i of tile t is key
// 32G + 8(i/4) + 4t + i%4: "pair rows"), which makes the state directly the B operand of the
// next chunk's K h / Q h products.  Token-indexed results (X_K, v_new, o) use the same mapping
// over tokens, so v_new feeds P v_new and K^T v_new directly too.
#include "gdn_chunk.h"

namespace gdn {

namespace {

using namespace chunk;

constexpr int kThreads = 256;  // 4 waves
constexpr int kBV = 64;        // value columns per fp32 scan workgroup

hipError_t launch_varlen_tables_impl(const int* cu, int N, int* offs, int* idx, hipStream_t stream);

// ======================================================================================
// chunk_prep_kernel: one workgroup per chunk.
// ======================================================================================
template <typename TI, int K, bool PK>
struct __attribute__((aligned(16))) PrepSmem {
  typedef typename OpT<TI>::type TO;
  typedef typename QKT<TI, PK>::type TQ;
  static constexpr int kKP = K + Pad<TQ>::kE;
  static constexpr int kTP = kC + Pad<TO>::kE;
  static constexpr int kAP = kC + 4;
  TQ q[kC][kKP];
  TQ k[kC][kKP];
  TQ kb[PK ? kC : 1][kKP];
  TQ kh[PK ? kC : 1][kKP];  // per-key gate: K e^{gamma_last - gamma}
  TO tm[kC][kTP];
  TO p[kC][kTP];
  float a[kC][kAP];
  float x[32][36];
  float gam[kC], beta[kC], g[kC];
};

template <typename TI, int K, bool VARLEN, bool PK>
__global__ __launch_bounds__(kThreads) void chunk_prep_kernel(const FwdParams p) {
  typedef typename OpT<TI>::type TO;
  typedef typename QKT<TI, PK>::type TQ;
  typedef typename Vec8<TQ>::type Q8;
  typedef PrepSmem<TI, K, PK> SM;
  typedef SlotF SL;
  constexpr int kG = K / 32;
  constexpr int kE = Pad<TI>::kE;
  constexpr int kCPR = K / kE;
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
  const long HK = (long)p.H * K;
  const TI* q = static_cast<const TI*>(p.q);
  const TI* k = static_cast<const TI*>(p.k);

  // strict upper 16x16 tiles of A / Tm / P stay zero
  for (int e = tid; e < 6 * 256; e += kThreads) {
    const int t = e >> 8, r = (e >> 4) & 15, c = e & 15;
    const int I = (t >= 3) + (t >= 5);
    const int J = (t < 3) ? t + 1 : (t < 5 ? t - 1 : 3);
    s.a[16 * I + r][16 * J + c] = 0.f;
    s.tm[16 * I + r][16 * J + c] = to_t<TO>(0.f);
    s.p[16 * I + r][16 * J + c] = to_t<TO>(0.f);
  }
  // q, k rows (16-byte loads, 16 lanes per row); rows past the end are zero
#pragma unroll
  for (int i = 0; i < kC * kCPR / kThreads; ++i) {
    const int c = tid + kThreads * i;
    const int row = c / kCPR, cc = c % kCPR;
    uint4 zq = make_uint4(0, 0, 0, 0), zk = zq;
    if (row < rows) {
      const long off = (cp.tok0 + t0 + row) * HK + (long)h * K + cc * kE;
      zq = *reinterpret_cast<const uint4*>(q + off);
      zk = *reinterpret_cast<const uint4*>(k + off);
    }
    if constexpr (PK) {
      const TI* eq = reinterpret_cast<const TI*>(&zq);
      const TI* ek = reinterpret_cast<const TI*>(&zk);
#pragma unroll
      for (int j = 0; j < kE; ++j) {
        s.q[row][cc * kE + j] = to_t<TQ>(to_f(eq[j]));
        s.k[row][cc * kE + j] = to_t<TQ>(to_f(ek[j]));
      }
    } else {
      *reinterpret_cast<uint4*>(&s.q[row][cc * kE]) = zq;
      *reinterpret_cast<uint4*>(&s.k[row][cc * kE]) = zk;
    }
  }
  if (tid < kC) {
    const bool ok = tid < rows;
    const long gi = (cp.tok0 + t0 + tid) * p.H + h;
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
      gkr[i] = t < rows ? p.gk[((cp.tok0 + t0 + t) * p.H + h) * (long)K + d] : 0.f;
    }
  }
  __syncthreads();

  // 16-bit inputs: the slot holds LDS images for the 16-bit scan (Slot16); fp32: SlotF
  constexpr bool k16 = sizeof(TI) == 2;
  typedef Slot16<K, PK> S16;
  constexpr size_t kSlotBytes = k16 ? S16::kBytes : SL::kBytes;
  char* slot = static_cast<char*>(p.ws) + (cp.slot0 + n) * kSlotBytes;
  float* vec = reinterpret_cast<float*>(slot + (k16 ? S16::kVec : SL::kEg));
  if constexpr (PK) {
    // per-key gamma and the scaled Gram / Q K^T operands, in place; the state-update
    // operand K e^{gamma_last - gamma}; beta, e^{gamma_mid}, e^{gamma_last} to the slot
    const int d = tid / kTPK, part = tid % kTPK;
    float gam[kGT], gm, gL;
    key_cumsum<K, kGT>(gkr, [&](int t) { return s.g[t]; }, part, gam, gm, gL);
#pragma unroll
    for (int i = 0; i < kGT; ++i) {
      const int t = part * kGT + i;
      const float up = __expf(gam[i] - gm), dn = __expf(gm - gam[i]);
      const float kk = to_f(s.k[t][d]), qq = to_f(s.q[t][d]);
      s.k[t][d] = to_t<TQ>(kk * up);
      s.q[t][d] = to_t<TQ>(qq * up);
      s.kb[t][d] = to_t<TQ>(kk * dn);
      s.kh[t][d] = to_t<TQ>(kk * __expf(gL - gam[i]));
    }
    if (part == 0) {
      vec[S16::kEmid + d] = __expf(gm);
      vec[S16::kEglk + d] = __expf(gL);
    }
    if (tid < kC) vec[S16::kBeta + tid] = s.beta[tid];
  } else if (wave == 0) {
    const float gam = wave_incl_scan(s.g[lane], lane);
    const float gl = __shfl(gam, 63, 64);
    s.gam[lane] = gam;
    if constexpr (k16) {
      vec[S16::kEg + lane] = __expf(gam);
      vec[S16::kEl + lane] = __expf(gl - gam);
      vec[S16::kBeta + lane] = s.beta[lane];
      if (lane == 0) vec[S16::kEgl] = __expf(gl);
    } else {
      vec[lane] = __expf(gam);
      vec[kC + lane] = __expf(gl - gam);
      if (lane == 0) vec[2 * kC] = __expf(gl);
    }
  }
  __syncthreads();

  // Gram (-> A) and Q K^T (-> P), lower 16x16 tiles
#pragma unroll
  for (int ji = 0; ji < 5; ++ji) {
    const int job = wave + 4 * ji;
    const bool is_qk = job >= 10;
    int I, J;
    tri_tile(is_qk ? job - 10 : job, I, J);
    const TQ* arow = is_qk ? &s.q[16 * I + li][0] : &s.k[16 * I + li][0];
    const TQ* brow = PK ? &s.kb[(16 * J + li) % (PK ? kC : 1)][0] : &s.k[16 * J + li][0];
    Q8 av[kG], bv[kG];
#pragma unroll
    for (int kk = 0; kk < kG; ++kk) {
      av[kk] = lds8(arow + 32 * kk + 8 * lq);
      bv[kk] = lds8(brow + 32 * kk + 8 * lq);
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
      if (is_qk) s.p[r][sc] = to_t<TO>(sc <= r ? dd * acc[e] : 0.f);
      else s.a[r][sc] = sc < r ? br[e] * dd * acc[e] : 0.f;
    }
  }
  __syncthreads();
  solve_unit_lower(s, wave, lane);

  // Tm, P -> slot, 16-byte pieces (16-bit: in the scan's pair-row tile layout)
  constexpr int kOE = Pad<TO>::kE;
  TO* tslot = reinterpret_cast<TO*>(slot);
  for (int c = tid; c < 2 * kC * kC / kOE; c += kThreads) {
    const int which = c / (kC * kC / kOE), cc = c % (kC * kC / kOE);
    const int r = cc / (kC / kOE), c0 = (cc % (kC / kOE)) * kOE;
    const TO* src = which ? &s.p[r][c0] : &s.tm[r][c0];
    int dst = r * kC + c0;
    if constexpr (k16) dst = tix_s32<kC>(r, c0);
    *reinterpret_cast<uint4*>(tslot + (which ? kC * kC : 0) + dst) = *reinterpret_cast<const uint4*>(src);
  }
  if constexpr (PK) {
    // scaled Q, K and the update operand, in the scan's column-split tile layout
    constexpr int kPieces = kC * K / 8;
    for (int c = tid; c < 3 * kPieces; c += kThreads) {
      const int which = c / kPieces, cc = c % kPieces;
      const int r = cc / (K / 8), c0 = (cc % (K / 8)) * 8;
      const TQ* src = which == 0 ? &s.q[r][c0] : (which == 1 ? &s.k[r][c0] : &s.kh[r][c0]);
      const size_t base = which == 0 ? S16::kQ : (which == 1 ? S16::kK : S16::kKh);
      *reinterpret_cast<uint4*>(slot + base + 2 * tix_s32<kC>(r, c0)) =
          *reinterpret_cast<const uint4*>(src);
    }
  } else if constexpr (k16) {
    // K as fp16 (exact for bf16 values in fp16's normal range), column-split layout
    for (int c = tid; c < kC * K / 8; c += kThreads) {
      const int r = c / (K / 8), c0 = (c % (K / 8)) * 8;
      typename Vec8<f16>::type h;
#pragma unroll
      for (int j = 0; j < 8; ++j) h[j] = (f16)to_f(s.k[r][c0 + j]);
      *reinterpret_cast<typename Vec8<f16>::type*>(slot + S16::kK + 2 * tix_s32<kC>(r, c0)) = h;
    }
  }
}

// ======================================================================================
// scan_kernel: one workgroup per (chain, 64-wide value block), chunks in order.
// ======================================================================================
template <typename TI, int K, bool PK>
struct __attribute__((aligned(16))) ScanBuf {
  typedef typename OpT<TI>::type TO;
  typedef typename QKT<TI, PK>::type TQ;
  TQ q[Lay<TQ, K>::kElems(kC)];   // Q rows (per-key: Q e^{gamma - gamma_mid})
  TQ k[Lay<TQ, K>::kElems(kC)];   // K rows (per-key: K e^{gamma - gamma_mid})
  TO kt[Lay<TO, kC>::kElems(K)];  // K^T (per-key: (K e^{gl - gamma})^T)
  TI vt[Lay<TI, kC>::kElems(kBV)];
  TO tm[Lay<TO, kC>::kElems(kC)];
  TO p[Lay<TO, kC>::kElems(kC)];
  float eg[kC], el[kC], beta[kC], g[kC];
  float egl;
  float emid[PK ? K : 1], eglk[PK ? K : 1];
};

template <typename TI, int K, bool PK>
struct __attribute__((aligned(16))) ScanSmem {
  static constexpr bool kDB = sizeof(TI) == 2;  // double-buffered (16-bit operands)
  ScanBuf<TI, K, PK> buf[kDB ? 2 : 1];
  TI stg[4][kC * 16];  // per-wave output staging
};

// register staging of one chunk for scan_kernel
template <typename TI, int K, bool PK>
struct ScanStage {
  typedef typename OpT<TI>::type TO;
  static constexpr int kE = Pad<TI>::kE;
  static constexpr int kCPR = K / kE;
  static constexpr int kNQ = kC * kCPR / kThreads;
  static constexpr int kNV = (kBV / kE) / 4;
  static constexpr int kOE = Pad<TO>::kE;
  static constexpr int kNT = kC * kC / kOE / kThreads;  // Tm / P 16-byte loads per thread
  static constexpr int kTPK = kThreads / K, kGT = kC / kTPK;
  uint4 q[kNQ], k[kNQ], v[kNV], tm[kNT], p[kNT];
  float vec;  // thread t < 64: e^gamma[t]; < 128: e^{gl-gamma}; < 192: beta; < 256: g
  float egl;
  float gk[PK ? kGT : 1];
};

template <typename TI, int K, bool PK>
__device__ __forceinline__ void scan_load(ScanStage<TI, K, PK>& st, const FwdParams& p,
                                          const ChunkPos& cp, int h, int n, int v0, int tid,
                                          int wave, int lane) {
  typedef ScanStage<TI, K, PK> St;
  typedef typename OpT<TI>::type TO;
  typedef SlotF SL;
  constexpr int kE = St::kE;
  const TI* q = static_cast<const TI*>(p.q);
  const TI* k = static_cast<const TI*>(p.k);
  const TI* v = static_cast<const TI*>(p.v);
  const long HK = (long)p.H * K, HV = (long)p.H * p.V;
  const int t0 = n * kC, rows = cp.len - t0;
#pragma unroll
  for (int i = 0; i < St::kNQ; ++i) {
    const int c = tid + kThreads * i;
    const int row = c / St::kCPR, cc = c % St::kCPR;
    st.q[i] = row < rows ? *reinterpret_cast<const uint4*>(q + (cp.tok0 + t0 + row) * HK + (long)h * K + cc * kE)
                         : make_uint4(0, 0, 0, 0);
  }
  const bool ok = lane < rows;
  const TI* krow = k + (cp.tok0 + t0 + lane) * HK + (long)h * K;
  const TI* vrow = v + (cp.tok0 + t0 + lane) * HV + (long)h * p.V + v0;
#pragma unroll
  for (int i = 0; i < St::kNQ; ++i)
    st.k[i] = ok ? *reinterpret_cast<const uint4*>(krow + (wave + 4 * i) * kE) : make_uint4(0, 0, 0, 0);
#pragma unroll
  for (int i = 0; i < St::kNV; ++i)
    st.v[i] = ok ? *reinterpret_cast<const uint4*>(vrow + (wave + 4 * i) * kE) : make_uint4(0, 0, 0, 0);
  const char* slot = static_cast<const char*>(p.ws) + (cp.slot0 + n) * SL::kBytes;
#pragma unroll
  for (int i = 0; i < St::kNT; ++i) {
    const int c = tid + kThreads * i;
    st.tm[i] = *reinterpret_cast<const uint4*>(slot + SL::kTm + c * 16);
    st.p[i] = *reinterpret_cast<const uint4*>(slot + SL::kP + c * 16);
  }
  const int t = tid & 63;
  const long gi = (cp.tok0 + t0 + t) * p.H + h;
  const float* fs = reinterpret_cast<const float*>(slot + SL::kEg);
  if (tid < 128) st.vec = PK ? 0.f : fs[tid];  // e^gamma, then e^{gl - gamma}
  else if (tid < 192) st.vec = t < rows ? p.beta[gi] : 0.f;
  else st.vec = (t < rows && p.g) ? p.g[gi] : 0.f;  // a prefetch: floored where it lands
  st.egl = PK ? 0.f : fs[2 * kC];
  if constexpr (PK) {
    const int d = tid / St::kTPK, part = tid % St::kTPK;
#pragma unroll
    for (int i = 0; i < St::kGT; ++i) {
      const int tt = part * St::kGT + i;
      st.gk[i] = tt < rows ? p.gk[((cp.tok0 + t0 + tt) * p.H + h) * (long)K + d] : 0.f;
    }
  }
}

// Registers -> LDS buffer.  Per-key gate: stores raw q / k; scan_scale_pk then rescales.
template <typename TI, int K, bool PK>
__device__ __forceinline__ void scan_store(const ScanStage<TI, K, PK>& st, ScanBuf<TI, K, PK>& b,
                                           int tid, int wave, int lane) {
  typedef ScanStage<TI, K, PK> St;
  typedef typename OpT<TI>::type TO;
  typedef typename QKT<TI, PK>::type TQ;
  typedef Lay<TQ, K> LQ;
  typedef Lay<TO, kC> LO;
  typedef Lay<TI, kC> LV;
  constexpr int kE = St::kE, kOE = St::kOE;
#pragma unroll
  for (int i = 0; i < St::kNQ; ++i) {
    const int c = tid + kThreads * i;
    const int row = c / St::kCPR, cc = c % St::kCPR;
    if constexpr (PK) {
      const TI* e = reinterpret_cast<const TI*>(&st.q[i]);
#pragma unroll
      for (int j = 0; j < kE; ++j) b.q[LQ::pair(row, cc * kE + j)] = to_t<TQ>(to_f(e[j]));
    } else {
      *reinterpret_cast<uint4*>(&b.q[LQ::pair(row, cc * kE)]) = st.q[i];
    }
  }
#pragma unroll
  for (int i = 0; i < St::kNQ; ++i) {
    const int cc = wave + 4 * i;
    const TI* e = reinterpret_cast<const TI*>(&st.k[i]);
    if constexpr (PK) {
#pragma unroll
      for (int j = 0; j < kE; ++j) b.k[LQ::pair(lane, cc * kE + j)] = to_t<TQ>(to_f(e[j]));
    } else {
      *reinterpret_cast<uint4*>(&b.k[LQ::pair(lane, cc * kE)]) = st.k[i];
#pragma unroll
      for (int j = 0; j < kE; ++j) b.kt[LO::pair(cc * kE + j, lane)] = to_t<TO>(to_f(e[j]));
    }
  }
#pragma unroll
  for (int i = 0; i < St::kNV; ++i) {
    const int cc = wave + 4 * i;
    const TI* e = reinterpret_cast<const TI*>(&st.v[i]);
#pragma unroll
    for (int j = 0; j < kE; ++j) b.vt[LV::seq(cc * kE + j, lane)] = e[j];
  }
#pragma unroll
  for (int i = 0; i < St::kNT; ++i) {
    const int c = tid + kThreads * i;
    const int r = c / (kC / kOE), c0 = (c % (kC / kOE)) * kOE;
    *reinterpret_cast<uint4*>(&b.tm[LO::pair(r, c0)]) = st.tm[i];
    *reinterpret_cast<uint4*>(&b.p[LO::pair(r, c0)]) = st.p[i];
  }
  const int t = tid & 63;
  if (tid < 64) b.eg[t] = st.vec;
  else if (tid < 128) b.el[t] = st.vec;
  else if (tid < 192) b.beta[t] = st.vec;
  else b.g[t] = floor_gate(st.vec);
  if (tid == 0) b.egl = st.egl;
}

// Per-key gate: gamma per key from b.g and the thread's gk, then K, Q rescaled in place, the
// state-update operand (K e^{gl - gamma})^T, e^{gamma_mid} and e^{gl} per key.
template <typename TI, int K, bool PK>
__device__ __forceinline__ void scan_scale_pk(const ScanStage<TI, K, PK>& st,
                                              ScanBuf<TI, K, PK>& b, int tid) {
  typedef ScanStage<TI, K, PK> St;
  typedef typename OpT<TI>::type TO;
  typedef typename QKT<TI, PK>::type TQ;
  typedef Lay<TQ, K> LQ;
  typedef Lay<TO, kC> LO;
  const int d = tid / St::kTPK, part = tid % St::kTPK;
  float gam[St::kGT], gm, gL;
  key_cumsum<K, St::kGT>(st.gk, [&](int t) { return b.g[t]; }, part, gam, gm, gL);
  const float el_mid = __expf(gL - gm);
  if (part == 0) {
    b.emid[d] = __expf(gm);
    b.eglk[d] = __expf(gL);
  }
#pragma unroll
  for (int i = 0; i < St::kGT; ++i) {
    const int t = part * St::kGT + i;
    const float up = __expf(gam[i] - gm), dn = __expf(gm - gam[i]);
    const float kk = to_f(b.k[LQ::pair(t, d)]), qq = to_f(b.q[LQ::pair(t, d)]);
    b.k[LQ::pair(t, d)] = to_t<TQ>(kk * up);
    b.q[LQ::pair(t, d)] = to_t<TQ>(qq * up);
    b.kt[LO::pair(d, t)] = to_t<TO>(kk * dn * el_mid);
  }
}

// Writes a wave's [rows x 16] staging tile (row-major, TI) to global memory with 16-byte
// stores: row r goes to dst + r * row_stride; rows r >= valid_rows are skipped.
template <typename TI>
__device__ __forceinline__ void flush_tile(const TI* stg, int rows, TI* dst, long row_stride,
                                           int lane, int valid_rows) {
  constexpr int kE = Pad<TI>::kE;
  constexpr int kCPR = 16 / kE;  // 16-byte chunks per 16-column row
  for (int c = lane; c < rows * kCPR; c += 64) {
    const int r = c / kCPR, part = c % kCPR;
    if (r < valid_rows)
      *reinterpret_cast<uint4*>(dst + r * row_stride + part * kE) =
          *reinterpret_cast<const uint4*>(stg + r * 16 + part * kE);
  }
}

template <typename TI, int K, bool VARLEN, bool PK>
__global__ __launch_bounds__(kThreads) void scan_kernel(const FwdParams p) {
  typedef typename OpT<TI>::type TO;
  typedef typename QKT<TI, PK>::type TQ;
  typedef typename Vec8<TI>::type V8;
  typedef typename Vec8<TO>::type W8;
  typedef typename Vec8<TQ>::type Q8;
  typedef ScanSmem<TI, K, PK> SM;
  typedef ScanBuf<TI, K, PK> BUF;
  typedef ScanStage<TI, K, PK> St;
  typedef Lay<TQ, K> LQ;
  typedef Lay<TO, kC> LO;
  typedef Lay<TI, kC> LV;
  constexpr int kG = K / 32;  // key groups of 32
  constexpr bool kDB = SM::kDB;
  __shared__ SM s;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int li = lane & 15, lq = lane >> 4;

  // Workgroup -> (chain, value block).  Consecutive workgroup ids are dealt round-robin to
  // the 8 XCDs; remap so that the value blocks of one chain sit on one XCD and share its L2.
  const int nwg = gridDim.x;
  int logical = blockIdx.x;
  if ((nwg & 7) == 0) logical = (blockIdx.x & 7) * (nwg >> 3) + (blockIdx.x >> 3);
  const int chain = logical / p.nvb;
  const int v0 = (logical % p.nvb) * kBV;
  const int h = chain % p.H;
  const ChunkPos cp = chain_pos(p, chain, VARLEN);
  const int nchunks = (cp.len + kC - 1) / kC;
  const int col = v0 + 16 * wave + li;  // this lane's value column
  const long HV = (long)p.H * p.V;

  // State: hs[G][t] holds keys 32G + 8lq + 4t + e (e = 0..3) of column col.
  f32x4 hs[kG][2];
#pragma unroll
  for (int G = 0; G < kG; ++G)
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int e = 0; e < 4; ++e)
        hs[G][t][e] = p.h0 ? p.h0[((long)chain * K + 32 * G + 8 * lq + 4 * t + e) * p.V + col] : 0.f;

  TI* o = static_cast<TI*>(p.o);
  TI* vnew_out = static_cast<TI*>(p.v_new);
  TI* hch = static_cast<TI*>(p.h_chunks);
  TI* stg = s.stg[wave];

  // Pipeline (16-bit operands, double-buffered LDS): chunk n+1's global loads are issued at
  // the top of iteration n and written to the other LDS buffer halfway through it, before
  // this chunk's output stores.  Global loads and stores share one completion counter on this
  // architecture, so consuming the loads before issuing the stores keeps the wait for them
  // from also waiting on the previous chunk's output writes.
  St st;
  scan_load<TI, K, PK>(st, p, cp, h, 0, v0, tid, wave, lane);
  if constexpr (kDB) {
    scan_store<TI, K, PK>(st, s.buf[0], tid, wave, lane);
    __syncthreads();
    if constexpr (PK) {
      scan_scale_pk<TI, K, PK>(st, s.buf[0], tid);
      __syncthreads();
    }
  }

  for (int n = 0; n < nchunks; ++n) {
    const int t0 = n * kC;
    BUF& b = s.buf[kDB ? (n & 1) : 0];
    if constexpr (kDB) {
      if (n + 1 < nchunks) scan_load<TI, K, PK>(st, p, cp, h, n + 1, v0, tid, wave, lane);
    } else {
      scan_store<TI, K, PK>(st, b, tid, wave, lane);
      __syncthreads();
      if constexpr (PK) {
        scan_scale_pk<TI, K, PK>(st, b, tid);
        __syncthreads();
      }
      if (n + 1 < nchunks) scan_load<TI, K, PK>(st, p, cp, h, n + 1, v0, tid, wave, lane);
    }

    // B operand of the K h / Q h products (per-key gate: rows scaled by e^{gamma_mid})
    Q8 bh[kG];
#pragma unroll
    for (int G = 0; G < kG; ++G) {
      if constexpr (PK) {
        f32x4 a = hs[G][0], c = hs[G][1];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          a[e] *= b.emid[32 * G + 8 * lq + e];
          c[e] *= b.emid[32 * G + 8 * lq + 4 + e];
        }
        bh[G] = pack8<TQ>(a, c);
      } else {
        bh[G] = pack8<TQ>(hs[G][0], hs[G][1]);
      }
    }
    if (hch) {
      // state entering this chunk -> h_chunks[.., n, :, cols], 64 key rows per pass
#pragma unroll
      for (int half = 0; half < K / 64; ++half) {
#pragma unroll
        for (int G = 2 * half; G < 2 * half + 2; ++G)
#pragma unroll
          for (int t = 0; t < 2; ++t)
#pragma unroll
            for (int e = 0; e < 4; ++e)
              stg[(32 * (G - 2 * half) + 8 * lq + 4 * t + e) * 16 + li] = to_t<TI>(hs[G][t][e]);
        wave_lds_sync();
        flush_tile<TI>(stg, kC, hch + ((cp.slot0 + n) * K + 64 * half) * (long)p.V + v0 + 16 * wave,
                       p.V, lane, kC);
        wave_lds_sync();
      }
    }

    f32x4 xk[2][2], xq[2][2];
#pragma unroll
    for (int P = 0; P < 2; ++P)
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        const int r = pair_row(P, t, li);
        f32x4 ak = {0.f, 0.f, 0.f, 0.f}, aq = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int G = 0; G < kG; ++G) {
          ak = mma16(lds8(&b.k[LQ::pair(r, 32 * G + 8 * lq)]), bh[G], ak);
          aq = mma16(lds8(&b.q[LQ::pair(r, 32 * G + 8 * lq)]), bh[G], aq);
        }
        xk[P][t] = ak;
        xq[P][t] = aq;
      }

    // Y = diag(beta) (V - diag(e^gamma) X_K), rows 32P + 8lq + j of column col.
    W8 by[2];
#pragma unroll
    for (int P = 0; P < 2; ++P) {
      const int r0 = 32 * P + 8 * lq;
      const V8 vv = lds8(&b.vt[LV::seq(16 * wave + li, r0)]);
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const float xkj = j < 4 ? xk[P][0][j] : xk[P][1][j - 4];
        const float eg = PK ? 1.f : b.eg[r0 + j];
        by[P][j] = to_t<TO>(b.beta[r0 + j] * (to_f(vv[j]) - eg * xkj));
      }
    }

    // v_new = Tm Y (Tm lower triangular: token group P contributes to groups G >= P).
    f32x4 vn[2][2];
#pragma unroll
    for (int G = 0; G < 2; ++G)
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        const int r = pair_row(G, t, li);
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int P = 0; P <= G; ++P) acc = mma16(lds8(&b.tm[LO::pair(r, 32 * P + 8 * lq)]), by[P], acc);
        vn[G][t] = acc;
      }

    W8 bv[2], bvs[2];
#pragma unroll
    for (int P = 0; P < 2; ++P) {
      bv[P] = pack8<TO>(vn[P][0], vn[P][1]);
      const int r0 = 32 * P + 8 * lq;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const float vj = j < 4 ? vn[P][0][j] : vn[P][1][j - 4];
        bvs[P][j] = to_t<TO>(PK ? vj : vj * b.el[r0 + j]);
      }
    }

    if constexpr (kDB) {
      // stage chunk n+1 into the other buffer (last read in iteration n-1)
      if (n + 1 < nchunks) {
        BUF& nb = s.buf[(n + 1) & 1];
        scan_store<TI, K, PK>(st, nb, tid, wave, lane);
        if constexpr (PK) {
          __syncthreads();
          scan_scale_pk<TI, K, PK>(st, nb, tid);
        }
      }
    }

    // o = scale (diag(e^gamma) X_Q + P v_new) -> staging tile -> 16-byte stores
    const int rows_left = cp.len - t0;
#pragma unroll
    for (int G = 0; G < 2; ++G)
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        const int r = pair_row(G, t, li);
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int P = 0; P <= G; ++P) acc = mma16(lds8(&b.p[LO::pair(r, 32 * P + 8 * lq)]), bv[P], acc);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int tl = 32 * G + 8 * lq + 4 * t + e;
          const float eg = PK ? 1.f : b.eg[tl];
          stg[tl * 16 + li] = to_t<TI>(p.scale * (eg * xq[G][t][e] + acc[e]));
        }
      }
    wave_lds_sync();
    flush_tile<TI>(stg, kC, o + (cp.tok0 + t0) * HV + (long)h * p.V + v0 + 16 * wave, HV, lane,
                   rows_left);
    if (vnew_out) {
      wave_lds_sync();
#pragma unroll
      for (int G = 0; G < 2; ++G)
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
          for (int e = 0; e < 4; ++e) stg[(32 * G + 8 * lq + 4 * t + e) * 16 + li] = to_t<TI>(vn[G][t][e]);
      wave_lds_sync();
      flush_tile<TI>(stg, kC, vnew_out + (cp.tok0 + t0) * HV + (long)h * p.V + v0 + 16 * wave, HV,
                     lane, rows_left);
    }
    wave_lds_sync();

    // h <- e^gl h + K^T diag(e^{gl - gamma}) v_new
    const float egl = b.egl;
#pragma unroll
    for (int G = 0; G < kG; ++G)
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        const int kr = pair_row(G, t, li);
        f32x4 acc = hs[G][t] * egl;
        if constexpr (PK) {
#pragma unroll
          for (int e = 0; e < 4; ++e) acc[e] = hs[G][t][e] * b.eglk[32 * G + 8 * lq + 4 * t + e];
        }
#pragma unroll
        for (int P = 0; P < 2; ++P) acc = mma16(lds8(&b.kt[LO::pair(kr, 32 * P + 8 * lq)]), bvs[P], acc);
        hs[G][t] = acc;
      }
    __syncthreads();
  }

  if (p.ht) {
#pragma unroll
    for (int G = 0; G < kG; ++G)
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int e = 0; e < 4; ++e)
          p.ht[((long)chain * K + 32 * G + 8 * lq + 4 * t + e) * p.V + col] = hs[G][t][e];
  }
}

// Varlen tables: chunk_offsets[i] = chunks before sequence i; chunk_indices = (i, c) rows.
__global__ __launch_bounds__(256) void varlen_tables_kernel(const int* cu, int N, int* offs,
                                                            int* idx) {
  __shared__ int part[257];
  const int tid = threadIdx.x;
  const int per = (N + 255) / 256;
  const int lo = min(N, tid * per), hi = min(N, lo + per);
  int sum = 0;
  for (int i = lo; i < hi; ++i) sum += (cu[i + 1] - cu[i] + kC - 1) / kC;
  part[tid + 1] = sum;
  if (tid == 0) part[0] = 0;
  __syncthreads();
  if (tid == 0)
    for (int i = 1; i <= 256; ++i) part[i] += part[i - 1];
  __syncthreads();
  int run = part[tid];
  for (int i = lo; i < hi; ++i) {
    const int nc = (cu[i + 1] - cu[i] + kC - 1) / kC;
    if (offs) offs[i] = run;
    if (idx)
      for (int c = 0; c < nc; ++c) {
        idx[2 * (run + c)] = i;
        idx[2 * (run + c) + 1] = c;
      }
    run += nc;
  }
  if (tid == 255 && offs) offs[N] = part[256];
}

hipError_t launch_varlen_tables_impl(const int* cu, int N, int* offs, int* idx, hipStream_t stream) {
  hipLaunchKernelGGL(varlen_tables_kernel, dim3(1), dim3(256), 0, stream, cu, N, offs, idx);
  return hipGetLastError();
}

template <typename TI, int K, bool VL, bool PK>
hipError_t launch_pair(const FwdParams& p, long nslots, int nchains, hipStream_t stream) {
  if constexpr (sizeof(TI) == 2) {
    const hipError_t e = launch_prep16(p, K, VL, PK, nslots, stream);
    if (e != hipSuccess) return e;
    return launch_scan16(p, K, VL, PK, nchains, stream);
  } else {
    hipLaunchKernelGGL((chunk_prep_kernel<TI, K, VL, PK>), dim3(nslots), dim3(kThreads), 0, stream, p);
    hipLaunchKernelGGL((scan_kernel<TI, K, VL, PK>), dim3(nchains * p.nvb), dim3(kThreads), 0, stream, p);
    return hipGetLastError();
  }
}

}  // namespace

size_t fwd_slot_bytes(int dtype, int K, bool pk) {
  if (dtype != 1) return chunk::SlotF::kBytes;
  if (K == 128) return pk ? chunk::Slot16<128, true>::kBytes : chunk::Slot16<128, false>::kBytes;
  return pk ? chunk::Slot16<64, true>::kBytes : chunk::Slot16<64, false>::kBytes;
}

size_t fwd_workspace_bytes(long nslots, int nseq, int dtype, int K, bool pk, bool fused) {
  // the single fused kernel keeps every per-chunk term on chip; a packed batch needs its
  // sequence rank table (nseq ints)
  if (fused) return nseq > 0 ? (((size_t)nseq * sizeof(int) + 255) & ~(size_t)255) : 0;
  size_t b = (size_t)nslots * fwd_slot_bytes(dtype, K, pk);
  if (nseq > 0) b += ((size_t)(nseq + 1) * sizeof(int) + 255) & ~(size_t)255;
  return b;
}

hipError_t launch_gdn_fwd(const FwdParams& p, int dtype, int K, bool varlen, hipStream_t stream) {
  const int nchains = varlen ? p.nseq * p.H : p.B * p.H;
  const long nslots = varlen ? (long)p.H * p.nt_total : (long)p.B * p.H * ((p.T + kC - 1) / kC);
  // bf16 with a scalar gate and nothing saved per chunk: one fused kernel, no workspace traffic
  if (dtype == 1 && !p.gk && !p.v_new && !p.h_chunks) return launch_fused16(p, K, varlen, nchains, stream);
  if (varlen) {
    hipError_t e = launch_varlen_tables_impl(p.cu, p.nseq, p.coffs, nullptr, stream);
    if (e != hipSuccess) return e;
  }
  const bool pk = p.gk != nullptr;
  if (dtype == 1) {
    if (K == 128) {
      if (pk) return varlen ? launch_pair<bf16, 128, true, true>(p, nslots, nchains, stream)
                            : launch_pair<bf16, 128, false, true>(p, nslots, nchains, stream);
      return varlen ? launch_pair<bf16, 128, true, false>(p, nslots, nchains, stream)
                    : launch_pair<bf16, 128, false, false>(p, nslots, nchains, stream);
    }
    if (pk) return varlen ? launch_pair<bf16, 64, true, true>(p, nslots, nchains, stream)
                          : launch_pair<bf16, 64, false, true>(p, nslots, nchains, stream);
    return varlen ? launch_pair<bf16, 64, true, false>(p, nslots, nchains, stream)
                  : launch_pair<bf16, 64, false, false>(p, nslots, nchains, stream);
  }
  return varlen ? launch_pair<float, 64, true, false>(p, nslots, nchains, stream)
                : launch_pair<float, 64, false, false>(p, nslots, nchains, stream);
}

hipError_t launch_varlen_tables(const int* cu, int N, int* offs, int* idx, hipStream_t stream) {
  return launch_varlen_tables_impl(cu, N, offs, idx, stream);
}

}  // namespace gdn

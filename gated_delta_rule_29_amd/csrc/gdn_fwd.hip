// gdn_fwd.hip -- fused chunkwise gated delta-rule forward for gfx950.
//
// One workgroup owns one chain (a (batch, head) pair, or a (sequence, head) pair of a packed
// batch) and one 64-wide block of the value dimension, and walks the chain's 64-token chunks
// in order.  Per chunk it does all of the method in LDS and registers:
//
//   gamma_r = sum_{i<=r} g_i (chunk-local inclusive cumsum),  gl = gamma of the last row
//   A   = strict_lower( diag(beta) (K K^T o D) ),  D[r,s] = exp(gamma_r - gamma_s)
//   Tm  = (I + A)^-1                                   (unit lower triangular, fp32)
//   P   = lower( Q K^T o D )
//   X_K = diag(e^gamma) K h,    X_Q = diag(e^gamma) Q h           (h = state entering chunk)
//   v_new = Tm ( diag(beta) (V - X_K) )        ( = u - w h of the WY form )
//   o   = scale (X_Q + P v_new)
//   h  <- e^gl h + K^T diag(e^{gl - gamma}) v_new
//
// This is the WY/chunkwise form of the recurrence: the state-pass lines are the ones in the
// chunk_gated_delta_rule_fwd_h fragments on the hyper-parallel "Diff Coverage" page (v_new =
// u - w h, decay by the last gate, state += K^T (v_new * e^{g_last - g})); the intra-chunk
// solve and the masked output follow from unrolling the recurrence over one chunk.  Here w h
// is evaluated as Tm (diag(beta e^gamma) K h), so w is never formed.
//
// Layout of the state in registers.  Wave w owns value columns 16w..16w+15 of the block and
// every key row.  Keys are grouped by 32; for group G a lane holds keys 32G+8lq+j, j=0..7, of
// its column li, split over two 16x16 accumulators (j<4 and j>=4).  The MFMA tiles that
// produce the state pick A-operand rows so that this holds (row i of tile t is key
// 32G + 8(i/4) + 4t + i%4), which makes the state directly usable as the B operand of the
// next chunk's K h / Q h products with no data movement.  Token-indexed results (X_K, v_new,
// o) use the same mapping over tokens, so v_new feeds P v_new and K^T v_new directly too.
#include <type_traits>

#include "gdn_device.h"
#include "gdn_internal.h"

namespace gdn {

namespace {

constexpr int kThreads = 256;  // 4 waves
constexpr int kBV = 64;        // value columns per workgroup
constexpr int kC = 64;         // chunk length

template <typename TI>
struct Pad {
  static constexpr int kE = 16 / sizeof(TI);  // elements per 16 bytes
};

// Operand type of the intra-chunk products (Tm Y, P v_new, K^T v_new).  For bf16 inputs these
// use fp16 operands: the factors are bounded (unit-norm keys give |P|, |A| <= 1, and Y, v_new
// stay O(|v|)), and fp16's 11 significant bits keep the stored bf16 output within tolerance
// where 8-bit operands would not.  The fp32 path stays fp32 throughout.
template <typename TI>
struct OpT;
template <>
struct OpT<bf16> {
  typedef f16 type;
};
template <>
struct OpT<float> {
  typedef float type;
};

// Row of the 16-row A-operand tile t (0/1) of 32-group G that lane row li supplies.
__device__ __forceinline__ int pair_row(int G, int t, int li) {
  return 32 * G + 8 * (li >> 2) + 4 * t + (li & 3);
}

// Type of the q / k tiles: the inputs as given for a scalar gate; for a per-key gate they
// hold the decay-scaled operands, so they take the intra-chunk operand type.
template <typename TI, bool PK>
struct QKT {
  typedef typename std::conditional<PK, typename OpT<TI>::type, TI>::type type;
};

template <typename TI, int K, bool PK>
struct __attribute__((aligned(16))) Smem {
  typedef typename OpT<TI>::type TO;
  typedef typename QKT<TI, PK>::type TQ;
  static constexpr int kE = Pad<TI>::kE;
  static constexpr int kKP = K + kE;    // row stride of [token][key] tiles
  static constexpr int kTP = kC + kE;   // row stride of [.][token] tiles
  static constexpr int kAP = kC + 4;    // row stride of the fp32 solve buffer
  TQ q[kC][kKP];    // Q, or per-key gate: Q * e^{gamma - gamma_mid}
  TQ k[kC][kKP];    // K, or per-key gate: K * e^{gamma - gamma_mid}
  TQ kb[PK ? kC : 1][kKP];  // per-key gate: K * e^{gamma_mid - gamma}
  TO kt[K][kTP];    // K^T, or per-key gate: (K * e^{gamma_last - gamma})^T
  TI vt[kBV][kTP];
  TO tm[kC][kTP];   // (I + A)^-1 as MFMA operand (bf16 path)
  TO p[kC][kTP];    // masked decayed Q K^T
  float a[kC][kAP]; // fp32: A, then overwritten in place by (I + A)^-1
  float x[32][36];  // fp32 scratch of the solve's last merge
  float gam[kC], eg[kC], el[kC], beta[kC];
  float egl;
  // per-key gate: e^{gamma_mid}, e^{gamma_last} per key, and the cumsum exchange
  float emid[PK ? K : 1], eglk[PK ? K : 1], gpart[PK ? kThreads / K : 1][PK ? K : 1];
  float gmid[PK ? K : 1], glast[PK ? K : 1];
};

// Global -> register staging of one chunk, 16 bytes per load.
template <typename TI, int K, bool PK>
struct Stage {
  static constexpr int kE = Pad<TI>::kE;
  static constexpr int kCPR = K / kE;                  // 16-byte chunks per q/k row
  static constexpr int kNQ = kC * kCPR / kThreads;     // per thread, per tensor
  static constexpr int kVPR = kBV / kE;                // 16-byte chunks per v row block
  static constexpr int kNV = kC * kVPR / kThreads;
  // per-key gate: thread tid owns key tid % K and kGT consecutive tokens
  static constexpr int kTPK = kThreads / K;
  static constexpr int kGT = kC / kTPK;
  uint4 q[kNQ], k[kNQ], v[kNV];
  float g, beta;
  float gk[PK ? kGT : 1];
};

template <typename TI, int K, bool PK>
__device__ __forceinline__ void load_chunk(Stage<TI, K, PK>& st, const FwdParams& p, long tok0,
                                           int h, int t0, int len, int v0, int tid) {
  typedef Stage<TI, K, PK> St;
  constexpr int kE = Pad<TI>::kE;
  const TI* q = static_cast<const TI*>(p.q);
  const TI* k = static_cast<const TI*>(p.k);
  const TI* v = static_cast<const TI*>(p.v);
#pragma unroll
  for (int i = 0; i < St::kNQ; ++i) {
    const int c = tid + kThreads * i;
    const int row = c / St::kCPR, cc = c % St::kCPR;
    const int t = t0 + row;
    uint4 zq = make_uint4(0, 0, 0, 0), zk = zq;
    if (t < len) {
      const long off = ((tok0 + t) * p.H + h) * (long)K + cc * kE;
      zq = *reinterpret_cast<const uint4*>(q + off);
      zk = *reinterpret_cast<const uint4*>(k + off);
    }
    st.q[i] = zq;
    st.k[i] = zk;
  }
#pragma unroll
  for (int i = 0; i < St::kNV; ++i) {
    const int c = tid + kThreads * i;
    const int row = c / St::kVPR, cc = c % St::kVPR;
    const int t = t0 + row;
    uint4 z = make_uint4(0, 0, 0, 0);
    if (t < len) z = *reinterpret_cast<const uint4*>(v + ((tok0 + t) * p.H + h) * (long)p.V + v0 + cc * kE);
    st.v[i] = z;
  }
  st.g = 0.f;
  st.beta = 0.f;
  if (tid < kC) {
    const int t = t0 + tid;
    if (t < len) {
      const long gi = (tok0 + t) * p.H + h;
      st.g = p.g ? p.g[gi] : 0.f;
      st.beta = p.beta[gi];
    }
  }
  if constexpr (PK) {
    const int d = tid % K, t1 = (tid / K) * St::kGT;
#pragma unroll
    for (int i = 0; i < St::kGT; ++i) {
      const int t = t0 + t1 + i;
      st.gk[i] = t < len ? p.gk[((tok0 + t) * p.H + h) * (long)K + d] : 0.f;
    }
  }
}

template <typename TI, int K, bool PK>
__device__ __forceinline__ void store_chunk(const Stage<TI, K, PK>& st, Smem<TI, K, PK>& s, int tid) {
  typedef typename OpT<TI>::type TO;
  typedef Stage<TI, K, PK> St;
  constexpr int kE = Pad<TI>::kE;
#pragma unroll
  for (int i = 0; i < St::kNQ; ++i) {
    const int c = tid + kThreads * i;
    const int row = c / St::kCPR, cc = c % St::kCPR;
    if constexpr (PK) {
      // raw q / k converted to the operand type; the scaling pass rescales them in place
      const TI* eq = reinterpret_cast<const TI*>(&st.q[i]);
      const TI* ek = reinterpret_cast<const TI*>(&st.k[i]);
#pragma unroll
      for (int j = 0; j < kE; ++j) {
        s.q[row][cc * kE + j] = to_t<TO>(to_f(eq[j]));
        s.k[row][cc * kE + j] = to_t<TO>(to_f(ek[j]));
      }
    } else {
      *reinterpret_cast<uint4*>(&s.q[row][cc * kE]) = st.q[i];
      *reinterpret_cast<uint4*>(&s.k[row][cc * kE]) = st.k[i];
      const TI* e = reinterpret_cast<const TI*>(&st.k[i]);
#pragma unroll
      for (int j = 0; j < kE; ++j) s.kt[cc * kE + j][row] = to_t<TO>(to_f(e[j]));
    }
  }
#pragma unroll
  for (int i = 0; i < St::kNV; ++i) {
    const int c = tid + kThreads * i;
    const int row = c / St::kVPR, cc = c % St::kVPR;
    const TI* e = reinterpret_cast<const TI*>(&st.v[i]);
#pragma unroll
    for (int j = 0; j < kE; ++j) s.vt[cc * kE + j][row] = e[j];
  }
  if (tid < kC) {
    s.gam[tid] = st.g;
    s.beta[tid] = st.beta;
  }
}

// Lower-triangular 16x16 tile enumeration: (0,0),(1,0),(1,1),(2,0),(2,1),(2,2),(3,0),...
__device__ __forceinline__ void tri_tile(int idx, int& I, int& J) {
  I = (idx >= 1) + (idx >= 3) + (idx >= 6);
  J = idx - I * (I + 1) / 2;
}

// (I + A)^-1 for the strictly lower 64x64 A held in s.a, in place, fp32.  Diagonal 16x16
// blocks by forward substitution, then blocks merged with
//   T_hi,lo = -T_hi,hi A_hi,lo T_lo,lo       (first for 16-blocks, then for 32-blocks).
template <typename SM>
__device__ __forceinline__ void solve_unit_lower(SM& s, int wave, int lane) {
  const int li = lane & 15, lq = lane >> 4;
  if (wave == 0) {
    // lane -> (block b = lq, column c = li): forward substitution down column c.
    const int b0 = 16 * lq;
    float x[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      float acc = (i == li) ? 1.f : 0.f;
#pragma unroll
      for (int j = 0; j < i; ++j) acc -= s.a[b0 + i][b0 + j] * x[j];
      x[i] = acc;
    }
#pragma unroll
    for (int i = 0; i < 16; ++i) s.a[b0 + i][b0 + li] = x[i];
  }
  __syncthreads();
  if (wave < 2) {
    // wave 0: block (1,0); wave 1: block (3,2).
    const int hi = 16 * (1 + 2 * wave), lo = hi - 16;
    f32x4 m = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kk = 0; kk < 4; ++kk)
      m = mma4(s.a[hi + li][lo + 4 * kk + lq], s.a[lo + 4 * kk + lq][lo + li], m);
    f32x4 t = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) t = mma4(s.a[hi + li][hi + 4 * lq + kk], m[kk], t);
#pragma unroll
    for (int e = 0; e < 4; ++e) s.a[hi + 4 * lq + e][lo + li] = -t[e];
  }
  __syncthreads();
  {
    // X = A[32:64, 0:32] T[0:32, 0:32]; wave -> tile (ti, tj) of X.
    const int ti = wave >> 1, tj = wave & 1;
    f32x4 x = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int m = 0; m < 2; ++m) {
      if (m < tj) continue;
#pragma unroll
      for (int kk = 0; kk < 4; ++kk)
        x = mma4(s.a[32 + 16 * ti + li][16 * m + 4 * kk + lq], s.a[16 * m + 4 * kk + lq][16 * tj + li], x);
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) s.x[16 * ti + 4 * lq + e][16 * tj + li] = x[e];
  }
  __syncthreads();
  {
    // T[32:64, 0:32] = -T[32:64, 32:64] X.
    const int ti = wave >> 1, tj = wave & 1;
    f32x4 y = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int m = 0; m < 2; ++m) {
      if (m > ti) continue;
#pragma unroll
      for (int kk = 0; kk < 4; ++kk)
        y = mma4(s.a[32 + 16 * ti + li][32 + 16 * m + 4 * kk + lq], s.x[16 * m + 4 * kk + lq][16 * tj + li], y);
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) s.a[32 + 16 * ti + 4 * lq + e][16 * tj + li] = -y[e];
  }
  __syncthreads();
}

template <typename TI, int K, bool VARLEN, bool PK>
__global__ __launch_bounds__(kThreads) void gdn_fwd_kernel(const FwdParams p) {
  typedef typename OpT<TI>::type TO;
  typedef typename QKT<TI, PK>::type TQ;
  typedef typename Vec8<TI>::type V8;
  typedef typename Vec8<TO>::type W8;
  typedef typename Vec8<TQ>::type Q8;
  typedef Smem<TI, K, PK> SM;
  typedef Stage<TI, K, PK> St;
  constexpr int kG = K / 32;  // key groups of 32
  __shared__ SM s;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int li = lane & 15, lq = lane >> 4;

  // Workgroup -> (chain, value block).  Consecutive workgroup ids are dealt round-robin to
  // the 8 XCDs; remap so that the value blocks of one chain sit on one XCD and share its L2
  // for the chain's q/k/g/beta reads.
  const int nwg = gridDim.x;
  int logical = blockIdx.x;
  if ((nwg & 7) == 0) logical = (blockIdx.x & 7) * (nwg >> 3) + (blockIdx.x >> 3);
  const int chain = logical / p.nvb;
  const int v0 = (logical % p.nvb) * kBV;
  const int h = chain % p.H;
  const int bs = chain / p.H;

  long tok0;
  int len;
  long hbase;  // index of this chain's first chunk state in h_chunks
  if (VARLEN) {
    tok0 = p.cu[bs];
    len = p.cu[bs + 1] - p.cu[bs];
    long before = 0;
    for (int j = 0; j < bs; ++j) before += (p.cu[j + 1] - p.cu[j] + kC - 1) / kC;
    hbase = (long)h * p.nt_total + before;
  } else {
    tok0 = (long)bs * p.T;
    len = p.T;
    hbase = (long)chain * ((p.T + kC - 1) / kC);
  }
  const int nchunks = (len + kC - 1) / kC;
  const int col = v0 + 16 * wave + li;  // this lane's value column

  // Strict upper 16x16 tiles of A / Tm / P are never written by the chunk loop: zero once.
  for (int e = tid; e < 6 * 256; e += kThreads) {
    const int t = e >> 8, r = (e >> 4) & 15, c = e & 15;
    const int I = (t >= 3) + (t >= 5);
    const int J = (t < 3) ? t + 1 : (t < 5 ? t - 1 : 3);
    s.a[16 * I + r][16 * J + c] = 0.f;
    s.tm[16 * I + r][16 * J + c] = to_t<TO>(0.f);
    s.p[16 * I + r][16 * J + c] = to_t<TO>(0.f);
  }

  // State: h[G][t] holds keys 32G + 8lq + 4t + e (e = 0..3) of column col.
  f32x4 hs[kG][2];
#pragma unroll
  for (int G = 0; G < kG; ++G)
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int e = 0; e < 4; ++e)
        hs[G][t][e] = p.h0 ? p.h0[((long)chain * K + 32 * G + 8 * lq + 4 * t + e) * p.V + col] : 0.f;

  St st;
  load_chunk<TI, K, PK>(st, p, tok0, h, 0, len, v0, tid);

  TI* o = static_cast<TI*>(p.o);
  TI* vnew_out = static_cast<TI*>(p.v_new);
  TI* hch = static_cast<TI*>(p.h_chunks);

  for (int n = 0; n < nchunks; ++n) {
    const int t0 = n * kC;
    store_chunk<TI, K, PK>(st, s, tid);
    float gkl[PK ? St::kGT : 1];  // this chunk's per-key log decays (before the prefetch reuses st)
    if constexpr (PK) {
#pragma unroll
      for (int i = 0; i < St::kGT; ++i) gkl[i] = st.gk[i];
    }
    __syncthreads();
    if (n + 1 < nchunks) load_chunk<TI, K, PK>(st, p, tok0, h, t0 + kC, len, v0, tid);

    if constexpr (PK) {
      // ---- per-key cumulative gate gamma[t][d] = sum_{i<=t} (g_i + gk_{i,d}) and the
      // decay-scaled operands.  Thread tid owns key d = tid % K and tokens t1..t1+kGT-1.
      const int d = tid % K, part = tid / K, t1 = part * St::kGT;
      float gam[St::kGT];
      float run = 0.f;
#pragma unroll
      for (int i = 0; i < St::kGT; ++i) {
        run += s.gam[t1 + i] + gkl[i];
        gam[i] = run;
      }
      s.gpart[part][d] = run;
      __syncthreads();
      float off = 0.f;
      for (int pp = 0; pp < part; ++pp) off += s.gpart[pp][d];
#pragma unroll
      for (int i = 0; i < St::kGT; ++i) {
        gam[i] += off;
        if (t1 + i == kC / 2 - 1) s.gmid[d] = gam[i];
        if (t1 + i == kC - 1) s.glast[d] = gam[i];  // padded rows add 0: last valid row's value
      }
      __syncthreads();
      const float gm = s.gmid[d], gL = s.glast[d];
      const float el_mid = __expf(gL - gm);
      if (part == 0) {
        s.emid[d] = __expf(gm);
        s.eglk[d] = __expf(gL);
      }
#pragma unroll
      for (int i = 0; i < St::kGT; ++i) {
        const int t = t1 + i;
        const float up = __expf(gam[i] - gm), dn = __expf(gm - gam[i]);
        const float kk = to_f(s.k[t][d]), qq = to_f(s.q[t][d]);
        s.k[t][d] = to_t<TQ>(kk * up);
        s.q[t][d] = to_t<TQ>(qq * up);
        s.kb[t][d] = to_t<TQ>(kk * dn);
        s.kt[d][t] = to_t<TO>(kk * dn * el_mid);
      }
    } else if (wave == 0) {
      const float gam = wave_incl_scan(s.gam[lane], lane);
      const float gl = __shfl(gam, 63, 64);  // padded rows carry g = 0, so this is the last valid row
      s.gam[lane] = gam;
      s.eg[lane] = __expf(gam);
      s.el[lane] = __expf(gl - gam);
      if (lane == 0) s.egl = __expf(gl);
    }
    __syncthreads();

    // ---- Gram (-> A) and Q K^T (-> P), lower 16x16 tiles.  Scalar gate: the decay
    // e^{gamma_r - gamma_s} is applied in the epilogue.  Per-key gate: it is inside the
    // operands (rows e^{gamma - gamma_mid} against columns e^{gamma_mid - gamma}).
    for (int job = wave; job < 20; job += 4) {
      const bool is_qk = job >= 10;
      int I, J;
      tri_tile(job % 10, I, J);
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
      const TQ* arow = is_qk ? &s.q[16 * I + li][0] : &s.k[16 * I + li][0];
      const TQ* brow = PK ? &s.kb[(16 * J + li) % (PK ? kC : 1)][0] : &s.k[16 * J + li][0];
#pragma unroll
      for (int kk = 0; kk < kG; ++kk) acc = mma16(lds8(arow + 32 * kk + 8 * lq), lds8(brow + 32 * kk + 8 * lq), acc);
      const int sc = 16 * J + li;
      const float gs = s.gam[sc];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int r = 16 * I + 4 * lq + e;
        const float d = PK ? 1.f : __expf(s.gam[r] - gs);
        if (is_qk) s.p[r][sc] = to_t<TO>(sc <= r ? d * acc[e] : 0.f);
        else s.a[r][sc] = sc < r ? s.beta[r] * d * acc[e] : 0.f;
      }
    }
    __syncthreads();

    solve_unit_lower(s, wave, lane);
    // (bf16) operand copy of the inverse; fp32 reads it from s.a directly.
    if (sizeof(TI) == 2) {
      for (int e = tid; e < 10 * 256; e += kThreads) {
        int I, J;
        tri_tile(e >> 8, I, J);
        const int r = 16 * I + ((e >> 4) & 15), c = 16 * J + (e & 15);
        s.tm[r][c] = to_t<TO>(s.a[r][c]);
      }
      __syncthreads();
    }

    // ---- per-wave: outputs and the state update for columns 16w..16w+15
    // B operand of the K h / Q h products (per-key gate: rows scaled by e^{gamma_mid})
    Q8 bh[kG];
#pragma unroll
    for (int G = 0; G < kG; ++G) {
      if constexpr (PK) {
        f32x4 a = hs[G][0], b = hs[G][1];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          a[e] *= s.emid[32 * G + 8 * lq + e];
          b[e] *= s.emid[32 * G + 8 * lq + 4 + e];
        }
        bh[G] = pack8<TQ>(a, b);
      } else {
        bh[G] = pack8<TQ>(hs[G][0], hs[G][1]);
      }
    }
    if (hch) {
#pragma unroll
      for (int G = 0; G < kG; ++G)
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
          for (int e = 0; e < 4; ++e)
            hch[((hbase + n) * K + 32 * G + 8 * lq + 4 * t + e) * p.V + col] = to_t<TI>(hs[G][t][e]);
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
          ak = mma16(lds8(&s.k[r][32 * G + 8 * lq]), bh[G], ak);
          aq = mma16(lds8(&s.q[r][32 * G + 8 * lq]), bh[G], aq);
        }
        xk[P][t] = ak;
        xq[P][t] = aq;
      }

    // Y = diag(beta) (V - diag(e^gamma) X_K), rows 32P + 8lq + j of column col.
    W8 by[2];
#pragma unroll
    for (int P = 0; P < 2; ++P) {
      const int r0 = 32 * P + 8 * lq;
      const V8 vv = lds8(&s.vt[16 * wave + li][r0]);
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const float xkj = j < 4 ? xk[P][0][j] : xk[P][1][j - 4];
        const float eg = PK ? 1.f : s.eg[r0 + j];
        by[P][j] = to_t<TO>(s.beta[r0 + j] * (to_f(vv[j]) - eg * xkj));
      }
    }

    const TO* tmb = (sizeof(TI) == 2) ? &s.tm[0][0] : reinterpret_cast<const TO*>(&s.a[0][0]);
    const int tstride = (sizeof(TI) == 2) ? SM::kTP : SM::kAP;

    // v_new = Tm Y (Tm lower triangular: token group P contributes to groups G >= P).
    f32x4 vn[2][2];
#pragma unroll
    for (int G = 0; G < 2; ++G)
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        const int r = pair_row(G, t, li);
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int P = 0; P <= G; ++P) acc = mma16(lds8(tmb + r * tstride + 32 * P + 8 * lq), by[P], acc);
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
        bvs[P][j] = to_t<TO>(PK ? vj : vj * s.el[r0 + j]);
      }
    }

    // o = scale (diag(e^gamma) X_Q + P v_new)
#pragma unroll
    for (int G = 0; G < 2; ++G)
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        const int r = pair_row(G, t, li);
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int P = 0; P <= G; ++P) acc = mma16(lds8(&s.p[r][32 * P + 8 * lq]), bv[P], acc);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int tl = 32 * G + 8 * lq + 4 * t + e;
          if (t0 + tl < len) {
            const long oi = ((tok0 + t0 + tl) * p.H + h) * (long)p.V + col;
            const float eg = PK ? 1.f : s.eg[tl];
            o[oi] = to_t<TI>(p.scale * (eg * xq[G][t][e] + acc[e]));
            if (vnew_out) vnew_out[oi] = to_t<TI>(vn[G][t][e]);
          }
        }
      }

    // h <- e^gl h + K^T diag(e^{gl - gamma}) v_new
    const float egl = s.egl;
#pragma unroll
    for (int G = 0; G < kG; ++G)
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        const int kr = pair_row(G, t, li);
        f32x4 acc = hs[G][t] * egl;
        if constexpr (PK) {
#pragma unroll
          for (int e = 0; e < 4; ++e) acc[e] = hs[G][t][e] * s.eglk[32 * G + 8 * lq + 4 * t + e];
        }
#pragma unroll
        for (int P = 0; P < 2; ++P) acc = mma16(lds8(&s.kt[kr][32 * P + 8 * lq]), bvs[P], acc);
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

}  // namespace

hipError_t launch_gdn_fwd(const FwdParams& p, int dtype, int K, bool varlen, hipStream_t stream) {
  const int nchains = varlen ? p.nseq * p.H : p.B * p.H;
  const dim3 grid(nchains * p.nvb), block(kThreads);
#define GDN_LAUNCH(TI, KK, VL, PK) \
  hipLaunchKernelGGL((gdn_fwd_kernel<TI, KK, VL, PK>), grid, block, 0, stream, p)
  const bool pk = p.gk != nullptr;
  if (dtype == 1) {
    if (K == 128) {
      if (pk) {
        if (varlen) GDN_LAUNCH(bf16, 128, true, true); else GDN_LAUNCH(bf16, 128, false, true);
      } else {
        if (varlen) GDN_LAUNCH(bf16, 128, true, false); else GDN_LAUNCH(bf16, 128, false, false);
      }
    } else {
      if (pk) {
        if (varlen) GDN_LAUNCH(bf16, 64, true, true); else GDN_LAUNCH(bf16, 64, false, true);
      } else {
        if (varlen) GDN_LAUNCH(bf16, 64, true, false); else GDN_LAUNCH(bf16, 64, false, false);
      }
    }
  } else {
    if (varlen) GDN_LAUNCH(float, 64, true, false); else GDN_LAUNCH(float, 64, false, false);
  }
#undef GDN_LAUNCH
  return hipGetLastError();
}

hipError_t launch_varlen_tables(const int* cu, int N, int* offs, int* idx, hipStream_t stream) {
  hipLaunchKernelGGL(varlen_tables_kernel, dim3(1), dim3(256), 0, stream, cu, N, offs, idx);
  return hipGetLastError();
}

}  // namespace gdn

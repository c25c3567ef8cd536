// gdn_scan16.hip -- state pass of the chunkwise gated delta-rule forward for bf16 inputs on
// gfx950.
//
// One workgroup walks the chunks of one chain for 64 value columns (four waves of 16).  Per
// chunk n, with h the fp32 state entering it (per chunk quantities as in gdn_fwd.hip):
//   X_K = K h, X_Q = Q h                         (bf16 / fp16 matrix-core products)
//   Y   = diag(beta) (V - diag(e^gamma) X_K)      -> v_new = Tm Y
//   o   = scale (diag(e^gamma) X_Q + P v_new)
//   h  <- e^gl h + K^T diag(e^{gl-gamma}) v_new
// (per-key gate: Q, K arrive pre-scaled per key, K^T carries e^{gamma_last-gamma}, the state
// rows are scaled by e^{gamma_mid} for the two products and decay by e^{gamma_last} per key).
//
// Data movement.  Every operand tile reaches LDS by buffer loads that write LDS directly
// (no register staging): q, k, v from the inputs, Tm, P and the per-token vectors from the
// chunk's workspace slot (which the prep kernel wrote as the exact LDS image).  The next
// chunk's transfers are issued right after the top-of-loop barrier into the other half of a
// double-buffered LDS and waited for at the next barrier with an explicit vmcnt; the only
// vector-memory operations issued after them in an iteration are this chunk's output stores,
// whose number is fixed, so the wait never includes the loads' successors' latency.  Loads
// and stores use buffer resources bounded to the chain's rows: rows past the end read as zero
// and stores to them are dropped, with no branches.
//
// Operand layouts.  K, Q rows feed the A operand of K h / Q h with 16-byte reads in the
// pair-row order (gdn_tiles.h).  K^T (state update) and the V values Y needs (four tokens of
// one column per lane, the accumulator layout) are read with the LDS transpose read
// ds_read_b64_tr_b16: within each 16-lane group, result lane n gets element j from source
// lane 4j + n/4, halfword n%4 (checked in bounds on gfx950).  Outputs go accumulator -> a
// per-wave [16 columns][64 rows] staging tile (8-byte writes) -> transpose reads -> 16-byte
// row stores.
#include "gdn_chunk.h"
#include "gdn_dma.h"

namespace gdn {
namespace {

using namespace chunk;
using namespace dma;

typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

constexpr int kNW = 2;   // compute waves per workgroup
constexpr int kNCT = 1;  // 16-column tiles per compute wave (each LDS operand read feeds kNCT products)
constexpr int kTW = 2;   // transfer waves per workgroup
constexpr int kWC = 16 * kNCT;  // value columns per compute wave
constexpr int kBV = kWC * kNW;  // value columns per workgroup
constexpr int kThr = 64 * (kNW + kTW);

// Transpose read (8 bytes per lane).  The result is consumed only as a whole vector (bit
// casts of the full vector, shuffles): element-wise casts of it have been miscompiled.
__device__ __forceinline__ u32x2 tr16(const u16* p) {
  return __builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(uintptr_t)lds_addr(p)));
}

// A operand of 8 fp16 values from two transpose reads (elements 0..3, then 4..7).
__device__ __forceinline__ f16x8 tr16_pair(const u16* p0, const u16* p1) {
  const u32x4 w = __builtin_shufflevector(tr16(p0), tr16(p1), 0, 1, 2, 3);
  return __builtin_bit_cast(f16x8, w);
}

__device__ __forceinline__ float bf_lo(unsigned w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf_hi(unsigned w) { return __uint_as_float(w & 0xffff0000u); }
// element e (0..3) of four bf16 values packed in two dwords
__device__ __forceinline__ float bf_at(const u32x2& v, int e) {
  return (e & 1) ? bf_hi(v[e >> 1]) : bf_lo(v[e >> 1]);
}

// four fp32 -> four bf16 (round to nearest even), packed for one 8-byte store
__device__ __forceinline__ u32x2 pack_bf16x4(float a, float b, float c, float d) {
  // built as one vector so that the conversions pair up into packed converts
  bf16x4 v;
  v[0] = (bf16)a;
  v[1] = (bf16)b;
  v[2] = (bf16)c;
  v[3] = (bf16)d;
  return __builtin_bit_cast(u32x2, v);
}

// All operand tiles use the column-split layout tix_s32<64> (gdn_tiles.h).
__device__ __forceinline__ int tix(int r, int c) { return tix_s32<kC>(r, c); }

template <int K, bool PK>
struct __attribute__((aligned(16))) S16Buf {
  u16 q[kC * K];  // bf16 Q (per-key gate: fp16 Q e^{gamma - gamma_mid})
  u16 k[kC * K];  // fp16 K (per-key gate: K e^{gamma - gamma_mid})
  u16 kh[PK ? kC * K : 8];  // per-key gate: fp16 K e^{gamma_last - gamma}
  u16 tm[kC * kC];
  u16 p[kC * kC];
  u16 v[kC * kBV];  // bf16 V columns of this workgroup
  float vec[Slot16<K, PK>::kVecBytes / 4];
};

constexpr int kSW = kC + 8;  // staging row length (elements): padded against bank conflicts

template <int K, bool PK>
struct __attribute__((aligned(16))) S16Smem {
  S16Buf<K, PK> buf[2];
  u16 stg[kNW][16 * kSW];           // per-wave staging of v_new, [16 columns][64 rows]
  u16 stgh[kNW][K / 64][16 * kSW];  // per-wave staging of the state, one tile per 64 keys
  unsigned sink[64];                // destination of the L2 prefetch loads (never read)
  unsigned hread;                   // staged states read by the transfer waves (one per wave and chunk)
};

// L2 prefetch distance in chunks: the transfer waves touch the lines of chunk n + kPF while
// chunk n is scanned, and that chunk's own transfers are issued kPF - 1 steps later.
constexpr int kPF = 2;

// The lane index, opaque to the optimiser: addresses derived from it inside the chunk loop are
// recomputed each iteration (a few integer operations) instead of being hoisted out of the
// loop and kept in registers.
__device__ __forceinline__ int opaque_lane() {
  int l = __lane_id();
  asm volatile("" : "+v"(l));
  return l;
}

// Keeps the compiler from moving LDS accesses across this point.  Within one wave the LDS
// executes accesses in issue order, so this is all a wave's write -> read (or read -> write)
// of its own staging tile needs; unlike a fence it leaves arithmetic free to move across.
__device__ __forceinline__ void lds_order() { asm volatile("" : : : "memory"); }

// Per-wave output of a 64-row x 16-column fp32 block held in accumulator layout (rows
// 32G + 8lq + 4t + e of column li in acc[G][t][e]) as bf16 rows, in two halves that can sit
// apart in the step: stage_rows writes the block to a staging tile [16 columns][kSW] (one
// 16-byte write per lane and G: rows 32G + 8lq .. +7 of its column), flush_rows reads it back
// transposed and stores two 16-byte row pieces per lane at rsrc offset
// row * row_bytes + col0_bytes.  Within one wave the LDS performs accesses in issue order, so
// the write -> read order needs no wait; lds_order keeps the compiler from reordering them.
template <typename F>
__device__ __forceinline__ void stage_rows(u16* stg, F val, int lane) {
  const int li = lane & 15, lq = lane >> 4;
#pragma unroll
  for (int G = 0; G < 2; ++G) {
    const u32x2 w0 = pack_bf16x4(val(G, 0, 0), val(G, 0, 1), val(G, 0, 2), val(G, 0, 3));
    const u32x2 w1 = pack_bf16x4(val(G, 1, 0), val(G, 1, 1), val(G, 1, 2), val(G, 1, 3));
    *reinterpret_cast<u32x4*>(&stg[li * kSW + 32 * G + 8 * lq]) = __builtin_shufflevector(w0, w1, 0, 1, 2, 3);
  }
  lds_order();
}

__device__ __forceinline__ void flush_rows(const u16* stg, __amdgpu_buffer_rsrc_t r, uint32_t row_bytes,
                                           uint32_t col0_bytes, int lane) {
  const int li = lane & 15, lq = lane >> 4, trj = (lane >> 2) & 3, trc = lane & 3;
#pragma unroll
  for (int s = 0; s < 2; ++s) {
    const u32x4 d = __builtin_shufflevector(tr16(&stg[(8 * s + trj) * kSW + 16 * lq + 4 * trc]),
                                            tr16(&stg[(8 * s + 4 + trj) * kSW + 16 * lq + 4 * trc]),
                                            0, 1, 2, 3);
    __builtin_amdgcn_raw_buffer_store_b128(d, r, (16 * lq + li) * row_bytes + col0_bytes + 16 * s,
                                           0, 0);
  }
  lds_order();
}

// ---------------------------------------------------------------------------------------
// the kernel
// ---------------------------------------------------------------------------------------

template <int K, bool VARLEN, bool PK, bool VN>
__global__ __launch_bounds__(kThr) void scan16_kernel(const FwdParams p) {
  typedef Slot16<K, PK> SL;
  typedef typename QKT<bf16, PK>::type TQ;  // Q tile type
  typedef typename Vec8<TQ>::type Q8;
  typedef S16Buf<K, PK> BUF;
  constexpr int kG = K / 32;
  constexpr int kVecB = SL::kVecBytes / 1024;
  constexpr int kVB = kC * kBV * 2 / 1024;  // 1 KiB blocks of the v tile
  __shared__ S16Smem<K, PK> s;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int li = lane & 15, lq = lane >> 4;
  const int trj = (lane >> 2) & 3, trc = lane & 3;

  // Workgroup -> (chain, value block).  Consecutive workgroup ids go round-robin to the 8
  // XCDs; remap so the value blocks of one chain sit on one XCD and share its L2.
  const int nwg = gridDim.x;
  int logical = blockIdx.x;
  if ((nwg & 7) == 0) logical = (blockIdx.x & 7) * (nwg >> 3) + (blockIdx.x >> 3);
  const int chain = logical / p.nvb;
  const int v0 = (logical % p.nvb) * kBV;
  const int h = chain % p.H;
  const ChunkPos cp = chain_pos(p, chain, VARLEN);
  const int nchunks = (cp.len + kC - 1) / kC;
  const uint32_t qk_row = (uint32_t)p.H * K * 2, v_row = (uint32_t)p.H * p.V * 2;

  if (tid == 0) s.hread = 0u;  // ordered before every use by the first barrier
  if (wave >= kNW) {
    // ---- transfer waves: chunk n+1's tiles into the other LDS buffer while chunk n is used.
    // One wave sustains only a fraction of a CU's load bandwidth, so the 1 KiB blocks of a
    // chunk are dealt round-robin to kTW waves.
    const int tw = wave - kNW;
    const bf16* qg = static_cast<const bf16*>(p.q);
    const bf16* vg = static_cast<const bf16*>(p.v);
    const char* wsg = static_cast<const char*>(p.ws);
    // Per-lane source offsets of the input tiles.  LDS block b (1 KiB) of a column-split tile
    // holds sub-tile b / 4, rows 16 (b % 4) .. +15; lane L writes its octet L % 4 of row
    // 16 (b % 4) + L / 4, which holds the row's logical octet (L % 4) ^ swz64(row).
    uint32_t voff_q[PK ? 1 : 4 * kG], voff_v[kVB];
#pragma unroll
    for (int b = 0; b < 4 * kG; ++b) {
      const int r = 16 * (b & 3) + (lane >> 2), lo = (lane & 3) ^ swz64(r);
      if constexpr (!PK) voff_q[b] = r * qk_row + (4 * (b >> 2) + lo) * 16;
      if (b < kVB) voff_v[b] = r * v_row + (4 * (b >> 2) + lo) * 16;
    }
    const uint32_t l16 = 16u * lane;
    auto issue = [&](int n, BUF& B) {
      int slot = 0;  // running block number; this wave issues blocks slot % kTW == tw
      auto dma = [&](const i32x4& r, uint32_t voff, uint32_t soff, uint32_t lds) {
        if (slot++ % kTW == tw) dma16(r, voff, soff, lds);
      };
      const long tok = cp.tok0 + (long)n * kC;
      const uint32_t rows = (uint32_t)(cp.len - n * kC);
      const i32x4 rw = make_rsrc(wsg + (cp.slot0 + n) * (long)SL::kBytes, (uint32_t)SL::kBytes);
#pragma unroll
      for (int b = 0; b < kVecB; ++b)
        dma(rw, l16, (uint32_t)SL::kVec + 1024u * b, lds_addr(B.vec) + 1024u * b);
      if constexpr (!PK) {
        const i32x4 rq = make_rsrc(qg + (tok * p.H + h) * K, rows * qk_row);
#pragma unroll
        for (int b = 0; b < 4 * kG; ++b) dma(rq, voff_q[b], 0, lds_addr(B.q) + 1024u * b);
      } else {
#pragma unroll
        for (int b = 0; b < 4 * kG; ++b) dma(rw, l16, (uint32_t)SL::kQ + 1024u * b, lds_addr(B.q) + 1024u * b);
      }
#pragma unroll
      for (int b = 0; b < 4 * kG; ++b) dma(rw, l16, (uint32_t)SL::kK + 1024u * b, lds_addr(B.k) + 1024u * b);
#pragma unroll
      for (int b = 0; b < 8; ++b) {
        dma(rw, l16, (uint32_t)SL::kTm + 1024u * b, lds_addr(B.tm) + 1024u * b);
        dma(rw, l16, (uint32_t)SL::kP + 1024u * b, lds_addr(B.p) + 1024u * b);
      }
      const i32x4 rv = make_rsrc(vg + (tok * p.H + h) * p.V + v0, rows * v_row);
#pragma unroll
      for (int b = 0; b < kVB; ++b) dma(rv, voff_v[b], 0, lds_addr(B.v) + 1024u * b);
      if constexpr (PK) {
#pragma unroll
        for (int b = 0; b < 4 * kG; ++b) dma(rw, l16, (uint32_t)SL::kKh + 1024u * b, lds_addr(B.kh) + 1024u * b);
      }
    };
    // L2 prefetch of chunk c: one-dword loads, one per 128-byte line, into a dummy LDS area
    // (no register is written, so nothing waits for them until the next step's count).  The
    // value blocks of a chain split the slot's lines between them; each workgroup also
    // touches its own v rows.  Two loads per wave: wave 0 lines [0, 128) of its share, wave 1
    // lines [128, 192) and the v rows.  Lines past the share or rows past the chain read
    // nothing (offsets beyond the buffer resource).
    constexpr uint32_t kLines = (uint32_t)(SL::kBytes / 128);
    const uint32_t vb = (uint32_t)(logical % p.nvb);
    const uint32_t share = (kLines + p.nvb - 1) / p.nvb;
    const uint32_t sink = lds_addr(s.sink);
    auto touch = [&](int c) {
      const long tok = cp.tok0 + (long)c * kC;
      const i32x4 rw = make_rsrc(wsg + (cp.slot0 + c) * (long)SL::kBytes, (uint32_t)SL::kBytes);
      const uint32_t l0 = 128u * tw + (uint32_t)lane;
      auto line_off = [&](uint32_t l) { return l < share ? (vb * share + l) * 128u : 0xffffffffu; };
      dma4(rw, line_off(l0), 0, sink);
      // (a select, not a branch: the branch form does not compile)
      const i32x4 rv = make_rsrc(vg + (tok * p.H + h) * p.V + v0, (uint32_t)(cp.len - c * kC) * v_row);
      dma4(tw == 0 ? rw : rv, tw == 0 ? line_off(l0 + 64) : (uint32_t)lane * v_row, 0, sink);
    };
    // The state entering chunk m -> h_chunks: the compute waves stage it (one tile per wave and
    // 64 keys) during step m; transfer wave tw stores the key half tw of both compute waves'
    // tiles in step m + 1 (after the loop for the last chunk).  Once its staging reads have
    // completed it counts them in s.hread, which the compute waves wait for before they stage
    // the next chunk's state.  The global stores are issued before the chunk's transfers, so
    // the count-based wait of the next step covers them too.
    bf16* hcg = static_cast<bf16*>(p.h_chunks);
    auto flush_h = [&](int m) {
      const __amdgpu_buffer_rsrc_t rh =
          store_rsrc(hcg + (cp.slot0 + m) * (long)K * p.V + v0, (uint32_t)(K * p.V - v0) * 2u);
      // Each store writes 16 rows x 64 bytes (the block's 32 columns): within a 16-lane group,
      // lane n = 4m + r receives row R0 + r, columns 8m .. 8m+7, from two transpose reads in
      // which source lane 4j + m points at column 8m + j (+4 for the second), rows R0 .. R0+3
      // (columns 0-15 in compute wave 0's tile, 16-31 in wave 1's).
      static_assert(kNW == 2 && kWC == 16, "two 16-column staging tiles per key half");
      const int n16 = lane & 15, grp = lane >> 4;
      const int src_m = n16 & 3, src_j = n16 >> 2;
      const int res_r = n16 & 3, res_m = n16 >> 2;
#pragma unroll
      for (int half = 0; half < K / 64; ++half) {
        if (half % kTW != tw) continue;
        const u16* tile = s.stgh[src_m >> 1][half] + (8 * (src_m & 1) + src_j) * kSW + 4 * grp;
        u32x4 d[4];
#pragma unroll
        for (int i = 0; i < 4; ++i)
          d[i] = __builtin_shufflevector(tr16(tile + 16 * i), tr16(tile + 4 * kSW + 16 * i), 0, 1, 2, 3);
        asm volatile("s_waitcnt lgkmcnt(0)" : : : "memory");
        if (lane == 0) __hip_atomic_fetch_add(&s.hread, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
#pragma unroll
        for (int i = 0; i < 4; ++i)
          __builtin_amdgcn_raw_buffer_store_b128(
              d[i], rh, (uint32_t)(64 * half + 16 * i + 4 * grp + res_r) * (uint32_t)p.V * 2u + 16u * res_m, 0, 0);
      }
    };
    bool touched = false;  // two prefetch loads were issued after the last transfers
    if (nchunks > 0) issue(0, s.buf[0]);
    for (int n = 0; n < nchunks; ++n) {
      // this wave's transfers of chunk n have landed in LDS (loads complete in issue order;
      // only the two prefetch loads issued after them may still be pending)
      if (touched) wait_vm<2>();
      else wait_vm0();
      __syncthreads();  // ... and every compute wave is done with chunk n-1
      if (hcg && n > 0) flush_h(n - 1);
      if (n + 1 < nchunks) issue(n + 1, s.buf[(n + 1) & 1]);
      touched = n + kPF < nchunks;
      if (touched) touch(n + kPF);
    }
    __syncthreads();  // the compute waves have staged the last chunk's state
    if (hcg && nchunks > 0) flush_h(nchunks - 1);
    wait_vm0();
    return;
  }

  // ---- compute waves: wave w owns value columns 32w + 16c + li (tile c < kNCT) of the block
  // State: hs[c][G][t] holds keys 32G + 8lq + 4t + e (e = 0..3) of column v0 + 32w + 16c + li.
  f32x4 hs[kNCT][kG][2];
#pragma unroll
  for (int c = 0; c < kNCT; ++c)
#pragma unroll
    for (int G = 0; G < kG; ++G)
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int e = 0; e < 4; ++e)
          hs[c][G][t][e] = p.h0 ? p.h0[((long)chain * K + 32 * G + 8 * lq + 4 * t + e) * p.V + v0 +
                                       kWC * wave + 16 * c + li]
                                : 0.f;

  bf16* og = static_cast<bf16*>(p.o);
  bf16* vng = static_cast<bf16*>(p.v_new);
  bf16* hcg = static_cast<bf16*>(p.h_chunks);

  static_assert(kNCT == 1, "one 16-column tile per compute wave");
  for (int n = 0; n < nchunks; ++n) {
    __syncthreads();  // chunk n is in buffer n & 1
    const int lane = opaque_lane(), li = lane & 15, lq = lane >> 4;
    const int trj = (lane >> 2) & 3, trc = lane & 3;
    const BUF& B = s.buf[n & 1];
    const long tok = cp.tok0 + (long)n * kC;
    const uint32_t rows = (uint32_t)(cp.len - n * kC);
    const f16* kt = reinterpret_cast<const f16*>(B.k);
    const TQ* qt = reinterpret_cast<const TQ*>(B.q);
    const f16* tmt = reinterpret_cast<const f16*>(B.tm);
    const f16* pt = reinterpret_cast<const f16*>(B.p);
    const u16* kht = PK ? B.kh : B.k;
    const int col = kWC * wave;  // this wave's first value column within the block

    // The step is software-pipelined in stages: each stage issues the LDS reads of a later
    // stage before its own products, and scheduling barriers keep the compiler from sinking
    // those reads next to their uses, so LDS latency overlaps matrix and vector work.

    // ---- stage 0: K rows (A operand of K h) in flight; the state entering the chunk ->
    // h_chunks; the B operands of K h and Q h (per-key gate: rows scaled by e^{gamma_mid})
    f16x8 kfr[2][2][kG];
#pragma unroll
    for (int G = 0; G < kG; ++G)
#pragma unroll
      for (int P = 0; P < 2; ++P)
#pragma unroll
        for (int t = 0; t < 2; ++t) kfr[P][t][G] = lds8(kt + tix(pair_row(P, t, li), 32 * G + 8 * lq));
    f16x8 bk[kG];
    Q8 bq[kG];
#pragma unroll
    for (int G = 0; G < kG; ++G) {
      if constexpr (PK) {
        const f32x4 m0 = *reinterpret_cast<const f32x4*>(&B.vec[SL::kEmid + 32 * G + 8 * lq]);
        const f32x4 m1 = *reinterpret_cast<const f32x4*>(&B.vec[SL::kEmid + 32 * G + 8 * lq + 4]);
        bk[G] = pack8<f16>(hs[0][G][0] * m0, hs[0][G][1] * m1);
        bq[G] = bk[G];
      } else {
        bk[G] = pack8<f16>(hs[0][G][0], hs[0][G][1]);
        bq[G] = pack8<TQ>(hs[0][G][0], hs[0][G][1]);
      }
    }
    __builtin_amdgcn_sched_barrier(0);

    // ---- stage 1: X_K = K h (tokens 32P + 8lq + 4t + e of this lane's column), a contraction
    // round at a time; under it, reads of the Q rows, V, the Y gates and the Tm rows
    Q8 qfr[2][2][kG];
    u32x2 vv[2][2];
    f32x4 be[2][2], eg[2][2];
    f16x8 tmf[2][2][2];
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
        for (int t = 0; t < 2; ++t) xk[P][t] = mma16(kfr[P][t][G], bk[G], xk[P][t]);
      if (G == 0) {
#pragma unroll
        for (int Gk = 0; Gk < kG; ++Gk)
#pragma unroll
          for (int Gr = 0; Gr < 2; ++Gr)
#pragma unroll
            for (int t = 0; t < 2; ++t) qfr[Gr][t][Gk] = lds8(qt + tix(pair_row(Gr, t, li), 32 * Gk + 8 * lq));
      }
      if (G == kG - 1) {
#pragma unroll
        for (int P = 0; P < 2; ++P)
#pragma unroll
          for (int t = 0; t < 2; ++t) {
            const int r0 = 32 * P + 8 * lq + 4 * t;
            vv[P][t] = tr16(&B.v[tix(r0 + trj, col + 4 * trc)]);
            be[P][t] = *reinterpret_cast<const f32x4*>(&B.vec[SL::kBeta + r0]);
            eg[P][t] = PK ? f32x4{1.f, 1.f, 1.f, 1.f} : *reinterpret_cast<const f32x4*>(&B.vec[SL::kEg + r0]);
          }
#pragma unroll
        for (int P = 0; P < 2; ++P)
#pragma unroll
          for (int Gr = P; Gr < 2; ++Gr)
#pragma unroll
            for (int t = 0; t < 2; ++t) tmf[Gr][t][P] = lds8(tmt + tix(pair_row(Gr, t, li), 32 * P + 8 * lq));
      }
      __builtin_amdgcn_sched_barrier(0);
    }

    // ---- stage 2: Y = diag(beta) (V - diag(e^gamma) X_K) (fp16 B operand of Tm Y); the Q h
    // part of o (value columns 4lq..4lq+3 of token pair_row(G, t, li), the state as the A
    // operand) fills the matrix pipe meanwhile; reads of the first token half of the update
    // operand K^T (transpose reads)
    f16x8 khf[kG][2][2];
    auto read_kh = [&](int P) {
#pragma unroll
      for (int G = 0; G < kG; ++G)
#pragma unroll
        for (int t = 0; t < 2; ++t) {
          const int c0 = 32 * G + 8 * trc + 4 * t;
          khf[G][t][P] = tr16_pair(&kht[tix(32 * P + 8 * lq + trj, c0)], &kht[tix(32 * P + 8 * lq + 4 + trj, c0)]);
        }
    };
    f32x4 oacc[2][2];
#pragma unroll
    for (int G = 0; G < 2; ++G)
#pragma unroll
      for (int t = 0; t < 2; ++t) oacc[G][t] = f32x4{0.f, 0.f, 0.f, 0.f};
    f16x8 by[2];
#pragma unroll
    for (int Gk = 0; Gk < kG; ++Gk) {
#pragma unroll
      for (int G = 0; G < 2; ++G)
#pragma unroll
        for (int t = 0; t < 2; ++t) oacc[G][t] = mma16(bq[Gk], qfr[G][t][Gk], oacc[G][t]);
      if (Gk == 0) {
#pragma unroll
        for (int P = 0; P < 2; ++P)
#pragma unroll
          for (int t = 0; t < 2; ++t)
#pragma unroll
            for (int e = 0; e < 4; ++e)
              by[P][4 * t + e] = (f16)(be[P][t][e] * (bf_at(vv[P][t], e) - eg[P][t][e] * xk[P][t][e]));
      }
      if (Gk == 1) read_kh(0);
      __builtin_amdgcn_sched_barrier(0);
    }

    // ---- stage 3: reads of the second half of K^T, the P rows and the update / o gates;
    // v_new = Tm Y (Tm lower triangular: token group P feeds groups G >= P)
    read_kh(1);
    f16x8 pfr[2][2][2];
    float ego[2][2];
#pragma unroll
    for (int G = 0; G < 2; ++G)
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        const int r = pair_row(G, t, li);
#pragma unroll
        for (int P = 0; P <= G; ++P) pfr[G][t][P] = lds8(pt + tix(r, 32 * P + 8 * lq));
        ego[G][t] = PK ? 1.f : B.vec[SL::kEg + r];
      }
    f32x4 l0[2], l1[2], dec[kG][2];
#pragma unroll
    for (int P = 0; P < 2; ++P) {
      l0[P] = PK ? f32x4{1.f, 1.f, 1.f, 1.f} : *reinterpret_cast<const f32x4*>(&B.vec[SL::kEl + 32 * P + 8 * lq]);
      l1[P] = PK ? f32x4{1.f, 1.f, 1.f, 1.f} : *reinterpret_cast<const f32x4*>(&B.vec[SL::kEl + 32 * P + 8 * lq + 4]);
    }
#pragma unroll
    for (int G = 0; G < kG; ++G)
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        if constexpr (PK) {
          dec[G][t] = *reinterpret_cast<const f32x4*>(&B.vec[SL::kEglk + 32 * G + 8 * lq + 4 * t]);
        } else {
          const float egl = B.vec[SL::kEgl];
          dec[G][t] = f32x4{egl, egl, egl, egl};
        }
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

    // the state entering the chunk -> staging tiles, which the transfer waves store to
    // h_chunks in the next step; the previous chunk's tiles must have been read first
    if (hcg) {
      const unsigned target = (unsigned)(K / 64) * (unsigned)n;
      while (__hip_atomic_load(&s.hread, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP) < target)
        __builtin_amdgcn_s_sleep(1);
      lds_order();
#pragma unroll
      for (int half = 0; half < K / 64; ++half)
        stage_rows(s.stgh[wave][half], [&](int G, int t, int e) { return hs[0][2 * half + G][t][e]; }, lane);
    }

    // ---- stage 4: bv = v_new (fp16) for P v_new; bu = the update's B operand (scalar gate:
    // v_new e^{gl-gamma}); h <- decay h + K^T diag(...) v_new, a token half at a time
    f16x8 bv[2], bu[2];
#pragma unroll
    for (int P = 0; P < 2; ++P) {
      bv[P] = pack8<f16>(vn[P][0], vn[P][1]);
      if constexpr (PK) bu[P] = bv[P];
      else bu[P] = pack8<f16>(vn[P][0] * l0[P], vn[P][1] * l1[P]);
    }
#pragma unroll
    for (int G = 0; G < kG; ++G)
#pragma unroll
      for (int t = 0; t < 2; ++t) hs[0][G][t] = hs[0][G][t] * dec[G][t];
#pragma unroll
    for (int P = 0; P < 2; ++P) {
#pragma unroll
      for (int G = 0; G < kG; ++G)
#pragma unroll
        for (int t = 0; t < 2; ++t) hs[0][G][t] = mma16(khf[G][t][P], bu[P], hs[0][G][t]);
      __builtin_amdgcn_sched_barrier(0);
    }

    // ---- stage 5: o^T = scale ((Q h)^T diag(e^gamma) + (P v_new)^T), 8-byte row stores;
    // v_new -> its output rows
    const __amdgpu_buffer_rsrc_t ro = store_rsrc(og + (tok * p.H + h) * p.V + v0, rows * v_row);
#pragma unroll
    for (int G = 0; G < 2; ++G)
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        f32x4 acc = oacc[G][t] * ego[G][t];
#pragma unroll
        for (int P = 0; P <= G; ++P) acc = mma16(bv[P], pfr[G][t][P], acc);
        const f32x4 ov = acc * p.scale;
        __builtin_amdgcn_raw_buffer_store_b64(pack_bf16x4(ov[0], ov[1], ov[2], ov[3]), ro,
                                              pair_row(G, t, li) * v_row + (col + 4 * lq) * 2, 0, 0);
      }
    if constexpr (VN) {
      const __amdgpu_buffer_rsrc_t rv = store_rsrc(vng + (tok * p.H + h) * p.V + v0, rows * v_row);
      stage_rows(s.stg[wave], [&](int G, int t, int e) { return vn[G][t][e]; }, lane);
      flush_rows(s.stg[wave], rv, v_row, (uint32_t)col * 2u, lane);
    }
  }
  __syncthreads();  // the transfer waves store the last chunk's staged state after this

  if (p.ht) {
#pragma unroll
    for (int c = 0; c < kNCT; ++c)
#pragma unroll
      for (int G = 0; G < kG; ++G)
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
          for (int e = 0; e < 4; ++e)
            p.ht[((long)chain * K + 32 * G + 8 * lq + 4 * t + e) * p.V + v0 + kWC * wave + 16 * c + li] =
                hs[c][G][t][e];
  }
}

template <int K, bool VL, bool PK>
hipError_t launch_k(const FwdParams& p0, int nchains, hipStream_t stream) {
  FwdParams p = p0;
  p.nvb = p.V / kBV;
  const dim3 grid(nchains * p.nvb), block(kThr);
  if (p.v_new)
    hipLaunchKernelGGL((scan16_kernel<K, VL, PK, true>), grid, block, 0, stream, p);
  else
    hipLaunchKernelGGL((scan16_kernel<K, VL, PK, false>), grid, block, 0, stream, p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_scan16(const FwdParams& p, int K, bool varlen, bool pk, int nchains,
                         hipStream_t stream) {
  if (K == 128) {
    if (pk) return varlen ? launch_k<128, true, true>(p, nchains, stream) : launch_k<128, false, true>(p, nchains, stream);
    return varlen ? launch_k<128, true, false>(p, nchains, stream) : launch_k<128, false, false>(p, nchains, stream);
  }
  if (pk) return varlen ? launch_k<64, true, true>(p, nchains, stream) : launch_k<64, false, true>(p, nchains, stream);
  return varlen ? launch_k<64, true, false>(p, nchains, stream) : launch_k<64, false, false>(p, nchains, stream);
}

}  // namespace gdn

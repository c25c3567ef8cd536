// gdn_chunk.h -- definitions shared by the chunkwise forward kernels (prep, state scans):
// chunk geometry, operand types, chain positions, workspace slot layouts and LDS tile layouts.
#pragma once

#include <stdint.h>

#include <type_traits>

#include "gdn_device.h"
#include "gdn_internal.h"
#include "gdn_tiles.h"

namespace gdn {
namespace chunk {

constexpr int kC = 64;  // chunk length (tokens)

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

// Type of the q / k tiles: the inputs as given for a scalar gate; for a per-key gate they
// hold the decay-scaled operands, so they take the intra-chunk operand type.
template <typename TI, bool PK>
struct QKT {
  typedef typename std::conditional<PK, typename OpT<TI>::type, TI>::type type;
};

// Row of the 16-row A-operand tile t (0/1) of 32-group G that lane row li supplies.
__device__ __forceinline__ int pair_row(int G, int t, int li) {
  return 32 * G + 8 * (li >> 2) + 4 * t + (li & 3);
}

// Makes one wave's LDS writes visible to its other lanes before they read.
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Tile layouts: 16-bit tiles are unpadded and XOR-swizzled (gdn_tiles.h); fp32 tiles are
// padded by 16 bytes per row.
template <typename T, int COLS>
struct Lay {
  static constexpr bool kSwz = sizeof(T) == 2;
  static constexpr int kStride = kSwz ? COLS : COLS + 16 / (int)sizeof(T);
  static constexpr int kElems(int rows) { return rows * kStride; }
  __device__ static int pair(int r, int c) {
    if constexpr (kSwz) return tix_pair<COLS>(r, c);
    else return r * kStride + c;
  }
  __device__ static int seq(int r, int c) {
    if constexpr (kSwz) {
      static_assert(!kSwz || COLS == 64, "sequential-row swizzle is defined for 64 columns");
      return tix_seq64(r, c);
    } else {
      return r * kStride + c;
    }
  }
};

// Workspace slot of one chunk, fp32 inputs: Tm, P (64x64 fp32, row-major), e^gamma,
// e^{gl - gamma}, e^gl.
struct SlotF {
  static constexpr size_t kTm = 0;
  static constexpr size_t kP = (size_t)kC * kC * sizeof(float);
  static constexpr size_t kEg = 2 * kP;
  static constexpr size_t kEl = kEg + kC * 4;
  static constexpr size_t kEgl = kEl + kC * 4;
  static constexpr size_t kBytes = (kEgl + 16 + 255) & ~(size_t)255;
};

// Workspace slot of one chunk, 16-bit inputs.  Every region is the exact image of the LDS
// tile the scan keeps it in (column-split layout tix_s32<64>), so the scan copies it with
// linear 16-byte transfers:
//   Tm, P     [64][64] fp16
//   vec       scalar gate: e^gamma[64], e^{gl-gamma}[64], beta[64], e^gl, padding
//             per-key gate: beta[64], e^{gamma_mid}[K], e^{gamma_last}[K], padding
//   K         [64][K] fp16: K itself (scalar gate) or K e^{gamma-gamma_mid} (per-key gate)
//   per-key gate only: Q e^{gamma-gamma_mid} and K e^{gamma_last-gamma}, [64][K] fp16
template <int K, bool PK>
struct Slot16 {
  static constexpr size_t kTile = (size_t)kC * K * 2;
  static constexpr size_t kTm = 0;
  static constexpr size_t kP = kC * kC * 2;
  static constexpr size_t kVec = 2 * kP;
  static constexpr size_t kVecBytes = PK ? (((kC + 2 * K) * 4 + 1023) & ~(size_t)1023) : 1024;
  static constexpr size_t kK = kVec + kVecBytes;
  static constexpr size_t kQ = kK + kTile;
  static constexpr size_t kKh = kQ + (PK ? kTile : 0);
  static constexpr size_t kBytes = kKh + (PK ? kTile : 0);
  // float offsets inside vec
  static constexpr int kEg = 0, kEl = kC, kBeta = PK ? 0 : 2 * kC, kEgl = 3 * kC;
  static constexpr int kEmid = kC, kEglk = kC + K;
  static_assert(kBytes % 1024 == 0, "slot regions are whole 1 KiB blocks");
};

// Where a chain lives: first token, token count, workspace / h_chunks index of chunk 0.
struct ChunkPos {
  long tok0;
  int len;
  long slot0;
};

__device__ __forceinline__ ChunkPos chain_pos(const FwdParams& p, int chain, bool varlen) {
  ChunkPos c;
  const int h = chain % p.H, bs = chain / p.H;
  if (varlen) {
    c.tok0 = p.cu[bs];
    c.len = p.cu[bs + 1] - p.cu[bs];
    c.slot0 = (long)h * p.nt_total + p.coffs[bs];
  } else {
    c.tok0 = (long)bs * p.T;
    c.len = p.T;
    c.slot0 = (long)chain * ((p.T + kC - 1) / kC);
  }
  return c;
}

// Lower-triangular 16x16 tile enumeration: (0,0),(1,0),(1,1),(2,0),(2,1),(2,2),(3,0),...
__device__ __forceinline__ void tri_tile(int idx, int& I, int& J) {
  I = (idx >= 1) + (idx >= 3) + (idx >= 6);
  J = idx - I * (I + 1) / 2;
}

// Per-key gate, column pass.  Thread tid owns key d = tid / TPK and tokens part*GT..+GT-1
// (TPK adjacent lanes per key).  gk holds this thread's log decays; g_at(t) gives g_t.  On
// return gam[] holds gamma[t][d] for its tokens, and gm / gL the key's gamma at tokens 31
// and 63 (padded rows carry zero decays, so gL is the last valid row's value).
template <int K, int GT, typename GF>
__device__ __forceinline__ void key_cumsum(const float* gk, GF g_at, int part, float* gam,
                                           float& gm, float& gL) {
  constexpr int kTPK = 256 / K;
  float run = 0.f;
#pragma unroll
  for (int i = 0; i < GT; ++i) {
    run += g_at(part * GT + i) + gk[i];
    gam[i] = run;
  }
  // exclusive prefix over the TPK parts of this key (adjacent lanes of one wave)
  const int lane0 = (threadIdx.x & 63) & ~(kTPK - 1);
  float tot[kTPK];
#pragma unroll
  for (int q = 0; q < kTPK; ++q) tot[q] = __shfl(run, lane0 + q, 64);
  float off = 0.f;
#pragma unroll
  for (int q = 0; q < kTPK; ++q) off += q < part ? tot[q] : 0.f;
#pragma unroll
  for (int i = 0; i < GT; ++i) gam[i] += off;
  float cum[kTPK];
  float acc = 0.f;
#pragma unroll
  for (int q = 0; q < kTPK; ++q) {
    acc += tot[q];
    cum[q] = acc;
  }
  static_assert((kC / 2) % GT == 0, "the middle token must end a part");
  gm = cum[kC / 2 / GT - 1];  // gamma at token 31 (the parts up to it sum exactly to it)
  gL = cum[kTPK - 1];
}

// (I + A)^-1 for the strictly lower 64x64 A held in s.a, fp32.  Diagonal 16x16 blocks by
// forward substitution, then blocks merged with
//   T_hi,lo = -T_hi,hi A_hi,lo T_lo,lo       (first for 16-blocks, then for 32-blocks).
// Every final block is written to s.tm (operand type) as it is produced; s.a keeps the fp32
// blocks the later merges read.
template <typename SM>
__device__ __forceinline__ void solve_unit_lower(SM& s, int wave, int lane) {
  typedef typename SM::TO TO;
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
    for (int i = 0; i < 16; ++i) {
      s.a[b0 + i][b0 + li] = x[i];
      s.tm[b0 + i][b0 + li] = to_t<TO>(x[i]);
    }
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
    for (int e = 0; e < 4; ++e) {
      s.a[hi + 4 * lq + e][lo + li] = -t[e];
      s.tm[hi + 4 * lq + e][lo + li] = to_t<TO>(-t[e]);
    }
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
    for (int e = 0; e < 4; ++e) s.tm[32 + 16 * ti + 4 * lq + e][16 * tj + li] = to_t<TO>(-y[e]);
  }
  __syncthreads();
}

}  // namespace chunk

// Per-chunk prep of 16-bit inputs (gdn_prep16.hip): one workgroup per chunk slot.
hipError_t launch_prep16(const FwdParams& p, int K, bool varlen, bool pk, long nslots,
                         hipStream_t stream);

// Single-kernel forward of bf16 inputs with a scalar gate and no saved states
// (gdn_fused16.hip): one workgroup per (chain, 32-column value block).
hipError_t launch_fused16(const FwdParams& p, int K, bool varlen, int nchains, hipStream_t stream);

// Scan of 16-bit inputs (gdn_scan16.hip).
hipError_t launch_scan16(const FwdParams& p, int K, bool varlen, bool pk, int nchains,
                         hipStream_t stream);

}  // namespace gdn

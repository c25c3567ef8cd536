// gdn_device.h -- device-side building blocks shared by the gfx950 kernels.
//
// Matrix-core conventions (CDNA4, wave64).  Every product here is issued as 16x16 output
// tiles with a 32-long contraction slice:
//   - bf16: one v_mfma_f32_16x16x32_bf16;  fp16: one v_mfma_f32_16x16x32_f16;
//   - fp32: eight v_mfma_f32_16x16x4_f32, instruction j taking element j of each lane.
// In both cases lane l = 16*lq + li supplies, for the A operand, row li and contraction
// indices 8*lq .. 8*lq+7 of the slice; for the B operand, column li and the same contraction
// indices.  The 16x16 fp32 accumulator holds, in lane l, column li and rows 4*lq .. 4*lq+3.
// (Verified by an in-bounds layout check on gfx950.)  Because the contraction index a lane
// supplies is the same for A and B, any fixed assignment of real indices to (lq, j) gives
// the same sum; the kernels use "8*lq + j" throughout so each lane's operand is one
// contiguous 16- or 32-byte LDS read.
#pragma once

#include <hip/hip_runtime.h>

#include <type_traits>
#include <stdint.h>

namespace gdn {

typedef __bf16 bf16;
typedef _Float16 f16;
typedef bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef f16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x8 __attribute__((ext_vector_type(8)));

template <typename T>
struct Vec8;
template <>
struct Vec8<bf16> {
  typedef bf16x8 type;
};
template <>
struct Vec8<f16> {
  typedef f16x8 type;
};
template <>
struct Vec8<float> {
  typedef f32x8 type;
};

__device__ __forceinline__ f32x4 mma16(const bf16x8& a, const bf16x8& b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ f32x4 mma16(const f16x8& a, const f16x8& b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ f32x4 mma16(const f32x8& a, const f32x8& b, f32x4 c) {
#pragma unroll
  for (int j = 0; j < 8; ++j) c = __builtin_amdgcn_mfma_f32_16x16x4f32(a[j], b[j], c, 0, 0, 0);
  return c;
}

// One fp32 16x16x4 step (contraction 4), used by the small fp32 products of the solve.
__device__ __forceinline__ f32x4 mma4(float a, float b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

// 8 contiguous elements from LDS (16-byte aligned address).
__device__ __forceinline__ bf16x8 lds8(const bf16* p) { return *reinterpret_cast<const bf16x8*>(p); }
__device__ __forceinline__ f16x8 lds8(const f16* p) { return *reinterpret_cast<const f16x8*>(p); }
__device__ __forceinline__ f32x8 lds8(const float* p) {
  const f32x4 a = *reinterpret_cast<const f32x4*>(p);
  const f32x4 b = *reinterpret_cast<const f32x4*>(p + 4);
  f32x8 r;
  r[0] = a[0]; r[1] = a[1]; r[2] = a[2]; r[3] = a[3];
  r[4] = b[0]; r[5] = b[1]; r[6] = b[2]; r[7] = b[3];
  return r;
}

template <typename T>
__device__ __forceinline__ T to_t(float x);
template <>
__device__ __forceinline__ bf16 to_t<bf16>(float x) { return (bf16)x; }
template <>
__device__ __forceinline__ f16 to_t<f16>(float x) { return (f16)x; }
template <>
__device__ __forceinline__ float to_t<float>(float x) { return x; }

__device__ __forceinline__ float to_f(bf16 x) { return (float)x; }
__device__ __forceinline__ float to_f(f16 x) { return (float)x; }
__device__ __forceinline__ float to_f(float x) { return x; }

// Pack a lane's 8 rows of a tile pair (rows 0..3 from accumulator a, 4..7 from b) as an MFMA
// operand.
template <typename T>
__device__ __forceinline__ typename Vec8<T>::type pack8(const f32x4& a, const f32x4& b) {
  typename Vec8<T>::type r;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    r[j] = to_t<T>(a[j]);
    r[4 + j] = to_t<T>(b[j]);
  }
  return r;
}

// Gate floors.  A per-token log decay of -inf (a hard reset of the state, alpha = 0) would
// turn the differences of cumulative decays into inf - inf.  Every kernel therefore reads a
// scalar gate as max(g, kGateFloor): e^-40 = 4.2e-18 leaves at most that fraction of the state
// it erases, below fp32 resolution.  With a per-key gate the combined per-key log decay
// g + gk of one token is floored at kKeyGateFloor instead: the per-key intra-chunk products
// factor e^{gamma_r - gamma_s} around a reference token inside each 16-token block, and the
// factors stay inside the fp32 / bf16 exponent range (|x| <= e^88) only while 8 tokens of
// decay span at most 80; a floored token keeps at most e^-10 = 4.5e-5 of what it erases.
constexpr float kGateFloor = -40.f;
constexpr float kKeyGateFloor = -10.f;
__device__ __forceinline__ float floor_gate(float g) { return fmaxf(g, kGateFloor); }
__device__ __forceinline__ float floor_key_gate(float lam) { return fmaxf(lam, kKeyGateFloor); }

// Split bf16 operands.  x = hi + lo with hi = bf16(x) and lo = bf16(x - hi) keeps about 16
// mantissa bits and fp32's exponent range; a product of two split operands is summed as
// hi*hi + hi*lo + lo*hi (the lo*lo term is below 2^-16 of the result).
#define GDN_SPLIT(x, H, L)           \
  do {                               \
    const float x_ = (x);            \
    H = (bf16)x_;                    \
    L = (bf16)(x_ - (float)(bf16)H); \
  } while (0)

// c + (ah + al)(bh + bl) without the al bl term
__device__ __forceinline__ f32x4 mma3(const bf16x8& ah, const bf16x8& al, const bf16x8& bh,
                                      const bf16x8& bl, f32x4 c) {
  c = mma16(al, bh, c);
  c = mma16(ah, bl, c);
  return mma16(ah, bh, c);
}

// 8 consecutive inputs as fp32
template <typename TI>
__device__ __forceinline__ void load8f(const TI* p, float (&x)[8]) {
  if constexpr (std::is_same<TI, float>::value) {
    const f32x4 a = *reinterpret_cast<const f32x4*>(p), b = *reinterpret_cast<const f32x4*>(p + 4);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      x[j] = a[j];
      x[4 + j] = b[j];
    }
  } else {
    const bf16x8 a = *reinterpret_cast<const bf16x8*>(p);
#pragma unroll
    for (int j = 0; j < 8; ++j) x[j] = (float)a[j];
  }
}

// Inclusive prefix sum across the 64 lanes of a wave.
__device__ __forceinline__ float wave_incl_scan(float x, int lane) {
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const float y = __shfl_up(x, off, 64);
    if (lane >= off) x += y;
  }
  return x;
}

}  // namespace gdn

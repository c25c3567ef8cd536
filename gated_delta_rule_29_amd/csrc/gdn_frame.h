// gdn_frame.h -- operand layouts shared by the frame-level scans (BiGDN and the camera
// branch): the lane orders in which the frame statistics G and U are written for the scan,
// and the LDS transpose read used to form operands that contract over a tile's rows.
#pragma once

#include "gdn_device.h"

namespace gdn {

// Workspace layouts of G and U (written by frame_stats, read by scan), per (b, h, frame),
// with kRT = D / 64 row tiles per scan wave and 32-column scan blocks:
//   G: A-operand order, element (r, c) at ((((r / (D/4)) kRT + (r % (D/4)) / 16) (D/32)
//      + c / 32) 64 + ((c / 8) % 4) 16 + r % 16) 8 + c % 8, so a scan lane's 16-byte
//      operand is one load and a wave's loads are contiguous;
//   U: accumulator order, element (r, c) at (c / 32) 32D + ((((r / (D/4)) kRT
//      + (r % (D/4)) / 16) 2 + (c % 32) / 16) 64 + ((r % 16) / 4) 16 + c % 16) 4 + r % 4.
template <int D>
__device__ __forceinline__ long g_lane_index(int r, int c) {
  constexpr int kRT = D / 64;
  return ((((long)(r / (D / 4)) * kRT + (r % (D / 4)) / 16) * (D / 32) + c / 32) * 64 +
          ((c / 8) & 3) * 16 + (r & 15)) * 8 + (c & 7);
}
template <int D>
__device__ __forceinline__ long u_lane_index(int r, int c) {
  constexpr int kRT = D / 64;
  return (long)(c >> 5) * (32 * D) +
         ((((long)(r / (D / 4)) * kRT + (r % (D / 4)) / 16) * 2 + ((c >> 4) & 1)) * 64 +
          ((r & 15) >> 2) * 16 + (c & 15)) * 4 +
         (r & 3);
}

typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef f16 f16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
typedef unsigned u32x2v __attribute__((ext_vector_type(2)));
typedef unsigned u32x4v __attribute__((ext_vector_type(4)));

// Two 8-byte LDS transpose reads (ds_read_b64_tr_b16) joined into one 8-element operand.
// Within a 16-lane group, lane n of one read receives element j (j = 0..3) from halfword
// n % 4 of the 8-byte piece addressed by lane 4j + n / 4.
__device__ __forceinline__ f16x8 tr_pair(const f16* p0, const f16* p1) {
  auto rd = [](const f16* p) {
    return __builtin_bit_cast(u32x2v, __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (lds_i16x4*)(uintptr_t)(const __attribute__((address_space(3))) char*)p));
  };
  const u32x4v w = __builtin_shufflevector(rd(p0), rd(p1), 0, 1, 2, 3);
  return __builtin_bit_cast(f16x8, w);
}

}  // namespace gdn

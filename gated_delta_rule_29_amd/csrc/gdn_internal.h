// gdn_internal.h -- host-side launch interface between the C ABI and the kernels.
#pragma once

#include <hip/hip_runtime.h>

namespace gdn {

struct FwdParams {
  const void* q;
  const void* k;
  const void* v;
  const float* g;     // [tokens, H] or nullptr
  const float* gk;    // [tokens, H, K] or nullptr
  const float* beta;  // [tokens, H]
  const float* h0;    // [chains, K, V] or nullptr
  void* o;
  float* ht;          // [chains, K, V] or nullptr
  void* h_chunks;     // [.., H, NT, K, V] or nullptr
  void* v_new;        // [tokens, H, V] or nullptr
  const int* cu;      // packed batches: [nseq + 1] device offsets
  float scale;
  int B, T, H, V;
  int nvb;            // V / 64 value blocks
  int nseq;           // packed batches: number of sequences
  int nt_total;       // packed batches: total chunks (h_chunks indexing)
};

hipError_t launch_gdn_fwd(const FwdParams& p, int dtype, int K, bool varlen, hipStream_t stream);
hipError_t launch_varlen_tables(const int* cu, int N, int* offs, int* idx, hipStream_t stream);

}  // namespace gdn

// gdn_bwd_params.h -- host/device parameter blocks of the frame-scan backward kernels that
// are not shared with the forward (the forward's translation units do not include this file).
#pragma once

#include <hip/hip_runtime.h>

#include "gdn_internal.h"

namespace gdn {

// Workgroup ids are dealt to the eight XCDs round-robin.  When the grid is a multiple of eight,
// XCD x takes the contiguous range [x n/8, (x+1) n/8) of logical indices in order, so logical
// neighbours (which read the same slabs or matrices) run close in time on one XCD's L2.
__device__ __forceinline__ int xcd_logical(int bid, int n) {
  return n % 8 ? bid : (bid % 8) * (n / 8) + bid / 8;
}

// The state / gradient scan of the camera-scan backward alone (gdn_cambwd.hip): the forward
// states and the state gradients from the frame statistics G, U, W in p's workspace views.
// The BiGDN direction backward reuses it for its S stream.
hipError_t launch_cam_bwd_scan(const CamBwdParams& p, hipStream_t stream);

// Backward of one BiGDN direction (gdn_bigdnbwd.hip).  Prepped tensors token-major bf16
// [B,H,N,D]; dnum [B,N,H,D] and dden [B,H,N] fp32; gradients fp32 (dq_rot .. dv [B,H,N,D],
// dbeta [B,H,F,S], ddecay [B,H,F]).  cam holds the S stream's workspace views (G = K_rot
// diag(beta) K_rot^T, U = K_rot diag(beta) V^T, W = Q_rot dnum^T, the saved states and
// their gradients); the z stream adds its own.
struct BigdnBwdParams {
  CamBwdParams cam;       // S stream: q, k, v, dout unused here (token-major copies below)
  const __bf16* q_rot;
  const __bf16* k_rot;
  const __bf16* q_pos;
  const __bf16* k_pos;
  const __bf16* v;
  const float* dnum;      // [B,N,H,D]
  const float* dden;      // [B,H,N]
  float* dq_rot;
  float* dk_rot;
  float* dq_pos;
  float* dk_pos;
  float* dv;
  // z stream workspace, per (b, h, frame or step)
  float* Gpos;            // K_pos diag(beta) K_pos^T, D x D
  float* upos;            // K_pos^T beta, D
  float* wz;              // Q_pos^T dden, D
  float* zs;              // z after every step, D
  float* as;              // gradient of z after every step's update, D
  float* ddz;             // the z stream's part of ddecay, per absorbed frame
  int acc;                // dbeta and ddecay are added to the arrays' contents
};
hipError_t launch_bigdn_dir_bwd(const BigdnBwdParams& p, hipStream_t stream);

// Backward of the BiGDN front end (gdn_prepbwd.hip): the scan directions' gradients of the
// prepped tensors, summed, taken back through RoPE, ReLU, k-scale and the full-channel
// RMSNorm to qkv and the norm weights.
struct PrepBwdParams {
  const __bf16* qkv;      // [B,N,3,H,D]
  const float* q_norm_w;  // [H*D]
  const float* k_norm_w;
  const float* rope_cos;  // [N,D]
  const float* rope_sin;
  float k_scale, eps;
  int ndir;               // 1 or 2 directions in each gradient tensor
  const float* dq_rot;    // [ndir,B,H,N,D]
  const float* dk_rot;
  const float* dq_pos;
  const float* dk_pos;
  const float* dv;
  float* dqkv;            // [B,N,3,H,D]
  float* dq_norm_w;       // [H*D]
  float* dk_norm_w;
  float* part;            // workspace: the norm weights' partial gradients [nwg][2][H*D]
  int nwg;                // token groups (one workgroup each)
  int B, N, H, D;
};
hipError_t launch_prep_bwd(const PrepBwdParams& p, hipStream_t stream);

// Backward of the merge out = num / (den + eps) * SiLU(gate) (gdn_prepbwd.hip).
struct MergeBwdParams {
  const __bf16* num;      // [B,N,H,D] (the sums over both directions, as bigdn_fwd stores them)
  const __bf16* den;      // [B,H,N]
  const __bf16* gate;     // [B,N,H,D] or nullptr
  const float* dout;      // [B,N,H,D]
  float eps;
  float* dnum;            // [B,N,H,D]
  float* dden;            // [B,H,N]
  float* dgate;           // [B,N,H,D], given with gate
  int B, N, H, D;
};
hipError_t launch_merge_bwd(const MergeBwdParams& p, hipStream_t stream);

// State columns per workgroup of the backward frame scan (gdn_cambwd.hip); the decay
// gradient's partial sums come one per column block, D / kScanCB per (b, h, frame).
constexpr int kScanCB = 16;

// Backward of the camera-branch prep (gdn_prepbwd.hip).
struct CamPrepBwdParams {
  const float* q;          // [B,N,H,D] fp32, the raw inputs of the prep
  const float* k;
  const float* q_norm_w;   // [H*D]
  const float* k_norm_w;
  const float* proj_q;     // [B,N,4,4]
  const float* proj_kv;
  const float* rope_cos;   // [N,D/2]
  const float* rope_sin;
  float k_scale, eps;
  int ndir;                // 1 or 2 directions in each upstream gradient tensor
  const float* dq_t;       // [ndir,B,H,D,N] gradients of the prep's outputs
  const float* dk_t;
  const float* dv_t;
  const float* dinfl;      // [B,H,N] gradient of the inflation, or nullptr
  float* k_inv_rms;        // [B,N] workspace (written first when dinfl is given)
  float* dq;               // [B,N,H,D]: the gradient before the RMSNorm first, then dq in place
  float* dk;
  float* dv;
  float* dq_norm_w;        // [H*D]
  float* dk_norm_w;
  float* part;             // workspace: the norm weights' partial gradients [nwg][2][H*D]
  int nwg;                 // token groups of the RMSNorm backward (one workgroup each)
  int B, N, H, D;
};
hipError_t launch_cam_prep_bwd(const CamPrepBwdParams& p, hipStream_t stream);

}  // namespace gdn

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
  void* ws;           // workspace: per-chunk slots, then (packed batches) chunk offsets
  int* coffs;         // packed batches: chunk offsets table inside the workspace
  const int* order;   // packed batches, single-kernel path: sequences, longest first
};

// Workspace of a forward call with `nslots` chunk slots (B*H*NT dense, H*NT_total packed)
// and, for packed batches, nseq + 1 chunk offsets; `fused`: the single-kernel path, whose
// only scratch is the rank table of a packed batch (nseq ints).
size_t fwd_workspace_bytes(long nslots, int nseq, int dtype, int K, bool per_key, bool fused);
size_t fwd_slot_bytes(int dtype, int K, bool per_key);

hipError_t launch_gdn_fwd(const FwdParams& p, int dtype, int K, bool varlen, hipStream_t stream);
hipError_t launch_varlen_tables(const int* cu, int N, int* offs, int* idx, hipStream_t stream);

// fragment state summary helpers (gdn_summary.hip)
hipError_t launch_zero(void* p, size_t bytes, hipStream_t stream);  // bytes a multiple of 16
hipError_t launch_identity(float* m, long BH, int K, hipStream_t stream);
hipError_t launch_apply(const float* c, const float* M, const float* h_in, float* h_out, int BH,
                        int K, int V, hipStream_t stream);
// M [B,H,K,K] fp32 from k (dtype 0 fp32, 1 bf16), g, gk (each may be null), beta; K in {64, 128}.
// wy: transition_ws_bytes(B, T, H, K, dtype, gk != null) bytes of workspace (256-byte aligned).
hipError_t launch_transition(const void* k, const float* g, const float* gk, const float* beta,
                             float* M, int B, int T, int H, int K, int dtype, void* wy,
                             hipStream_t stream);
size_t transition_ws_bytes(int B, int T, int H, int K, int dtype, bool per_key);
constexpr int kApplyMaxK = 256;

}  // namespace gdn

namespace gdn {

struct PrepParams {
  const void* qkv;  // [B, N, 3, H, D] bf16
  const float* q_norm_w;
  const float* k_norm_w;
  const float* rope_cos;
  const float* rope_sin;
  float k_scale, eps;
  float* q_inv_rms;  // [B, N] or nullptr
  float* k_inv_rms;
  void* q_rot;  // [B, H, N, D] bf16 outputs, each nullable
  void* k_rot;
  void* q_pos;
  void* k_pos;
  void* v_hm;
  _Float16* rope_h;  // [N, D, 2] (cos, sin) fp16 pairs, or nullptr
  int B, N, H, D;
};

struct BigdnParams {
  const void* qkv;
  const void* qkv_bwd;     // [B, N, 3, H, D] q, k, v of the reverse direction, or nullptr (= qkv)
  const float* beta;       // [B, H, F, S]
  const float* decay;      // [B, H, F]
  const float* decay_bwd;  // [B, H, F] decay of the reverse direction, or nullptr (= decay)
  const float* beta_bwd;   // [B, H, F, S] beta of the reverse direction, or nullptr (= beta)
  const float* q_norm_w;
  const float* k_norm_w;
  const float* rope_cos;
  const float* rope_sin;
  float k_scale, eps;
  void* num;  // [B, N, H, D] bf16, or nullptr
  void* den;  // [B, H, N] bf16, or nullptr
  // merge epilogue: out = num / (den + merge_eps) * SiLU(gate) (gate nullable), when out is set
  const void* gate;  // [B, N, H, D] bf16
  void* out;         // [B, N, H, D] bf16
  float merge_eps;
  int B, F, S, H, D, N;
  // workspace views
  float* q_inv_rms;  // [B, N]
  float* k_inv_rms;  // [B, N]
  float* q_inv_rms_b;  // [B, N] of qkv_bwd (when set)
  float* k_inv_rms_b;  // [B, N]
  _Float16* rope_h;  // [N, D, 2]  RoPE tables as (cos, sin) fp16 pairs
  _Float16* G;       // [B, H, F, D, D]
  _Float16* Gz;      // [B, H, F, D, D]
  float* U;          // [B, H, F, D, D]
  float* uz;         // [B, H, F, D]
  // statistics of the reverse direction (the same buffers unless beta or qkv is overridden
  // for it)
  _Float16* G_b;
  _Float16* Gz_b;
  float* U_b;
  float* uz_b;
  _Float16* SdT;     // [dir_slots, B, H, F, D, D]  S_f^T (forward) and R_f^T (reverse)
  float* zd;         // [2, B, H, F, D]     z_f and zR_f
  // scan set-up: directions run (1 forward, 2 reverse, 3 both), whether the z block runs,
  // SdT direction slots (2: indexed by direction; 1: the one direction run), and the forward
  // state in / out ([B*H, D, D] fp32, keys as rows; nullable)
  int scan_dirs, scan_z, dir_slots;
  const float* s_init;
  float* s_final;
};

// camera branch (gdn_cam.hip)
struct CamPrepParams {
  const float* q;  // [B, N, H, D] fp32
  const float* k;
  const float* v;
  const float* q_norm_w;  // [H*D]
  const float* k_norm_w;
  const float* proj_q;    // [B, N, 4, 4]
  const float* proj_kv;
  const float* rope_cos;  // [N, D/2]
  const float* rope_sin;
  float k_scale, eps;
  float* q_out;  // [B, H, D, N] fp32
  float* k_out;
  float* v_out;
  float* inflation;  // [B, H, N]
  float* q_inv_rms;  // [B, N] workspace
  float* k_inv_rms;
  int B, N, H, D;
};
struct CamScanParams {
  const float* q;  // [B, H, D, N] fp32
  const float* k;
  const float* v;
  const float* beta;   // [B, H, F, S]
  const float* decay;  // [B, H, F]
  int reverse;              // one direction: 0 forward, 1 reverse; 2: both (bidirectional)
  const float* decay_bwd;   // [B, H, F] decay of the reverse direction (both), or nullptr
  const float* init_state;  // [B*H, D, D] or nullptr (forward only)
  float* final_state;       // [B*H, D, D] or nullptr (forward only)
  float* out;               // [B, H, D, N] fp32 (the direction run; forward when both)
  float* out_rev;           // [B, H, D, N] fp32 (reverse, when both)
  int B, H, D, F, S;
  // workspace views
  _Float16* G;    // [B, H, F, D, D]
  float* U;       // [B, H, F, D, D]
  _Float16* SdT;  // [dirs, B, H, F, D, D]
};
// state-gradient pass of the chunked backward (gdn_bwd.hip)
struct DhuParams {
  const void* q;    // [B, T, H, K] (fp32 or bf16, as every input here)
  const void* k;
  const void* w;    // [B, T, H, K] the WY w of the forward
  const void* do_;  // [B, T, H, V]
  const void* dv;   // [B, T, H, V] the intra-chunk gradient of v_new
  const float* g;   // [B, T, H] per-token log gates, or nullptr
  const float* gk;  // [B, T, H, K] per-key log gates, or nullptr (bf16 inputs only)
  const float* dht; // [B, H, K, V] or nullptr
  float scale;
  float* dh_chunks; // [B, H, NT, K, V] or nullptr
  void* dv2;        // [B, T, H, V] (input dtype)
  float* dh0;       // [B, H, K, V] or nullptr
  int B, T, H, V;
  // packed sequences (B = number of sequences, T = total tokens): cu [B + 1] token offsets and
  // coffs [B + 1] chunk offsets on the device; dh_chunks is then [1, H, nt_total, K, V]
  const int* cu;
  const int* coffs;
  int nt_total;
};
hipError_t launch_dhu(const DhuParams& p, int dtype, hipStream_t stream);  // K = 128; dtype 0 fp32, 1 bf16
// Inputs of the state-gradient pass (gdn_bwdprep.hip): w [B,T,H,K] and dv = P^T do [B,T,H,V]
// from q, k [B,T,H,K], beta, g [B,T,H] (g may be null) and do [B,T,H,V]; scalar gate only.
struct BwdPrepParams {
  const void* q;
  const void* k;
  const float* beta;
  const float* g;
  const void* do_;
  float scale;
  void* w;
  void* dv;
  int B, T, H;
};
hipError_t launch_bwd_prep(const BwdPrepParams& p, int K, int V, int dtype, hipStream_t stream);
// grad_out = grad_ext + M^T grad_in (grad_in may be null: zero)
hipError_t launch_grad_apply(const float* grad_ext, const float* M, const float* grad_in,
                             float* grad_out, int BH, int K, int V, hipStream_t stream);

// backward of the camera-branch scan (gdn_cambwd.hip)
struct CamBwdParams {
  const float* q;     // [B, H, D, N] fp32
  const float* k;
  const float* v;
  const float* beta;  // [B, H, F, S]
  const float* decay; // [B, H, F]
  const float* dout;  // [B, H, D, N]
  int reverse;
  int acc;            // add dbeta and ddecay to the arrays' contents
  int reuse;          // G and U are in the workspace already (only W is formed)
  float* dq;          // [B, H, D, N]
  float* dk;
  float* dv;
  float* dbeta;       // [B, H, F, S]
  float* ddecay;      // [B, H, F]
  int B, H, D, F, S;
  // workspace views, per (b, h, frame or step) D x D
  float* G;           // frame statistics K diag(beta) K^T (stored as a hi/lo bf16 pair in its
                      // fp32 slot), K diag(beta) V^T, Q dout^T (fp32)
  float* U;
  float* W;
  float* Spf;         // state after each step (fp32)
  // bf16 operand pairs: element e of a matrix is hi[e] + lo[e] with hi[e] = bf16(x) and
  // lo[e] = bf16(x - hi[e]); the lo half of each array starts `lo` elements after the hi half
  __bf16* Sp;         // state after each step, row-major and transposed
  __bf16* SpT;
  __bf16* Ab;         // gradient of the state after each step's update, both orientations
  __bf16* AbT;
  size_t lo;          // B * H * F * D * D
  float* ddecay_part; // [B, H, F, D/kScanCB] (gdn_bwd_params.h) partial sums of the decay gradient (one per
                      // column block of the scan)
};
hipError_t launch_cam_scan_bwd(const CamBwdParams& p, hipStream_t stream);

hipError_t launch_cam_prep(const CamPrepParams& p, hipStream_t stream);
hipError_t launch_cam_scan(const CamScanParams& p, hipStream_t stream);
// the frame scan of gdn_bigdn.hip, for one direction without z
hipError_t launch_frame_scan(const BigdnParams& p, hipStream_t stream);

hipError_t launch_prep(const PrepParams& p, hipStream_t stream);
hipError_t launch_bigdn(const BigdnParams& p, hipStream_t stream);

}  // namespace gdn

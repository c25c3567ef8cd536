/*
 * gdn.h -- C ABI of libgdn, a gfx950 (MI355X) implementation of the chunkwise gated
 * delta-rule forward pass.
 *
 * Method.  Per (batch, head) a K x V state S evolves token by token as
 *     S_t = diag(a_t) S_{t-1} + k_t d_t^T,  d_t = beta_t (v_t - (diag(a_t) S_{t-1})^T k_t),
 *     o_t = scale * S_t^T q_t,              a_{t,d} = exp(g_t + gk_{t,d}),
 * i.e. S_t = a_t (I - beta_t k_t k_t^T) S_{t-1} + beta_t k_t v_t^T for a scalar gate.  The
 * library computes it chunk by chunk (64 tokens): a WY form of each chunk from a unit-lower-
 * triangular solve, the sequential inter-chunk state pass v_new = u - w h,
 * h <- diag(e^{g_last}) h + (k * e^{g_last - g})^T v_new (the state-pass fragments of
 * chunk_gated_delta_rule_fwd_h on the hyper-parallel "Diff Coverage" page), and the masked
 * intra-chunk output.  The result equals the token recurrence up to rounding.
 *
 * Entry points, in the order declared below:
 *  - the forward, dense (gdn_fwd) and packed (gdn_fwd_varlen, gdn_varlen_num_chunks), and the
 *    packed forward for callers that cannot allocate (gdn_fwd_varlen_noalloc);
 *  - the BiGDN video block of the SANA pages: its front end (gdn_prep), the frame-level scan
 *    in both directions (bigdn_fwd) and the block output with reverse-direction overrides and
 *    the merge (bigdn_fwd_merged);
 *  - a fragment's state summary and the joining of fragments (gdn_state_summary,
 *    gdn_state_apply), and their gradient counterparts (gdn_state_grad_summary,
 *    gdn_state_grad_apply): the single-GPU part of context parallelism;
 *  - the camera branch of the video block (cam_prep, cam_scan, cam_scan_bidi) and the
 *    backward of its scan (cam_scan_bwd) and of its prep (cam_prep_bwd); the backward of a BiGDN direction (bigdn_dir_bwd),
 *    of the block's merge (bigdn_merge_bwd) and of its front end (gdn_prep_bwd);
 *  - the backward's inputs (gdn_bwd_prep) and state-gradient pass (gdn_bwd_dhu,
 *    gdn_bwd_dhu_varlen).
 *
 * Conventions shared by every entry point.
 *  - All tensor pointers are DEVICE pointers unless the name ends in _host.  The caller owns
 *    all memory, including any workspace; the library keeps no device allocation between
 *    calls and has no other global mutable state, except the static scratch array of
 *    gdn_fwd_varlen_noalloc (one per GPU, held until the process ends).
 *  - Tensors are dense and row-major in the shapes given (no strides).
 *  - dtype: GDN_DTYPE_F32 (fp32 inputs, fp32 MFMA, fp32 state) or GDN_DTYPE_BF16 (bf16 q/k/v
 *    and bf16 outputs, bf16 MFMA operands, fp32 accumulation and fp32 state).  Gates (g, gk,
 *    beta), initial and final states are always fp32.  Gates are natural-log decays: a base-2
 *    gate x is passed as x * ln 2.
 *  - stream is a hipStream_t (0 = the null stream).  Calls are asynchronous on that stream
 *    and never synchronise the device.
 *  - Every argument is validated on the host before anything is launched; on an error
 *    nothing is written.  The return value is a status code below, and gdn_last_error()
 *    returns a message for the calling thread's most recent failure.
 *  - Results are deterministic: no entry point uses atomics, so two identical calls give
 *    bitwise-identical outputs.
 */
#ifndef GDN_H_
#define GDN_H_

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

#if defined(__GNUC__)
#define GDN_API __attribute__((visibility("default")))
#else
#define GDN_API
#endif

#define GDN_ABI_VERSION 6
#define GDN_CHUNK 64
#define GDN_BWD_ACCUMULATE 2  /* bigdn_dir_bwd: add dbeta, ddecay into the outputs */
#define GDN_BWD_REUSE_STATS 4 /* the workspace holds this call's frame statistics already */

/* Status codes (the pages' wrappers raise ValueError / NotImplementedError / RuntimeError
 * for these classes, SANA fused_gdn.py page, fused_gdn_func argument checks). */
#define GDN_OK 0
#define GDN_ERR_INVALID 1     /* bad pointer, size, shape or table (ValueError)            */
#define GDN_ERR_UNSUPPORTED 2 /* valid but not implemented combination (NotImplementedError) */
#define GDN_ERR_WORKSPACE 3   /* workspace missing or smaller than the size query returns   */
#define GDN_ERR_HIP 4         /* a HIP launch or runtime call failed (RuntimeError)          */

#define GDN_DTYPE_F32 0
#define GDN_DTYPE_BF16 1

/* Flags of the forward workspace queries: what the call they size will ask for. */
#define GDN_FWD_PER_KEY 1u /* gk is given                                */
#define GDN_FWD_SAVES 2u   /* h_chunks or v_new is requested             */

/* ABI version (GDN_ABI_VERSION) of the loaded library. */
GDN_API int gdn_abi_version(void);

/* Message for the calling thread's most recent failed call ("" if none).  The pointer stays
 * valid until the thread's next library call. */
GDN_API const char* gdn_last_error(void);

/*
 * gdn_fwd -- dense batch forward.
 *
 *   q, k      [B, T, H, K]  dtype      queries and keys (the method assumes unit-norm keys for
 *                                      stability; nothing here enforces it)
 *   v         [B, T, H, V]  dtype
 *   g         [B, T, H]     fp32       scalar log decay per token and head; NULL = 0
 *   gk        [B, T, H, K]  fp32       per-key log decay, added to g in log space (the per-key
 *                                      gate row-scaling of the state in the Diff Coverage page's
 *                                      state pass); NULL = none.  bf16 only.
 *   beta      [B, T, H]     fp32       write strength
 *   scale                              output scale (o = scale * S^T q)
 *   h0        [B, H, K, V]  fp32       state at the end of a prefix, before any further decay
 *                                      (SANA fused_cam_gdn.py page, LOAD_INIT_STATE); NULL = 0
 *   o         [B, T, H, V]  dtype      output (required)
 *   ht        [B, H, K, V]  fp32       final state; NULL = not written
 *   h_chunks  [B, H, NT, K, V] dtype   state entering each chunk, NT = ceil(T / 64),
 *                                      h_chunks[.., 0, ..] = h0; NULL = not written
 *   v_new     [B, T, H, V]  dtype      per-token delta d_t = beta_t (v_t - S'^T k_t), the
 *                                      v_new = u - w h of the state pass; NULL = not written
 *   workspace, workspace_bytes          caller-owned device scratch, 256-byte aligned, of at
 *                                      least gdn_fwd_workspace_bytes(B, T, H, K, V, dtype,
 *                                      flags) bytes, flags = GDN_FWD_PER_KEY if gk is given |
 *                                      GDN_FWD_SAVES if h_chunks or v_new is.  The call fills
 *                                      it with per-chunk terms (WY inverse, masked Q K^T,
 *                                      decays) and reads them back; it is free again once the
 *                                      call's work on `stream` has completed.  Smaller than
 *                                      that, or NULL when that is not 0: GDN_ERR_WORKSPACE.
 *                                      A bf16 call with neither flag needs none (0 bytes).
 * Supported: K in {64, 128}, V in {64, 128} for bf16; K = 64 and V in {64, 128} for fp32
 * (gk is bf16 only).  B, T, H >= 1 and B*H*(V/32) <= 2^31 - 1 (else GDN_ERR_INVALID); bf16
 * also needs T*H*max(K, V)*2 < 2^32, the byte span of one head's rows (else
 * GDN_ERR_UNSUPPORTED).  The size query returns 0 for arguments it cannot size.
 */
GDN_API size_t gdn_fwd_workspace_bytes(int B, int T, int H, int K, int V, int dtype,
                                       unsigned flags);
GDN_API int gdn_fwd(const void* q, const void* k, const void* v, const float* g, const float* gk,
            const float* beta, float scale, const float* h0, void* o, float* ht, void* h_chunks,
            void* v_new, int B, int T, int H, int K, int V, int dtype, void* workspace,
            size_t workspace_bytes, void* stream);

/*
 * Packed variable-length batch (batch 1), the IS_VARLEN layout of the state-pass fragments:
 * sequence i covers tokens [cu[i], cu[i+1]) of [1, T_total, H, .] tensors; the state
 * (from h0[i] or zero) and the 64-token chunk grid restart at every sequence.
 *
 * gdn_varlen_num_chunks: host-only helper, returns sum_i ceil((cu[i+1]-cu[i]) / 64) for a
 * HOST array of N+1 offsets, or -1 if cu is malformed (cu[0] != 0, a sequence is empty, or
 * N < 1).
 */
GDN_API int gdn_varlen_num_chunks(const int* cu_seqlens_host, int N);

/* Workspace of a packed call with N sequences, T_total tokens and NT_total chunks
 * (gdn_varlen_num_chunks); NT_total <= 0 gives a bound for any packing (T_total / 64 + N
 * chunks).  flags as for gdn_fwd_workspace_bytes. */
GDN_API size_t gdn_fwd_varlen_workspace_bytes(int T_total, int N, int NT_total, int H, int K,
                                              int V, int dtype, unsigned flags);

/*
 *   cu_seqlens       [N+1] int32 device   offsets, cu[0] = 0, strictly increasing,
 *                                          cu[N] = T_total (copied from cu_seqlens_host)
 *   cu_seqlens_host  [N+1] int32 host     the same offsets; validated and used for sizing
 *   h0, ht           [N, H, K, V] fp32    per-sequence initial / final state (nullable)
 *   h_chunks         [1, H, NT_total, K, V] dtype; chunk c of sequence i at index
 *                                          chunk_offsets[i] + c (nullable)
 *   chunk_offsets    [N+1] int32 device   OUT: chunks before sequence i (nullable)
 *   chunk_indices    [NT_total, 2] int32  OUT: (sequence, chunk within sequence) per chunk
 *                                          in order (nullable)
 * Other arguments as in gdn_fwd with B = 1 and T = T_total.
 */
GDN_API int gdn_fwd_varlen(const void* q, const void* k, const void* v, const float* g,
                   const float* gk, const float* beta, float scale, const int* cu_seqlens,
                   const int* cu_seqlens_host, int N, const float* h0, void* o, float* ht,
                   void* h_chunks, void* v_new, int* chunk_offsets, int* chunk_indices,
                   int T_total, int H, int K, int V, int dtype, void* workspace,
                   size_t workspace_bytes, void* stream);

/*
 * gdn_fwd_varlen_noalloc -- gdn_fwd_varlen for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid allocation).  The
 * arguments are those of gdn_fwd_varlen without the workspace: the call's scratch (the
 * sequence rank table of the single-kernel path; the per-chunk slots and chunk offsets of the
 * two-kernel path) lives in a static device array of GDN_NOALLOC_SCRATCH_BYTES per GPU, which
 * the library holds until the process ends.  The call itself allocates nothing.
 *   - A call whose scratch (gdn_fwd_varlen_workspace_bytes with its own NT_total and flags)
 *     exceeds GDN_NOALLOC_SCRATCH_BYTES returns GDN_ERR_WORKSPACE and launches nothing.
 *     bf16 calls without gk or saves need 4 bytes per sequence; the others about 66 KB
 *     (74 KB with gk) per chunk and head.
 *   - Every call on one GPU shares that GPU's array.  Calls that overlap on one GPU (on
 *     different streams, or from different threads without ordering) race on it; calls
 *     ordered on one stream do not.  No call relies on the array's previous contents.
 *   - The first call on a device looks up the array's device address (once per device).
 * Results are bitwise those of gdn_fwd_varlen.
 */
#define GDN_NOALLOC_SCRATCH_BYTES ((size_t)32 << 20)
GDN_API int gdn_fwd_varlen_noalloc(const void* q, const void* k, const void* v, const float* g,
                                   const float* gk, const float* beta, float scale,
                                   const int* cu_seqlens, const int* cu_seqlens_host, int N,
                                   const float* h0, void* o, float* ht, void* h_chunks,
                                   void* v_new, int* chunk_offsets, int* chunk_indices,
                                   int T_total, int H, int K, int V, int dtype, void* stream);

/*
 * gdn_prep -- BiGDN front end (SANA fused_gdn.py page: _fused_qk_inv_rms_kernel,
 * prepare_rope_tables and the load path of _fused_gdn_kernel):
 *   inv_rms[b,n] = 1 / sqrt(sum_{c < H*D} x[b,n,c]^2 / (H*D) + norm_eps)   for q and for k
 *   x_hat = x * inv_rms * w[h*D + d];  q_pos = relu(q_hat);  k_pos = relu(k_hat) * k_scale
 *   x_rot[d] = x_pos[d] * cos[n,d] + x_pos[d^1] * sin[n,d]
 *
 *   qkv                [B, N, 3, H, D] bf16
 *   q_norm_w, k_norm_w [H*D] fp32
 *   rope_cos, rope_sin [N, D] fp32     expanded tables (sin[2i] = -sin, sin[2i+1] = +sin)
 *   q_inv_rms, k_inv_rms [B, N] fp32   OUT (nullable)
 *   q_rot, k_rot, q_pos, k_pos, v_hm   [B, H, N, D] bf16 OUT, head-major (each nullable)
 * Supported: D in {64, 128}, H*D <= 4096.
 */
GDN_API int gdn_prep(const void* qkv, const float* q_norm_w, const float* k_norm_w,
             const float* rope_cos, const float* rope_sin, float k_scale, float norm_eps,
             float* q_inv_rms, float* k_inv_rms, void* q_rot, void* k_rot, void* q_pos,
             void* k_pos, void* v_hm, int B, int N, int H, int D, void* stream);

/*
 * gdn_state_summary -- the state summary of one fragment of a sequence, so that the
 * fragments of a long sequence can run separately and be joined (the context-parallel GDN /
 * KDA state summary of the MindSpore hyper-parallel "Diff Coverage" page: a per-chunk
 * transition diag(decay) - K^T W composed over the fragment, plus the state reached from a
 * zero start).  Over a fragment the final state is affine in the initial state:
 *     ht(h0) = transition h0 + state_ext,
 *     state_ext  = ht with h0 = 0                                   [B,H,K,V] fp32 OUT
 *     transition = A_T ... A_1,  A_t = (I - beta_t k_t k_t^T) diag(exp(g_t + gk_t))
 *                                                                    [B,H,K,K] fp32 OUT
 *   k [B,T,H,K], v [B,T,H,V] (dtype), g [B,T,H] or NULL, gk [B,T,H,K] or NULL, beta [B,T,H]
 *   as in gdn_fwd (q is not needed).  transition may be NULL (not formed).  state_ext comes
 *   from the forward kernels.  The transition decays like the product of all the fragment's
 *   decays, so values below fp32 range become zero, as they would in any fp32 result.  With a
 *   scalar (or no) gate it is e^{sum_t g_t} times the ordered product of the ungated chunk
 *   maps I - K^T W (W = Tm diag(beta) K, the chunk's WY factor), formed on matrix cores with
 *   split bf16 operands (each fp32 value as hi + lo, about 16 mantissa bits, fp32's exponent
 *   range); with a per-key gate it is the token recurrence in fp32 with a power-of-two
 *   exponent per column.
 *   workspace  at least gdn_state_summary_workspace_bytes(B, T, H, K, V, dtype, flags)
 *              (flags = GDN_FWD_PER_KEY if gk is given)
 *              bytes, 256-byte aligned, caller-owned
 * Supported and errors: as gdn_fwd.
 */
GDN_API size_t gdn_state_summary_workspace_bytes(int B, int T, int H, int K, int V, int dtype,
                                                 unsigned flags);
GDN_API int gdn_state_summary(const void* k, const void* v, const float* g, const float* gk,
                              const float* beta, float* state_ext, float* transition, int B,
                              int T, int H, int K, int V, int dtype, void* workspace,
                              size_t workspace_bytes, void* stream);

/*
 * gdn_state_apply -- joins a fragment to the state before it: per (b, h),
 *     h_out = transition h_in + state_ext          ([K,K] x [K,V] + [K,V], fp32)
 * state_ext [BH,K,V], transition [BH,K,K], h_in [BH,K,V] (NULL = zero: h_out = state_ext),
 * h_out [BH,K,V] OUT, all fp32 device pointers; h_out must not overlap h_in.
 * Supported: K <= 256, BH <= 65535.  GDN_ERR_INVALID on null/overlapping pointers or
 * non-positive sizes.
 */
GDN_API int gdn_state_apply(const float* state_ext, const float* transition, const float* h_in,
                            float* h_out, int BH, int K, int V, void* stream);

/*
 * gdn_state_grad_summary -- the reverse (gradient) summary of one fragment, for the
 * context-parallel backward (the KDA state-gradient summary of the hyper-parallel "Diff
 * Coverage" page): the gradient of the loss with respect to the state entering the fragment,
 * counting only the fragment's own outputs (a zero gradient for the state leaving it),
 *     grad_state_ext = dh0 of gdn_bwd_dhu with dht = 0           [B,H,K,V] fp32 OUT.
 * The gradient for a nonzero gradient of the leaving state follows from gdn_state_grad_apply
 * with the fragment's forward transition.  Inputs, dtype, gates, Supported and errors as
 * gdn_bwd_dhu (q, k, w, do_, dv of the fragment alone, with its own 64-token chunk grid).
 *   workspace  at least gdn_state_grad_summary_workspace_bytes(B, T, H, V, dtype) bytes,
 *              256-byte aligned (the pass's per-token dv2, which is not returned)
 */
GDN_API size_t gdn_state_grad_summary_workspace_bytes(int B, int T, int H, int V, int dtype);
GDN_API int gdn_state_grad_summary(const void* q, const void* k, const void* w, const void* do_,
                                   const void* dv, const float* g, const float* gk, float scale,
                                   float* grad_state_ext, int B, int T, int H, int K, int V,
                                   int dtype, void* workspace, size_t workspace_bytes,
                                   void* stream);

/*
 * gdn_state_grad_apply -- joins a fragment's gradient to the gradient after it: per (b, h),
 *     grad_out = transition^T grad_in + grad_state_ext     ([K,K]^T x [K,V] + [K,V], fp32)
 * where transition is the fragment's forward transition (gdn_state_summary) and grad_in the
 * gradient of the state leaving the fragment (NULL = zero).  grad_out is the gradient of the
 * state entering it.  Layouts, Supported and errors as gdn_state_apply.
 */
GDN_API int gdn_state_grad_apply(const float* grad_state_ext, const float* transition,
                                 const float* grad_in, float* grad_out, int BH, int K, int V,
                                 void* stream);

/*
 * bigdn_fwd -- frame-level bidirectional GDN block forward (SANA fused_gdn.py page,
 * _fused_gdn_kernel run forward and REVERSE, summed as in fused_bigdn_func).  N = F * S
 * tokens form F frames of S tokens; every token of a frame reads the same decayed state.
 * Forward, per frame f: S,z *= decay[f]; S += K_rot^T (beta (V - K_rot S)),
 * z += K_pos^T (beta (1 - K_pos z)) (both from the decayed pre-update state);
 * num = Q_rot S, den = Q_pos . z.  Reverse: frame f reads the state built from frames > f
 * (flip-and-shift, SANA fused_cam_gdn.py page).  Returned: the sums of both directions.
 *
 *   qkv     [B, N, 3, H, D] bf16;  beta [B, H, F, S] fp32;  decay [B, H, F] fp32 in (0, 1]
 *   q_norm_w, k_norm_w, rope_cos, rope_sin, k_scale, norm_eps   as in gdn_prep
 *   num     [B, N, H, D] bf16 OUT;  den [B, H, N] bf16 OUT
 *   workspace  at least bigdn_fwd_workspace_bytes(B, F, S, H, D) bytes, 256-byte aligned
 * Supported: D in {64, 128}, S a multiple of 64, H*D <= 4096, F <= 65535 (GDN_ERR_UNSUPPORTED
 * otherwise).
 */
GDN_API size_t bigdn_fwd_workspace_bytes(int B, int F, int S, int H, int D);
GDN_API int bigdn_fwd(const void* qkv, const float* beta, const float* decay, const float* q_norm_w,
              const float* k_norm_w, const float* rope_cos, const float* rope_sin,
              float k_scale, float norm_eps, void* num, void* den, int B, int F, int S, int H,
              int D, void* workspace, size_t workspace_bytes, void* stream);

/*
 * bigdn_fwd_merged -- bigdn_fwd with the options of the [SANA fused_gdn.py page]
 * block wrapper (fused_bigdn_func and fused_bidi_merge):
 *   - chunk-causal overrides of the REVERSE direction, each NULL = the forward one:
 *     qkv_bwd [B,N,3,H,D] bf16 (its own q, k, v; the inverse RMS of its q and k is computed
 *     from it), beta_bwd [B,H,F,S] and decay_bwd [B,H,F] fp32.  A zero decay_bwd at frame f
 *     resets the reverse state when frame f is absorbed, so frames before f see no frame
 *     after f; zeroed k or v (qkv_bwd) or beta_bwd at a frame keep that frame out of it.
 *     With qkv_bwd the outputs sum Q_fwd S_f + Q_bwd R_f and q_fwd z_f + q_bwd zR_f.
 *   - the bidirectional merge epilogue, fused into the output kernel:
 *       out = (num_fwd + num_bwd) / (den_fwd + den_bwd + merge_eps) * SiLU(gate)
 *     out [B,N,H,D] bf16 OUT; gate [B,N,H,D] bf16 or NULL (no gate); the division uses the
 *     fp32 sums before they are rounded.
 *   num [B,N,H,D], den [B,H,N] bf16 OUT as in bigdn_fwd; either may be NULL when out is set.
 *   workspace  at least bigdn_fwd_merged_workspace_bytes(B, F, S, H, D, has_rev_inputs),
 *              has_rev_inputs = (qkv_bwd != NULL || beta_bwd != NULL)
 * Errors as bigdn_fwd; GDN_ERR_INVALID also when out and num/den are all NULL, when gate is
 * given without out, or merge_eps < 0.
 */
GDN_API size_t bigdn_fwd_merged_workspace_bytes(int B, int F, int S, int H, int D,
                                                int has_rev_inputs);
GDN_API int bigdn_fwd_merged(const void* qkv, const void* qkv_bwd, const float* beta,
                             const float* decay,
                             const float* beta_bwd, const float* decay_bwd,
                             const float* q_norm_w, const float* k_norm_w,
                             const float* rope_cos, const float* rope_sin, float k_scale,
                             float norm_eps, const void* gate, float merge_eps, void* out,
                             void* num, void* den, int B, int F, int S, int H, int D,
                             void* workspace, size_t workspace_bytes, void* stream);

/*
 * cam_prep -- camera-branch prep of the SANA video block ([SANA fused_cam_gdn.py page],
 * _cam_prep_kernel and cam_prep_func), per token n and head h:
 *   q_n = relu(q * inv_rms_q * q_norm_w),  k_n = relu(k * inv_rms_k * k_norm_w) * k_scale,
 *   v_n = v, with inv_rms = 1/sqrt(mean over all H*D channels of the token of x^2 + norm_eps);
 *   channels [0, D/2): groups of four mixed by the token's camera matrix,
 *     y[4g+i] = sum_j P[i][j] x[4g+j]  (P = proj_q for q, proj_kv for k and v);
 *   channels [D/2, D): interleaved-pair RoPE, y[D/2+r] = x[D/2+r] cos[n,r] + x[D/2+(r^1)] sin[n,r];
 *   inflation = max(|k_out|^2, 1e-12) / max(|k_n|^2, 1e-12).
 *   q, k, v            [B,N,H,D] fp32 IN (device)
 *   q_norm_w, k_norm_w [H*D] fp32 IN
 *   proj_q, proj_kv    [B,N,4,4] fp32 IN (row i, column j)
 *   rope_cos, rope_sin [N,D/2] fp32 IN: expanded interleaved-pair tables (sin[n,2i] = -sin,
 *                      sin[n,2i+1] = +sin of the pair's angle)
 *   q_out, k_out, v_out [B,H,D,N] fp32 OUT (channel-major); inflation [B,H,N] fp32 OUT
 *   workspace          at least cam_prep_workspace_bytes(B, N), 256-byte aligned (inverse RMS)
 * Supported: D in {64, 128}, N a multiple of 4 (GDN_ERR_UNSUPPORTED otherwise).
 * GDN_ERR_INVALID for null pointers, non-positive sizes, norm_eps <= 0.
 */
GDN_API size_t cam_prep_workspace_bytes(int B, int N);
GDN_API int cam_prep(const float* q, const float* k, const float* v, const float* q_norm_w,
                     const float* k_norm_w, const float* proj_q, const float* proj_kv,
                     const float* rope_cos, const float* rope_sin, float k_scale, float norm_eps,
                     float* q_out, float* k_out, float* v_out, float* inflation, int B, int N,
                     int H, int D, void* workspace, size_t workspace_bytes, void* stream);

/*
 * cam_scan -- camera-branch numerator-only frame scan ([SANA fused_cam_gdn.py page],
 * _cam_scan_kernel and cam_scan_func).  Per (b, h), state St [D_k rows, D_v columns]:
 *   forward: for each frame f: St *= decay[f]; St += K_f diag(beta_f) (V_f - K_f^T St)^T with
 *            every token of the frame predicting from the same decayed St; the frame's
 *            outputs are out[:, n] = St^T q_n (after the update).
 *   reverse: frame f reads the state built from the frames after it (zero for the last);
 *            absorbing frame f+1 first multiplies the state by decay[f+1].
 *   q, k, v     [B,H,D,N] fp32 IN (channel-major, N = F*S); beta [B,H,F,S], decay [B,H,F] fp32 IN
 *   init_state  [B*H,D,D] fp32 IN or NULL: state at the end of a prefix (decayed by decay[0]
 *               at the first frame); forward only
 *   final_state [B*H,D,D] fp32 OUT or NULL: St after the last frame; forward only
 *   out         [B,H,D,N] fp32 OUT
 *   workspace   at least cam_scan_workspace_bytes(B, H, D, F), 256-byte aligned
 * Products use fp16 operands with fp32 accumulation (the page's scan uses TF32 dots) and the
 * state is kept in fp32; operands must lie within fp16 range (the prep's outputs do).
 * Supported: D in {64, 128}, S a multiple of 64, F <= 65535 (GDN_ERR_UNSUPPORTED otherwise);
 * GDN_ERR_UNSUPPORTED also for reverse != 0 with init_state or final_state (the page raises
 * NotImplementedError there).  GDN_ERR_INVALID for null pointers or non-positive sizes.
 */
GDN_API size_t cam_scan_workspace_bytes(int B, int H, int D, int F);
GDN_API int cam_scan(const float* q, const float* k, const float* v, const float* beta,
                     const float* decay, int reverse, const float* init_state, float* final_state,
                     float* out, int B, int H, int D, int F, int S, void* workspace,
                     size_t workspace_bytes, void* stream);

/*
 * cam_scan_bidi -- both directions of cam_scan over the same q, k, v and beta in one call:
 * out_fwd is cam_scan(reverse=0) (with init_state / final_state as there) and out_rev is
 * cam_scan(reverse=1), the reverse direction using decay_bwd [B,H,F] when it is non-NULL
 * (chunk-causal resets: a zero at frame f+1 cuts frames > f off from frame f) and decay
 * otherwise.  The frame statistics are computed once, the two scans run concurrently and
 * one read of q serves both outputs.
 *   out_fwd, out_rev  [B,H,D,N] fp32 OUT
 *   workspace         at least cam_scan_bidi_workspace_bytes(B, H, D, F), 256-byte aligned
 * Errors as cam_scan (GDN_ERR_INVALID also for a null out_rev).
 */
GDN_API size_t cam_scan_bidi_workspace_bytes(int B, int H, int D, int F);
GDN_API int cam_scan_bidi(const float* q, const float* k, const float* v, const float* beta,
                          const float* decay, const float* decay_bwd, const float* init_state,
                          float* final_state, float* out_fwd, float* out_rev, int B, int H,
                          int D, int F, int S, void* workspace, size_t workspace_bytes,
                          void* stream);

/*
 * cam_scan_bwd -- backward of cam_scan (one direction, no initial or final state): the
 * gradients of L = sum(out * dout) for out = cam_scan(q, k, v, beta, decay, reverse)
 * (SANA fused_cam_gdn.py page, "Backward Triton kernel": _cam_scan_bwd_kernel, and its
 * per-iteration derivation).  The forward states are recomputed here, so the call needs only
 * the forward's inputs.  reverse | GDN_BWD_ACCUMULATE adds this direction's dbeta and ddecay
 * to the arrays' contents instead of writing them (both directions of cam_scan_bidi share beta
 * and, unless decay_bwd is given, decay); dq, dk, dv are always written.  The per-frame
 * statistics K diag(beta) K^T and K diag(beta) V^T do not depend on the direction:
 * reverse | GDN_BWD_REUSE_STATS takes them from the workspace, where a previous call with the
 * same q, k, v, beta, B, H, D, F, S (the other direction's) left them, and forms only
 * Q dout^T (the caller guarantees the match; nothing checks it).
 *   q, k, v, dout [B,H,D,N] fp32 channel-major, N = F*S; beta [B,H,F,S]; decay [B,H,F]
 *   dq, dk, dv    [B,H,D,N] fp32 OUT;  dbeta [B,H,F,S] fp32 OUT;  ddecay [B,H,F] fp32 OUT
 *   Tokens never absorbed (frame 0 of the reverse scan) get zero dk, dv, dbeta; a decay that
 *   is never applied, or that multiplies the zero initial state, gets ddecay = 0.
 *   Precision: every product splits each fp32 operand x into bf16 hi = bf16(x) and
 *   lo = bf16(x - hi) and sums hi*hi + hi*lo + lo*hi with fp32 accumulation (about 16
 *   mantissa bits per operand; the page's backward takes plain bf16 operands, whose
 *   rounding alone moves the gradients by up to 4e-2 of their RMS); the recomputed forward
 *   states and their gradients are scanned in fp32.
 *   workspace  at least cam_scan_bwd_workspace_bytes(B, H, D, F) bytes, 256-byte aligned
 *   (per (b, h, frame) three D x D fp32 statistics, the fp32 state, and hi/lo bf16 pairs of
 *   the state and its gradient in both orientations).
 * Supported: D in {64, 128}, S a multiple of 64.
 */
GDN_API size_t cam_scan_bwd_workspace_bytes(int B, int H, int D, int F);
GDN_API int cam_scan_bwd(const float* q, const float* k, const float* v, const float* beta,
                         const float* decay, const float* dout, int reverse, float* dq,
                         float* dk, float* dv, float* dbeta, float* ddecay, int B, int H, int D,
                         int F, int S, void* workspace, size_t workspace_bytes, void* stream);

/*
 * bigdn_dir_bwd -- backward of one BiGDN direction (SANA fused_gdn.py page, "Backward /
 * autograd Functions": the reverse replay of the frame recurrence behind
 * FusedBiGDNFunction.backward): gradients of L = sum(num * dnum) + sum(den * dden) for the
 * num, den of one direction of bigdn_fwd on the prepped tensors (reverse = 0 forward, 1
 * reverse; the block's outputs sum both directions, so the caller runs both and adds).
 * reverse | GDN_BWD_ACCUMULATE adds this direction's dbeta and ddecay to the arrays' contents
 * instead of writing them (the two directions share beta and decay unless the reverse one is
 * overridden); the token gradients are always written (gdn_prep_bwd sums directions).
 * reverse | GDN_BWD_REUSE_STATS skips the per-frame statistics (they do not depend on the
 * direction): the workspace must hold those of a previous call with the same prepped tensors,
 * beta, dnum, dden and sizes (the other direction's; the caller guarantees the match).
 * With S, z the states and A, a their gradients after a step's update (S_pre = g S_prev,
 * z_pre = g z_prev for the frame the step absorbs), per token:
 *   output frame:   dq_rot = S dnum,  dq_pos = dden z
 *   absorbed frame: dv = beta A^T k_rot,  dk_rot = A (beta r) - beta S_pre (A^T k_rot),
 *                   r = v - S_pre^T k_rot;  dk_pos = a (beta e) - beta (a . k_pos) z_pre,
 *                   e = 1 - k_pos . z_pre;  dbeta = (A^T k_rot) . r + (a . k_pos) e
 *   ddecay[f] = <dS_pre, S_prev> + <dz_pre, z_prev> for the frame f absorbed with decay[f].
 * Frames a direction never absorbs (frame 0 of the reverse one) get zero k, v, beta
 * gradients; the decay applied to the zero initial state gets 0.
 *   q_rot, k_rot, q_pos, k_pos, v   [B,H,N,D] bf16 IN (as gdn_prep writes them), N = F * S
 *   beta [B,H,F,S], decay [B,H,F] fp32 IN; dnum [B,N,H,D], dden [B,H,N] fp32 IN
 *   dq_rot, dk_rot, dq_pos, dk_pos, dv [B,H,N,D], dbeta [B,H,F,S], ddecay [B,H,F] fp32 OUT
 *   Products take split bf16 operands (as cam_scan_bwd); the z stream is fp32 arithmetic.
 *   workspace  at least bigdn_dir_bwd_workspace_bytes(B, H, D, F) bytes, 256-byte aligned
 *   (per (b, h, frame) the D x D statistics and saved states of the S stream, G_pos and the
 *   z stream's vectors).
 * Supported: D in {64, 128}, S a multiple of 64.
 */
GDN_API size_t bigdn_dir_bwd_workspace_bytes(int B, int H, int D, int F);
GDN_API int bigdn_dir_bwd(const void* q_rot, const void* k_rot, const void* q_pos,
                          const void* k_pos, const void* v, const float* beta,
                          const float* decay, const float* dnum, const float* dden, int reverse,
                          float* dq_rot, float* dk_rot, float* dq_pos, float* dk_pos, float* dv,
                          float* dbeta, float* ddecay, int B, int H, int D, int F, int S,
                          void* workspace, size_t workspace_bytes, void* stream);

/*
 * bigdn_merge_bwd -- backward of the BiGDN block's merge (SANA fused_gdn.py page: the dnum and
 * dden that FusedBiGDNFunction.backward forms from the upstream gradient, with the SiLU gate of
 * fused_bidi_merge):
 *   out   = num / (den + merge_eps) * silu(gate)       (silu = 1 when gate is NULL)
 *   dnum  = dout silu(gate) / (den + merge_eps)
 *   dden  = -sum_d dout silu(gate) num / (den + merge_eps)^2
 *   dgate = dout num / (den + merge_eps) * s (1 + gate (1 - s)),  s = sigmoid(gate)
 *   num [B,N,H,D], den [B,H,N] bf16 IN (the sums over both directions, as bigdn_fwd /
 *   bigdn_fwd_merged store them); gate [B,N,H,D] bf16 IN or NULL; dout [B,N,H,D] fp32 IN;
 *   dnum [B,N,H,D], dden [B,H,N] fp32 OUT (the inputs of bigdn_dir_bwd for either direction);
 *   dgate [B,N,H,D] fp32 OUT, given exactly when gate is.
 * Supported: D in {64, 128}, H*D <= 4096.  GDN_ERR_INVALID when merge_eps < 0 or when only one
 * of gate and dgate is given.
 */
GDN_API int bigdn_merge_bwd(const void* num, const void* den, const void* gate, const float* dout,
                            float merge_eps, float* dnum, float* dden, float* dgate, int B, int N,
                            int H, int D, void* stream);

/*
 * gdn_prep_bwd -- backward of gdn_prep (SANA fused_gdn.py page, "Backward / autograd
 * Functions": the RoPE inverse, ReLU and k-scale backward of _fused_gdn_bwd_kernel and the
 * full-channel RMSNorm backward of FusedBiGDNFunction.backward).  The gradients of the
 * prepped tensors from ndir scan directions (each tensor [ndir,B,H,N,D], the directions
 * summed; bigdn_dir_bwd writes one direction's slice) are taken back to qkv and the norm
 * weights.  Per token, C = H*D, r the inverse RMS, x_hat = x r w:
 *   g_pos[d] = dpos[d] + drot[d] cos[n,d] + drot[d^1] sin[n,d^1]
 *   g        = g_pos (times k_scale for k) where x_hat > 0, else 0
 *   dx[c]    = r w[c] g[c] - r^3 / C x[c] sum_c' w[c'] g[c'] x[c'],   dv passes through
 *   dw[c]    = sum over all tokens of g[c] x[c] r
 *   qkv [B,N,3,H,D] bf16, q_norm_w, k_norm_w [H*D], rope_cos, rope_sin [N,D] fp32 IN (as given
 *   to gdn_prep); dq_rot, dk_rot, dq_pos, dk_pos, dv [ndir,B,H,N,D] fp32 IN, ndir in {1, 2};
 *   dqkv [B,N,3,H,D], dq_norm_w, dk_norm_w [H*D] fp32 OUT.
 *   workspace  at least gdn_prep_bwd_workspace_bytes(B, N, H, D) bytes, 256-byte aligned (the
 *   weight gradients' per-workgroup partial sums, added in a fixed order).
 * Supported: D in {64, 128}, H*D <= 4096.  GDN_ERR_INVALID for ndir outside {1, 2} or
 * norm_eps <= 0.
 */
GDN_API size_t gdn_prep_bwd_workspace_bytes(int B, int N, int H, int D);
GDN_API int gdn_prep_bwd(const void* qkv, const float* q_norm_w, const float* k_norm_w,
                         const float* rope_cos, const float* rope_sin, float k_scale,
                         float norm_eps, int ndir, const float* dq_rot, const float* dk_rot,
                         const float* dq_pos, const float* dk_pos, const float* dv, float* dqkv,
                         float* dq_norm_w, float* dk_norm_w, int B, int N, int H, int D,
                         void* workspace, size_t workspace_bytes, void* stream);

/*
 * cam_prep_bwd -- backward of cam_prep (SANA fused_cam_gdn.py page: _cam_prep_bwd_kernel and
 * _cam_prep_bwd_dispatch): the gradients of q, k, v and of the two norm weights from those of
 * cam_prep's outputs q_t, k_t, v_t (each [ndir,B,H,D,N], the directions summed, so the two
 * directions' cam_scan_bwd results go in unchanged) and, optionally, of the inflation.  With
 * x_n = relu(x r w) (times k_scale for k; v is not normed), y = T x_n the output (T the token's
 * 4x4 camera matrix on each group of four of channels [0, D/2), RoPE on [D/2, D)), pre =
 * |x_n,k|^2, post = |y_k|^2 per (b, h, n):
 *   d_post = dinfl [post >= 1e-12] / max(pre, 1e-12)
 *   d_pre  = -dinfl max(post, 1e-12) / max(pre, 1e-12)^2 [pre >= 1e-12]
 *   dx_n   = T^T (dy + 2 y d_post) (+ 2 x_n d_pre for k);  dv = T^T dy_v
 *   T^T:  dx_n[4g + j] = sum_i P[i][j] dy[4g + i],
 *         dx_n[D/2 + r] = dy[D/2 + r] cos[n,r] + dy[D/2 + (r^1)] sin[n,r^1]
 *   g      = dx_n (times k_scale for k) where x w > 0, else 0
 *   dx[c]  = r w[c] g[c] - r^3 / C x[c] sum_c' w[c'] g[c'] x[c'],  C = H*D
 *   dw[c]  = sum over all tokens of g[c] x[c] r
 *   q, k [B,N,H,D], q_norm_w, k_norm_w [H*D], proj_q, proj_kv [B,N,4,4], rope_cos, rope_sin
 *   [N,D/2] fp32 IN (as given to cam_prep); dq_t, dk_t, dv_t [ndir,B,H,D,N] fp32 IN, ndir in
 *   {1, 2}; dinfl [B,H,N] fp32 IN or NULL (no inflation gradient);
 *   dq, dk, dv [B,N,H,D], dq_norm_w, dk_norm_w [H*D] fp32 OUT.  Tensors 16-byte aligned.
 *   workspace  at least cam_prep_bwd_workspace_bytes(B, N, H, D) bytes, 256-byte aligned (k's
 *   inverse RMS and the weight gradients' per-workgroup partial sums, added in a fixed order).
 * Supported: D in {64, 128}, H*D <= 4096, N a multiple of 4.  GDN_ERR_INVALID for ndir outside
 * {1, 2} or norm_eps <= 0.
 */
GDN_API size_t cam_prep_bwd_workspace_bytes(int B, int N, int H, int D);
GDN_API int cam_prep_bwd(const float* q, const float* k, const float* q_norm_w,
                         const float* k_norm_w, const float* proj_q, const float* proj_kv,
                         const float* rope_cos, const float* rope_sin, float k_scale,
                         float norm_eps, int ndir, const float* dq_t, const float* dk_t,
                         const float* dv_t, const float* dinfl, float* dq, float* dk, float* dv,
                         float* dq_norm_w, float* dk_norm_w, int B, int N, int H, int D,
                         void* workspace, size_t workspace_bytes, void* stream);

/*
 * gdn_bwd_prep -- the inputs of the state-gradient pass, from the forward's inputs
 * ([hyper-parallel "Diff Coverage" page]: the chunk state pass v_new = u - w h and its dhu
 * backward).  Per 64-token chunk, gamma the chunk-local inclusive cumsum of g:
 *     A_{r,s} = beta_r e^{gamma_r - gamma_s} (k_r . k_s)   (s < r)
 *     w       = (I + A)^-1 diag(beta e^gamma) K                      [B,T,H,K] OUT (dtype)
 *     P_{r,s} = scale e^{gamma_r - gamma_s} (q_r . k_s)    (s <= r)
 *     dv      = P^T do                                               [B,T,H,V] OUT (dtype)
 *   q, k [B,T,H,K], do_ [B,T,H,V] (dtype); beta, g [B,T,H] fp32 (g NULL: no decay); gk must
 *   be NULL.  Products take split bf16 operands with fp32 accumulation, so the results are
 *   near fp32 before they are stored in dtype.
 * Supported: K, V in {64, 128}; scalar gates (GDN_ERR_UNSUPPORTED for gk).
 */
GDN_API int gdn_bwd_prep(const void* q, const void* k, const float* beta, const float* g,
                         const float* gk, const void* do_, float scale, void* w, void* dv, int B,
                         int T, int H, int K, int V, int dtype, void* stream);

/*
 * gdn_bwd_dhu -- state-gradient pass of the chunked backward ([hyper-parallel "Diff Coverage"
 * page], the dhu fragments): the adjoint of the chunk state pass of gdn_fwd, over 64-token
 * chunks in reverse.  With dh the gradient of the state leaving chunk n (dht, or 0, after
 * the last chunk), gamma the chunk-local inclusive cumsum of g and gamma_L its value at the
 * chunk's last token:
 *     dv2_t = dv_t + e^{gamma_L - gamma_t} (dh^T k_t)
 *     dh    = e^{gamma_L} dh + scale sum_t e^{gamma_t} q_t do_t^T - sum_t w_t dv2_t^T
 *     dh_chunks[n] = dh   (the gradient of h[n], the state entering chunk n, as gdn_fwd saves it)
 * and dh0 = dh after chunk 0.
 *   q, k, w   [B,T,H,K] IN; w is the forward's WY w (v_new = u - w h)
 *   do_, dv   [B,T,H,V] IN: the output gradient, and the intra-chunk gradient of v_new (P^T do)
 *   g         [B,T,H] fp32 IN per-token log gates, or NULL (no decay)
 *   gk        [B,T,H,K] fp32 IN per-key log gates, or NULL; bf16 inputs only (the chunk-local
 *             cumsum is of g_t + gk_{t,d}: dv2 takes e^{gamma_L,d - gamma_{t,d}} inside the sum
 *             over keys, dh's row d decays by e^{gamma_L,d}, q_t is scaled per key)
 *   dht       [B,H,K,V] fp32 IN or NULL (zero)
 *   dh_chunks [B,H,NT,K,V] fp32 OUT or NULL (NT = ceil(T/64)); dv2 [B,T,H,V] OUT (dtype);
 *   dh0       [B,H,K,V] fp32 OUT or NULL
 *   dtype     GDN_DTYPE_F32 or GDN_DTYPE_BF16 for q, k, w, do_, dv and dv2.  fp32: fp32
 *             arithmetic.  bf16: fp16 matrix-core operands (dh and dv2 rounded to fp16 where
 *             they enter a product) with fp32 accumulation and an fp32 dh
 * Supported: K = 128, V a multiple of 32, gk only with bf16 (GDN_ERR_UNSUPPORTED otherwise).
 * GDN_ERR_INVALID for null required pointers, non-positive sizes or an unknown dtype.
 */
GDN_API int gdn_bwd_dhu(const void* q, const void* k, const void* w, const void* do_,
                        const void* dv, const float* g, const float* gk, const float* dht,
                        float scale,
                        float* dh_chunks, void* dv2, float* dh0, int B, int T, int H, int K,
                        int V, int dtype, void* stream);

/*
 * gdn_bwd_dhu_varlen -- gdn_bwd_dhu over packed sequences (the layout of gdn_fwd_varlen):
 * every (sequence, head) is its own chain, with chunks restarting at each sequence start.
 *   q, k, w [1,T_total,H,K]; do_, dv, dv2 [1,T_total,H,V]; g [1,T_total,H] or NULL;
 *   gk [1,T_total,H,K] or NULL
 *   cu_seqlens [N+1] int32 on the device and cu_seqlens_host, the same offsets on the host
 *   dht, dh0 [N,H,K,V] fp32 (nullable); dh_chunks [1,H,NT_total,K,V] fp32 (nullable), chunk
 *   c = chunk_offsets[i] + n of sequence i as in gdn_fwd_varlen (NT_total = gdn_varlen_num_chunks)
 *   workspace  at least gdn_bwd_dhu_varlen_workspace_bytes(N, NT_total), 256-byte aligned
 *              (the chunk tables, built on the device)
 * Errors as gdn_bwd_dhu and gdn_fwd_varlen (malformed cu_seqlens: GDN_ERR_INVALID).
 */
GDN_API size_t gdn_bwd_dhu_varlen_workspace_bytes(int N, int NT_total);
GDN_API int gdn_bwd_dhu_varlen(const void* q, const void* k, const void* w, const void* do_,
                               const void* dv, const float* g, const float* gk,
                               const float* dht, float scale, const int* cu_seqlens, const int* cu_seqlens_host, int N,
                               float* dh_chunks, void* dv2, float* dh0, int T_total, int H,
                               int K, int V, int dtype, void* workspace, size_t workspace_bytes,
                               void* stream);

#ifdef __cplusplus
}
#endif

#endif /* GDN_H_ */

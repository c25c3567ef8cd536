/*
 * gdn_oracle.c -- plain fp64 CPU oracle for the gated delta rule (TEST INFRASTRUCTURE ONLY).
 *
 * This file is the correctness reference for the HIP library.  Only the test suite, the
 * smoke check and the CPU-baseline leg of the benchmark may load it.  It shares no code,
 * header, table or helper with the GPU path, and nothing in the GPU path calls it.
 *
 * Everything here is the plain definition of the method, written token by token in double
 * precision, with no blocking, fusion or reordering beyond what the definition states.  The
 * only parallelism is an OpenMP loop over chains that are independent by definition
 * (distinct (batch, head) pairs, distinct packed sequences, the two BiGDN directions).
 *
 * Sources (pages, as named by their addresses):
 *  - chunk_gated_delta_rule_fwd_h fragments on the hyper-parallel "Diff Coverage" page
 *    (MindSpore): the per-chunk state pass (decay by the last gate, optional per-key gate
 *    row-scaling of the state, v_new = u - w h), the varlen offsets (bos, chunk tables),
 *    and the [B, H, K, V] fp32 state layout.
 *  - SANA fused_gdn.py page, section "Unified forward Triton Mega-Kernel"
 *    (_fused_gdn_kernel): full-channel RMSNorm, ReLU, k-scale, interleaved-pair RoPE,
 *    the frame-level update (all tokens of a frame read the decayed pre-update state),
 *    the z normaliser, inclusive outputs, and the reverse direction's frame indexing.
 *  - SANA fused_gdn.py page, prepare_rope_tables / _precompute_inv_rms: the expanded
 *    (N, D) cos/sin table format and the full-channel inverse RMS with eps.
 *  - SANA fused_cam_gdn.py page, "Torch reference implementations" section
 *    (_flip_and_shift, _torch_cam_scan_reference): reverse = flip-and-shift.
 *
 * Readings where the pages are silent (each is listed in the design notes):
 *  - gates are natural-log: the decay factor of token t on key row d is
 *    exp(g_t + gk_{t,d}) (a missing g or gk contributes 0);
 *  - h_chunks[n] is the state entering chunk n, i.e. before token n*C's decay;
 *  - v_new_t = beta_t (v_t - S'^T k_t) with S' the decayed state (the delta itself);
 *  - the initial state h0 is the state at the end of a prefix, before any further decay.
 */
#include <math.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

int oracle_abi_version(void) { return 1; }

int oracle_max_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}

void oracle_set_threads(int n) {
#ifdef _OPENMP
  if (n > 0) omp_set_num_threads(n);
#else
  (void)n;
#endif
}

/*
 * One chain of the token recurrence (the definition given with the method):
 *     S_t = diag(a_t) S_{t-1} + k_t d_t^T,   d_t = beta_t (v_t - (diag(a_t) S_{t-1})^T k_t),
 *     o_t = scale * S_t^T q_t,               a_{t,d} = exp(g_t + gk_{t,d}).
 * S is K x V with the key dimension as rows.  Pointers address token 0 of this chain; the
 * token strides say how far apart consecutive tokens are (in elements).
 *   q, k  : K values per token, stride sqk     g    : 1 value per token, stride sg
 *   v     : V values per token, stride sv      gk   : K values per token, stride sqk
 *   beta  : 1 value per token, stride sg       o,vnew: V values per token, stride sv
 *   h0/ht : K*V (row-major), may be NULL       hch  : NT*K*V states entering each chunk
 * S is a caller-provided K*V work array.
 */
static void gdn_chain(int T, int K, int V, int C,
                      const double* q, const double* k, const double* v, long sqk, long sv,
                      const double* g, const double* gk, const double* beta, long sg,
                      double scale, const double* h0, double* o, double* ht, double* hch,
                      double* vnew, double* S, double* a, double* d) {
  if (h0) memcpy(S, h0, sizeof(double) * (size_t)K * V);
  else memset(S, 0, sizeof(double) * (size_t)K * V);
  for (int t = 0; t < T; ++t) {
    const double* qt = q + (long)t * sqk;
    const double* kt = k + (long)t * sqk;
    const double* vt = v + (long)t * sv;
    const double bt = beta[(long)t * sg];
    if (hch && (t % C) == 0)  /* state entering chunk t/C, before this token's decay */
      memcpy(hch + (size_t)(t / C) * K * V, S, sizeof(double) * (size_t)K * V);
    /* decay: S <- diag(a_t) S */
    for (int r = 0; r < K; ++r) {
      double lam = 0.0;
      if (g) lam += g[(long)t * sg];
      if (gk) lam += gk[(long)t * sqk + r];
      a[r] = exp(lam);
    }
    for (int r = 0; r < K; ++r)
      for (int c = 0; c < V; ++c) S[(size_t)r * V + c] *= a[r];
    /* delta: d = beta (v - S^T k) */
    for (int c = 0; c < V; ++c) d[c] = 0.0;
    for (int r = 0; r < K; ++r)
      for (int c = 0; c < V; ++c) d[c] += S[(size_t)r * V + c] * kt[r];
    for (int c = 0; c < V; ++c) d[c] = bt * (vt[c] - d[c]);
    /* rank-one write: S <- S + k d^T */
    for (int r = 0; r < K; ++r)
      for (int c = 0; c < V; ++c) S[(size_t)r * V + c] += kt[r] * d[c];
    /* inclusive output o_t = scale S_t^T q_t */
    double* ot = o + (long)t * sv;
    for (int c = 0; c < V; ++c) ot[c] = 0.0;
    for (int r = 0; r < K; ++r)
      for (int c = 0; c < V; ++c) ot[c] += S[(size_t)r * V + c] * qt[r];
    for (int c = 0; c < V; ++c) ot[c] *= scale;
    if (vnew)
      for (int c = 0; c < V; ++c) vnew[(long)t * sv + c] = d[c];
  }
  if (ht) memcpy(ht, S, sizeof(double) * (size_t)K * V);
}

/*
 * Dense batch: q,k [B,T,H,K], v [B,T,H,V], g,beta [B,T,H], gk [B,T,H,K], h0/ht [B,H,K,V],
 * o/vnew [B,T,H,V], hch [B,H,NT,K,V] with NT = ceil(T/C).  g, gk, h0, ht, hch, vnew may be
 * NULL.  Returns 0, or -1 on bad sizes.
 */
int oracle_gdn(int B, int T, int H, int K, int V, int C,
               const double* q, const double* k, const double* v, const double* g,
               const double* gk, const double* beta, double scale, const double* h0,
               double* o, double* ht, double* hch, double* vnew) {
  if (B <= 0 || T <= 0 || H <= 0 || K <= 0 || V <= 0 || C <= 0) return -1;
  const int NT = (T + C - 1) / C;
  int fail = 0;
#pragma omp parallel
  {
    double* S = (double*)malloc(sizeof(double) * (size_t)K * V);
    double* a = (double*)malloc(sizeof(double) * (size_t)K);
    double* d = (double*)malloc(sizeof(double) * (size_t)V);
    if (!S || !a || !d) {
#pragma omp atomic write
      fail = 1;
    } else {
#pragma omp for schedule(dynamic, 1)
      for (int bh = 0; bh < B * H; ++bh) {
        const int b = bh / H, h = bh % H;
        const long tok0 = (long)b * T * H + h;
        gdn_chain(T, K, V, C, q + tok0 * K, k + tok0 * K, v + tok0 * V, (long)H * K,
                  (long)H * V, g ? g + tok0 : NULL, gk ? gk + tok0 * K : NULL, beta + tok0,
                  (long)H, scale, h0 ? h0 + (size_t)bh * K * V : NULL, o + tok0 * V,
                  ht ? ht + (size_t)bh * K * V : NULL,
                  hch ? hch + (size_t)bh * NT * K * V : NULL, vnew ? vnew + tok0 * V : NULL,
                  S, a, d);
      }
    }
    free(S);
    free(a);
    free(d);
  }
  return fail ? -1 : 0;
}

/*
 * Transition of one chain: the linear part of the map h0 -> ht of the recurrence above.
 * Each token applies S <- A_t S + beta_t k_t v_t^T with
 *     A_t = (I - beta_t k_t k_t^T) diag(a_t),
 * so ht(h0) = M h0 + ht(0) with M = A_T ... A_1 (K x K).  M is formed by running the same
 * token steps on a K x K state that starts as the identity and has no value term.
 *   k, gk : K values per token, stride sk     g, beta : 1 value per token, stride sg
 * M is K*K row-major; a, w are K-element work arrays.
 */
static void transition_chain(int T, int K, const double* k, long sk, const double* g,
                             const double* gk, const double* beta, long sg, double* M,
                             double* a, double* w) {
  for (int r = 0; r < K; ++r)
    for (int c = 0; c < K; ++c) M[(size_t)r * K + c] = (r == c) ? 1.0 : 0.0;
  for (int t = 0; t < T; ++t) {
    const double* kt = k + (long)t * sk;
    const double bt = beta[(long)t * sg];
    for (int r = 0; r < K; ++r) {
      double lam = 0.0;
      if (g) lam += g[(long)t * sg];
      if (gk) lam += gk[(long)t * sk + r];
      a[r] = exp(lam);
    }
    /* M <- diag(a_t) M */
    for (int r = 0; r < K; ++r)
      for (int c = 0; c < K; ++c) M[(size_t)r * K + c] *= a[r];
    /* M <- M - beta k (k^T M) */
    for (int c = 0; c < K; ++c) w[c] = 0.0;
    for (int r = 0; r < K; ++r)
      for (int c = 0; c < K; ++c) w[c] += kt[r] * M[(size_t)r * K + c];
    for (int r = 0; r < K; ++r)
      for (int c = 0; c < K; ++c) M[(size_t)r * K + c] -= bt * kt[r] * w[c];
  }
}

/*
 * Dense batch transitions: k [B,T,H,K], g, beta [B,T,H], gk [B,T,H,K] (g, gk may be NULL)
 * -> M [B,H,K,K].  Returns 0, or -1 on bad sizes.
 */
int oracle_gdn_transition(int B, int T, int H, int K, const double* k, const double* g,
                          const double* gk, const double* beta, double* M) {
  if (B <= 0 || T <= 0 || H <= 0 || K <= 0) return -1;
  int fail = 0;
#pragma omp parallel
  {
    double* a = (double*)malloc(sizeof(double) * (size_t)K);
    double* w = (double*)malloc(sizeof(double) * (size_t)K);
    if (!a || !w) {
#pragma omp atomic write
      fail = 1;
    } else {
#pragma omp for schedule(dynamic, 1)
      for (int bh = 0; bh < B * H; ++bh) {
        const int b = bh / H, h = bh % H;
        const long tok0 = (long)b * T * H + h;
        transition_chain(T, K, k + tok0 * K, (long)H * K, g ? g + tok0 : NULL,
                         gk ? gk + tok0 * K : NULL, beta + tok0, (long)H,
                         M + (size_t)bh * K * K, a, w);
      }
    }
    free(a);
    free(w);
  }
  return fail ? -1 : 0;
}

/*
 * Varlen chunk tables (the chunk_indices / chunk_offsets the state-pass fragments index
 * with): chunk_offsets[i] = number of chunks in sequences before i, so it has N+1 entries;
 * chunk_indices holds one (sequence, chunk-within-sequence) pair per chunk, in order.
 * Returns the total number of chunks, or -1 if cu is malformed (cu[0] != 0 or a sequence
 * is empty).  Either output may be NULL.
 */
int oracle_varlen_tables(const int* cu, int N, int C, int* chunk_offsets, int* chunk_indices) {
  if (N <= 0 || C <= 0 || cu[0] != 0) return -1;
  int total = 0;
  for (int i = 0; i < N; ++i) {
    const int len = cu[i + 1] - cu[i];
    if (len <= 0) return -1;
    if (chunk_offsets) chunk_offsets[i] = total;
    const int nc = (len + C - 1) / C;
    for (int c = 0; c < nc; ++c) {
      if (chunk_indices) {
        chunk_indices[2 * (total + c)] = i;
        chunk_indices[2 * (total + c) + 1] = c;
      }
    }
    total += nc;
  }
  if (chunk_offsets) chunk_offsets[N] = total;
  return total;
}

/*
 * Packed variable-length batch (batch 1): tensors are [1, T_total, H, .]; sequence i covers
 * tokens [cu[i], cu[i+1]) and restarts both the state (from h0[i] or zero) and the chunk
 * grid.  h0/ht are [N,H,K,V]; hch is [1,H,NT_total,K,V] indexed by chunk_offsets.
 */
int oracle_gdn_varlen(const int* cu, int N, int H, int K, int V, int C,
                      const double* q, const double* k, const double* v, const double* g,
                      const double* gk, const double* beta, double scale, const double* h0,
                      double* o, double* ht, double* hch, double* vnew) {
  const int NT = oracle_varlen_tables(cu, N, C, NULL, NULL);
  if (NT < 0 || H <= 0 || K <= 0 || V <= 0) return -1;
  int* offs = (int*)malloc(sizeof(int) * (size_t)(N + 1));
  if (!offs) return -1;
  oracle_varlen_tables(cu, N, C, offs, NULL);
  int fail = 0;
#pragma omp parallel
  {
    double* S = (double*)malloc(sizeof(double) * (size_t)K * V);
    double* a = (double*)malloc(sizeof(double) * (size_t)K);
    double* d = (double*)malloc(sizeof(double) * (size_t)V);
    if (!S || !a || !d) {
#pragma omp atomic write
      fail = 1;
    } else {
#pragma omp for schedule(dynamic, 1)
      for (int ih = 0; ih < N * H; ++ih) {
        const int i = ih / H, h = ih % H;
        const long tok0 = (long)cu[i] * H + h;
        gdn_chain(cu[i + 1] - cu[i], K, V, C, q + tok0 * K, k + tok0 * K, v + tok0 * V,
                  (long)H * K, (long)H * V, g ? g + tok0 : NULL, gk ? gk + tok0 * K : NULL,
                  beta + tok0, (long)H, scale, h0 ? h0 + (size_t)ih * K * V : NULL,
                  o + tok0 * V, ht ? ht + (size_t)ih * K * V : NULL,
                  hch ? hch + ((size_t)h * NT + offs[i]) * K * V : NULL,
                  vnew ? vnew + tok0 * V : NULL, S, a, d);
      }
    }
    free(S);
    free(a);
    free(d);
  }
  free(offs);
  return fail ? -1 : 0;
}

/*
 * BiGDN front end (SANA fused_gdn.py page: _precompute_inv_rms, prepare_rope_tables and the
 * load path of _fused_gdn_kernel).  qkv is [B,N,3,H,D]; weights are [H*D]; cos/sin are the
 * expanded [N,D] tables with y[d] = x[d] cos[n,d] + x[d^1] sin[n,d].
 *   inv_rms = 1 / sqrt(sum over all H*D channels of x^2 / (H*D) + eps), per (b, n)
 *   x_hat   = x * inv_rms * w[h*D + d]
 *   q_pos   = relu(q_hat),  k_pos = relu(k_hat) * k_scale
 *   x_rot   = x_pos[d] cos[n,d] + x_pos[d^1] sin[n,d]
 * Outputs (each may be NULL): q_inv_rms/k_inv_rms [B,N]; q_rot, k_rot, q_pos, k_pos, v_hm
 * [B,H,N,D] (head-major).  D must be even.
 */
int oracle_prep(int B, int N, int H, int D, const double* qkv, const double* qw,
                const double* kw, const double* cosv, const double* sinv, double k_scale,
                double eps, double* q_inv_rms, double* k_inv_rms, double* q_rot, double* k_rot,
                double* q_pos, double* k_pos, double* v_hm) {
  if (B <= 0 || N <= 0 || H <= 0 || D <= 0 || (D % 2) != 0) return -1;
  const long C = (long)H * D;
#pragma omp parallel for schedule(static)
  for (long bn = 0; bn < (long)B * N; ++bn) {
    const long b = bn / N, n = bn % N;
    const double* row = qkv + bn * 3 * C;
    double inv[2];
    for (int which = 0; which < 2; ++which) {
      double ss = 0.0;
      for (long c = 0; c < C; ++c) ss += row[which * C + c] * row[which * C + c];
      inv[which] = 1.0 / sqrt(ss / (double)C + eps);
    }
    if (q_inv_rms) q_inv_rms[bn] = inv[0];
    if (k_inv_rms) k_inv_rms[bn] = inv[1];
    for (int h = 0; h < H; ++h) {
      const long o0 = (((long)b * H + h) * N + n) * D;
      for (int dd = 0; dd < D; ++dd) {
        const int pd = dd ^ 1;
        const long c = (long)h * D + dd, pc = (long)h * D + pd;
        const double cs = cosv[n * D + dd], sn = sinv[n * D + dd];
        double qx = row[c] * inv[0] * qw[c], qp = row[pc] * inv[0] * qw[pc];
        double kx = row[C + c] * inv[1] * kw[c], kp = row[C + pc] * inv[1] * kw[pc];
        qx = qx > 0.0 ? qx : 0.0;
        qp = qp > 0.0 ? qp : 0.0;
        kx = (kx > 0.0 ? kx : 0.0) * k_scale;
        kp = (kp > 0.0 ? kp : 0.0) * k_scale;
        if (q_pos) q_pos[o0 + dd] = qx;
        if (k_pos) k_pos[o0 + dd] = kx;
        if (q_rot) q_rot[o0 + dd] = qx * cs + qp * sn;
        if (k_rot) k_rot[o0 + dd] = kx * cs + kp * sn;
        if (v_hm) v_hm[o0 + dd] = row[2 * C + c];
      }
    }
  }
  return 0;
}

/*
 * Absorb one frame into (S, z) in place, following the frame-level update of
 * _fused_gdn_kernel: every token of the frame predicts from the same (already decayed)
 * state snapshot Sp / zp, and the frame's corrections are summed:
 *     S += sum_s k_rot_s (beta_s (v_s - Sp^T k_rot_s))^T
 *     z += sum_s k_pos_s  beta_s (1 - k_pos_s . zp)
 * Pointers address the frame's first token of one (b, h) in [.., N, D] head-major tensors.
 */
static void absorb_frame(int S_, int D, const double* kr, const double* kp, const double* vv,
                         const double* bt, double* S, double* z, double* Sp, double* zp,
                         double* dv) {
  memcpy(Sp, S, sizeof(double) * (size_t)D * D);
  memcpy(zp, z, sizeof(double) * (size_t)D);
  for (int s = 0; s < S_; ++s) {
    const double* k = kr + (long)s * D;
    const double* kq = kp + (long)s * D;
    const double* v = vv + (long)s * D;
    for (int c = 0; c < D; ++c) dv[c] = 0.0;
    for (int r = 0; r < D; ++r)
      for (int c = 0; c < D; ++c) dv[c] += Sp[(size_t)r * D + c] * k[r];
    for (int c = 0; c < D; ++c) dv[c] = bt[s] * (v[c] - dv[c]);
    for (int r = 0; r < D; ++r)
      for (int c = 0; c < D; ++c) S[(size_t)r * D + c] += k[r] * dv[c];
    double zh = 0.0;
    for (int r = 0; r < D; ++r) zh += kq[r] * zp[r];
    const double dz = bt[s] * (1.0 - zh);
    for (int r = 0; r < D; ++r) z[r] += kq[r] * dz;
  }
}

/* Inclusive outputs of one frame: num_s = S^T q_rot_s, den_s = q_pos_s . z (accumulated). */
static void emit_frame(int S_, int D, const double* qr, const double* qp, const double* S,
                       const double* z, double* num, long num_stride, double* den) {
  for (int s = 0; s < S_; ++s) {
    const double* q = qr + (long)s * D;
    const double* qq = qp + (long)s * D;
    double* o = num + (long)s * num_stride;
    for (int r = 0; r < D; ++r)
      for (int c = 0; c < D; ++c) o[c] += S[(size_t)r * D + c] * q[r];
    double dn = 0.0;
    for (int r = 0; r < D; ++r) dn += qq[r] * z[r];
    den[s] += dn;
  }
}

/*
 * One BiGDN direction on prepped head-major tensors q_rot, k_rot, q_pos, k_pos, v
 * [B,H,N,D] (N = F*S), beta [B,H,F,S], decay [B,H,F] (multiplicative, in (0,1]).
 * Results are ADDED into num [B,N,H,D] and den [B,H,N] (callers zero them first).
 *   forward : for f = 0..F-1: S,z *= decay[f]; absorb frame f; emit frame f.
 *   reverse : frame f is emitted from the state built from frames > f, where absorbing
 *             frame f+1 first multiplies the state by decay[f+1]; the last frame emits
 *             from the zero state.
 */
int oracle_bigdn_dir(int B, int F, int S_, int H, int D, int reverse, const double* q_rot,
                     const double* k_rot, const double* q_pos, const double* k_pos,
                     const double* v, const double* beta, const double* decay, double* num,
                     double* den) {
  if (B <= 0 || F <= 0 || S_ <= 0 || H <= 0 || D <= 0) return -1;
  const long N = (long)F * S_;
  int fail = 0;
#pragma omp parallel
  {
    double* St = (double*)malloc(sizeof(double) * (size_t)D * D);
    double* Sp = (double*)malloc(sizeof(double) * (size_t)D * D);
    double* z = (double*)malloc(sizeof(double) * (size_t)D);
    double* zp = (double*)malloc(sizeof(double) * (size_t)D);
    double* dv = (double*)malloc(sizeof(double) * (size_t)D);
    if (!St || !Sp || !z || !zp || !dv) {
#pragma omp atomic write
      fail = 1;
    } else {
#pragma omp for schedule(dynamic, 1)
      for (int bh = 0; bh < B * H; ++bh) {
        const int b = bh / H, h = bh % H;
        const long base = (long)bh * N * D;
        memset(St, 0, sizeof(double) * (size_t)D * D);
        memset(z, 0, sizeof(double) * (size_t)D);
        for (int it = 0; it < F; ++it) {
          const int f = reverse ? F - 1 - it : it;
          if (!reverse || it > 0) {
            const int fa = reverse ? f + 1 : f; /* frame absorbed at this step */
            const double dcy = decay[(long)bh * F + fa];
            for (long e = 0; e < (long)D * D; ++e) St[e] *= dcy;
            for (int r = 0; r < D; ++r) z[r] *= dcy;
            const long t0 = (long)fa * S_;
            absorb_frame(S_, D, k_rot + base + t0 * D, k_pos + base + t0 * D,
                         v + base + t0 * D, beta + (long)bh * N + t0, St, z, Sp, zp, dv);
          }
          const long t0 = (long)f * S_;
          emit_frame(S_, D, q_rot + base + t0 * D, q_pos + base + t0 * D, St, z,
                     num + (((long)b * N + t0) * H + h) * D, (long)H * D,
                     den + (long)bh * N + t0);
        }
      }
    }
    free(St);
    free(Sp);
    free(z);
    free(zp);
    free(dv);
  }
  return fail ? -1 : 0;
}

/*
 * Whole BiGDN block forward: prep, then both directions, summed (the sums that
 * fused_bigdn_func divides; the divide itself is not part of this call).
 * qkv [B,N,3,H,D]; beta [B,H,F,S]; decay [B,H,F]; outputs num [B,N,H,D], den [B,H,N].
 */
int oracle_bigdn(int B, int F, int S_, int H, int D, const double* qkv, const double* beta,
                 const double* decay, const double* qw, const double* kw, const double* cosv,
                 const double* sinv, double k_scale, double eps, double* num, double* den) {
  const long N = (long)F * S_;
  const size_t n = (size_t)B * H * N * D;
  double* buf = (double*)malloc(sizeof(double) * n * 5);
  if (!buf) return -1;
  double *qr = buf, *kr = buf + n, *qp = buf + 2 * n, *kp = buf + 3 * n, *vv = buf + 4 * n;
  int rc = oracle_prep(B, (int)N, H, D, qkv, qw, kw, cosv, sinv, k_scale, eps, NULL, NULL,
                       qr, kr, qp, kp, vv);
  if (rc == 0) {
    memset(num, 0, sizeof(double) * n);
    memset(den, 0, sizeof(double) * (size_t)B * H * N);
    rc = oracle_bigdn_dir(B, F, S_, H, D, 0, qr, kr, qp, kp, vv, beta, decay, num, den);
    if (rc == 0)
      rc = oracle_bigdn_dir(B, F, S_, H, D, 1, qr, kr, qp, kp, vv, beta, decay, num, den);
  }
  free(buf);
  return rc;
}

/*
 * Camera-branch prep (SANA fused_cam_gdn.py page: _cam_prep_kernel, cam_prep_func and the
 * torch reference of the prep).  Inputs q, k, v [B,N,H,D]; qw, kw [H*D]; pq, pkv [B,N,4,4]
 * (row i, column j); cosv, sinv [N, D/2] (the expanded interleaved-pair tables, sin already
 * signed).  Per token n and head h, with inverse RMS over all H*D channels of the token:
 *   q_n = relu(q * inv_q * qw),  k_n = relu(k * inv_k * kw) * k_scale,  v_n = v
 *   first D/2 channels, in groups of four:  y[4g + i] = sum_j P[i][j] x[4g + j]
 *       (P = pq for q, pkv for k and v)
 *   last D/2 channels:  y[D/2 + r] = x[D/2 + r] cos[n, r] + x[D/2 + (r ^ 1)] sin[n, r]
 *   inflation = max(|k_out|^2, 1e-12) / max(|k_n|^2, 1e-12)
 * Outputs q_t, k_t, v_t [B,H,D,N] (channel-major); inflation [B,H,N].  D/2 must be a
 * multiple of 4.
 */
int oracle_cam_prep(int B, int N, int H, int D, const double* q, const double* k,
                    const double* v, const double* qw, const double* kw, const double* pq,
                    const double* pkv, const double* cosv, const double* sinv, double k_scale,
                    double eps, double* q_t, double* k_t, double* v_t, double* inflation) {
  if (B <= 0 || N <= 0 || H <= 0 || D <= 0 || (D % 8) != 0) return -1;
  const long C = (long)H * D;
  const int Dh = D / 2;
#pragma omp parallel for schedule(static)
  for (long bn = 0; bn < (long)B * N; ++bn) {
    const long b = bn / N, n = bn % N;
    const double* xr[3] = {q + bn * C, k + bn * C, v + bn * C};
    double inv[2];
    for (int which = 0; which < 2; ++which) {
      double ss = 0.0;
      for (long c = 0; c < C; ++c) ss += xr[which][c] * xr[which][c];
      inv[which] = 1.0 / sqrt(ss / (double)C + eps);
    }
    const double* P[3] = {pq + bn * 16, pkv + bn * 16, pkv + bn * 16};
    double* outs[3] = {q_t, k_t, v_t};
    double xn[512], y[512];
    for (int h = 0; h < H; ++h) {
      double pre = 0.0, post = 0.0;
      for (int which = 0; which < 3; ++which) {
        const double* x = xr[which] + (long)h * D;
        for (int d = 0; d < D; ++d) {
          if (which == 2) {
            xn[d] = x[d];
          } else {
            const double w = (which == 0 ? qw : kw)[(long)h * D + d];
            double t = x[d] * inv[which] * w;
            t = t > 0.0 ? t : 0.0;
            xn[d] = which == 1 ? t * k_scale : t;
          }
        }
        for (int g = 0; g < Dh / 4; ++g)
          for (int i = 0; i < 4; ++i) {
            double acc = 0.0;
            for (int j = 0; j < 4; ++j) acc += P[which][i * 4 + j] * xn[4 * g + j];
            y[4 * g + i] = acc;
          }
        for (int r = 0; r < Dh; ++r)
          y[Dh + r] = xn[Dh + r] * cosv[n * Dh + r] + xn[Dh + (r ^ 1)] * sinv[n * Dh + r];
        if (which == 1)
          for (int d = 0; d < D; ++d) {
            pre += xn[d] * xn[d];
            post += y[d] * y[d];
          }
        for (int d = 0; d < D; ++d) outs[which][(((long)b * H + h) * D + d) * N + n] = y[d];
      }
      inflation[((long)b * H + h) * N + n] = (post > 1e-12 ? post : 1e-12) / (pre > 1e-12 ? pre : 1e-12);
    }
  }
  return 0;
}

/*
 * Camera-branch scan (SANA fused_cam_gdn.py page: _cam_scan_kernel and cam_scan_func), the
 * numerator-only frame-level delta rule on channel-major tensors q, k, v [B,H,D,N] (N = F*S),
 * beta [B,H,F,S], decay [B,H,F].  The state St is [D_k rows, D_v columns] per (b, h).
 *   forward: for f = 0..F-1: St *= decay[f]; Sp = St; for every token s of frame f:
 *            St += k_s (beta_s (v_s - Sp^T k_s))^T; then out[:, s] = St^T q_s for the tokens
 *            of frame f (after the frame's update).
 *   reverse: frame f reads the state built from the frames after it (frame F-1 reads the
 *            zero state); absorbing frame f+1 first multiplies the state by decay[f+1].
 *   init   : forward only, may be NULL: [B*H, D, D] state at the end of a prefix, decayed by
 *            decay[0] at the first frame like any other state.
 *   final  : forward only, may be NULL: St after the last frame's update.
 * Returns -1 for a reverse scan with init or final (there is no cross-prefix reverse state).
 */
int oracle_cam_scan(int B, int H, int D, int F, int S_, int reverse, const double* q,
                    const double* k, const double* v, const double* beta, const double* decay,
                    const double* init, double* out, double* final_state) {
  if (B <= 0 || H <= 0 || D <= 0 || F <= 0 || S_ <= 0) return -1;
  if (reverse && (init || final_state)) return -1;
  const long N = (long)F * S_;
  int fail = 0;
#pragma omp parallel
  {
    double* St = (double*)malloc(sizeof(double) * (size_t)D * D);
    double* Sp = (double*)malloc(sizeof(double) * (size_t)D * D);
    double* dv = (double*)malloc(sizeof(double) * (size_t)D);
    if (!St || !Sp || !dv) {
#pragma omp atomic write
      fail = 1;
    } else {
#pragma omp for schedule(dynamic, 1)
      for (int bh = 0; bh < B * H; ++bh) {
        const long base = (long)bh * D * N;
        if (init)
          memcpy(St, init + (long)bh * D * D, sizeof(double) * (size_t)D * D);
        else
          memset(St, 0, sizeof(double) * (size_t)D * D);
        for (int it = 0; it < F; ++it) {
          const int f = reverse ? F - 1 - it : it;
          if (!reverse || it > 0) {
            const int fa = reverse ? f + 1 : f; /* frame absorbed at this step */
            const double g = decay[(long)bh * F + fa];
            for (long e = 0; e < (long)D * D; ++e) St[e] *= g;
            memcpy(Sp, St, sizeof(double) * (size_t)D * D);
            for (int s = 0; s < S_; ++s) {
              const long t = (long)fa * S_ + s;
              for (int c = 0; c < D; ++c) {
                double pred = 0.0;
                for (int r = 0; r < D; ++r) pred += k[base + (long)r * N + t] * Sp[(size_t)r * D + c];
                dv[c] = beta[(long)bh * N + t] * (v[base + (long)c * N + t] - pred);
              }
              for (int r = 0; r < D; ++r) {
                const double kr = k[base + (long)r * N + t];
                for (int c = 0; c < D; ++c) St[(size_t)r * D + c] += kr * dv[c];
              }
            }
          }
          for (int s = 0; s < S_; ++s) {
            const long t = (long)f * S_ + s;
            for (int c = 0; c < D; ++c) {
              double o = 0.0;
              for (int r = 0; r < D; ++r) o += St[(size_t)r * D + c] * q[base + (long)r * N + t];
              out[base + (long)c * N + t] = o;
            }
          }
        }
        if (final_state) memcpy(final_state + (long)bh * D * D, St, sizeof(double) * (size_t)D * D);
      }
    }
    free(St);
    free(Sp);
    free(dv);
  }
  return fail ? -1 : 0;
}

/*
 * Backward of the camera-branch scan (SANA fused_cam_gdn.py page, "Backward Triton kernel":
 * _cam_scan_bwd_kernel): the gradients of L = sum(out * dout) with respect to q, k, v, beta
 * and decay, for the scan of oracle_cam_scan without an initial state (one direction).
 * The forward steps are replayed, keeping the state after each step's decay (Sp) and after
 * its update (St); then, step by step in reverse order, with dSt the gradient of the state
 * after the step's update:
 *   output of frame f (out_s = St^T q_s):   dq_s = St dout_s,   dSt += q_s dout_s^T
 *   absorption of frame fa (St = Sp + sum_s k_s d_s^T, d_s = beta_s (v_s - Sp^T k_s)):
 *       dd_s = dSt^T k_s,  dv_s = beta_s dd_s,  dbeta_s = dd_s . (v_s - Sp^T k_s),
 *       dk_s = dSt d_s + Sp (-beta_s dd_s),  dSp = dSt + sum_s k_s (-beta_s dd_s)^T
 *   decay (Sp = g St_prev):  ddecay[fa] = sum(dSp * St_prev),  dSt_prev = g dSp.
 * Tokens of a frame that is never absorbed (frame 0 of the reverse scan) get zero k, v, beta
 * gradients, and a decay that is never applied (or that multiplies the zero initial state)
 * gets ddecay = 0.
 */
int oracle_cam_scan_bwd(int B, int H, int D, int F, int S_, int reverse, const double* q,
                        const double* k, const double* v, const double* beta,
                        const double* decay, const double* dout, double* dq, double* dk,
                        double* dv, double* dbeta, double* ddecay) {
  if (B <= 0 || H <= 0 || D <= 0 || F <= 0 || S_ <= 0) return -1;
  const long N = (long)F * S_;
  const size_t DD = (size_t)D * D;
  int fail = 0;
#pragma omp parallel
  {
    double* Sp = (double*)malloc(sizeof(double) * DD * F);  /* per step: after the decay */
    double* St = (double*)malloc(sizeof(double) * DD * F);  /* per step: after the update */
    double* dS = (double*)malloc(sizeof(double) * DD);
    double* dP = (double*)malloc(sizeof(double) * DD);
    double* vec = (double*)malloc(sizeof(double) * 4 * (size_t)D);
    if (!Sp || !St || !dS || !dP || !vec) {
#pragma omp atomic write
      fail = 1;
    } else {
#pragma omp for schedule(dynamic, 1)
      for (int bh = 0; bh < B * H; ++bh) {
        const long base = (long)bh * D * N;
        double* r_ = vec;           /* v_s - Sp^T k_s */
        double* dd = vec + D;       /* dd_s */
        double* d_ = vec + 2 * D;   /* d_s */
        /* ---- forward replay ---- */
        for (int it = 0; it < F; ++it) {
          double* sp = Sp + (size_t)it * DD;
          double* st = St + (size_t)it * DD;
          if (it == 0) memset(st, 0, sizeof(double) * DD);
          else memcpy(st, St + (size_t)(it - 1) * DD, sizeof(double) * DD);
          memcpy(sp, st, sizeof(double) * DD);
          const int f = reverse ? F - 1 - it : it;
          if (reverse && it == 0) continue;  /* the reverse scan absorbs nothing first */
          const int fa = reverse ? f + 1 : f;
          const double g = decay[(long)bh * F + fa];
          for (size_t e = 0; e < DD; ++e) sp[e] = g * sp[e];
          memcpy(st, sp, sizeof(double) * DD);
          for (int s = 0; s < S_; ++s) {
            const long t = (long)fa * S_ + s;
            for (int c = 0; c < D; ++c) {
              double pred = 0.0;
              for (int r = 0; r < D; ++r) pred += k[base + (long)r * N + t] * sp[(size_t)r * D + c];
              d_[c] = beta[(long)bh * N + t] * (v[base + (long)c * N + t] - pred);
            }
            for (int r = 0; r < D; ++r)
              for (int c = 0; c < D; ++c) st[(size_t)r * D + c] += k[base + (long)r * N + t] * d_[c];
          }
        }
        /* ---- reverse pass ---- */
        for (long e = 0; e < (long)D * N; ++e) {
          dk[base + e] = 0.0;
          dv[base + e] = 0.0;
        }
        for (long t = 0; t < N; ++t) dbeta[(long)bh * N + t] = 0.0;
        for (int f = 0; f < F; ++f) ddecay[(long)bh * F + f] = 0.0;
        memset(dS, 0, sizeof(double) * DD);
        for (int it = F - 1; it >= 0; --it) {
          const double* sp = Sp + (size_t)it * DD;
          const double* st = St + (size_t)it * DD;
          const int f = reverse ? F - 1 - it : it;
          /* output of frame f */
          for (int s = 0; s < S_; ++s) {
            const long t = (long)f * S_ + s;
            for (int r = 0; r < D; ++r) {
              double acc = 0.0;
              for (int c = 0; c < D; ++c) acc += st[(size_t)r * D + c] * dout[base + (long)c * N + t];
              dq[base + (long)r * N + t] = acc;
            }
            for (int r = 0; r < D; ++r)
              for (int c = 0; c < D; ++c)
                dS[(size_t)r * D + c] += q[base + (long)r * N + t] * dout[base + (long)c * N + t];
          }
          if (reverse && it == 0) continue;
          const int fa = reverse ? f + 1 : f;
          const double g = decay[(long)bh * F + fa];
          memcpy(dP, dS, sizeof(double) * DD);
          for (int s = 0; s < S_; ++s) {
            const long t = (long)fa * S_ + s;
            const double bt = beta[(long)bh * N + t];
            for (int c = 0; c < D; ++c) {
              double pred = 0.0, g_ = 0.0;
              for (int r = 0; r < D; ++r) {
                pred += k[base + (long)r * N + t] * sp[(size_t)r * D + c];
                g_ += dS[(size_t)r * D + c] * k[base + (long)r * N + t];
              }
              r_[c] = v[base + (long)c * N + t] - pred;
              d_[c] = bt * r_[c];
              dd[c] = g_;
            }
            double db = 0.0;
            for (int c = 0; c < D; ++c) {
              dv[base + (long)c * N + t] = bt * dd[c];
              db += dd[c] * r_[c];
            }
            dbeta[(long)bh * N + t] = db;
            for (int r = 0; r < D; ++r) {
              double acc = 0.0;
              for (int c = 0; c < D; ++c)
                acc += dS[(size_t)r * D + c] * d_[c] - sp[(size_t)r * D + c] * bt * dd[c];
              dk[base + (long)r * N + t] = acc;
            }
            for (int r = 0; r < D; ++r)
              for (int c = 0; c < D; ++c)
                dP[(size_t)r * D + c] -= k[base + (long)r * N + t] * bt * dd[c];
          }
          /* decay: Sp = g * (state before the step); that state is St of the previous step
             (zero before the first) */
          double dg = 0.0;
          if (it > 0) {
            const double* prev = St + (size_t)(it - 1) * DD;
            for (size_t e = 0; e < DD; ++e) dg += dP[e] * prev[e];
          }
          ddecay[(long)bh * F + fa] = dg;
          for (size_t e = 0; e < DD; ++e) dS[e] = g * dP[e];
        }
      }
    }
    free(Sp);
    free(St);
    free(dS);
    free(dP);
    free(vec);
  }
  return fail ? -1 : 0;
}

/*
 * State-gradient pass of the chunked backward (the dhu fragments on the hyper-parallel
 * "Diff Coverage" page): the adjoint of the chunk state pass
 *     v_new = u - w h,   o = scale (e^gamma q)^T h + P v_new,   h_next = diag(e^{gamma_L}) h + K~^T v_new
 * run over chunks in reverse.  gamma_{t,d} is the chunk-local inclusive cumsum of
 * g_t + gk_{t,d} (either may be absent), gamma_L,d its value at the chunk's last token.  Per
 * chain, with dh = dht (or 0) on entry and for each chunk n from last to first:
 *     dv2_t = dv_t + sum_d k_{t,d} e^{gamma_L,d - gamma_{t,d}} dh[d, :]   (the gradient of v_new_t)
 *     dh    = diag(e^{gamma_L}) dh + scale sum_t (e^{gamma_t} * q_t) do_t^T - sum_t w_t dv2_t^T
 *     dh_chunks[n] = dh    (the gradient of the state entering chunk n)
 * and dh0 = dh at the end.  q, k, w [B,T,H,K]; do_, dv, dv2 [B,T,H,V]; g [B,T,H] or NULL;
 * gk [B,T,H,K] or NULL; dht, dh0 [B,H,K,V] (dht may be NULL); dh_chunks [B,H,NT,K,V] (may be
 * NULL).
 */
int oracle_gdn_dhu(int B, int T, int H, int K, int V, int C, const double* q, const double* k,
                   const double* w, const double* g, const double* gk, const double* do_,
                   const double* dv, const double* dht, double scale, double* dh_chunks,
                   double* dv2, double* dh0) {
  if (B <= 0 || T <= 0 || H <= 0 || K <= 0 || V <= 0 || C <= 0) return -1;
  const int NT = (T + C - 1) / C;
  int fail = 0;
#pragma omp parallel
  {
    double* dh = (double*)malloc(sizeof(double) * (size_t)K * V);
    double* gam = (double*)malloc(sizeof(double) * (size_t)C * K);
    if (!dh || !gam) {
#pragma omp atomic write
      fail = 1;
    } else {
#pragma omp for schedule(dynamic, 1)
      for (int bh = 0; bh < B * H; ++bh) {
        const int b = bh / H, h = bh % H;
        if (dht)
          memcpy(dh, dht + (long)bh * K * V, sizeof(double) * (size_t)K * V);
        else
          memset(dh, 0, sizeof(double) * (size_t)K * V);
        for (int n = NT - 1; n >= 0; --n) {
          const int t0 = n * C, L = (T - t0 < C) ? T - t0 : C;
          for (int d = 0; d < K; ++d) {
            double acc = 0.0;
            for (int i = 0; i < L; ++i) {
              const long tk = ((long)b * T + t0 + i) * H + h;
              acc += (g ? g[tk] : 0.0) + (gk ? gk[tk * K + d] : 0.0);
              gam[(size_t)i * K + d] = acc;
            }
          }
          const double* gl = gam + (size_t)(L - 1) * K;
          /* dv2 from the gradient of the state leaving the chunk */
          for (int i = 0; i < L; ++i) {
            const long tk = ((long)b * T + t0 + i) * H + h;
            for (int c = 0; c < V; ++c) {
              double s = 0.0;
              for (int r = 0; r < K; ++r)
                s += k[tk * K + r] * exp(gl[r] - gam[(size_t)i * K + r]) * dh[(size_t)r * V + c];
              dv2[tk * V + c] = dv[tk * V + c] + s;
            }
          }
          for (int r = 0; r < K; ++r) {
            const double el = exp(gl[r]);
            for (int c = 0; c < V; ++c) dh[(size_t)r * V + c] *= el;
          }
          for (int i = 0; i < L; ++i) {
            const long tk = ((long)b * T + t0 + i) * H + h;
            for (int r = 0; r < K; ++r) {
              const double qr = scale * exp(gam[(size_t)i * K + r]) * q[tk * K + r], wr = w[tk * K + r];
              for (int c = 0; c < V; ++c)
                dh[(size_t)r * V + c] += qr * do_[tk * V + c] - wr * dv2[tk * V + c];
            }
          }
          if (dh_chunks)
            memcpy(dh_chunks + ((long)bh * NT + n) * K * V, dh, sizeof(double) * (size_t)K * V);
        }
        if (dh0) memcpy(dh0 + (long)bh * K * V, dh, sizeof(double) * (size_t)K * V);
      }
    }
    free(dh);
    free(gam);
  }
  return fail ? -1 : 0;
}

/*
 * Inputs of the state-gradient pass formed from the forward's inputs, per chunk of C tokens
 * ([hyper-parallel "Diff Coverage" page]: the WY factor w that the chunk state pass takes in
 * v_new = u - w h, and the intra-chunk part of the gradient of v_new).  With gamma the
 * chunk-local inclusive cumsum of lambda_{t,d} = g_t + gk_{t,d}:
 *     A_{r,s} = beta_r sum_d k_{r,d} k_{s,d} e^{gamma_{r,d} - gamma_{s,d}}    (s < r, else 0)
 *     w       = (I + A)^-1 diag(beta) (e^{gamma} * K)     (forward substitution, row by row)
 *     P_{r,s} = scale sum_d q_{r,d} k_{s,d} e^{gamma_{r,d} - gamma_{s,d}}    (s <= r, else 0)
 *     dv      = P^T do.
 * q, k, w [B,T,H,K]; do_, dv [B,T,H,V]; beta, g [B,T,H] (g may be NULL); gk [B,T,H,K] or NULL.
 */
int oracle_gdn_bwd_prep(int B, int T, int H, int K, int V, int C, const double* q,
                        const double* k, const double* beta, const double* g, const double* gk,
                        const double* do_, double scale, double* w, double* dv) {
  if (B <= 0 || T <= 0 || H <= 0 || K <= 0 || V <= 0 || C <= 0) return -1;
  const int NT = (T + C - 1) / C;
  int fail = 0;
#pragma omp parallel
  {
    double* gam = (double*)malloc(sizeof(double) * (size_t)C * K);
    if (!gam) {
#pragma omp atomic write
      fail = 1;
    } else {
#pragma omp for schedule(dynamic, 1) collapse(2)
      for (int bh = 0; bh < B * H; ++bh)
        for (int n = 0; n < NT; ++n) {
          const int b = bh / H, h = bh % H;
          const int t0 = n * C, L = (T - t0 < C) ? T - t0 : C;
#define TOK(i) (((long)b * T + t0 + (i)) * H + h)
          for (int d = 0; d < K; ++d) {
            double acc = 0.0;
            for (int i = 0; i < L; ++i) {
              acc += (g ? g[TOK(i)] : 0.0) + (gk ? gk[TOK(i) * K + d] : 0.0);
              gam[(size_t)i * K + d] = acc;
            }
          }
          /* w row r = beta_r e^{gamma_r} k_r - sum_{s<r} A_{r,s} w_s, rows in order */
          for (int r = 0; r < L; ++r) {
            const double br = beta[TOK(r)];
            for (int d = 0; d < K; ++d)
              w[TOK(r) * K + d] = br * exp(gam[(size_t)r * K + d]) * k[TOK(r) * K + d];
            for (int s = 0; s < r; ++s) {
              double a = 0.0;
              for (int d = 0; d < K; ++d)
                a += k[TOK(r) * K + d] * k[TOK(s) * K + d] *
                     exp(gam[(size_t)r * K + d] - gam[(size_t)s * K + d]);
              a *= br;
              for (int d = 0; d < K; ++d) w[TOK(r) * K + d] -= a * w[TOK(s) * K + d];
            }
          }
          /* dv_s = sum_{r >= s} P_{r,s} do_r */
          for (int s = 0; s < L; ++s)
            for (int c = 0; c < V; ++c) dv[TOK(s) * V + c] = 0.0;
          for (int r = 0; r < L; ++r)
            for (int s = 0; s <= r; ++s) {
              double p = 0.0;
              for (int d = 0; d < K; ++d)
                p += q[TOK(r) * K + d] * k[TOK(s) * K + d] *
                     exp(gam[(size_t)r * K + d] - gam[(size_t)s * K + d]);
              p *= scale;
              for (int c = 0; c < V; ++c) dv[TOK(s) * V + c] += p * do_[TOK(r) * V + c];
            }
#undef TOK
        }
    }
    free(gam);
  }
  return fail ? -1 : 0;
}

/*
 * Backward of one BiGDN direction (SANA fused_gdn.py page, "Backward / autograd Functions":
 * the reverse replay of the frame recurrence behind FusedBiGDNFunction.backward): gradients of
 * L = sum(num * dnum) + sum(den * dden) for (num, den) = oracle_bigdn_dir(..., reverse).
 * With A and a the gradients of S and z after a step's update (num_s = S^T q_rot_s and
 * den_s = q_pos_s . z of the step's output frame), per step in reverse:
 *   A += sum_s q_rot_s dnum_s^T,  a += sum_s dden_s q_pos_s;
 *   dq_rot_s = S dnum_s,  dq_pos_s = dden_s z                       (output frame's tokens)
 * and, when the step absorbs frame fa with decay g from the states S_prev, z_prev
 * (S_pre = g S_prev, z_pre = g z_prev), for its tokens s:
 *   r_s = v_s - S_pre^T k_rot_s,  dd_s = A^T k_rot_s:
 *     dv_s = beta_s dd_s,  dk_rot_s = A (beta_s r_s) - beta_s S_pre dd_s
 *   e_s = 1 - k_pos_s . z_pre,    ee_s = a . k_pos_s:
 *     dk_pos_s = a (beta_s e_s) - beta_s ee_s z_pre
 *   dbeta_s = dd_s . r_s + ee_s e_s
 *   dS_pre = A - sum_s beta_s k_rot_s dd_s^T,  dz_pre = a - sum_s beta_s ee_s k_pos_s
 *   ddecay[fa] = <dS_pre, S_prev> + <dz_pre, z_prev>;  A = g dS_pre,  a = g dz_pre.
 * Frames that are never absorbed (frame 0 of the reverse direction) get zero k, v and beta
 * gradients and ddecay 0.  Layouts as oracle_bigdn_dir; dnum [B,N,H,D], dden [B,H,N];
 * outputs dq_rot, dk_rot, dq_pos, dk_pos, dv [B,H,N,D], dbeta [B,H,F,S], ddecay [B,H,F].
 */
int oracle_bigdn_dir_bwd(int B, int F, int S_, int H, int D, int reverse, const double* q_rot,
                         const double* k_rot, const double* q_pos, const double* k_pos,
                         const double* v, const double* beta, const double* decay,
                         const double* dnum, const double* dden, double* dq_rot,
                         double* dk_rot, double* dq_pos, double* dk_pos, double* dv,
                         double* dbeta, double* ddecay) {
  if (B <= 0 || F <= 0 || S_ <= 0 || H <= 0 || D <= 0) return -1;
  const long N = (long)F * S_;
  const size_t DD = (size_t)D * D;
  int fail = 0;
#pragma omp parallel
  {
    /* states after every step (S, z), the running gradients, scratch vectors */
    double* Ss = (double*)malloc(sizeof(double) * DD * F);
    double* zs = (double*)malloc(sizeof(double) * (size_t)D * F);
    double* A = (double*)malloc(sizeof(double) * DD);
    double* dSp = (double*)malloc(sizeof(double) * DD);
    double* a = (double*)malloc(sizeof(double) * D);
    double* dzp = (double*)malloc(sizeof(double) * D);
    double* Sp = (double*)malloc(sizeof(double) * DD);
    double* zp = (double*)malloc(sizeof(double) * D);
    double* vec = (double*)malloc(sizeof(double) * 3 * D);
    if (!Ss || !zs || !A || !dSp || !a || !dzp || !Sp || !zp || !vec) {
#pragma omp atomic write
      fail = 1;
    } else {
#pragma omp for schedule(dynamic, 1)
      for (int bh = 0; bh < B * H; ++bh) {
        const int b = bh / H, h = bh % H;
        const long base = (long)bh * N * D;
        /* forward replay, keeping the state after every step */
        double* St = Sp; /* reused below; the replay's running state */
        memset(St, 0, sizeof(double) * DD);
        memset(zp, 0, sizeof(double) * D);
        for (int it = 0; it < F; ++it) {
          const int f = reverse ? F - 1 - it : it;
          if (!reverse || it > 0) {
            const int fa = reverse ? f + 1 : f;
            const double g = decay[(long)bh * F + fa];
            for (size_t e = 0; e < DD; ++e) St[e] *= g;
            for (int r = 0; r < D; ++r) zp[r] *= g;
            const long t0 = (long)fa * S_;
            absorb_frame(S_, D, k_rot + base + t0 * D, k_pos + base + t0 * D, v + base + t0 * D,
                         beta + (long)bh * N + t0, St, zp, dSp, dzp, vec);
          }
          memcpy(Ss + (size_t)it * DD, St, sizeof(double) * DD);
          memcpy(zs + (size_t)it * D, zp, sizeof(double) * D);
        }
        /* reverse pass */
        memset(A, 0, sizeof(double) * DD);
        memset(a, 0, sizeof(double) * D);
        for (int it = F - 1; it >= 0; --it) {
          const int f = reverse ? F - 1 - it : it;
          const double* Sa = Ss + (size_t)it * DD;
          const double* za = zs + (size_t)it * D;
          for (int s = 0; s < S_; ++s) {
            const long t = (long)f * S_ + s;
            const double* qr = q_rot + base + t * D;
            const double* qp = q_pos + base + t * D;
            const double* dn = dnum + (((long)b * N + t) * H + h) * D;
            const double dd = dden[(long)bh * N + t];
            for (int r = 0; r < D; ++r) {
              double acc = 0.0;
              for (int c = 0; c < D; ++c) {
                A[(size_t)r * D + c] += qr[r] * dn[c];
                acc += Sa[(size_t)r * D + c] * dn[c];
              }
              dq_rot[base + t * D + r] = acc;
              a[r] += dd * qp[r];
              dq_pos[base + t * D + r] = dd * za[r];
            }
          }
          if (reverse && it == 0) break; /* frame 0 of the reverse direction is not absorbed */
          const int fa = reverse ? f + 1 : f;
          const double g = decay[(long)bh * F + fa];
          /* S_prev, z_prev: the state after the previous step (zero before the first) */
          if (it > 0) {
            for (size_t e = 0; e < DD; ++e) Sp[e] = g * Ss[(size_t)(it - 1) * DD + e];
            for (int r = 0; r < D; ++r) zp[r] = g * zs[(size_t)(it - 1) * D + r];
          } else {
            memset(Sp, 0, sizeof(double) * DD);
            memset(zp, 0, sizeof(double) * D);
          }
          memcpy(dSp, A, sizeof(double) * DD);
          memcpy(dzp, a, sizeof(double) * D);
          for (int s = 0; s < S_; ++s) {
            const long t = (long)fa * S_ + s;
            const double* kr = k_rot + base + t * D;
            const double* kp = k_pos + base + t * D;
            const double* vv = v + base + t * D;
            const double bt = beta[(long)bh * N + t];
            double* r_ = vec;
            double* dd_ = vec + D;
            double db = 0.0;
            for (int c = 0; c < D; ++c) {
              double pr = 0.0, q = 0.0;
              for (int r = 0; r < D; ++r) {
                pr += Sp[(size_t)r * D + c] * kr[r];
                q += A[(size_t)r * D + c] * kr[r];
              }
              r_[c] = vv[c] - pr;
              dd_[c] = q;
              dv[base + t * D + c] = bt * q;
              db += q * r_[c];
            }
            for (int r = 0; r < D; ++r) {
              double acc = 0.0;
              for (int c = 0; c < D; ++c)
                acc += A[(size_t)r * D + c] * bt * r_[c] - Sp[(size_t)r * D + c] * bt * dd_[c];
              dk_rot[base + t * D + r] = acc;
              for (int c = 0; c < D; ++c) dSp[(size_t)r * D + c] -= bt * kr[r] * dd_[c];
            }
            double zh = 0.0, ee = 0.0;
            for (int r = 0; r < D; ++r) {
              zh += kp[r] * zp[r];
              ee += a[r] * kp[r];
            }
            const double e1 = 1.0 - zh;
            for (int r = 0; r < D; ++r) {
              dk_pos[base + t * D + r] = a[r] * bt * e1 - bt * ee * zp[r];
              dzp[r] -= bt * ee * kp[r];
            }
            dbeta[(long)bh * N + t] = db + ee * e1;
          }
          double gd = 0.0;
          if (it > 0) {
            for (size_t e = 0; e < DD; ++e) gd += dSp[e] * Ss[(size_t)(it - 1) * DD + e];
            for (int r = 0; r < D; ++r) gd += dzp[r] * zs[(size_t)(it - 1) * D + r];
          }
          ddecay[(long)bh * F + fa] = gd;
          for (size_t e = 0; e < DD; ++e) A[e] = g * dSp[e];
          for (int r = 0; r < D; ++r) a[r] = g * dzp[r];
        }
        if (reverse) {
          /* frame 0 is never absorbed */
          for (long t = 0; t < S_; ++t) {
            for (int r = 0; r < D; ++r) {
              dk_rot[base + t * D + r] = 0.0;
              dk_pos[base + t * D + r] = 0.0;
              dv[base + t * D + r] = 0.0;
            }
            dbeta[(long)bh * N + t] = 0.0;
          }
          ddecay[(long)bh * F] = 0.0;
        }
      }
    }
    free(Ss);
    free(zs);
    free(A);
    free(dSp);
    free(a);
    free(dzp);
    free(Sp);
    free(zp);
    free(vec);
  }
  return fail ? -1 : 0;
}

/*
 * Backward of the BiGDN front end (oracle_prep), following the backward of the SANA
 * fused_gdn.py page ("Backward / autograd Functions": the RoPE inverse, ReLU and k-scale
 * backward inside _fused_gdn_bwd_kernel, and the full-channel RMSNorm backward of
 * FusedBiGDNFunction.backward).  Inputs are the gradients of the prepped tensors from ndir
 * scan directions, each [ndir, B, H, N, D] (the directions' contributions are summed);
 * outputs dqkv [B, N, 3, H, D] and the norm weights' gradients dqw, dkw [H*D].
 * Per token, with C = H*D, r the inverse RMS and x_hat = x r w:
 *   g_pos[d] = dpos[d] + drot[d] cos[d] + drot[d^1] sin[d^1]      (x_rot = x_pos cos + x_pos[d^1] sin)
 *   g[c]     = g_pos * (k_scale for k) * [x_hat > 0]               (the gradient of x_hat)
 *   dx[c]    = r w[c] g[c] - r^3 / C * x[c] * sum_c' w[c'] g[c'] x[c']
 *   dw[c]   += g[c] x[c] r
 * The token loop is serial so that the weight gradients are summed in token order.
 */
int oracle_prep_bwd(int B, int N, int H, int D, const double* qkv, const double* qw,
                    const double* kw, const double* cosv, const double* sinv, double k_scale,
                    double eps, int ndir, const double* dq_rot, const double* dk_rot,
                    const double* dq_pos, const double* dk_pos, const double* dv,
                    double* dqkv, double* dqw, double* dkw) {
  if (B <= 0 || N <= 0 || H <= 0 || D <= 0 || (D % 2) != 0 || ndir < 1) return -1;
  const long C = (long)H * D;
  const long dirs = (long)B * H * N * D;  /* elements of one direction's gradient */
  double* g = (double*)malloc(sizeof(double) * 2 * C);
  if (!g) return -1;
  for (long c = 0; c < C; ++c) dqw[c] = dkw[c] = 0.0;
  for (long bn = 0; bn < (long)B * N; ++bn) {
    const long b = bn / N, n = bn % N;
    const double* row = qkv + bn * 3 * C;
    double* out = dqkv + bn * 3 * C;
    for (int which = 0; which < 2; ++which) {
      const double* x = row + which * C;
      const double* w = which ? kw : qw;
      const double* drot = which ? dk_rot : dq_rot;
      const double* dpos = which ? dk_pos : dq_pos;
      double ss = 0.0;
      for (long c = 0; c < C; ++c) ss += x[c] * x[c];
      const double r = 1.0 / sqrt(ss / (double)C + eps);
      double s = 0.0;
      for (int h = 0; h < H; ++h) {
        for (int dd = 0; dd < D; ++dd) {
          const int pd = dd ^ 1;
          const long c = (long)h * D + dd;
          double gp = 0.0;
          for (int dir = 0; dir < ndir; ++dir) {
            const long o = dir * dirs + (((long)b * H + h) * N + n) * D;
            gp += dpos[o + dd] + drot[o + dd] * cosv[n * D + dd] + drot[o + pd] * sinv[n * D + pd];
          }
          const double xhat = x[c] * r * w[c];
          g[which * C + c] = xhat > 0.0 ? gp * (which ? k_scale : 1.0) : 0.0;
          s += w[c] * g[which * C + c] * x[c];
        }
      }
      double* dw = which ? dkw : dqw;
      for (long c = 0; c < C; ++c) {
        out[which * C + c] = r * w[c] * g[which * C + c] - r * r * r / (double)C * x[c] * s;
        dw[c] += g[which * C + c] * x[c] * r;
      }
    }
    for (int h = 0; h < H; ++h)
      for (int dd = 0; dd < D; ++dd) {
        double a = 0.0;
        for (int dir = 0; dir < ndir; ++dir) a += dv[dir * dirs + (((long)b * H + h) * N + n) * D + dd];
        out[2 * C + (long)h * D + dd] = a;
      }
  }
  free(g);
  return 0;
}

/*
 * Backward of the BiGDN merge (SANA fused_gdn.py page: the dnum / dden of
 * FusedBiGDNFunction.backward, with the SiLU gate of fused_bidi_merge):
 *   out = num / (den + eps) * silu(gate)     (silu = 1 without a gate)
 *   dnum  = dout silu(gate) / (den + eps)
 *   dden  = -sum_d dout silu(gate) num / (den + eps)^2
 *   dgate = dout num / (den + eps) * silu'(gate),  silu'(x) = s(x) (1 + x (1 - s(x)))
 * num, dout, gate, dnum, dgate [B, N, H, D]; den, dden [B, H, N].
 */
int oracle_bigdn_merge_bwd(int B, int N, int H, int D, const double* num, const double* den,
                           const double* gate, const double* dout, double eps, double* dnum,
                           double* dden, double* dgate) {
  if (B <= 0 || N <= 0 || H <= 0 || D <= 0) return -1;
  for (long b = 0; b < B; ++b)
    for (long n = 0; n < N; ++n)
      for (long h = 0; h < H; ++h) {
        const double inv = 1.0 / (den[(b * H + h) * N + n] + eps);
        const long o = ((b * N + n) * H + h) * D;
        double acc = 0.0;
        for (int d = 0; d < D; ++d) {
          double sl = 1.0;
          if (gate) {
            const double x = gate[o + d], sg = 1.0 / (1.0 + exp(-x));
            sl = x * sg;
            if (dgate) dgate[o + d] = dout[o + d] * num[o + d] * inv * sg * (1.0 + x * (1.0 - sg));
          }
          dnum[o + d] = dout[o + d] * sl * inv;
          acc += dout[o + d] * sl * num[o + d];
        }
        dden[(b * H + h) * N + n] = -acc * inv * inv;
      }
  return 0;
}

/*
 * Backward of the camera-branch prep (oracle_cam_prep), following the SANA fused_cam_gdn.py
 * page (_cam_prep_bwd_kernel, _cam_prep_bwd_dispatch): gradients of q, k, v [B,N,H,D] and of
 * the norm weights [H*D] from the gradients of the outputs q_t, k_t, v_t [B,H,D,N] and of the
 * inflation [B,H,N] (dinfl may be NULL: no inflation gradient).  Per token (serial, so the
 * weight gradients are summed in token order) and head, with xn the post-ReLU (k: times
 * k_scale) vector, y = T xn the output (UCPE 4x4 blocks on channels [0, D/2), RoPE on
 * [D/2, D)), pre = |xn_k|^2, post = |y_k|^2, inflation = max(post, 1e-12) / max(pre, 1e-12):
 *   d_post = dinfl [post >= 1e-12] / max(pre, 1e-12)
 *   d_pre  = -dinfl max(post, 1e-12) / max(pre, 1e-12)^2 [pre >= 1e-12]
 * (the indicators of the two clamps include equality, as the page's dispatch states them)
 *   dxn    = T^T dy   (dy_k = dk_t + 2 y_k d_post);   dxn_k += 2 xn_k d_pre
 *   T^T:  dxn[4g+j] = sum_i P[i][j] dy[4g+i];  dxn[D/2+r] = dy[D/2+r] cos[r] + dy[D/2+(r^1)] sin[r^1]
 *   g = dxn (times k_scale for k) where x_hat > 0;  dv = dxn_v
 * then the full-channel RMSNorm backward of oracle_prep_bwd.
 */
int oracle_cam_prep_bwd(int B, int N, int H, int D, const double* q, const double* k,
                        const double* qw, const double* kw, const double* pq, const double* pkv,
                        const double* cosv, const double* sinv, double k_scale, double eps,
                        const double* dq_t, const double* dk_t, const double* dv_t,
                        const double* dinfl, double* dq, double* dk, double* dv, double* dqw,
                        double* dkw) {
  if (B <= 0 || N <= 0 || H <= 0 || D <= 0 || (D % 8) != 0 || D > 512) return -1;
  const long C = (long)H * D;
  const int Dh = D / 2;
  double* g = (double*)malloc(sizeof(double) * 2 * C);
  if (!g) return -1;
  for (long c = 0; c < C; ++c) dqw[c] = dkw[c] = 0.0;
  for (long bn = 0; bn < (long)B * N; ++bn) {
    const long b = bn / N, n = bn % N;
    const double* xr[2] = {q + bn * C, k + bn * C};
    double inv[2];
    for (int which = 0; which < 2; ++which) {
      double ss = 0.0;
      for (long c = 0; c < C; ++c) ss += xr[which][c] * xr[which][c];
      inv[which] = 1.0 / sqrt(ss / (double)C + eps);
    }
    const double* P[3] = {pq + bn * 16, pkv + bn * 16, pkv + bn * 16};
    const double* dyt[3] = {dq_t, dk_t, dv_t};
    for (int h = 0; h < H; ++h) {
      double xn[2][512], y[512], dy[512], dx[512];
      for (int which = 0; which < 2; ++which)
        for (int d = 0; d < D; ++d) {
          const double w = (which ? kw : qw)[(long)h * D + d];
          const double t = xr[which][(long)h * D + d] * inv[which] * w;
          xn[which][d] = (t > 0.0 ? t : 0.0) * (which ? k_scale : 1.0);
        }
      /* the k output and the inflation's two squared norms */
      double pre = 0.0, post = 0.0;
      for (int gi = 0; gi < Dh / 4; ++gi)
        for (int i = 0; i < 4; ++i) {
          double acc = 0.0;
          for (int j = 0; j < 4; ++j) acc += P[1][i * 4 + j] * xn[1][4 * gi + j];
          y[4 * gi + i] = acc;
        }
      for (int r = 0; r < Dh; ++r)
        y[Dh + r] = xn[1][Dh + r] * cosv[n * Dh + r] + xn[1][Dh + (r ^ 1)] * sinv[n * Dh + r];
      for (int d = 0; d < D; ++d) {
        pre += xn[1][d] * xn[1][d];
        post += y[d] * y[d];
      }
      double d_post = 0.0, d_pre = 0.0;
      if (dinfl) {
        const double di = dinfl[((long)b * H + h) * N + n];
        const double prec = pre > 1e-12 ? pre : 1e-12, postc = post > 1e-12 ? post : 1e-12;
        d_post = post >= 1e-12 ? di / prec : 0.0;
        d_pre = pre >= 1e-12 ? -di * postc / (prec * prec) : 0.0;
      }
      for (int which = 0; which < 3; ++which) {
        for (int d = 0; d < D; ++d) {
          dy[d] = dyt[which][(((long)b * H + h) * D + d) * N + n];
          if (which == 1) dy[d] += 2.0 * y[d] * d_post;
        }
        for (int gi = 0; gi < Dh / 4; ++gi)
          for (int j = 0; j < 4; ++j) {
            double acc = 0.0;
            for (int i = 0; i < 4; ++i) acc += P[which][i * 4 + j] * dy[4 * gi + i];
            dx[4 * gi + j] = acc;
          }
        for (int r = 0; r < Dh; ++r)
          dx[Dh + r] = dy[Dh + r] * cosv[n * Dh + r] + dy[Dh + (r ^ 1)] * sinv[n * Dh + (r ^ 1)];
        for (int d = 0; d < D; ++d) {
          const long c = (long)h * D + d;
          if (which == 2) {
            dv[bn * C + c] = dx[d];
          } else {
            double gv = dx[d];
            if (which == 1) gv = (gv + 2.0 * xn[1][d] * d_pre) * k_scale;
            const double w = (which ? kw : qw)[c];
            g[which * C + c] = xr[which][c] * inv[which] * w > 0.0 ? gv : 0.0;
          }
        }
      }
    }
    for (int which = 0; which < 2; ++which) {
      const double* x = xr[which];
      const double* w = which ? kw : qw;
      double s = 0.0;
      for (long c = 0; c < C; ++c) s += w[c] * g[which * C + c] * x[c];
      const double r = inv[which];
      double* out = which ? dk : dq;
      double* dw = which ? dkw : dqw;
      for (long c = 0; c < C; ++c) {
        out[bn * C + c] = r * w[c] * g[which * C + c] - r * r * r / (double)C * x[c] * s;
        dw[c] += g[which * C + c] * x[c] * r;
      }
    }
  }
  free(g);
  return 0;
}

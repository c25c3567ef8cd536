// gdn_abi.hip -- the extern "C" boundary of libgdn: argument validation, dispatch and error
// reporting.  Declarations and the contract of every entry point are in include/gdn.h.
//
// Argument classes follow the wrappers on the pages (SANA fused_gdn.py page, fused_gdn_func
// and fused_bigdn_func checks; hyper-parallel "Diff Coverage" page, KDA state validation):
// malformed input is GDN_ERR_INVALID (their ValueError), valid-but-unimplemented
// combinations are GDN_ERR_UNSUPPORTED (their NotImplementedError), runtime failures are
// GDN_ERR_HIP (their RuntimeError).  Validation always completes before any launch.
#include <stdarg.h>
#include <stdint.h>
#include <stdio.h>

#include <mutex>

#include "../../include/gdn.h"
#include "gdn_bwd_params.h"
#include "gdn_internal.h"

namespace {

thread_local char g_err[512];

int fail(int code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return code;
}

int ok() {
  g_err[0] = '\0';
  return GDN_OK;
}

int hip_fail(hipError_t e, const char* what) {
  return fail(GDN_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

bool kv_supported(int dtype, int K, int V, bool per_key) {
  if (V != 64 && V != 128) return false;
  if (dtype == GDN_DTYPE_BF16) return K == 64 || K == 128;
  return K == 64 && !per_key;
}

// Checks shared by the dense and packed forward passes.
int check_fwd_common(const void* q, const void* k, const void* v, const float* beta, const void* o,
                     const float* gk, int H, int K, int V, int dtype) {
  if (!q || !k || !v || !beta || !o)
    return fail(GDN_ERR_INVALID, "q, k, v, beta and o must be non-null device pointers");
  if (H <= 0 || K <= 0 || V <= 0) return fail(GDN_ERR_INVALID, "H, K, V must be positive (got %d, %d, %d)", H, K, V);
  if (dtype != GDN_DTYPE_F32 && dtype != GDN_DTYPE_BF16)
    return fail(GDN_ERR_INVALID, "dtype must be GDN_DTYPE_F32 (0) or GDN_DTYPE_BF16 (1), got %d", dtype);
  if (!kv_supported(dtype, K, V, gk != nullptr))
    return fail(GDN_ERR_UNSUPPORTED,
                "unsupported combination: dtype=%s K=%d V=%d%s (bf16: K,V in {64,128}; fp32: K=64, "
                "V in {64,128}, no per-key gate)",
                dtype == GDN_DTYPE_BF16 ? "bf16" : "f32", K, V, gk ? " with gk" : "");
  return GDN_OK;
}

// 16-bit inputs are addressed with 32-bit buffer offsets over one head's rows.
int check_row_span(int64_t tokens, int H, int K, int V, int dtype) {
  const int64_t span = tokens * H * (K > V ? K : V) * 2;
  if (dtype == GDN_DTYPE_BF16 && span >= ((int64_t)1 << 32))
    return fail(GDN_ERR_UNSUPPORTED, "tokens*H*max(K,V)*2 = %lld bytes exceeds 32-bit buffer offsets",
                (long long)span);
  return GDN_OK;
}

// Flags implied by a forward call's arguments (what its workspace must be sized for).
unsigned fwd_flags(const float* gk, const void* h_chunks, const void* v_new) {
  return (gk ? GDN_FWD_PER_KEY : 0u) | ((h_chunks || v_new) ? GDN_FWD_SAVES : 0u);
}

// bf16 with a scalar gate and nothing saved per chunk runs the single fused kernel, which
// keeps every per-chunk term on chip (its only scratch is the rank table of a packed batch).
bool fused_path(int dtype, unsigned flags) {
  return dtype == GDN_DTYPE_BF16 && !(flags & (GDN_FWD_PER_KEY | GDN_FWD_SAVES));
}

int check_workspace(const void* ws, size_t bytes, size_t need) {
  if (need == 0) return GDN_OK;
  if (!ws || bytes < need)
    return fail(GDN_ERR_WORKSPACE, "workspace of %zu bytes needed, got %zu", need, ws ? bytes : (size_t)0);
  if (reinterpret_cast<uintptr_t>(ws) % 256) return fail(GDN_ERR_INVALID, "workspace must be 256-byte aligned");
  return GDN_OK;
}

}  // namespace

extern "C" {

int gdn_abi_version(void) { return GDN_ABI_VERSION; }

const char* gdn_last_error(void) { return g_err; }

size_t gdn_fwd_workspace_bytes(int B, int T, int H, int K, int V, int dtype, unsigned flags) {
  const bool per_key = flags & GDN_FWD_PER_KEY;
  if (B <= 0 || T <= 0 || H <= 0 || !kv_supported(dtype, K, V, per_key)) return 0;
  return gdn::fwd_workspace_bytes((long)B * H * ((T + GDN_CHUNK - 1) / GDN_CHUNK), 0, dtype, K,
                                  per_key, fused_path(dtype, flags));
}

int gdn_fwd(const void* q, const void* k, const void* v, const float* g, const float* gk,
            const float* beta, float scale, const float* h0, void* o, float* ht, void* h_chunks,
            void* v_new, int B, int T, int H, int K, int V, int dtype, void* workspace,
            size_t workspace_bytes, void* stream) {
  int rc = check_fwd_common(q, k, v, beta, o, gk, H, K, V, dtype);
  if (rc) return rc;
  if (B <= 0 || T <= 0) return fail(GDN_ERR_INVALID, "B and T must be positive (got %d, %d)", B, T);
  rc = check_row_span(T, H, K, V, dtype);
  if (rc) return rc;
  const int64_t wgs = (int64_t)B * H * (V / 32), nslots = (int64_t)B * H * ((T + GDN_CHUNK - 1) / GDN_CHUNK);
  if (wgs > INT32_MAX || nslots > INT32_MAX)
    return fail(GDN_ERR_INVALID, "B*H*(V/32) = %lld or B*H*chunks = %lld exceeds the grid limit",
                (long long)wgs, (long long)nslots);
  const size_t need = gdn_fwd_workspace_bytes(B, T, H, K, V, dtype, fwd_flags(gk, h_chunks, v_new));
  rc = check_workspace(workspace, workspace_bytes, need);
  if (rc) return rc;
  gdn::FwdParams p{};
  p.q = q; p.k = k; p.v = v; p.g = g; p.gk = gk; p.beta = beta; p.h0 = h0;
  p.o = o; p.ht = ht; p.h_chunks = h_chunks; p.v_new = v_new; p.cu = nullptr;
  p.scale = scale; p.B = B; p.T = T; p.H = H; p.V = V; p.nvb = V / 64;
  p.nseq = 0; p.nt_total = 0; p.ws = workspace; p.coffs = nullptr;
  hipError_t e = gdn::launch_gdn_fwd(p, dtype, K, false, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "gdn_fwd launch");
  return ok();
}

}  // extern "C"

namespace {

// gdn_state_summary workspace: the forward pass's own workspace and, except on the fused bf16
// path (which forms the state alone), its discarded per-token outputs.  Every view 256-byte
// aligned.
struct SummaryWs {
  size_t fwd, o, wy, total;
};

size_t al256s(size_t x) { return (x + 255) & ~(size_t)255; }

SummaryWs summary_ws(int B, int T, int H, int K, int V, int dtype, bool per_key) {
  SummaryWs w{};
  const size_t es = dtype == GDN_DTYPE_BF16 ? 2 : 4, tok = (size_t)B * T * H;
  size_t off = 0;
  w.fwd = off;
  off = al256s(off + gdn_fwd_workspace_bytes(B, T, H, K, V, dtype, per_key ? GDN_FWD_PER_KEY : 0u));
  w.o = off;
  if (!fused_path(dtype, per_key ? GDN_FWD_PER_KEY : 0u)) off = al256s(off + tok * (size_t)V * es);
  w.wy = off;
  off = al256s(off + gdn::transition_ws_bytes(B, T, H, K, dtype, per_key));
  w.total = off;
  return w;
}

}  // namespace

extern "C" {

size_t gdn_state_summary_workspace_bytes(int B, int T, int H, int K, int V, int dtype, unsigned flags) {
  const bool per_key = flags & GDN_FWD_PER_KEY;
  if (B <= 0 || T <= 0 || H <= 0 || !kv_supported(dtype, K, V, per_key)) return 0;
  return summary_ws(B, T, H, K, V, dtype, per_key).total;
}

int gdn_state_summary(const void* k, const void* v, const float* g, const float* gk,
                      const float* beta, float* state_ext, float* transition, int B, int T, int H,
                      int K, int V, int dtype, void* workspace, size_t workspace_bytes,
                      void* stream) {
  int rc = check_fwd_common(k, k, v, beta, state_ext, gk, H, K, V, dtype);
  if (rc) return rc;
  if (B <= 0 || T <= 0) return fail(GDN_ERR_INVALID, "B and T must be positive (got %d, %d)", B, T);
  rc = check_row_span(T, H, K, V, dtype);
  if (rc) return rc;
  const int64_t wgs = (int64_t)B * H * ((K > V ? K : V) / 32), nslots = (int64_t)B * H * ((T + GDN_CHUNK - 1) / GDN_CHUNK);
  if (wgs > INT32_MAX || nslots > INT32_MAX)
    return fail(GDN_ERR_INVALID, "B*H*(V/32) = %lld or B*H*chunks = %lld exceeds the grid limit",
                (long long)wgs, (long long)nslots);
  const SummaryWs w = summary_ws(B, T, H, K, V, dtype, gk != nullptr);
  if (!workspace || workspace_bytes < w.total)
    return fail(GDN_ERR_WORKSPACE, "workspace of %zu bytes needed, got %zu", w.total, workspace_bytes);
  if (reinterpret_cast<uintptr_t>(workspace) % 256)
    return fail(GDN_ERR_INVALID, "workspace must be 256-byte aligned");
  char* ws = static_cast<char*>(workspace);
  const hipStream_t st = static_cast<hipStream_t>(stream);
  // state_ext: the fragment from a zero initial state (the per-token outputs are discarded; the
  // fused bf16 path does not form them at all)
  gdn::FwdParams p{};
  p.q = k; p.k = k; p.v = v; p.g = g; p.gk = gk; p.beta = beta; p.h0 = nullptr;
  p.o = fused_path(dtype, gk ? GDN_FWD_PER_KEY : 0u) ? nullptr : ws + w.o; p.ht = state_ext; p.h_chunks = nullptr; p.v_new = nullptr; p.cu = nullptr;
  p.scale = 1.f; p.B = B; p.T = T; p.H = H; p.V = V; p.nvb = V / 64;
  p.nseq = 0; p.nt_total = 0; p.ws = ws + w.fwd; p.coffs = nullptr;
  hipError_t e = gdn::launch_gdn_fwd(p, dtype, K, false, st);
  if (e != hipSuccess) return hip_fail(e, "gdn_state_summary launch");
  if (transition) {
    e = gdn::launch_transition(k, g, gk, beta, transition, B, T, H, K, dtype, ws + w.wy, st);
    if (e != hipSuccess) return hip_fail(e, "gdn_state_summary launch");
  }
  return ok();
}

int gdn_state_apply(const float* state_ext, const float* transition, const float* h_in,
                    float* h_out, int BH, int K, int V, void* stream) {
  if (!state_ext || !h_out || (h_in && !transition))
    return fail(GDN_ERR_INVALID, "state_ext and h_out must be non-null, and transition too when h_in is");
  if (BH <= 0 || K <= 0 || V <= 0) return fail(GDN_ERR_INVALID, "BH, K, V must be positive (got %d, %d, %d)", BH, K, V);
  if (K > gdn::kApplyMaxK) return fail(GDN_ERR_UNSUPPORTED, "K must be <= %d, got %d", gdn::kApplyMaxK, K);
  if (BH > 65535) return fail(GDN_ERR_INVALID, "BH must be <= 65535, got %d", BH);
  const uintptr_t bytes = (uintptr_t)BH * K * V * 4;
  const uintptr_t a0 = reinterpret_cast<uintptr_t>(h_out), b0 = reinterpret_cast<uintptr_t>(h_in);
  if (h_in && a0 < b0 + bytes && b0 < a0 + bytes) return fail(GDN_ERR_INVALID, "h_out must not overlap h_in");
  hipError_t e = gdn::launch_apply(state_ext, transition, h_in, h_out, BH, K, V, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "gdn_state_apply launch");
  return ok();
}

int gdn_varlen_num_chunks(const int* cu, int N) {
  if (!cu || N < 1 || cu[0] != 0) return -1;
  int64_t total = 0;
  for (int i = 0; i < N; ++i) {
    const int64_t len = (int64_t)cu[i + 1] - cu[i];
    if (len <= 0) return -1;
    total += (len + GDN_CHUNK - 1) / GDN_CHUNK;
  }
  return total > INT32_MAX ? -1 : (int)total;
}

size_t gdn_fwd_varlen_workspace_bytes(int T_total, int N, int NT_total, int H, int K, int V,
                                      int dtype, unsigned flags) {
  const bool per_key = flags & GDN_FWD_PER_KEY;
  if (T_total <= 0 || N <= 0 || H <= 0 || !kv_supported(dtype, K, V, per_key)) return 0;
  // chunks <= T_total / 64 + N (each sequence adds at most one partial chunk)
  const long nt = NT_total > 0 ? (long)NT_total : (long)T_total / GDN_CHUNK + N;
  return gdn::fwd_workspace_bytes((long)H * nt, N, dtype, K, per_key, fused_path(dtype, flags));
}

}  // extern "C"

namespace {

// Scratch of gdn_fwd_varlen_noalloc: a static device array, one copy per GPU, held until the
// process ends.  In host code `scratch` only names the symbol; its device address on the
// current GPU comes from hipGetSymbolAddress, looked up once per device on the first call
// there (with that device current) and kept in g_scratch_ptr.
__device__ __align__(256) unsigned char scratch[GDN_NOALLOC_SCRATCH_BYTES];
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];

int scratch_of_current_device(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices) return fail(GDN_ERR_UNSUPPORTED, "device index %d >= %d", dev, kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_fail(e, "hipGetSymbolAddress(scratch)");
    if (!ptr || reinterpret_cast<uintptr_t>(ptr) % 256)
      return fail(GDN_ERR_HIP, "static scratch has no usable device address");
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return GDN_OK;
}

// gdn_fwd_varlen with its scratch given (noalloc: the static array instead): validation,
// then the launches.
int fwd_varlen_impl(bool noalloc, const void* q, const void* k, const void* v, const float* g,
                    const float* gk, const float* beta, float scale, const int* cu_seqlens,
                    const int* cu_seqlens_host, int N, const float* h0, void* o, float* ht,
                    void* h_chunks, void* v_new, int* chunk_offsets, int* chunk_indices,
                    int T_total, int H, int K, int V, int dtype, void* workspace,
                    size_t workspace_bytes, void* stream) {
  int rc = check_fwd_common(q, k, v, beta, o, gk, H, K, V, dtype);
  if (rc) return rc;
  if (!cu_seqlens || !cu_seqlens_host)
    return fail(GDN_ERR_INVALID, "cu_seqlens (device) and cu_seqlens_host must be non-null");
  if (N < 1 || T_total < 1) return fail(GDN_ERR_INVALID, "N and T_total must be positive (got %d, %d)", N, T_total);
  rc = check_row_span(T_total, H, K, V, dtype);
  if (rc) return rc;
  if (cu_seqlens_host[0] != 0) return fail(GDN_ERR_INVALID, "cu_seqlens[0] must be 0 (got %d)", cu_seqlens_host[0]);
  for (int i = 0; i < N; ++i)
    if (cu_seqlens_host[i + 1] <= cu_seqlens_host[i])
      return fail(GDN_ERR_INVALID, "cu_seqlens must be strictly increasing (sequence %d is empty or negative)", i);
  if (cu_seqlens_host[N] != T_total)
    return fail(GDN_ERR_INVALID, "cu_seqlens[N] = %d differs from T_total = %d", cu_seqlens_host[N], T_total);
  const int nt = gdn_varlen_num_chunks(cu_seqlens_host, N);
  if (nt < 0) return fail(GDN_ERR_INVALID, "too many chunks");
  const int64_t wgs = (int64_t)N * H * (V / 32);
  if (wgs > INT32_MAX || (int64_t)H * nt > INT32_MAX)
    return fail(GDN_ERR_INVALID, "N*H*(V/32) or H*chunks exceeds the grid limit");
  const unsigned flags = fwd_flags(gk, h_chunks, v_new);
  const size_t need = gdn_fwd_varlen_workspace_bytes(T_total, N, nt, H, K, V, dtype, flags);
  if (noalloc) {
    if (need > GDN_NOALLOC_SCRATCH_BYTES)
      return fail(GDN_ERR_WORKSPACE,
                  "gdn_fwd_varlen_noalloc needs %zu bytes of scratch; the static scratch holds %zu "
                  "(GDN_NOALLOC_SCRATCH_BYTES)", need, (size_t)GDN_NOALLOC_SCRATCH_BYTES);
    rc = scratch_of_current_device(&workspace);
    if (rc) return rc;
    workspace_bytes = GDN_NOALLOC_SCRATCH_BYTES;
  }
  rc = check_workspace(workspace, workspace_bytes, need);
  if (rc) return rc;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  if (chunk_offsets || chunk_indices) {
    hipError_t e = gdn::launch_varlen_tables(cu_seqlens, N, chunk_offsets, chunk_indices, s);
    if (e != hipSuccess) return hip_fail(e, "varlen table launch");
  }
  gdn::FwdParams p{};
  p.q = q; p.k = k; p.v = v; p.g = g; p.gk = gk; p.beta = beta; p.h0 = h0;
  p.o = o; p.ht = ht; p.h_chunks = h_chunks; p.v_new = v_new; p.cu = cu_seqlens;
  p.scale = scale; p.B = 1; p.T = T_total; p.H = H; p.V = V; p.nvb = V / 64;
  p.nseq = N; p.nt_total = nt; p.ws = workspace;
  p.coffs = fused_path(dtype, flags)
                ? nullptr
                : reinterpret_cast<int*>(static_cast<char*>(workspace) +
                                         (size_t)H * nt * gdn::fwd_slot_bytes(dtype, K, gk != nullptr));
  hipError_t e = gdn::launch_gdn_fwd(p, dtype, K, true, s);
  if (e != hipSuccess) return hip_fail(e, "gdn_fwd_varlen launch");
  return ok();
}

}  // namespace

extern "C" {

int gdn_fwd_varlen(const void* q, const void* k, const void* v, const float* g,
                   const float* gk, const float* beta, float scale, const int* cu_seqlens,
                   const int* cu_seqlens_host, int N, const float* h0, void* o, float* ht,
                   void* h_chunks, void* v_new, int* chunk_offsets, int* chunk_indices,
                   int T_total, int H, int K, int V, int dtype, void* workspace,
                   size_t workspace_bytes, void* stream) {
  return fwd_varlen_impl(false, q, k, v, g, gk, beta, scale, cu_seqlens,
                         cu_seqlens_host, N, h0, o, ht, h_chunks, v_new, chunk_offsets,
                         chunk_indices, T_total, H, K, V, dtype, workspace, workspace_bytes,
                         stream);
}

int gdn_fwd_varlen_noalloc(const void* q, const void* k, const void* v, const float* g,
                           const float* gk, const float* beta, float scale, const int* cu_seqlens,
                           const int* cu_seqlens_host, int N, const float* h0, void* o,
                           float* ht, void* h_chunks, void* v_new, int* chunk_offsets,
                           int* chunk_indices, int T_total, int H, int K, int V, int dtype,
                           void* stream) {
  return fwd_varlen_impl(true, q, k, v, g, gk, beta, scale, cu_seqlens, cu_seqlens_host, N, h0,
                         o, ht, h_chunks, v_new, chunk_offsets, chunk_indices, T_total, H, K, V,
                         dtype, nullptr, 0, stream);
}

}  // extern "C"

namespace {

// bigdn_fwd workspace: every view 256-byte aligned, in the order of BigdnParams.
struct BigdnWs {
  size_t q_rms, k_rms, q_rms_b, k_rms_b, rope_h, G, Gz, U, uz, G_b, Gz_b, U_b, uz_b, SdT, zd,
      total;
};

size_t al256(size_t x) { return (x + 255) & ~(size_t)255; }

// rev_stats: room for the reverse direction's own statistics (its beta or its q, k, v
// overridden) and its inverse RMS
BigdnWs bigdn_ws(int B, int F, int S, int H, int D, bool rev_stats = false) {
  BigdnWs w{};
  const size_t N = (size_t)F * S, mats = (size_t)B * H * F * D * D, vecs = (size_t)B * H * F * D;
  size_t off = 0;
  w.q_rms = off; off = al256(off + (size_t)B * N * 4);
  w.k_rms = off; off = al256(off + (size_t)B * N * 4);
  if (rev_stats) {
    w.q_rms_b = off; off = al256(off + (size_t)B * N * 4);
    w.k_rms_b = off; off = al256(off + (size_t)B * N * 4);
  }
  w.rope_h = off; off = al256(off + N * D * 4);
  w.G = off; off = al256(off + mats * 2);
  w.Gz = off; off = al256(off + mats * 2);
  w.U = off; off = al256(off + mats * 4);
  w.uz = off; off = al256(off + vecs * 4);
  if (rev_stats) {
    w.G_b = off; off = al256(off + mats * 2);
    w.Gz_b = off; off = al256(off + mats * 2);
    w.U_b = off; off = al256(off + mats * 4);
    w.uz_b = off; off = al256(off + vecs * 4);
  }
  w.SdT = off; off = al256(off + 2 * mats * 2);
  w.zd = off; off = al256(off + 2 * vecs * 4);
  w.total = off;
  return w;
}

int check_bigdn_dims(int B, int N, int H, int D) {
  if (B <= 0 || N <= 0 || H <= 0 || D <= 0)
    return fail(GDN_ERR_INVALID, "B, N, H, D must be positive (got %d, %d, %d, %d)", B, N, H, D);
  if (D % 2) return fail(GDN_ERR_INVALID, "D must be even (RoPE pairs), got %d", D);
  if (D != 64 && D != 128) return fail(GDN_ERR_UNSUPPORTED, "D must be 64 or 128, got %d", D);
  if ((int64_t)H * D > 4096) return fail(GDN_ERR_UNSUPPORTED, "H*D must be <= 4096, got %d", H * D);
  if ((int64_t)B * N > INT32_MAX) return fail(GDN_ERR_INVALID, "B*N exceeds the grid limit");
  return GDN_OK;
}

}  // namespace

extern "C" {

int gdn_prep(const void* qkv, const float* q_norm_w, const float* k_norm_w,
             const float* rope_cos, const float* rope_sin, float k_scale, float norm_eps,
             float* q_inv_rms, float* k_inv_rms, void* q_rot, void* k_rot, void* q_pos,
             void* k_pos, void* v_hm, int B, int N, int H, int D, void* stream) {
  if (!qkv || !q_norm_w || !k_norm_w || !rope_cos || !rope_sin)
    return fail(GDN_ERR_INVALID, "qkv, norm weights and RoPE tables must be non-null");
  int rc = check_bigdn_dims(B, N, H, D);
  if (rc) return rc;
  if (!(norm_eps > 0.f)) return fail(GDN_ERR_INVALID, "norm_eps must be positive");
  gdn::PrepParams p{};
  p.qkv = qkv; p.q_norm_w = q_norm_w; p.k_norm_w = k_norm_w; p.rope_cos = rope_cos;
  p.rope_sin = rope_sin; p.k_scale = k_scale; p.eps = norm_eps; p.q_inv_rms = q_inv_rms;
  p.k_inv_rms = k_inv_rms; p.q_rot = q_rot; p.k_rot = k_rot; p.q_pos = q_pos; p.k_pos = k_pos;
  p.v_hm = v_hm; p.B = B; p.N = N; p.H = H; p.D = D;
  hipError_t e = gdn::launch_prep(p, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "gdn_prep launch");
  return ok();
}

size_t bigdn_fwd_workspace_bytes(int B, int F, int S, int H, int D) {
  if (B <= 0 || F <= 0 || S <= 0 || H <= 0 || D <= 0) return 0;
  return bigdn_ws(B, F, S, H, D).total;
}

int bigdn_fwd_merged(const void* qkv, const void* qkv_bwd, const float* beta, const float* decay,
                     const float* beta_bwd, const float* decay_bwd, const float* q_norm_w,
                     const float* k_norm_w, const float* rope_cos, const float* rope_sin,
                     float k_scale, float norm_eps, const void* gate, float merge_eps, void* out,
                     void* num, void* den, int B, int F, int S, int H, int D, void* workspace,
                     size_t workspace_bytes, void* stream) {
  if (!qkv || !beta || !decay || !q_norm_w || !k_norm_w || !rope_cos || !rope_sin)
    return fail(GDN_ERR_INVALID, "qkv, beta, decay, norm weights and RoPE tables must be non-null");
  if (!out && !(num && den))
    return fail(GDN_ERR_INVALID, "out, or both num and den, must be non-null");
  if (gate && !out) return fail(GDN_ERR_INVALID, "gate needs out");
  if (F <= 0 || S <= 0) return fail(GDN_ERR_INVALID, "F and S must be positive (got %d, %d)", F, S);
  if ((int64_t)F * S > INT32_MAX) return fail(GDN_ERR_INVALID, "F*S too large");
  // the scan addresses one (b, h)'s per-frame statistics with 32-bit byte offsets
  if (F > 65535) return fail(GDN_ERR_UNSUPPORTED, "F must be <= 65535, got %d", F);
  const int N = F * S;
  int rc = check_bigdn_dims(B, N, H, D);
  if (rc) return rc;
  if (S % 64) return fail(GDN_ERR_UNSUPPORTED, "S (tokens per frame) must be a multiple of 64, got %d", S);
  if (!(norm_eps > 0.f)) return fail(GDN_ERR_INVALID, "norm_eps must be positive");
  if (out && !(merge_eps >= 0.f)) return fail(GDN_ERR_INVALID, "merge_eps must be >= 0");
  const bool rev = beta_bwd || qkv_bwd;
  const BigdnWs w = bigdn_ws(B, F, S, H, D, rev);
  if (!workspace || workspace_bytes < w.total)
    return fail(GDN_ERR_WORKSPACE, "workspace of %zu bytes needed, got %zu", w.total, workspace_bytes);
  if (reinterpret_cast<uintptr_t>(workspace) % 256)
    return fail(GDN_ERR_INVALID, "workspace must be 256-byte aligned");
  char* ws = static_cast<char*>(workspace);
  gdn::BigdnParams p{};
  p.qkv = qkv; p.qkv_bwd = qkv_bwd; p.beta = beta; p.decay = decay; p.beta_bwd = beta_bwd; p.decay_bwd = decay_bwd;
  p.q_norm_w = q_norm_w; p.k_norm_w = k_norm_w;
  p.rope_cos = rope_cos; p.rope_sin = rope_sin; p.k_scale = k_scale; p.eps = norm_eps;
  p.num = num; p.den = den; p.gate = gate; p.out = out; p.merge_eps = merge_eps;
  p.B = B; p.F = F; p.S = S; p.H = H; p.D = D; p.N = N;
  p.q_inv_rms = reinterpret_cast<float*>(ws + w.q_rms);
  p.k_inv_rms = reinterpret_cast<float*>(ws + w.k_rms);
  p.rope_h = reinterpret_cast<_Float16*>(ws + w.rope_h);
  p.G = reinterpret_cast<_Float16*>(ws + w.G);
  p.Gz = reinterpret_cast<_Float16*>(ws + w.Gz);
  p.U = reinterpret_cast<float*>(ws + w.U);
  p.uz = reinterpret_cast<float*>(ws + w.uz);
  if (rev) {
    p.q_inv_rms_b = reinterpret_cast<float*>(ws + w.q_rms_b);
    p.k_inv_rms_b = reinterpret_cast<float*>(ws + w.k_rms_b);
    p.G_b = reinterpret_cast<_Float16*>(ws + w.G_b);
    p.Gz_b = reinterpret_cast<_Float16*>(ws + w.Gz_b);
    p.U_b = reinterpret_cast<float*>(ws + w.U_b);
    p.uz_b = reinterpret_cast<float*>(ws + w.uz_b);
  }
  p.SdT = reinterpret_cast<_Float16*>(ws + w.SdT);
  p.zd = reinterpret_cast<float*>(ws + w.zd);
  hipError_t e = gdn::launch_bigdn(p, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "bigdn_fwd launch");
  return ok();
}

size_t bigdn_fwd_merged_workspace_bytes(int B, int F, int S, int H, int D, int has_rev_inputs) {
  if (B <= 0 || F <= 0 || S <= 0 || H <= 0 || D <= 0) return 0;
  return bigdn_ws(B, F, S, H, D, has_rev_inputs != 0).total;
}

int bigdn_fwd(const void* qkv, const float* beta, const float* decay, const float* q_norm_w,
              const float* k_norm_w, const float* rope_cos, const float* rope_sin,
              float k_scale, float norm_eps, void* num, void* den, int B, int F, int S, int H,
              int D, void* workspace, size_t workspace_bytes, void* stream) {
  if (!num || !den)
    return fail(GDN_ERR_INVALID, "qkv, beta, decay, norm weights, RoPE tables, num and den must be non-null");
  return bigdn_fwd_merged(qkv, nullptr, beta, decay, nullptr, nullptr, q_norm_w, k_norm_w, rope_cos,
                          rope_sin, k_scale, norm_eps, nullptr, 0.f, nullptr, num, den, B, F, S, H,
                          D, workspace, workspace_bytes, stream);
}


// ---- camera branch ----------------------------------------------------------------------

size_t cam_prep_workspace_bytes(int B, int N) {
  if (B <= 0 || N <= 0) return 0;
  return 2 * al256((size_t)B * N * 4);
}

int cam_prep(const float* q, const float* k, const float* v, const float* q_norm_w,
             const float* k_norm_w, const float* proj_q, const float* proj_kv,
             const float* rope_cos, const float* rope_sin, float k_scale, float norm_eps,
             float* q_out, float* k_out, float* v_out, float* inflation, int B, int N, int H,
             int D, void* workspace, size_t workspace_bytes, void* stream) {
  if (!q || !k || !v || !q_norm_w || !k_norm_w || !proj_q || !proj_kv || !rope_cos || !rope_sin ||
      !q_out || !k_out || !v_out || !inflation)
    return fail(GDN_ERR_INVALID, "every input and output pointer of cam_prep must be non-null");
  if (B <= 0 || N <= 0 || H <= 0 || D <= 0)
    return fail(GDN_ERR_INVALID, "B, N, H, D must be positive (got %d, %d, %d, %d)", B, N, H, D);
  if (D % 8) return fail(GDN_ERR_INVALID, "D must be even with D/2 a multiple of 4, got %d", D);
  if (D != 64 && D != 128) return fail(GDN_ERR_UNSUPPORTED, "D must be 64 or 128, got %d", D);
  if (N % 4) return fail(GDN_ERR_UNSUPPORTED, "N must be a multiple of 4, got %d", N);
  if ((int64_t)B * N > INT32_MAX || (int64_t)B * H * ((N + 63) / 64) > INT32_MAX)
    return fail(GDN_ERR_INVALID, "B*N exceeds the grid limit");
  if (!(norm_eps > 0.f)) return fail(GDN_ERR_INVALID, "norm_eps must be positive");
  const size_t need = cam_prep_workspace_bytes(B, N);
  if (!workspace || workspace_bytes < need)
    return fail(GDN_ERR_WORKSPACE, "workspace of %zu bytes needed, got %zu", need, workspace_bytes);
  if (reinterpret_cast<uintptr_t>(workspace) % 256)
    return fail(GDN_ERR_INVALID, "workspace must be 256-byte aligned");
  gdn::CamPrepParams p{};
  p.q = q; p.k = k; p.v = v; p.q_norm_w = q_norm_w; p.k_norm_w = k_norm_w;
  p.proj_q = proj_q; p.proj_kv = proj_kv; p.rope_cos = rope_cos; p.rope_sin = rope_sin;
  p.k_scale = k_scale; p.eps = norm_eps;
  p.q_out = q_out; p.k_out = k_out; p.v_out = v_out; p.inflation = inflation;
  p.q_inv_rms = static_cast<float*>(workspace);
  p.k_inv_rms = reinterpret_cast<float*>(static_cast<char*>(workspace) + al256((size_t)B * N * 4));
  p.B = B; p.N = N; p.H = H; p.D = D;
  hipError_t e = gdn::launch_cam_prep(p, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "cam_prep launch");
  return ok();
}

size_t cam_scan_workspace_bytes(int B, int H, int D, int F) {
  if (B <= 0 || H <= 0 || D <= 0 || F <= 0) return 0;
  const size_t mats = (size_t)B * H * F * D * D;
  return al256(mats * 2) + al256(mats * 4) + al256(mats * 2);
}

size_t cam_scan_bidi_workspace_bytes(int B, int H, int D, int F) {
  if (B <= 0 || H <= 0 || D <= 0 || F <= 0) return 0;
  const size_t mats = (size_t)B * H * F * D * D;
  return al256(mats * 2) + al256(mats * 4) + al256(2 * mats * 2);
}

}  // extern "C"

namespace {

// mode: 0 forward, 1 reverse, 2 both (out = forward, out_rev = reverse)
int cam_scan_impl(const float* q, const float* k, const float* v, const float* beta,
                  const float* decay, const float* decay_bwd, int mode, const float* init_state,
                  float* final_state, float* out, float* out_rev, int B, int H, int D, int F,
                  int S, void* workspace, size_t workspace_bytes, void* stream) {
  if (!q || !k || !v || !beta || !decay || !out || (mode == 2 && !out_rev))
    return fail(GDN_ERR_INVALID, "q, k, v, beta, decay and the outputs must be non-null");
  if (B <= 0 || H <= 0 || D <= 0 || F <= 0 || S <= 0)
    return fail(GDN_ERR_INVALID, "B, H, D, F, S must be positive (got %d, %d, %d, %d, %d)", B, H,
                D, F, S);
  if (mode == 1 && (init_state || final_state))
    return fail(GDN_ERR_UNSUPPORTED,
                "state in / out is defined for the forward scan only (reverse=1 with a state)");
  if (D != 64 && D != 128) return fail(GDN_ERR_UNSUPPORTED, "D must be 64 or 128, got %d", D);
  if (S % 64) return fail(GDN_ERR_UNSUPPORTED, "S (tokens per frame) must be a multiple of 64, got %d", S);
  if (F > 65535) return fail(GDN_ERR_UNSUPPORTED, "F must be <= 65535, got %d", F);
  if ((int64_t)F * S > INT32_MAX || (int64_t)B * H * F * (S / 64) > INT32_MAX)
    return fail(GDN_ERR_INVALID, "F*S exceeds the grid limit");
  const size_t mats = (size_t)B * H * F * D * D;
  const size_t need = mode == 2 ? cam_scan_bidi_workspace_bytes(B, H, D, F)
                                : cam_scan_workspace_bytes(B, H, D, F);
  if (!workspace || workspace_bytes < need)
    return fail(GDN_ERR_WORKSPACE, "workspace of %zu bytes needed, got %zu", need, workspace_bytes);
  if (reinterpret_cast<uintptr_t>(workspace) % 256)
    return fail(GDN_ERR_INVALID, "workspace must be 256-byte aligned");
  char* ws = static_cast<char*>(workspace);
  gdn::CamScanParams p{};
  p.q = q; p.k = k; p.v = v; p.beta = beta; p.decay = decay; p.decay_bwd = decay_bwd;
  p.reverse = mode; p.init_state = init_state; p.final_state = final_state;
  p.out = out; p.out_rev = out_rev;
  p.B = B; p.H = H; p.D = D; p.F = F; p.S = S;
  p.G = reinterpret_cast<_Float16*>(ws);
  p.U = reinterpret_cast<float*>(ws + al256(mats * 2));
  p.SdT = reinterpret_cast<_Float16*>(ws + al256(mats * 2) + al256(mats * 4));
  hipError_t e = gdn::launch_cam_scan(p, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "cam_scan launch");
  return ok();
}

}  // namespace

extern "C" {

int cam_scan(const float* q, const float* k, const float* v, const float* beta,
             const float* decay, int reverse, const float* init_state, float* final_state,
             float* out, int B, int H, int D, int F, int S, void* workspace,
             size_t workspace_bytes, void* stream) {
  return cam_scan_impl(q, k, v, beta, decay, nullptr, reverse ? 1 : 0, init_state, final_state,
                       out, nullptr, B, H, D, F, S, workspace, workspace_bytes, stream);
}

int cam_scan_bidi(const float* q, const float* k, const float* v, const float* beta,
                  const float* decay, const float* decay_bwd, const float* init_state,
                  float* final_state, float* out_fwd, float* out_rev, int B, int H, int D, int F,
                  int S, void* workspace, size_t workspace_bytes, void* stream) {
  return cam_scan_impl(q, k, v, beta, decay, decay_bwd, 2, init_state, final_state, out_fwd,
                       out_rev, B, H, D, F, S, workspace, workspace_bytes, stream);
}


// ---- backward of the camera-branch scan ----------------------------------------------------

size_t cam_scan_bwd_workspace_bytes(int B, int H, int D, int F) {
  if (B <= 0 || H <= 0 || (D != 64 && D != 128) || F <= 0) return 0;
  const size_t mats = (size_t)B * H * F * D * D;
  return 8 * al256(mats * 4) + al256((size_t)B * H * F * (D / gdn::kScanCB) * 4);
}

int cam_scan_bwd(const float* q, const float* k, const float* v, const float* beta,
                 const float* decay, const float* dout, int reverse, float* dq, float* dk,
                 float* dv, float* dbeta, float* ddecay, int B, int H, int D, int F, int S,
                 void* workspace, size_t workspace_bytes, void* stream) {
  if (!q || !k || !v || !beta || !decay || !dout || !dq || !dk || !dv || !dbeta || !ddecay)
    return fail(GDN_ERR_INVALID, "every input and gradient pointer must be non-null");
  if (B <= 0 || H <= 0 || D <= 0 || F <= 0 || S <= 0)
    return fail(GDN_ERR_INVALID, "B, H, D, F, S must be positive (got %d, %d, %d, %d, %d)", B, H,
                D, F, S);
  if (reverse & ~(1 | GDN_BWD_ACCUMULATE | GDN_BWD_REUSE_STATS))
    return fail(GDN_ERR_INVALID, "reverse must be 0 or 1, optionally with GDN_BWD_ACCUMULATE and GDN_BWD_REUSE_STATS, got %d", reverse);
  const int acc = (reverse & GDN_BWD_ACCUMULATE) ? 1 : 0;
  const int reuse = (reverse & GDN_BWD_REUSE_STATS) ? 1 : 0;
  reverse &= 1;
  if (D != 64 && D != 128) return fail(GDN_ERR_UNSUPPORTED, "D must be 64 or 128, got %d", D);
  if (S % 64) return fail(GDN_ERR_UNSUPPORTED, "S (tokens per frame) must be a multiple of 64, got %d", S);
  if ((int64_t)D * F * S > (int64_t(1) << 29) || (int64_t)B * H * F * 3 > INT32_MAX ||
      (int64_t)B * H * F * (S / 64) > INT32_MAX)
    return fail(GDN_ERR_INVALID, "D*F*S (a head's slab) or B*H*F exceeds the kernel limits");
  const size_t need = cam_scan_bwd_workspace_bytes(B, H, D, F);
  if (!workspace || workspace_bytes < need)
    return fail(GDN_ERR_WORKSPACE, "workspace of %zu bytes needed, got %zu", need, workspace_bytes);
  if (reinterpret_cast<uintptr_t>(workspace) % 256)
    return fail(GDN_ERR_INVALID, "workspace must be 256-byte aligned");
  const size_t mats = (size_t)B * H * F * D * D;
  char* ws = static_cast<char*>(workspace);
  gdn::CamBwdParams p{};
  p.q = q; p.k = k; p.v = v; p.beta = beta; p.decay = decay; p.dout = dout; p.reverse = reverse;
  p.acc = acc; p.reuse = reuse; p.dq = dq; p.dk = dk; p.dv = dv; p.dbeta = dbeta; p.ddecay = ddecay;
  p.B = B; p.H = H; p.D = D; p.F = F; p.S = S;
  size_t off = 0;
  auto take = [&](size_t bytes) { char* r = ws + off; off += al256(bytes); return r; };
  p.G = reinterpret_cast<float*>(take(mats * 4));
  p.U = reinterpret_cast<float*>(take(mats * 4));
  p.W = reinterpret_cast<float*>(take(mats * 4));
  p.Spf = reinterpret_cast<float*>(take(mats * 4));
  p.Sp = reinterpret_cast<__bf16*>(take(mats * 4));  // hi, then lo
  p.SpT = reinterpret_cast<__bf16*>(take(mats * 4));  // hi, then lo
  p.Ab = reinterpret_cast<__bf16*>(take(mats * 4));  // hi, then lo
  p.AbT = reinterpret_cast<__bf16*>(take(mats * 4));  // hi, then lo
  p.ddecay_part = reinterpret_cast<float*>(take((size_t)B * H * F * (D / gdn::kScanCB) * 4));
  p.lo = mats;
  hipError_t e = gdn::launch_cam_scan_bwd(p, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "cam_scan_bwd launch");
  return ok();
}

// ---- backward of one BiGDN direction ----------------------------------------------------------

size_t bigdn_dir_bwd_workspace_bytes(int B, int H, int D, int F) {
  if (B <= 0 || H <= 0 || (D != 64 && D != 128) || F <= 0) return 0;
  const size_t mats = (size_t)B * H * F * D * D, vecs = (size_t)B * H * F * D;
  return 9 * al256(mats * 4) + al256((size_t)B * H * F * (D / gdn::kScanCB) * 4) + 4 * al256(vecs * 4) +
         al256((size_t)B * H * F * 4);
}

int bigdn_dir_bwd(const void* q_rot, const void* k_rot, const void* q_pos, const void* k_pos,
                  const void* v, const float* beta, const float* decay, const float* dnum,
                  const float* dden, int reverse, float* dq_rot, float* dk_rot, float* dq_pos,
                  float* dk_pos, float* dv, float* dbeta, float* ddecay, int B, int H, int D, int F,
                  int S, void* workspace, size_t workspace_bytes, void* stream) {
  if (!q_rot || !k_rot || !q_pos || !k_pos || !v || !beta || !decay || !dnum || !dden || !dq_rot ||
      !dk_rot || !dq_pos || !dk_pos || !dv || !dbeta || !ddecay)
    return fail(GDN_ERR_INVALID, "every input and gradient pointer must be non-null");
  if (B <= 0 || H <= 0 || D <= 0 || F <= 0 || S <= 0)
    return fail(GDN_ERR_INVALID, "B, H, D, F, S must be positive (got %d, %d, %d, %d, %d)", B, H,
                D, F, S);
  if (reverse & ~(1 | GDN_BWD_ACCUMULATE | GDN_BWD_REUSE_STATS))
    return fail(GDN_ERR_INVALID, "reverse must be 0 or 1, optionally with GDN_BWD_ACCUMULATE and GDN_BWD_REUSE_STATS, got %d", reverse);
  const int acc = (reverse & GDN_BWD_ACCUMULATE) ? 1 : 0;
  const int reuse = (reverse & GDN_BWD_REUSE_STATS) ? 1 : 0;
  reverse &= 1;
  if (D != 64 && D != 128) return fail(GDN_ERR_UNSUPPORTED, "D must be 64 or 128, got %d", D);
  if (S % 64) return fail(GDN_ERR_UNSUPPORTED, "S (tokens per frame) must be a multiple of 64, got %d", S);
  if ((int64_t)F * S > INT32_MAX || (int64_t)B * H * F * 4 > INT32_MAX ||
      (int64_t)B * H * F * (S / 64) > INT32_MAX)
    return fail(GDN_ERR_INVALID, "F*S or B*H*F exceeds the grid limit");
  const size_t need = bigdn_dir_bwd_workspace_bytes(B, H, D, F);
  if (!workspace || workspace_bytes < need)
    return fail(GDN_ERR_WORKSPACE, "workspace of %zu bytes needed, got %zu", need, workspace_bytes);
  if (reinterpret_cast<uintptr_t>(workspace) % 256)
    return fail(GDN_ERR_INVALID, "workspace must be 256-byte aligned");
  const size_t mats = (size_t)B * H * F * D * D, vecs = (size_t)B * H * F * D;
  char* ws = static_cast<char*>(workspace);
  size_t off = 0;
  auto take = [&](size_t bytes) { char* r = ws + off; off += al256(bytes); return r; };
  gdn::BigdnBwdParams p{};
  gdn::CamBwdParams& c = p.cam;
  c.beta = beta; c.decay = decay; c.reverse = reverse; c.dbeta = dbeta; c.ddecay = ddecay;
  c.B = B; c.H = H; c.D = D; c.F = F; c.S = S;
  c.G = reinterpret_cast<float*>(take(mats * 4));
  c.U = reinterpret_cast<float*>(take(mats * 4));
  c.W = reinterpret_cast<float*>(take(mats * 4));
  c.Spf = reinterpret_cast<float*>(take(mats * 4));
  c.Sp = reinterpret_cast<__bf16*>(take(mats * 4));  // hi, then lo
  c.SpT = reinterpret_cast<__bf16*>(take(mats * 4));
  c.Ab = reinterpret_cast<__bf16*>(take(mats * 4));
  c.AbT = reinterpret_cast<__bf16*>(take(mats * 4));
  c.ddecay_part = reinterpret_cast<float*>(take((size_t)B * H * F * (D / gdn::kScanCB) * 4));
  c.lo = mats;
  p.Gpos = reinterpret_cast<float*>(take(mats * 4));
  p.upos = reinterpret_cast<float*>(take(vecs * 4));
  p.wz = reinterpret_cast<float*>(take(vecs * 4));
  p.zs = reinterpret_cast<float*>(take(vecs * 4));
  p.as = reinterpret_cast<float*>(take(vecs * 4));
  p.ddz = reinterpret_cast<float*>(take((size_t)B * H * F * 4));
  p.q_rot = static_cast<const __bf16*>(q_rot); p.k_rot = static_cast<const __bf16*>(k_rot);
  p.q_pos = static_cast<const __bf16*>(q_pos); p.k_pos = static_cast<const __bf16*>(k_pos);
  p.v = static_cast<const __bf16*>(v); p.dnum = dnum; p.dden = dden;
  p.dq_rot = dq_rot; p.dk_rot = dk_rot; p.dq_pos = dq_pos; p.dk_pos = dk_pos; p.dv = dv;
  p.acc = acc;
  c.reuse = reuse;
  hipError_t e = gdn::launch_bigdn_dir_bwd(p, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "bigdn_dir_bwd launch");
  return ok();
}

// ---- backward of the BiGDN front end and of the merge -------------------------------------

namespace {
constexpr long kPrepBwdGroups = 1024;  // token groups of gdn_prep_bwd (one workgroup each)
long prep_bwd_groups(int B, int N) {
  const long bn = (long)B * N;
  return bn < kPrepBwdGroups ? bn : kPrepBwdGroups;
}
}  // namespace

size_t gdn_prep_bwd_workspace_bytes(int B, int N, int H, int D) {
  if (B <= 0 || N <= 0 || H <= 0 || D <= 0) return 0;
  return al256((size_t)prep_bwd_groups(B, N) * 2 * H * D * 4);
}

int gdn_prep_bwd(const void* qkv, const float* q_norm_w, const float* k_norm_w,
                 const float* rope_cos, const float* rope_sin, float k_scale, float norm_eps,
                 int ndir, const float* dq_rot, const float* dk_rot, const float* dq_pos,
                 const float* dk_pos, const float* dv, float* dqkv, float* dq_norm_w,
                 float* dk_norm_w, int B, int N, int H, int D, void* workspace,
                 size_t workspace_bytes, void* stream) {
  if (!qkv || !q_norm_w || !k_norm_w || !rope_cos || !rope_sin || !dq_rot || !dk_rot || !dq_pos ||
      !dk_pos || !dv || !dqkv || !dq_norm_w || !dk_norm_w)
    return fail(GDN_ERR_INVALID, "every input and gradient pointer must be non-null");
  int rc = check_bigdn_dims(B, N, H, D);
  if (rc) return rc;
  if (ndir != 1 && ndir != 2) return fail(GDN_ERR_INVALID, "ndir must be 1 or 2, got %d", ndir);
  if (!(norm_eps > 0.f)) return fail(GDN_ERR_INVALID, "norm_eps must be positive");
  const size_t need = gdn_prep_bwd_workspace_bytes(B, N, H, D);
  if (!workspace || workspace_bytes < need)
    return fail(GDN_ERR_WORKSPACE, "workspace of %zu bytes needed, got %zu", need, workspace_bytes);
  if (reinterpret_cast<uintptr_t>(workspace) % 256)
    return fail(GDN_ERR_INVALID, "workspace must be 256-byte aligned");
  gdn::PrepBwdParams p{};
  p.qkv = static_cast<const __bf16*>(qkv); p.q_norm_w = q_norm_w; p.k_norm_w = k_norm_w;
  p.rope_cos = rope_cos; p.rope_sin = rope_sin; p.k_scale = k_scale; p.eps = norm_eps;
  p.ndir = ndir; p.dq_rot = dq_rot; p.dk_rot = dk_rot; p.dq_pos = dq_pos; p.dk_pos = dk_pos;
  p.dv = dv; p.dqkv = dqkv; p.dq_norm_w = dq_norm_w; p.dk_norm_w = dk_norm_w;
  p.part = static_cast<float*>(workspace); p.nwg = (int)prep_bwd_groups(B, N);
  p.B = B; p.N = N; p.H = H; p.D = D;
  hipError_t e = gdn::launch_prep_bwd(p, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "gdn_prep_bwd launch");
  return ok();
}

size_t cam_prep_bwd_workspace_bytes(int B, int N, int H, int D) {
  if (B <= 0 || N <= 0 || H <= 0 || D <= 0) return 0;
  return al256((size_t)B * N * 4) + al256((size_t)prep_bwd_groups(B, N) * 2 * H * D * 4);
}

int cam_prep_bwd(const float* q, const float* k, const float* q_norm_w, const float* k_norm_w,
                 const float* proj_q, const float* proj_kv, const float* rope_cos,
                 const float* rope_sin, float k_scale, float norm_eps, int ndir, const float* dq_t,
                 const float* dk_t, const float* dv_t, const float* dinfl, float* dq, float* dk,
                 float* dv, float* dq_norm_w, float* dk_norm_w, int B, int N, int H, int D,
                 void* workspace, size_t workspace_bytes, void* stream) {
  if (!q || !k || !q_norm_w || !k_norm_w || !proj_q || !proj_kv || !rope_cos || !rope_sin ||
      !dq_t || !dk_t || !dv_t || !dq || !dk || !dv || !dq_norm_w || !dk_norm_w)
    return fail(GDN_ERR_INVALID, "every input and gradient pointer except dinfl must be non-null");
  if (B <= 0 || N <= 0 || H <= 0 || D <= 0)
    return fail(GDN_ERR_INVALID, "B, N, H, D must be positive (got %d, %d, %d, %d)", B, N, H, D);
  if (D % 8) return fail(GDN_ERR_INVALID, "D must be even with D/2 a multiple of 4, got %d", D);
  if (D != 64 && D != 128) return fail(GDN_ERR_UNSUPPORTED, "D must be 64 or 128, got %d", D);
  if (N % 4) return fail(GDN_ERR_UNSUPPORTED, "N must be a multiple of 4, got %d", N);
  if ((int64_t)H * D > 4096) return fail(GDN_ERR_UNSUPPORTED, "H*D must be <= 4096, got %d", H * D);
  if ((int64_t)B * N > INT32_MAX || (int64_t)B * H * ((N + 63) / 64) > INT32_MAX)
    return fail(GDN_ERR_INVALID, "B*N exceeds the grid limit");
  if (ndir != 1 && ndir != 2) return fail(GDN_ERR_INVALID, "ndir must be 1 or 2, got %d", ndir);
  if (!(norm_eps > 0.f)) return fail(GDN_ERR_INVALID, "norm_eps must be positive");
  const size_t need = cam_prep_bwd_workspace_bytes(B, N, H, D);
  if (!workspace || workspace_bytes < need)
    return fail(GDN_ERR_WORKSPACE, "workspace of %zu bytes needed, got %zu", need, workspace_bytes);
  if (reinterpret_cast<uintptr_t>(workspace) % 256)
    return fail(GDN_ERR_INVALID, "workspace must be 256-byte aligned");
  gdn::CamPrepBwdParams p{};
  p.q = q; p.k = k; p.q_norm_w = q_norm_w; p.k_norm_w = k_norm_w; p.proj_q = proj_q;
  p.proj_kv = proj_kv; p.rope_cos = rope_cos; p.rope_sin = rope_sin; p.k_scale = k_scale;
  p.eps = norm_eps; p.ndir = ndir; p.dq_t = dq_t; p.dk_t = dk_t; p.dv_t = dv_t; p.dinfl = dinfl;
  p.dq = dq; p.dk = dk; p.dv = dv; p.dq_norm_w = dq_norm_w; p.dk_norm_w = dk_norm_w;
  p.k_inv_rms = static_cast<float*>(workspace);
  p.part = reinterpret_cast<float*>(static_cast<char*>(workspace) + al256((size_t)B * N * 4));
  p.nwg = (int)prep_bwd_groups(B, N);
  p.B = B; p.N = N; p.H = H; p.D = D;
  hipError_t e = gdn::launch_cam_prep_bwd(p, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "cam_prep_bwd launch");
  return ok();
}

int bigdn_merge_bwd(const void* num, const void* den, const void* gate, const float* dout,
                    float merge_eps, float* dnum, float* dden, float* dgate, int B, int N, int H,
                    int D, void* stream) {
  if (!num || !den || !dout || !dnum || !dden)
    return fail(GDN_ERR_INVALID, "num, den, dout, dnum and dden must be non-null");
  if (!gate != !dgate) return fail(GDN_ERR_INVALID, "gate and dgate must be given together");
  int rc = check_bigdn_dims(B, N, H, D);
  if (rc) return rc;
  if (!(merge_eps >= 0.f)) return fail(GDN_ERR_INVALID, "merge_eps must be >= 0");
  if ((int64_t)B * N * H > (int64_t)INT32_MAX * 4) return fail(GDN_ERR_INVALID, "B*N*H exceeds the grid limit");
  gdn::MergeBwdParams p{};
  p.num = static_cast<const __bf16*>(num); p.den = static_cast<const __bf16*>(den);
  p.gate = static_cast<const __bf16*>(gate); p.dout = dout; p.eps = merge_eps;
  p.dnum = dnum; p.dden = dden; p.dgate = dgate; p.B = B; p.N = N; p.H = H; p.D = D;
  hipError_t e = gdn::launch_merge_bwd(p, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "bigdn_merge_bwd launch");
  return ok();
}

// ---- backward: state-gradient pass --------------------------------------------------------

int gdn_bwd_dhu(const void* q, const void* k, const void* w, const void* do_, const void* dv,
                const float* g, const float* gk, const float* dht, float scale, float* dh_chunks, void* dv2,
                float* dh0, int B, int T, int H, int K, int V, int dtype, void* stream) {
  if (!q || !k || !w || !do_ || !dv || !dv2)
    return fail(GDN_ERR_INVALID, "q, k, w, do, dv and dv2 must be non-null");
  if (B <= 0 || T <= 0 || H <= 0 || K <= 0 || V <= 0)
    return fail(GDN_ERR_INVALID, "B, T, H, K, V must be positive (got %d, %d, %d, %d, %d)", B, T,
                H, K, V);
  if (dtype != GDN_DTYPE_F32 && dtype != GDN_DTYPE_BF16)
    return fail(GDN_ERR_INVALID, "dtype must be GDN_DTYPE_F32 or GDN_DTYPE_BF16, got %d", dtype);
  if (K != 128) return fail(GDN_ERR_UNSUPPORTED, "K must be 128, got %d", K);
  if (V % 32) return fail(GDN_ERR_UNSUPPORTED, "V must be a multiple of 32, got %d", V);
  if (gk && dtype == GDN_DTYPE_F32)
    return fail(GDN_ERR_UNSUPPORTED, "per-key gates need bf16 inputs");
  if ((int64_t)B * H * (V / 32) > INT32_MAX) return fail(GDN_ERR_INVALID, "B*H*V/32 exceeds the grid limit");
  gdn::DhuParams p{};
  p.q = q; p.k = k; p.w = w; p.do_ = do_; p.dv = dv; p.g = g; p.gk = gk; p.dht = dht; p.scale = scale;
  p.dh_chunks = dh_chunks; p.dv2 = dv2; p.dh0 = dh0;
  p.B = B; p.T = T; p.H = H; p.V = V;
  hipError_t e = gdn::launch_dhu(p, dtype == GDN_DTYPE_F32 ? 0 : 1, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "gdn_bwd_dhu launch");
  return ok();
}

int gdn_bwd_prep(const void* q, const void* k, const float* beta, const float* g, const float* gk,
                 const void* do_, float scale, void* w, void* dv, int B, int T, int H, int K, int V,
                 int dtype, void* stream) {
  if (!q || !k || !beta || !do_ || !w || !dv)
    return fail(GDN_ERR_INVALID, "q, k, beta, do, w and dv must be non-null");
  if (B <= 0 || T <= 0 || H <= 0 || K <= 0 || V <= 0)
    return fail(GDN_ERR_INVALID, "B, T, H, K, V must be positive (got %d, %d, %d, %d, %d)", B, T,
                H, K, V);
  if (dtype != GDN_DTYPE_F32 && dtype != GDN_DTYPE_BF16)
    return fail(GDN_ERR_INVALID, "dtype must be GDN_DTYPE_F32 or GDN_DTYPE_BF16, got %d", dtype);
  if ((K != 64 && K != 128) || (V != 64 && V != 128))
    return fail(GDN_ERR_UNSUPPORTED, "K and V must be 64 or 128 (got %d, %d)", K, V);
  if (gk) return fail(GDN_ERR_UNSUPPORTED, "gdn_bwd_prep takes scalar gates only (gk must be NULL)");
  if ((int64_t)B * H * ((T + GDN_CHUNK - 1) / GDN_CHUNK) > INT32_MAX)
    return fail(GDN_ERR_INVALID, "B*H*chunks exceeds the grid limit");
  gdn::BwdPrepParams p{};
  p.q = q; p.k = k; p.beta = beta; p.g = g; p.do_ = do_; p.scale = scale; p.w = w; p.dv = dv;
  p.B = B; p.T = T; p.H = H;
  hipError_t e = gdn::launch_bwd_prep(p, K, V, dtype == GDN_DTYPE_F32 ? 0 : 1,
                                      static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "gdn_bwd_prep launch");
  return ok();
}

size_t gdn_state_grad_summary_workspace_bytes(int B, int T, int H, int V, int dtype) {
  if (B <= 0 || T <= 0 || H <= 0 || V <= 0 || (dtype != GDN_DTYPE_F32 && dtype != GDN_DTYPE_BF16))
    return 0;
  return al256((size_t)B * T * H * V * (dtype == GDN_DTYPE_BF16 ? 2 : 4));
}

int gdn_state_grad_summary(const void* q, const void* k, const void* w, const void* do_,
                           const void* dv, const float* g, const float* gk, float scale,
                           float* grad_state_ext, int B, int T, int H, int K, int V, int dtype,
                           void* workspace, size_t workspace_bytes, void* stream) {
  if (!grad_state_ext) return fail(GDN_ERR_INVALID, "grad_state_ext must be non-null");
  if (T <= 0) return fail(GDN_ERR_INVALID, "a state summary needs a nonempty fragment (T = %d)", T);
  if (B <= 0 || H <= 0 || K <= 0 || V <= 0)
    return fail(GDN_ERR_INVALID, "B, H, K, V must be positive (got %d, %d, %d, %d)", B, H, K, V);
  const size_t need = gdn_state_grad_summary_workspace_bytes(B, T, H, V, dtype);
  if (need && (!workspace || workspace_bytes < need))
    return fail(GDN_ERR_WORKSPACE, "workspace of %zu bytes needed, got %zu", need, workspace_bytes);
  if (reinterpret_cast<uintptr_t>(workspace) % 256)
    return fail(GDN_ERR_INVALID, "workspace must be 256-byte aligned");
  return gdn_bwd_dhu(q, k, w, do_, dv, g, gk, nullptr, scale, nullptr, workspace, grad_state_ext,
                     B, T, H, K, V, dtype, stream);
}

int gdn_state_grad_apply(const float* grad_state_ext, const float* transition, const float* grad_in,
                         float* grad_out, int BH, int K, int V, void* stream) {
  if (!grad_state_ext || !grad_out || (grad_in && !transition))
    return fail(GDN_ERR_INVALID, "grad_state_ext and grad_out must be non-null, and transition too when grad_in is");
  if (BH <= 0 || K <= 0 || V <= 0) return fail(GDN_ERR_INVALID, "BH, K, V must be positive (got %d, %d, %d)", BH, K, V);
  if (K > gdn::kApplyMaxK) return fail(GDN_ERR_UNSUPPORTED, "K must be <= %d, got %d", gdn::kApplyMaxK, K);
  if (BH > 65535) return fail(GDN_ERR_INVALID, "BH must be <= 65535, got %d", BH);
  const uintptr_t bytes = (uintptr_t)BH * K * V * 4;
  const uintptr_t a0 = reinterpret_cast<uintptr_t>(grad_out), b0 = reinterpret_cast<uintptr_t>(grad_in);
  if (grad_in && a0 < b0 + bytes && b0 < a0 + bytes) return fail(GDN_ERR_INVALID, "grad_out must not overlap grad_in");
  hipError_t e = gdn::launch_grad_apply(grad_state_ext, transition, grad_in, grad_out, BH, K, V,
                                        static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "gdn_state_grad_apply launch");
  return ok();
}

size_t gdn_bwd_dhu_varlen_workspace_bytes(int N, int NT_total) {
  if (N <= 0 || NT_total <= 0) return 0;
  return al256((size_t)(N + 1) * 4) + al256((size_t)NT_total * 2 * 4);
}

int gdn_bwd_dhu_varlen(const void* q, const void* k, const void* w, const void* do_,
                       const void* dv, const float* g, const float* gk, const float* dht,
                       float scale, const int* cu_seqlens, const int* cu_seqlens_host, int N, float* dh_chunks,
                       void* dv2, float* dh0, int T_total, int H, int K, int V, int dtype,
                       void* workspace, size_t workspace_bytes, void* stream) {
  if (!q || !k || !w || !do_ || !dv || !dv2)
    return fail(GDN_ERR_INVALID, "q, k, w, do, dv and dv2 must be non-null");
  if (!cu_seqlens || !cu_seqlens_host)
    return fail(GDN_ERR_INVALID, "cu_seqlens (device) and cu_seqlens_host must be non-null");
  if (N < 1 || T_total < 1 || H <= 0 || K <= 0 || V <= 0)
    return fail(GDN_ERR_INVALID, "N, T_total, H, K, V must be positive (got %d, %d, %d, %d, %d)", N,
                T_total, H, K, V);
  if (dtype != GDN_DTYPE_F32 && dtype != GDN_DTYPE_BF16)
    return fail(GDN_ERR_INVALID, "dtype must be GDN_DTYPE_F32 or GDN_DTYPE_BF16, got %d", dtype);
  if (cu_seqlens_host[0] != 0) return fail(GDN_ERR_INVALID, "cu_seqlens[0] must be 0 (got %d)", cu_seqlens_host[0]);
  for (int i = 0; i < N; ++i)
    if (cu_seqlens_host[i + 1] <= cu_seqlens_host[i])
      return fail(GDN_ERR_INVALID, "cu_seqlens must be strictly increasing (sequence %d is empty or negative)", i);
  if (cu_seqlens_host[N] != T_total)
    return fail(GDN_ERR_INVALID, "cu_seqlens[N] = %d differs from T_total = %d", cu_seqlens_host[N], T_total);
  if (K != 128) return fail(GDN_ERR_UNSUPPORTED, "K must be 128, got %d", K);
  if (V % 32) return fail(GDN_ERR_UNSUPPORTED, "V must be a multiple of 32, got %d", V);
  if (gk && dtype == GDN_DTYPE_F32)
    return fail(GDN_ERR_UNSUPPORTED, "per-key gates need bf16 inputs");
  const int nt = gdn_varlen_num_chunks(cu_seqlens_host, N);
  if (nt < 0) return fail(GDN_ERR_INVALID, "too many chunks");
  if ((int64_t)N * H * (V / 32) > INT32_MAX) return fail(GDN_ERR_INVALID, "N*H*V/32 exceeds the grid limit");
  const size_t need = gdn_bwd_dhu_varlen_workspace_bytes(N, nt);
  if (!workspace || workspace_bytes < need)
    return fail(GDN_ERR_WORKSPACE, "workspace of %zu bytes needed, got %zu", need, workspace_bytes);
  if (reinterpret_cast<uintptr_t>(workspace) % 256)
    return fail(GDN_ERR_INVALID, "workspace must be 256-byte aligned");
  hipStream_t st = static_cast<hipStream_t>(stream);
  int* coffs = static_cast<int*>(workspace);
  int* cidx = reinterpret_cast<int*>(static_cast<char*>(workspace) + al256((size_t)(N + 1) * 4));
  hipError_t e = gdn::launch_varlen_tables(cu_seqlens, N, coffs, cidx, st);
  if (e != hipSuccess) return hip_fail(e, "varlen table launch");
  gdn::DhuParams p{};
  p.q = q; p.k = k; p.w = w; p.do_ = do_; p.dv = dv; p.g = g; p.gk = gk; p.dht = dht; p.scale = scale;
  p.dh_chunks = dh_chunks; p.dv2 = dv2; p.dh0 = dh0;
  p.B = N; p.T = T_total; p.H = H; p.V = V;
  p.cu = cu_seqlens; p.coffs = coffs; p.nt_total = nt;
  e = gdn::launch_dhu(p, dtype == GDN_DTYPE_F32 ? 0 : 1, st);
  if (e != hipSuccess) return hip_fail(e, "gdn_bwd_dhu_varlen launch");
  return ok();
}

}  // extern "C"

// C ABI of libwallattn: host-side validation, workspace carving, launches.
// Entry points and their contracts are documented in include/wallattn.h.
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include "../../include/wallattn.h"
#include "common.h"
#include "launch.h"

namespace {

thread_local char g_err[512] = "";

int fail(int code, const char *fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return code;
}

int ok() {
  g_err[0] = '\0';
  return WA_OK;
}

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Checks shared by the prefill entry points; fills the problem description.
int check_fwd_shape(int64_t B, int64_t T, int64_t HQ, int64_t H, int64_t K, int64_t V,
                    bool varlen, int64_t num_seqs, int64_t max_seqlen, int dtype,
                    wa::FwdProblem *p) {
  if (B < 1 || T < 1 || HQ < 1 || H < 1 || K < 1 || V < 1)
    return fail(WA_INVALID_ARG, "sizes must be positive (B=%lld T=%lld HQ=%lld H=%lld K=%lld V=%lld)",
                (long long)B, (long long)T, (long long)HQ, (long long)H, (long long)K, (long long)V);
  if (HQ % H != 0) return fail(WA_INVALID_ARG, "HQ (%lld) must be a multiple of H (%lld)", (long long)HQ, (long long)H);
  if (dtype != WA_BF16 && dtype != WA_F32) return fail(WA_UNSUPPORTED, "dtype %d not supported", dtype);
  if ((K != 64 && K != 128) || (V != 64 && V != 128))
    return fail(WA_UNSUPPORTED, "head dims K=%lld V=%lld not supported (64 or 128)", (long long)K, (long long)V);
  if (varlen) {
    if (B != 1) return fail(WA_INVALID_ARG, "cu_seqlens requires B == 1 (got B=%lld)", (long long)B);
    if (num_seqs < 1 || max_seqlen < 1 || max_seqlen > T)
      return fail(WA_INVALID_ARG, "cu_seqlens needs num_seqs >= 1 and 1 <= max_seqlen <= T");
  } else if (num_seqs != 0 || max_seqlen != 0) {
    // tolerated: ignored without cu_seqlens
  }
  // index arithmetic inside kernels uses 32-bit grid dimensions
  const int64_t nseg = varlen ? num_seqs : B;
  const int64_t maxlen = varlen ? max_seqlen : T;
  const int64_t ntok = varlen ? T : B * T;
  if (nseg > 65535 || HQ > 65535 || ((maxlen + 63) / 64 + 8) * HQ * nseg >= (int64_t)1 << 31)
    return fail(WA_UNSUPPORTED, "problem too large for the launch grid");
  // the bf16 attention kernel addresses one sequence's queries, values and
  // gate sums (token-major) and one head's rescaled keys (K+16 channels per
  // row) with 32-bit byte offsets
  const int64_t row_bf16 = HQ * (K > V ? K : V) > K + 16 ? HQ * (K > V ? K : V) : K + 16;
  if (dtype == WA_BF16 && maxlen * row_bf16 * 2 >= ((int64_t)1 << 31))
    return fail(WA_UNSUPPORTED,
                "sequence of %lld tokens too long for bf16 (max_seqlen*max(HQ*max(K,V), K+16)*2 must be < 2^31)",
                (long long)maxlen);
  if (p) {
    p->B = B; p->T = T; p->HQ = HQ; p->H = H; p->K = K; p->V = V;
    p->nseg = nseg; p->maxlen = maxlen; p->ntok = ntok; p->dtype = dtype;
  }
  return WA_OK;
}

}  // namespace

extern "C" {

const char *wall_attn_last_error(void) { return g_err; }

size_t wall_attn_fwd_workspace_bytes(int64_t B, int64_t T, int64_t HQ, int64_t H, int64_t K,
                                     int64_t V, int64_t num_seqs, int64_t max_seqlen, int dtype) {
  wa::FwdProblem p{};
  const bool varlen = num_seqs > 0;
  if (check_fwd_shape(B, T, HQ, H, K, V, varlen, num_seqs, max_seqlen, dtype, &p) != WA_OK) return 0;
  return wa::fwd_workspace_layout(p, nullptr, nullptr);
}

namespace {

enum FwdStage { STAGE_PREPARE = 1, STAGE_ATTEND = 2 };

int fwd_impl(int stages, const char *name, const void *q, const void *k, const void *v,
             const void *g, const void *g_scalar, const float *sink_bias, void *o, float *lse,
             int64_t B, int64_t T, int64_t HQ, int64_t H, int64_t K, int64_t V,
             const int32_t *cu_seqlens, int64_t num_seqs, int64_t max_seqlen,
             int64_t window_size, float scale, int dtype, void *workspace, size_t workspace_bytes,
             struct ihipStream_t *stream) {
  wa::FwdProblem p{};
  int rc = check_fwd_shape(B, T, HQ, H, K, V, cu_seqlens != nullptr, num_seqs, max_seqlen, dtype, &p);
  if (rc != WA_OK) return rc;
  const bool need_inputs = (stages & STAGE_PREPARE) != 0;
  const bool need_outputs = (stages & STAGE_ATTEND) != 0;
  // the attention stage reads q and g as well (it forms the rescaled queries)
  if ((need_inputs && (!q || !k || !g)) || (need_outputs && (!q || !g || !v || !o)) || !workspace)
    return fail(WA_INVALID_ARG, "%s: required pointers must be non-NULL", name);
  const void *ptrs[] = {q, k, v, g, g_scalar, sink_bias, o, lse, workspace};
  for (const void *ptr : ptrs)
    if (ptr && !aligned16(ptr)) return fail(WA_INVALID_ARG, "device pointers must be 16-byte aligned");
  const int64_t nblocks = ((p.maxlen + wa::CHUNK - 1) / wa::CHUNK) * p.nseg * HQ;
  if (nblocks > 2147483647LL) return fail(WA_UNSUPPORTED, "problem too large for the launch grid");
  const size_t need = wa::fwd_workspace_layout(p, nullptr, nullptr);
  if (workspace_bytes < need)
    return fail(WA_WORKSPACE_TOO_SMALL, "workspace has %zu bytes, needs %zu", workspace_bytes, need);
  p.q = q; p.k = k; p.v = v; p.g = g; p.g_scalar = g_scalar; p.sink = sink_bias;
  p.o = o; p.lse = lse; p.cu = cu_seqlens;
  p.window = window_size > 0 ? window_size : 0;
  p.scale = scale > 0.f ? scale : 1.0f / sqrtf((float)K);
  wa::FwdWorkspace ws{};
  wa::fwd_workspace_layout(p, &ws, static_cast<char *>(workspace));
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  hipError_t e = hipSuccess;
  if (stages & STAGE_PREPARE) e = wa::launch_prefix_phases(p, ws, st);
  if (e == hipSuccess && (stages & STAGE_ATTEND)) e = wa::launch_attn_fwd(p, ws, st);
  if (e != hipSuccess) return fail(WA_HIP_ERROR, "%s launch failed: %s", name, hipGetErrorString(e));
  return ok();
}

}  // namespace

int wall_attn_fwd(const void *q, const void *k, const void *v, const void *g, const void *g_scalar,
                  const float *sink_bias, void *o, float *lse, int64_t B, int64_t T, int64_t HQ,
                  int64_t H, int64_t K, int64_t V, const int32_t *cu_seqlens, int64_t num_seqs,
                  int64_t max_seqlen, int64_t window_size, float scale, int dtype, void *workspace,
                  size_t workspace_bytes, struct ihipStream_t *stream) {
  return fwd_impl(STAGE_PREPARE | STAGE_ATTEND, "wall_attn_fwd", q, k, v, g, g_scalar, sink_bias, o,
                  lse, B, T, HQ, H, K, V, cu_seqlens, num_seqs, max_seqlen, window_size, scale,
                  dtype, workspace, workspace_bytes, stream);
}

int wall_attn_fwd_prepare(const void *q, const void *k, const void *g, const void *g_scalar,
                          int64_t B, int64_t T, int64_t HQ, int64_t H, int64_t K, int64_t V,
                          const int32_t *cu_seqlens, int64_t num_seqs, int64_t max_seqlen,
                          float scale, int dtype, void *workspace, size_t workspace_bytes,
                          struct ihipStream_t *stream) {
  return fwd_impl(STAGE_PREPARE, "wall_attn_fwd_prepare", q, k, nullptr, g, g_scalar, nullptr,
                  nullptr, nullptr, B, T, HQ, H, K, V, cu_seqlens, num_seqs, max_seqlen, 0, scale,
                  dtype, workspace, workspace_bytes, stream);
}

int wall_attn_fwd_attend(const void *q, const void *v, const void *g, const void *g_scalar,
                         const float *sink_bias, void *o, float *lse, int64_t B, int64_t T,
                         int64_t HQ, int64_t H, int64_t K, int64_t V, const int32_t *cu_seqlens,
                         int64_t num_seqs, int64_t max_seqlen, int64_t window_size, float scale,
                         int dtype, void *workspace, size_t workspace_bytes,
                         struct ihipStream_t *stream) {
  return fwd_impl(STAGE_ATTEND, "wall_attn_fwd_attend", q, nullptr, v, g, g_scalar, sink_bias, o,
                  lse, B, T, HQ, H, K, V, cu_seqlens, num_seqs, max_seqlen, window_size, scale,
                  dtype, workspace, workspace_bytes, stream);
}

size_t wall_attn_prefix_log2_workspace_bytes(int64_t B, int64_t T, int64_t HQ, int64_t K,
                                             int64_t num_seqs, int64_t max_seqlen) {
  const bool varlen = num_seqs > 0;
  if (check_fwd_shape(B, T, HQ, 1, K, 64, varlen, num_seqs, max_seqlen, WA_F32, nullptr) != WA_OK) return 0;
  return wa::prefix_workspace_layout(varlen ? num_seqs : B, varlen ? max_seqlen : T, HQ, K, nullptr, nullptr);
}

int wall_attn_prefix_log2(const void *g, float *P2, int64_t B, int64_t T, int64_t HQ, int64_t K,
                          const int32_t *cu_seqlens, int64_t num_seqs, int64_t max_seqlen,
                          int dtype, void *workspace, size_t workspace_bytes,
                          struct ihipStream_t *stream) {
  const bool varlen = cu_seqlens != nullptr;
  int rc = check_fwd_shape(B, T, HQ, 1, K, 64, varlen, num_seqs, max_seqlen, dtype, nullptr);
  if (rc != WA_OK) return rc;
  if (!g || !P2 || !workspace) return fail(WA_INVALID_ARG, "g, P2 and workspace must be non-NULL");
  if (!aligned16(g) || !aligned16(P2) || !aligned16(workspace))
    return fail(WA_INVALID_ARG, "device pointers must be 16-byte aligned");
  const int64_t nseg = varlen ? num_seqs : B, maxlen = varlen ? max_seqlen : T;
  float *csum = nullptr;
  const size_t need = wa::prefix_workspace_layout(nseg, maxlen, HQ, K, &csum, static_cast<char *>(workspace));
  if (workspace_bytes < need)
    return fail(WA_WORKSPACE_TOO_SMALL, "workspace has %zu bytes, needs %zu", workspace_bytes, need);
  hipError_t e = wa::launch_prefix_log2(g, P2, cu_seqlens, T, HQ, K, nseg, maxlen, dtype, csum,
                                        reinterpret_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(WA_HIP_ERROR, "wall_attn_prefix_log2 launch failed: %s", hipGetErrorString(e));
  return ok();
}

int wall_attn_build_kv_cache(const void *k, const float *P2, void *k_tilde, float *r_cache,
                             int64_t B, int64_t T_kv, int64_t HQ, int64_t H, int64_t K,
                             int64_t chunk_size, int dtype, struct ihipStream_t *stream) {
  int rc = check_fwd_shape(B, T_kv, HQ, H, K, 64, false, 0, 0, dtype, nullptr);
  if (rc != WA_OK) return rc;
  if (chunk_size != wa::CHUNK) return fail(WA_UNSUPPORTED, "chunk_size %lld not supported (64)", (long long)chunk_size);
  if (!k || !P2 || !k_tilde || !r_cache) return fail(WA_INVALID_ARG, "k, P2, k_tilde and r_cache must be non-NULL");
  if (!aligned16(k) || !aligned16(P2) || !aligned16(k_tilde) || !aligned16(r_cache))
    return fail(WA_INVALID_ARG, "device pointers must be 16-byte aligned");
  if (((T_kv + 63) / 64 + 8) * HQ > 2147483647LL || B > 65535) return fail(WA_UNSUPPORTED, "problem too large for the launch grid");
  hipError_t e = wa::launch_build_cache(k, P2, k_tilde, r_cache, B, T_kv, HQ, H, K, dtype,
                                        reinterpret_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(WA_HIP_ERROR, "wall_attn_build_kv_cache launch failed: %s", hipGetErrorString(e));
  return ok();
}

size_t wall_attn_decode_workspace_bytes(int64_t B, int64_t T_kv, int64_t HQ, int64_t H, int64_t K,
                                        int64_t V, int64_t chunk_size) {
  if (check_fwd_shape(B, T_kv, HQ, H, K, V, false, 0, 0, WA_BF16, nullptr) != WA_OK) return 0;
  if (chunk_size != wa::CHUNK) return 0;
  return wa::decode_workspace_size(B, T_kv, HQ, H, V);
}

int wall_attn_decode(const void *q, const void *v, const float *p_curr, const void *k_tilde,
                     const float *r_cache, const float *sink_bias, void *o, float *lse, int64_t B,
                     int64_t T_kv, int64_t HQ, int64_t H, int64_t K, int64_t V, int64_t chunk_size,
                     float scale, int dtype, void *workspace, size_t workspace_bytes,
                     struct ihipStream_t *stream) {
  int rc = check_fwd_shape(B, T_kv, HQ, H, K, V, false, 0, 0, dtype, nullptr);
  if (rc != WA_OK) return rc;
  if (chunk_size != wa::CHUNK) return fail(WA_UNSUPPORTED, "chunk_size %lld not supported (64)", (long long)chunk_size);
  if (!q || !v || !p_curr || !k_tilde || !r_cache || !o || !workspace)
    return fail(WA_INVALID_ARG, "q, v, p_curr, k_tilde, r_cache, o and workspace must be non-NULL");
  const void *ptrs[] = {q, v, p_curr, k_tilde, r_cache, sink_bias, o, lse, workspace};
  for (const void *ptr : ptrs)
    if (ptr && !aligned16(ptr)) return fail(WA_INVALID_ARG, "device pointers must be 16-byte aligned");
  if (B > 65535) return fail(WA_UNSUPPORTED, "B too large for the launch grid");
  // the decode kernel addresses one batch row's k_tilde with 32-bit byte offsets
  if (T_kv * HQ * K * (dtype == WA_BF16 ? 2 : 4) >= ((int64_t)1 << 31))
    return fail(WA_UNSUPPORTED, "cache of %lld tokens too long (T_kv*HQ*K*operand bytes must be < 2^31)",
                (long long)T_kv);
  const size_t need = wa::decode_workspace_size(B, T_kv, HQ, H, V);
  if (workspace_bytes < need)
    return fail(WA_WORKSPACE_TOO_SMALL, "workspace has %zu bytes, needs %zu", workspace_bytes, need);
  wa::DecodeProblem p{};
  p.q = q; p.v = v; p.kt = k_tilde; p.p_curr = p_curr; p.rc = r_cache; p.sink = sink_bias;
  p.o = o; p.lse = lse; p.B = B; p.T = T_kv; p.HQ = HQ; p.H = H; p.K = K; p.V = V;
  p.scale = scale > 0.f ? scale : 1.0f / sqrtf((float)K);
  p.dtype = dtype;
  hipError_t e = wa::launch_decode(p, workspace, reinterpret_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(WA_HIP_ERROR, "wall_attn_decode launch failed: %s", hipGetErrorString(e));
  return ok();
}

}  // extern "C"

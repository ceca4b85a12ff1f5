// C ABI of libwallattn: host-side validation, workspace carving, launches.
// Entry points and their contracts are documented in include/wallattn.h.
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <mutex>

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

// A dispatch's work-items per grid dimension are a 32-bit count.
bool grid_fits(int64_t blocks, int64_t threads) { return blocks * threads < ((int64_t)1 << 32); }

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
  // grids: the attention kernel's (query tiles x segments x heads) and the
  // pre-pass's (chunk, head) pairs of 256-thread workgroups, plus padding
  if (nseg > 65535 || HQ > 65535 || !grid_fits(((maxlen + 63) / 64 + 8) * HQ * nseg, 256))
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
  // (the attention kernels also take the (segment, head) pairs the pre-pass
  // flagged as out of the anchored operands' range, on their exact path)
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

size_t wall_attn_bwd_workspace_bytes(int64_t B, int64_t T, int64_t HQ, int64_t H, int64_t K,
                                     int64_t V, int64_t num_seqs, int64_t max_seqlen, int dtype) {
  wa::FwdProblem p{};
  const bool varlen = num_seqs > 0;
  if (check_fwd_shape(B, T, HQ, H, K, V, varlen, num_seqs, max_seqlen, dtype, &p) != WA_OK) return 0;
  return wa::fwd_workspace_layout(p, nullptr, nullptr) + wa::bwd_workspace_layout(p, nullptr, nullptr);
}

int wall_attn_bwd(const void *q, const void *k, const void *v, const void *g,
                  const void *g_scalar, const float *sink_bias, const void *o, const float *lse,
                  const void *dO, void *dq, void *dk, void *dv, void *dg, void *dg_scalar,
                  float *dsink, int64_t B, int64_t T, int64_t HQ, int64_t H, int64_t K, int64_t V,
                  const int32_t *cu_seqlens, int64_t num_seqs, int64_t max_seqlen,
                  int64_t window_size, float scale, int dtype, void *workspace,
                  size_t workspace_bytes, struct ihipStream_t *stream) {
  wa::BwdProblem b{};
  int rc = check_fwd_shape(B, T, HQ, H, K, V, cu_seqlens != nullptr, num_seqs, max_seqlen, dtype, &b.f);
  if (rc != WA_OK) return rc;
  if (!q || !k || !v || !g || !o || !lse || !dO || !dq || !dk || !dv || !dg || !workspace)
    return fail(WA_INVALID_ARG, "wall_attn_bwd: q, k, v, g, o, lse, dO, dq, dk, dv, dg and workspace must be non-NULL");
  if ((g_scalar == nullptr) != (dg_scalar == nullptr))
    return fail(WA_INVALID_ARG, "wall_attn_bwd: g_scalar and dg_scalar must be given together");
  if (dsink != nullptr && sink_bias == nullptr)
    return fail(WA_INVALID_ARG, "wall_attn_bwd: dsink needs sink_bias");
  const void *ptrs[] = {q, k, v, g, g_scalar, sink_bias, o, lse, dO, dq, dk, dv, dg, dg_scalar,
                        dsink, workspace};
  for (const void *ptr : ptrs)
    if (ptr && !aligned16(ptr)) return fail(WA_INVALID_ARG, "device pointers must be 16-byte aligned");
  const size_t nf = wa::fwd_workspace_layout(b.f, nullptr, nullptr);
  const size_t need = nf + wa::bwd_workspace_layout(b.f, nullptr, nullptr);
  if (workspace_bytes < need)
    return fail(WA_WORKSPACE_TOO_SMALL, "workspace has %zu bytes, needs %zu", workspace_bytes, need);
  wa::FwdProblem &p = b.f;
  p.q = q; p.k = k; p.v = v; p.g = g; p.g_scalar = g_scalar; p.sink = sink_bias;
  p.o = nullptr; p.lse = nullptr; p.cu = cu_seqlens;
  p.window = window_size > 0 ? window_size : 0;
  p.scale = scale > 0.f ? scale : 1.0f / sqrtf((float)K);
  b.o = o; b.dO = dO; b.lse = lse; b.dq = dq; b.dk = dk; b.dv = dv; b.dg = dg; b.dgs = dg_scalar;
  b.dsink = dsink;
  wa::FwdWorkspace ws{};
  wa::fwd_workspace_layout(p, &ws, static_cast<char *>(workspace));
  wa::BwdWorkspace bw{};
  wa::bwd_workspace_layout(p, &bw, static_cast<char *>(workspace) + nf);
  ws.qbh = bw.qbh;  // the pre-pass also writes the backward's half query operand
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  // the running sums (chunk offsets, gate sums) come from the forward's pre-pass
  hipError_t e = wa::launch_prefix_phases(p, ws, st);
  if (e == hipSuccess) e = wa::launch_attn_bwd(b, ws, bw, st);
  if (e != hipSuccess) return fail(WA_HIP_ERROR, "wall_attn_bwd launch failed: %s", hipGetErrorString(e));
  return ok();
}

size_t wall_attn_prefix_log2_workspace_bytes(int64_t B, int64_t T, int64_t HQ, int64_t K,
                                             int64_t num_seqs, int64_t max_seqlen) {
  const bool varlen = num_seqs > 0;
  if (check_fwd_shape(B, T, HQ, 1, K, 64, varlen, num_seqs, max_seqlen, WA_F32, nullptr) != WA_OK) return 0;
  return wa::prefix_workspace_layout(varlen ? num_seqs : B, varlen ? max_seqlen : T, HQ, K);
}

int wall_attn_prefix_log2(const void *g, const void *g_scalar, float *P2, float *G2, int64_t B,
                          int64_t T, int64_t HQ, int64_t K, const int32_t *cu_seqlens,
                          int64_t num_seqs, int64_t max_seqlen, int dtype, void *workspace,
                          size_t workspace_bytes, struct ihipStream_t *stream) {
  const bool varlen = cu_seqlens != nullptr;
  int rc = check_fwd_shape(B, T, HQ, 1, K, 64, varlen, num_seqs, max_seqlen, dtype, nullptr);
  if (rc != WA_OK) return rc;
  if (!g || !P2 || !workspace) return fail(WA_INVALID_ARG, "g, P2 and workspace must be non-NULL");
  if ((g_scalar == nullptr) != (G2 == nullptr))
    return fail(WA_INVALID_ARG, "g_scalar and G2 must be given together");
  const void *ptrs[] = {g, g_scalar, P2, G2, workspace};
  for (const void *ptr : ptrs)
    if (ptr && !aligned16(ptr)) return fail(WA_INVALID_ARG, "device pointers must be 16-byte aligned");
  const int64_t nseg = varlen ? num_seqs : B, maxlen = varlen ? max_seqlen : T;
  const size_t need = wa::prefix_workspace_layout(nseg, maxlen, HQ, K);
  if (workspace_bytes < need)
    return fail(WA_WORKSPACE_TOO_SMALL, "workspace has %zu bytes, needs %zu", workspace_bytes, need);
  hipError_t e = wa::launch_prefix_log2(g, g_scalar, P2, G2, cu_seqlens, T, HQ, K, nseg, maxlen,
                                        dtype, workspace, reinterpret_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(WA_HIP_ERROR, "wall_attn_prefix_log2 launch failed: %s", hipGetErrorString(e));
  return ok();
}

}  // extern "C"

namespace {

size_t elem_bytes(int dt) { return dt == WA_F32 ? 4 : 2; }

// Shape checks shared by the decode-cache entry points.
int check_cache_shape(int64_t B, int64_t T, int64_t HQ, int64_t H, int64_t K, int64_t V,
                      int64_t chunk_size, int dtype, int cache_dtype) {
  if (B < 1 || T < 1 || HQ < 1 || H < 1 || K < 1 || V < 1)
    return fail(WA_INVALID_ARG, "sizes must be positive (B=%lld T=%lld HQ=%lld H=%lld K=%lld V=%lld)",
                (long long)B, (long long)T, (long long)HQ, (long long)H, (long long)K, (long long)V);
  if (HQ % H != 0) return fail(WA_INVALID_ARG, "HQ (%lld) must be a multiple of H (%lld)", (long long)HQ, (long long)H);
  if (dtype != WA_BF16 && dtype != WA_F32) return fail(WA_UNSUPPORTED, "dtype %d not supported", dtype);
  if (cache_dtype != WA_BF16 && cache_dtype != WA_F32 && cache_dtype != WA_F16)
    return fail(WA_UNSUPPORTED, "cache_dtype %d not supported", cache_dtype);
  if ((K != 64 && K != 128) || (V != 64 && V != 128))
    return fail(WA_UNSUPPORTED, "head dims K=%lld V=%lld not supported (64 or 128)", (long long)K, (long long)V);
  if (chunk_size != wa::CHUNK) return fail(WA_UNSUPPORTED, "chunk_size %lld not supported (64)", (long long)chunk_size);
  // grids: the cache build's (chunk, head) pairs and the decode combine's
  // (row, head) workgroups
  if (B > 65535 || HQ > 65535 || T >= ((int64_t)1 << 31) - wa::CHUNK ||
      !grid_fits(((T + 63) / 64 + 8) * HQ, 256) || !grid_fits(B * HQ, 128))
    return fail(WA_UNSUPPORTED, "problem too large for the launch grid or 32-bit token positions");
  // one chunk of one head is addressed with 32-bit byte offsets
  if ((int64_t)wa::CHUNK * HQ * K * 4 >= ((int64_t)1 << 31) || (int64_t)wa::CHUNK * H * V * 4 >= ((int64_t)1 << 31))
    return fail(WA_UNSUPPORTED, "HQ*K or H*V too large for 32-bit chunk offsets");
  return WA_OK;
}

// Paged-layout arguments: either block_table == NULL (contiguous rows of
// T tokens per batch row) or pages of page_size tokens.
int check_pages(const int32_t *block_table, int64_t max_blocks, int64_t page_size,
                int64_t num_pages, int64_t *T) {
  if (block_table == nullptr) return WA_OK;
  if (page_size < wa::CHUNK || page_size % wa::CHUNK != 0 || max_blocks < 1 || num_pages < 1 ||
      num_pages >= ((int64_t)1 << 31) / page_size || max_blocks * page_size >= ((int64_t)1 << 31) - wa::CHUNK)
    return fail(WA_INVALID_ARG, "paged cache needs page_size a positive multiple of 64, max_blocks >= 1, "
                                "1 <= num_pages and 32-bit token positions");
  if (!aligned16(block_table)) return fail(WA_INVALID_ARG, "device pointers must be 16-byte aligned");
  *T = max_blocks * page_size;
  return WA_OK;
}

int64_t decode_max_chunks(int64_t T, int64_t window) {
  const int64_t nc = (T + wa::CHUNK - 1) / wa::CHUNK;
  if (window <= 0) return nc;
  const int64_t nw = (window + wa::CHUNK - 2) / wa::CHUNK + 1;  // chunks a window of W keys can touch
  return nw < nc ? nw : nc;
}

int decode_impl(const char *name, const void *q, const void *v, const float *p_curr,
                const void *k_tilde, const float *r_cache, const float *sink_bias,
                const float *gate_cache, const float *gate_curr, void *o, float *lse, int64_t B,
                int64_t T_kv, int64_t HQ, int64_t H, int64_t K, int64_t V, int64_t chunk_size,
                float scale, int dtype, int cache_dtype, const int32_t *cache_seqlens,
                int64_t window_size, const int32_t *block_table, int64_t max_blocks,
                int64_t page_size, int64_t num_pages, void *workspace, size_t workspace_bytes,
                struct ihipStream_t *stream) {
  int64_t T = T_kv;
  int rc = check_pages(block_table, max_blocks, page_size, num_pages, &T);
  if (rc != WA_OK) return rc;
  rc = check_cache_shape(B, T, HQ, H, K, V, chunk_size, dtype, cache_dtype);
  if (rc != WA_OK) return rc;
  if (!q || !v || !p_curr || !k_tilde || !r_cache || !o || !workspace)
    return fail(WA_INVALID_ARG, "%s: q, v, p_curr, k_tilde, r_cache, o and workspace must be non-NULL", name);
  if ((gate_cache == nullptr) != (gate_curr == nullptr))
    return fail(WA_INVALID_ARG, "%s: gate_cache and gate_curr must be given together", name);
  if (window_size < 0) return fail(WA_INVALID_ARG, "%s: window_size must be >= 0 (0: none)", name);
  const void *ptrs[] = {q, v, p_curr, k_tilde, r_cache, sink_bias, gate_cache, gate_curr, o, lse,
                        cache_seqlens, workspace};
  for (const void *ptr : ptrs)
    if (ptr && !aligned16(ptr)) return fail(WA_INVALID_ARG, "device pointers must be 16-byte aligned");
  const int64_t nch = decode_max_chunks(T, window_size);
  const size_t need = wa::decode_workspace_size(B, (T + wa::CHUNK - 1) / wa::CHUNK, HQ, H, V);
  if (workspace_bytes < need)
    return fail(WA_WORKSPACE_TOO_SMALL, "workspace has %zu bytes, needs %zu", workspace_bytes, need);
  wa::DecodeProblem p{};
  p.q = q; p.v = v; p.kt = k_tilde; p.p_curr = p_curr; p.rc = r_cache; p.sink = sink_bias;
  p.gs_cache = gate_cache; p.gs_curr = gate_curr; p.seqlens = cache_seqlens;
  p.block_table = block_table; p.max_blocks = max_blocks; p.page_size = page_size;
  p.num_pages = num_pages; p.window = window_size >= T ? 0 : window_size; p.max_chunks = nch;
  p.o = o; p.lse = lse; p.B = B; p.T = T; p.HQ = HQ; p.H = H; p.K = K; p.V = V;
  p.scale = scale > 0.f ? scale : 1.0f / sqrtf((float)K);
  p.dtype = dtype;
  p.cache_dtype = cache_dtype;
  hipError_t e = wa::launch_decode(p, workspace, reinterpret_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(WA_HIP_ERROR, "%s launch failed: %s", name, hipGetErrorString(e));
  return ok();
}

}  // namespace

extern "C" {

int wall_attn_build_kv_cache(const void *k, const float *P2, void *k_tilde, float *r_cache,
                             int64_t B, int64_t T_kv, int64_t HQ, int64_t H, int64_t K,
                             int64_t chunk_size, int dtype, int cache_dtype,
                             struct ihipStream_t *stream) {
  int rc = check_cache_shape(B, T_kv, HQ, H, K, 64, chunk_size, dtype, cache_dtype);
  if (rc != WA_OK) return rc;
  if (!k || !P2 || !k_tilde || !r_cache) return fail(WA_INVALID_ARG, "k, P2, k_tilde and r_cache must be non-NULL");
  if (!aligned16(k) || !aligned16(P2) || !aligned16(k_tilde) || !aligned16(r_cache))
    return fail(WA_INVALID_ARG, "device pointers must be 16-byte aligned");
  hipError_t e = wa::launch_build_cache(k, P2, k_tilde, r_cache, B, T_kv, HQ, H, K, dtype,
                                        cache_dtype, reinterpret_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(WA_HIP_ERROR, "wall_attn_build_kv_cache launch failed: %s", hipGetErrorString(e));
  return ok();
}

size_t wall_attn_decode_workspace_bytes(int64_t B, int64_t T_kv, int64_t HQ, int64_t H, int64_t K,
                                        int64_t V, int64_t chunk_size) {
  if (check_cache_shape(B, T_kv, HQ, H, K, V, chunk_size, WA_BF16, WA_F32) != WA_OK) return 0;
  return wa::decode_workspace_size(B, (T_kv + wa::CHUNK - 1) / wa::CHUNK, HQ, H, V);
}

int wall_attn_decode(const void *q, const void *v, const float *p_curr, const void *k_tilde,
                     const float *r_cache, const float *sink_bias, void *o, float *lse, int64_t B,
                     int64_t T_kv, int64_t HQ, int64_t H, int64_t K, int64_t V, int64_t chunk_size,
                     float scale, int dtype, int cache_dtype, void *workspace,
                     size_t workspace_bytes, struct ihipStream_t *stream) {
  return decode_impl("wall_attn_decode", q, v, p_curr, k_tilde, r_cache, sink_bias, nullptr,
                     nullptr, o, lse, B, T_kv, HQ, H, K, V, chunk_size, scale, dtype, cache_dtype,
                     nullptr, 0, nullptr, 0, 0, 0, workspace, workspace_bytes, stream);
}

int wall_attn_decode_ext(const void *q, const void *v, const float *p_curr, const void *k_tilde,
                         const float *r_cache, const float *sink_bias, const float *gate_cache,
                         const float *gate_curr, void *o, float *lse, int64_t B, int64_t T_kv,
                         int64_t HQ, int64_t H, int64_t K, int64_t V, int64_t chunk_size,
                         float scale, int dtype, int cache_dtype, const int32_t *cache_seqlens,
                         int64_t window_size, const int32_t *block_table, int64_t max_blocks,
                         int64_t page_size, int64_t num_pages, void *workspace,
                         size_t workspace_bytes, struct ihipStream_t *stream) {
  return decode_impl("wall_attn_decode_ext", q, v, p_curr, k_tilde, r_cache, sink_bias, gate_cache,
                     gate_curr, o, lse, B, T_kv, HQ, H, K, V, chunk_size, scale, dtype, cache_dtype,
                     cache_seqlens, window_size, block_table, max_blocks, page_size, num_pages,
                     workspace, workspace_bytes, stream);
}

}  // extern "C"

namespace {

// Split partials of wall_attn_decode_noalloc: one array per GPU, held until
// the process ends.  In host code `scratch` names a host-side stand-in;
// kernels get the device address from hipGetSymbolAddress, taken once per
// device with that device current.
constexpr size_t kScratchBytes = size_t(32) << 20;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices] = {};

int scratch_address(void **out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(WA_HIP_ERROR, "hipGetDevice failed: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices) return fail(WA_UNSUPPORTED, "device %d beyond the scratch table", dev);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void *p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || p == nullptr)
      return fail(WA_HIP_ERROR, "hipGetSymbolAddress(scratch) failed: %s", hipGetErrorString(e));
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return WA_OK;
}

}  // namespace

extern "C" {

int wall_attn_decode_noalloc(const void *q, const void *v, const float *p_curr,
                             const void *k_tilde, const float *r_cache, const float *sink_bias,
                             const float *gate_cache, const float *gate_curr, void *o, float *lse,
                             int64_t B, int64_t T_kv, int64_t HQ, int64_t H, int64_t K, int64_t V,
                             int64_t chunk_size, float scale, int dtype, int cache_dtype,
                             const int32_t *cache_seqlens, int64_t window_size,
                             const int32_t *block_table, int64_t max_blocks, int64_t page_size,
                             int64_t num_pages, struct ihipStream_t *stream) {
  // size check first (host only): the partials must fit the static array
  int64_t T = T_kv;
  int rc = check_pages(block_table, max_blocks, page_size, num_pages, &T);
  if (rc != WA_OK) return rc;
  rc = check_cache_shape(B, T, HQ, H, K, V, chunk_size, dtype, cache_dtype);
  if (rc != WA_OK) return rc;
  const size_t need = wa::decode_workspace_size(B, (T + wa::CHUNK - 1) / wa::CHUNK, HQ, H, V);
  if (need > kScratchBytes)
    return fail(WA_UNSUPPORTED, "wall_attn_decode_noalloc: split partials need %zu bytes, above the "
                                "%zu-byte static scratch (use wall_attn_decode_ext with a workspace)",
                need, kScratchBytes);
  void *ws = nullptr;
  rc = scratch_address(&ws);
  if (rc != WA_OK) return rc;
  return decode_impl("wall_attn_decode_noalloc", q, v, p_curr, k_tilde, r_cache, sink_bias,
                     gate_cache, gate_curr, o, lse, B, T_kv, HQ, H, K, V, chunk_size, scale, dtype,
                     cache_dtype, cache_seqlens, window_size, block_table, max_blocks, page_size,
                     num_pages, ws, kScratchBytes, stream);
}

int wall_attn_cache_append(const void *k_new, const void *v_new, const float *p_new,
                           const float *gate_new, void *k_tilde, void *v_cache, float *r_cache,
                           float *gate_cache, int32_t *cache_seqlens, int64_t B, int64_t T_kv,
                           int64_t HQ, int64_t H, int64_t K, int64_t V, int64_t chunk_size,
                           int dtype, int cache_dtype, const int32_t *block_table,
                           int64_t max_blocks, int64_t page_size, int64_t num_pages,
                           struct ihipStream_t *stream) {
  int64_t T = T_kv;
  int rc = check_pages(block_table, max_blocks, page_size, num_pages, &T);
  if (rc != WA_OK) return rc;
  rc = check_cache_shape(B, T, HQ, H, K, V, chunk_size, dtype, cache_dtype);
  if (rc != WA_OK) return rc;
  if (!k_new || !v_new || !p_new || !k_tilde || !v_cache || !r_cache || !cache_seqlens)
    return fail(WA_INVALID_ARG, "wall_attn_cache_append: k_new, v_new, p_new, k_tilde, v_cache, r_cache "
                                "and cache_seqlens must be non-NULL");
  if ((gate_new == nullptr) != (gate_cache == nullptr))
    return fail(WA_INVALID_ARG, "wall_attn_cache_append: gate_new and gate_cache must be given together");
  const void *ptrs[] = {k_new, v_new, p_new, gate_new, k_tilde, v_cache, r_cache, gate_cache, cache_seqlens};
  for (const void *ptr : ptrs)
    if (ptr && !aligned16(ptr)) return fail(WA_INVALID_ARG, "device pointers must be 16-byte aligned");
  wa::AppendProblem p{};
  p.k = k_new; p.v = v_new; p.p_new = p_new; p.gs_new = gate_new; p.kt = k_tilde; p.vc = v_cache;
  p.rc = r_cache; p.gs_cache = gate_cache; p.seqlens = cache_seqlens; p.block_table = block_table;
  p.B = B; p.T = T; p.HQ = HQ; p.H = H; p.K = K; p.V = V; p.max_blocks = max_blocks;
  p.page_size = page_size; p.num_pages = num_pages; p.dtype = dtype; p.cache_dtype = cache_dtype;
  hipError_t e = wa::launch_cache_append(p, reinterpret_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(WA_HIP_ERROR, "wall_attn_cache_append launch failed: %s", hipGetErrorString(e));
  return ok();
}

}  // extern "C"

/*
 * libwallattn — exact causal Wall Attention on AMD Instinct MI355X (gfx950).
 *
 * C ABI.  Every pointer argument is a device pointer unless marked "host";
 * tensors are dense, contiguous, in the index order written, and at least
 * 16-byte aligned.  The caller owns every buffer, workspace included; the
 * library allocates nothing on the device, keeps no pointer after a call
 * returns and has no global state besides the thread-local error string.
 * Work is enqueued on `stream` (a hipStream_t; NULL is the null stream) and
 * no call synchronises the host.  Every argument is validated on the host
 * before anything is launched: on error nothing is launched, nothing is
 * written, and a non-zero status is returned with a message available from
 * wall_attn_last_error().
 *
 * Notation (Wall Attention README, introduction and "Usage"):
 *   B batch, T tokens per batch row (or total packed tokens with cu_seqlens),
 *   HQ query heads, H key/value heads (HQ % H == 0; query head hq reads
 *   key/value head hq / (HQ/H)), K key/query head dim, V value head dim.
 *   q [B,T,HQ,K], k [B,T,H,K], v [B,T,H,V], g [B,T,HQ,K] (natural-log decay),
 *   g_scalar [B,T,HQ], sink_bias [HQ], o [B,T,HQ,V], lse [B,T,HQ].
 *
 * The score of query i and key j (introduction of the README) is
 *   s(i,j) = scale * sum_n q[i,n] k[j,n] exp(P[i,n] - P[j,n]) + Gs[i] - Gs[j],
 * with P and Gs the inclusive running sums of g and g_scalar over the tokens
 * of the sequence; attention is causal, optionally restricted to the last
 * window_size keys (0 <= i - j < window_size, the FlexAttention article's
 * sliding-window rule), and optionally normalised together with a value-less
 * sink logit sink_bias[hq].
 */
#ifndef WALLATTN_H
#define WALLATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

struct ihipStream_t; /* hipStream_t is `struct ihipStream_t *` */

/* Status codes returned by every entry point. */
enum {
  WA_OK = 0,
  WA_INVALID_ARG = 1,        /* shapes, pointers or values that violate the contract */
  WA_UNSUPPORTED = 2,        /* a valid request the library has no kernel for */
  WA_HIP_ERROR = 3,          /* a HIP launch or query failed */
  WA_WORKSPACE_TOO_SMALL = 4 /* workspace_bytes below the matching *_workspace_bytes() */
};

/* Element types of q, k, v, g, g_scalar, o (README "Features": BF16 and FP32
 * inputs).  Statistics (P2, anchors, p_curr, r_cache, sink_bias, lse) are
 * always float32; the decode cache k_tilde is IEEE half for WA_BF16. */
enum { WA_BF16 = 0, WA_F32 = 1 };

/* Message for the last failing call on this host thread ("" if none). */
const char *wall_attn_last_error(void);

/*
 * Bytes of device workspace wall_attn_fwd needs for this problem (the
 * running sums, chunk anchors and rescaled q/k operands).  Returns 0 when
 * the arguments are invalid.  With cu_seqlens, pass B = 1, T = total packed
 * tokens, num_seqs and max_seqlen; without, num_seqs = 0 and max_seqlen = 0.
 */
size_t wall_attn_fwd_workspace_bytes(int64_t B, int64_t T, int64_t HQ, int64_t H, int64_t K,
                                     int64_t V, int64_t num_seqs, int64_t max_seqlen, int dtype);

/*
 * Prefill / training forward (README "Usage": wall_attn(q, k, v, g, scale,
 * g_scalar, sink_bias, window_size, cu_seqlens) -> o).
 *
 *   q, k, v, g     inputs in `dtype`, shapes as in the notation above.
 *   g_scalar       [B,T,HQ] in `dtype`, FoX-style additive gate; NULL = none.
 *   sink_bias      [HQ] float32 attention-sink logit; NULL = none.
 *   o              [B,T,HQ,V] output in `dtype`.
 *   lse            [B,T,HQ] float32 natural-log normaliser (log of the
 *                  softmax denominator, sink included); NULL = not written.
 *   cu_seqlens     int32 [num_seqs+1] packed sequence starts (0 first, T
 *                  last, non-decreasing); requires B == 1 (README "Usage").
 *                  NULL = each batch row is one sequence.
 *   max_seqlen     host: longest packed sequence (with cu_seqlens), else 0.
 *   window_size    host: > 0 keeps keys with 0 <= i - j < window_size; <= 0
 *                  means no window.
 *   scale          host: multiplies the decayed dot product only; <= 0 means
 *                  K^-0.5.
 *   workspace      device buffer of at least wall_attn_fwd_workspace_bytes().
 * Supported: K, V in {64, 128}; for WA_BF16,
 * max_seqlen*max(HQ*max(K,V), K+16)*2 < 2^31 (one sequence's operands
 * addressed with 32-bit offsets).
 * Errors: INVALID_ARG for HQ % H != 0,
 * cu_seqlens with B != 1, non-positive sizes, NULL required pointers or
 * misaligned pointers; UNSUPPORTED for other K, V or dtype, and for a launch
 * grid beyond the hardware's (segments or HQ above 65535, or
 * HQ*(ceil(max_seqlen/64)+8)*segments >= 2^31, segments = num_seqs or B);
 * WORKSPACE_TOO_SMALL; HIP_ERROR if a launch fails.
 */
int wall_attn_fwd(const void *q, const void *k, const void *v, const void *g,
                  const void *g_scalar, const float *sink_bias, void *o, float *lse,
                  int64_t B, int64_t T, int64_t HQ, int64_t H, int64_t K, int64_t V,
                  const int32_t *cu_seqlens, int64_t num_seqs, int64_t max_seqlen,
                  int64_t window_size, float scale, int dtype,
                  void *workspace, size_t workspace_bytes, struct ihipStream_t *stream);

/*
 * The two stages of wall_attn_fwd, for callers that time or schedule them
 * separately; wall_attn_fwd(...) is exactly prepare followed by attend on
 * the same stream and workspace.
 *
 * wall_attn_fwd_prepare: the running sums of g (and g_scalar) along each
 * sequence, the per-chunk anchors (README "Decode" and "Features": anchors
 * keep every exp2 argument bounded) and the rescaled keys (and, for WA_F32,
 * the rescaled queries), written into `workspace`.  Reads q, k, g,
 * g_scalar; arguments as in wall_attn_fwd.
 *
 * wall_attn_fwd_attend: the tiled causal attention over a prepared
 * workspace (README introduction: FlashAttention-style streaming softmax);
 * writes o and lse.  Reads q and g (for WA_BF16 each query tile's rescaled
 * queries are formed here from q, g and the prepared chunk offsets), v,
 * sink_bias and the workspace.  g_scalar is not read: pass non-NULL exactly
 * when the workspace was prepared with a gate.  Shape arguments, q, g,
 * scale, cu_seqlens and dtype must equal those given to prepare;
 * window_size may differ (it only selects keys).
 * Errors: as wall_attn_fwd.
 */
int wall_attn_fwd_prepare(const void *q, const void *k, const void *g, const void *g_scalar,
                          int64_t B, int64_t T, int64_t HQ, int64_t H, int64_t K, int64_t V,
                          const int32_t *cu_seqlens, int64_t num_seqs, int64_t max_seqlen,
                          float scale, int dtype, void *workspace, size_t workspace_bytes,
                          struct ihipStream_t *stream);
int wall_attn_fwd_attend(const void *q, const void *v, const void *g, const void *g_scalar,
                         const float *sink_bias, void *o, float *lse, int64_t B, int64_t T,
                         int64_t HQ, int64_t H, int64_t K, int64_t V, const int32_t *cu_seqlens,
                         int64_t num_seqs, int64_t max_seqlen, int64_t window_size, float scale,
                         int dtype, void *workspace, size_t workspace_bytes,
                         struct ihipStream_t *stream);

/* Bytes of device workspace wall_attn_prefix_log2 needs (0 on bad arguments). */
size_t wall_attn_prefix_log2_workspace_bytes(int64_t B, int64_t T, int64_t HQ, int64_t K,
                                             int64_t num_seqs, int64_t max_seqlen);

/*
 * Running sum of the decay in log2 units (README "Decode": the prefix P is
 * the chunked global cumulative sum of g scaled by 1/ln 2):
 *   P2[t,hq,n] = (1/ln 2) * sum_{u=bos..t} g[u,hq,n], restarting at every
 * sequence start bos.  g [B,T,HQ,K] in `dtype` -> P2 [B,T,HQ,K] float32.
 * cu_seqlens / num_seqs / max_seqlen as in wall_attn_fwd.
 */
int wall_attn_prefix_log2(const void *g, float *P2, int64_t B, int64_t T, int64_t HQ, int64_t K,
                          const int32_t *cu_seqlens, int64_t num_seqs, int64_t max_seqlen,
                          int dtype, void *workspace, size_t workspace_bytes,
                          struct ihipStream_t *stream);

/*
 * Decode cache build (README "Decode": build_wall_kv_cache(k, P, chunk_size)).
 * Chunk c covers tokens [c*C, min((c+1)*C, T_kv)); its anchor is
 *   r_cache[b,c,hq,:] = P2[b, min((c+1)*C, T_kv) - 1, hq, :]   (an exact copy)
 * and the decay is folded into the keys, one copy per query head:
 *   k_tilde[b,j,hq,n] = k[b,j,h(hq),n] * 2^(r_cache[b,c(j),hq,n] - P2[b,j,hq,n]).
 *   k [B,T_kv,H,K] (dtype), P2 [B,T_kv,HQ,K] float32
 *   -> k_tilde [B,T_kv,HQ,K] rounded to nearest even: IEEE half for WA_BF16
 *      inputs (same size as bfloat16 with 3 more mantissa bits; every stored
 *      factor 2^(R_c - P2[j]) spans at most one chunk's decay), float32 for
 *      WA_F32;  r_cache [B,ceil(T_kv/C),HQ,K] float32.
 * Supported: chunk_size == 64, K in {64, 128}; B <= 65535 and
 * HQ*(ceil(T_kv/64)+8)*B < 2^31 (launch grid); for WA_BF16 also
 * T_kv*HQ*K*2 < 2^31 (the forward's per-sequence limit, which the decode
 * shares); else UNSUPPORTED.
 */
int wall_attn_build_kv_cache(const void *k, const float *P2, void *k_tilde, float *r_cache,
                             int64_t B, int64_t T_kv, int64_t HQ, int64_t H, int64_t K,
                             int64_t chunk_size, int dtype, struct ihipStream_t *stream);

/* Bytes of device workspace wall_attn_decode needs (split partials). */
size_t wall_attn_decode_workspace_bytes(int64_t B, int64_t T_kv, int64_t HQ, int64_t H, int64_t K,
                                        int64_t V, int64_t chunk_size);

/*
 * Single-step decode over the pre-rescaled cache (README "Decode":
 * wall_attn_decode(q, v, p_curr, k_tilde, r_cache, sink_bias, scale,
 * cache_chunk_size) -> (o, lse)).  The query is the newest token, at
 * position T_kv - 1, and attends to all T_kv cached tokens itself included:
 *   s_j = scale * sum_n q[n] 2^(p_curr[n] - r_cache[c(j),n]) k_tilde[j,n]
 * followed by a softmax over j (and the optional sink logit) and the
 * weighted sum of v.  This equals the last row of wall_attn_fwd over the
 * same tokens (no window, no g_scalar).
 *   q [B,1,HQ,K] (dtype), v [B,T_kv,H,V] (dtype), p_curr [B,1,HQ,K] float32
 *   (P2 at the newest token), k_tilde (IEEE half for WA_BF16, float32 for
 *   WA_F32) and r_cache as built above,
 *   sink_bias [HQ] float32 or NULL -> o [B,1,HQ,V] (dtype),
 *   lse [B,1,HQ] float32 natural log, or NULL.
 * Supported: chunk_size == 64, K and V in {64, 128}; T_kv*HQ*K times the
 * k_tilde element size (2 or 4 bytes) < 2^31 (one batch row of the cache
 * addressed with 32-bit offsets), else UNSUPPORTED.
 */
int wall_attn_decode(const void *q, const void *v, const float *p_curr, const void *k_tilde,
                     const float *r_cache, const float *sink_bias, void *o, float *lse,
                     int64_t B, int64_t T_kv, int64_t HQ, int64_t H, int64_t K, int64_t V,
                     int64_t chunk_size, float scale, int dtype,
                     void *workspace, size_t workspace_bytes, struct ihipStream_t *stream);

#ifdef __cplusplus
}
#endif

#endif /* WALLATTN_H */

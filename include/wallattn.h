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

/* Element types.  q, k, v, g, g_scalar, o are WA_BF16 or WA_F32 (README
 * "Features": BF16 and FP32 inputs).  The decode cache k_tilde is any of the
 * three (the `cache_dtype` arguments): WA_BF16 is k's own type (the README's
 * cache), WA_F16 has 3 more mantissa bits in the same 2 bytes, WA_F32 keeps
 * 24 bits -- the format that holds long random-walk decays, whose decode
 * scores reach ~1e5 and whose softmax turns on score differences of a few
 * units (a 32K-token cache with g ~ 0.02 N(0,1): 16-bit caches move some
 * outputs by 0.07-3.5, float32 by < 2e-3).  Statistics (P2, G2, anchors,
 * p_curr, r_cache, gate caches, sink_bias, lse) are always float32. */
enum { WA_BF16 = 0, WA_F32 = 1, WA_F16 = 2 };

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
 * g_scalar, sink_bias, window_size, cu_seqlens) -> o).  With cu_seqlens, a
 * sequence longer than max_seqlen is processed only up to its first
 * ceil(max_seqlen/64)*64 tokens and its later rows of o and lse are not
 * written (nothing is read or written out of bounds).
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
 * HQ*(ceil(max_seqlen/64)+8)*segments*256 >= 2^32 work-items, segments =
 * num_seqs or B);
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

/* Bytes of device workspace wall_attn_bwd needs (0 on bad arguments);
 * arguments as wall_attn_fwd_workspace_bytes. */
size_t wall_attn_bwd_workspace_bytes(int64_t B, int64_t T, int64_t HQ, int64_t H, int64_t K,
                                     int64_t V, int64_t num_seqs, int64_t max_seqlen, int dtype);

/*
 * Backward pass of wall_attn_fwd (README introduction: analytic gradients
 * for q, k, v, g and the scalar gate; the FlashAttention papers'
 * recomputation from the stored o and lse).  For a loss with dL/do = dO,
 * with p_ij = exp(s_ij - lse_i), D_i = dO_i . o_i and
 * ds_ij = p_ij (dO_i . v_j - D_i):
 *   dv_j  = sum_i p_ij dO_i                        (summed over v's query heads)
 *   dq_in = scale sum_j ds_ij k_jn exp(P_in - P_jn)
 *   dk_jn = scale sum_i ds_ij q_in exp(P_in - P_jn) (summed over k's query heads)
 *   dg    = reverse running sum, within each sequence, of
 *           dP_tn = q_tn dq_tn - k_tn dk(hq)_tn   (dk(hq): the head's own share)
 *   dg_scalar = reverse running sum of sum_j ds_tj - sum_i ds_it
 *   dsink[hq] = -sum_i exp(sink_bias[hq] - lse_i) D_i.
 *   Inputs as wall_attn_fwd, plus o [B,T,HQ,V] and lse [B,T,HQ] from the
 *   forward and dO [B,T,HQ,V] (dtype).  Outputs (caller-owned): dq, dg
 *   [B,T,HQ,K], dk [B,T,H,K], dv [B,T,H,V] in dtype; dg_scalar [B,T,HQ]
 *   (given exactly when g_scalar is); dsink [HQ] float32 or NULL (needs
 *   sink_bias).  Every factor exp(P_in - P_jn) is formed per pair, so any
 *   decay rate is held; arithmetic in float32.  Rows past max_seqlen (see
 *   wall_attn_fwd) get unspecified gradients.
 * Errors: as wall_attn_fwd; INVALID_ARG for a gate or sink gradient without
 * its input.
 */
int wall_attn_bwd(const void *q, const void *k, const void *v, const void *g,
                  const void *g_scalar, const float *sink_bias, const void *o, const float *lse,
                  const void *dO, void *dq, void *dk, void *dv, void *dg, void *dg_scalar,
                  float *dsink, int64_t B, int64_t T, int64_t HQ, int64_t H, int64_t K, int64_t V,
                  const int32_t *cu_seqlens, int64_t num_seqs, int64_t max_seqlen,
                  int64_t window_size, float scale, int dtype, void *workspace,
                  size_t workspace_bytes, struct ihipStream_t *stream);

/* Bytes of device workspace wall_attn_prefix_log2 needs (0 on bad arguments). */
size_t wall_attn_prefix_log2_workspace_bytes(int64_t B, int64_t T, int64_t HQ, int64_t K,
                                             int64_t num_seqs, int64_t max_seqlen);

/*
 * Running sum of the decay in log2 units (README "Decode": the prefix P is
 * the chunked global cumulative sum of g scaled by 1/ln 2):
 *   P2[t,hq,n] = (1/ln 2) * sum_{u=bos..t} g[u,hq,n], restarting at every
 * sequence start bos.  g [B,T,HQ,K] in `dtype` -> P2 [B,T,HQ,K] float32.
 * Optionally the same for the scalar gate: g_scalar [B,T,HQ] -> G2 [B,T,HQ]
 * float32 (both NULL or both given; G2 feeds the gate cache of
 * wall_attn_decode_ext).  The sums are accumulated in double and each output
 * is rounded to float once.  cu_seqlens / num_seqs / max_seqlen as in
 * wall_attn_fwd; with cu_seqlens, at most ceil(max_seqlen/64) chunks of a
 * sequence are processed (tokens beyond max_seqlen are not written).
 */
int wall_attn_prefix_log2(const void *g, const void *g_scalar, float *P2, float *G2, int64_t B,
                          int64_t T, int64_t HQ, int64_t K, const int32_t *cu_seqlens,
                          int64_t num_seqs, int64_t max_seqlen, int dtype, void *workspace,
                          size_t workspace_bytes, struct ihipStream_t *stream);

/*
 * Decode cache build (README "Decode": build_wall_kv_cache(k, P, chunk_size)).
 * Chunk c covers tokens [c*C, min((c+1)*C, T_kv)); its anchor is
 *   r_cache[b,c,hq,:] = P2[b, min((c+1)*C, T_kv) - 1, hq, :]   (an exact copy)
 * and the decay is folded into the keys, one copy per query head:
 *   k_tilde[b,j,hq,n] = k[b,j,h(hq),n] * 2^(r_cache[b,c(j),hq,n] - P2[b,j,hq,n]).
 *   k [B,T_kv,H,K] (dtype), P2 [B,T_kv,HQ,K] float32
 *   -> k_tilde [B,T_kv,HQ,K] in cache_dtype (WA_BF16, WA_F16 or WA_F32),
 *      rounded to nearest even;  r_cache [B,ceil(T_kv/C),HQ,K] float32.
 * Supported: chunk_size == 64, K in {64, 128}; B, HQ <= 65535,
 * T_kv < 2^31 - 64, HQ*(ceil(T_kv/64)+8)*256 < 2^32; else UNSUPPORTED.
 */
int wall_attn_build_kv_cache(const void *k, const float *P2, void *k_tilde, float *r_cache,
                             int64_t B, int64_t T_kv, int64_t HQ, int64_t H, int64_t K,
                             int64_t chunk_size, int dtype, int cache_dtype,
                             struct ihipStream_t *stream);

/* Bytes of device workspace wall_attn_decode and wall_attn_decode_ext need
 * (split partials); T_kv is the cache's rows per batch row (paged: the
 * capacity max_blocks*page_size).  0 on bad arguments. */
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
 *   (P2 at the newest token), k_tilde [B,T_kv,HQ,K] (cache_dtype) and
 *   r_cache [B,ceil(T_kv/C),HQ,K] float32 (any anchors: they cancel),
 *   sink_bias [HQ] float32 or NULL -> o [B,1,HQ,V] (dtype),
 *   lse [B,1,HQ] float32 natural log, or NULL.
 *   workspace: at least wall_attn_decode_workspace_bytes(); its contents are
 *   scratch (split partials), overwritten by every call.
 * Supported: chunk_size == 64, K and V in {64, 128}; B, HQ <= 65535;
 * T_kv < 2^31 - 64; 64*HQ*K*4 and 64*H*V*4 < 2^31; B*HQ*128 < 2^32; else
 * UNSUPPORTED.
 */
int wall_attn_decode(const void *q, const void *v, const float *p_curr, const void *k_tilde,
                     const float *r_cache, const float *sink_bias, void *o, float *lse,
                     int64_t B, int64_t T_kv, int64_t HQ, int64_t H, int64_t K, int64_t V,
                     int64_t chunk_size, float scale, int dtype, int cache_dtype,
                     void *workspace, size_t workspace_bytes, struct ihipStream_t *stream);

/*
 * Decode with the serving options (README "Decode" and "Usage"; the
 * FlexAttention article's decode offset, sliding window and logical-to-
 * physical page table; the FlagAttention overview's paged decoding).  As
 * wall_attn_decode, plus (each may be left out with NULL / 0):
 *   cache_seqlens  int32 [B]: row b holds len_b cached tokens and its query
 *                  sits at position len_b - 1 (NULL: every row holds T_kv).
 *                  Values are clamped into [0, capacity]; a row with
 *                  len_b = 0 gets o = 0 and lse = sink_bias (or -inf).
 *   window_size    > 0: only keys j with len_b - 1 - j < window_size count
 *                  (the forward's window rule); 0: none.
 *   gate_cache     float32 running sums of g_scalar in log2 units per cached
 *                  token ([B,T_kv,HQ], or the page layout below) and
 *   gate_curr      float32 [B,1,HQ] the same at the query: the score gains
 *                  (gate_curr - gate_cache[j]) * ln 2, the forward's
 *                  Gs[i] - Gs[j].  Both NULL or both given.
 *   block_table    int32 [B, max_blocks]: logical page p of row b lives in
 *                  physical page block_table[b*max_blocks + p] of pools
 *                  k_tilde [num_pages, page_size, HQ, K], v [num_pages,
 *                  page_size, H, V], r_cache [num_pages, page_size/64, HQ, K]
 *                  and gate_cache [num_pages, page_size, HQ]; page_size a
 *                  multiple of 64; the capacity is max_blocks*page_size and
 *                  T_kv is ignored.  Entries outside [0, num_pages) are
 *                  clamped (such rows give undefined values, but no access
 *                  leaves the pools).  NULL: contiguous [B, T_kv] rows.
 * Errors: as wall_attn_decode; INVALID_ARG for a negative window_size, a
 * gate pointer without the other, or bad page arguments.
 */
int wall_attn_decode_ext(const void *q, const void *v, const float *p_curr, const void *k_tilde,
                         const float *r_cache, const float *sink_bias, const float *gate_cache,
                         const float *gate_curr, void *o, float *lse, int64_t B, int64_t T_kv,
                         int64_t HQ, int64_t H, int64_t K, int64_t V, int64_t chunk_size,
                         float scale, int dtype, int cache_dtype, const int32_t *cache_seqlens,
                         int64_t window_size, const int32_t *block_table, int64_t max_blocks,
                         int64_t page_size, int64_t num_pages, void *workspace,
                         size_t workspace_bytes, struct ihipStream_t *stream);

/*
 * wall_attn_decode_ext without a workspace, for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc).  Arguments as wall_attn_decode_ext.  The split
 * partials go to a static device array of 32 MiB per GPU (held until the
 * process ends; its address is taken once per device, with hipGetSymbolAddress,
 * on the first call with that device current -- the current device must be
 * the one the stream and tensors belong to).  No call allocates or frees
 * device memory.  Every call on one GPU shares that GPU's array: calls that
 * overlap on one GPU (other streams, other host threads) race and must be
 * ordered by the caller.  The array needs no clearing: every call writes all
 * the partials it reads.
 * Errors: as wall_attn_decode_ext; UNSUPPORTED when the partials
 * (wall_attn_decode_workspace_bytes) exceed 32 MiB.
 */
int wall_attn_decode_noalloc(const void *q, const void *v, const float *p_curr,
                             const void *k_tilde, const float *r_cache, const float *sink_bias,
                             const float *gate_cache, const float *gate_curr, void *o, float *lse,
                             int64_t B, int64_t T_kv, int64_t HQ, int64_t H, int64_t K, int64_t V,
                             int64_t chunk_size, float scale, int dtype, int cache_dtype,
                             const int32_t *cache_seqlens, int64_t window_size,
                             const int32_t *block_table, int64_t max_blocks, int64_t page_size,
                             int64_t num_pages, struct ihipStream_t *stream);

/*
 * Streaming append (README "Decode" and "Tests": the sequential-append
 * serving loop that reproduces the forward token by token).  For every batch
 * row b with len_b = cache_seqlens[b] < capacity, the new token goes to
 * position t = len_b:
 *   k_tilde[t] = k_new * 2^(R - p_new), R = rint(p_new) per channel,
 *   v_cache[t] = v_new,  gate_cache[t] = gate_new (if given),
 * the open chunk c = t/64 takes R as its anchor (r_cache[c] = R: the chunk
 * stays anchored at its newest token, rounded to an integer) and its rows
 * already cached are re-anchored, k_tilde[j] *= 2^(R - R_old) (an exact
 * power of two when R_old is an integer, as every anchor written here is);
 * then cache_seqlens[b] += 1.  Rows already at capacity are left unchanged.
 *   k_new [B,1,H,K], v_new [B,1,H,V] (dtype); p_new [B,1,HQ,K] float32 (P2 at
 *   the new token); gate_new [B,1,HQ] float32 or NULL (G2 at the new token);
 *   caches in the layouts of wall_attn_decode_ext (contiguous [B,T_kv,...]
 *   or paged through block_table, whose page for position t must be set).
 * Errors: as wall_attn_decode_ext.
 */
int wall_attn_cache_append(const void *k_new, const void *v_new, const float *p_new,
                           const float *gate_new, void *k_tilde, void *v_cache, float *r_cache,
                           float *gate_cache, int32_t *cache_seqlens, int64_t B, int64_t T_kv,
                           int64_t HQ, int64_t H, int64_t K, int64_t V, int64_t chunk_size,
                           int dtype, int cache_dtype, const int32_t *block_table,
                           int64_t max_blocks, int64_t page_size, int64_t num_pages,
                           struct ihipStream_t *stream);

#ifdef __cplusplus
}
#endif

#endif /* WALLATTN_H */

// Internal launchers of libwallattn (host side).  Arguments are validated by
// the C ABI layer before any of these is called.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace wa {

// One prefill problem, validated.  Token axis is packed: ntok = B*T, or the
// packed length with cu_seqlens (then B == 1).
struct FwdProblem {
  const void *q, *k, *v, *g, *g_scalar;
  const float *sink;
  void *o;
  float *lse;
  const int32_t *cu;
  int64_t B, T, HQ, H, K, V;
  int64_t nseg;     // segments: B, or num_seqs
  int64_t maxlen;   // longest segment (T without cu_seqlens)
  int64_t ntok;     // packed tokens
  int64_t window;   // <= 0: none
  float scale;
  int dtype;        // WA_BF16 / WA_F32
};

// Device workspace of the prefill path, carved from the caller's buffer.
struct FwdWorkspace {
  float *csum;     // [nseg*NCmax, HQ, K] chunk sums of g, then exclusive chunk offsets
  float *anch;     // [nseg*NCmax, HQ, K] chunk anchors (log2 units)
  float *csum_s;   // [nseg*NCmax, HQ] chunk sums / offsets of g_scalar
  void *qh;        // [ntok, HQ, K] rescaled queries (float operands only)
  void *kt;        // rescaled keys: bf16 path [HQ, ntok, K+16] half with extra
                   // channels, fp32 path [ntok, HQ, K] float
  float *gsum;     // [ntok, HQ] running gate sum (log2 units)
  int *wide;       // [nseg, HQ] 1: the (segment, head) leaves the anchored operands' range
  void *qbh;       // NULL, or the backward's half q_hat [HQ, ntok, K] (own-chunk anchor)
  float *mid;      // bf16 path: [nseg*NCmax, HQ, K] running sum of g (log2 units) at each
                   // chunk's row 31, where the second 32-row half of a query tile's chunk starts
};

size_t fwd_workspace_layout(const FwdProblem &p, FwdWorkspace *ws, char *base);
size_t prefix_workspace_layout(int64_t nseg, int64_t maxlen, int64_t HQ, int64_t K);

hipError_t launch_prefix_phases(const FwdProblem &p, const FwdWorkspace &ws, hipStream_t st);
hipError_t launch_prefix_log2(const void *g, const void *gs, float *P2, float *G2,
                              const int32_t *cu, int64_t T, int64_t HQ, int64_t K, int64_t nseg,
                              int64_t maxlen, int dtype, void *ws, hipStream_t st);
hipError_t launch_attn_fwd(const FwdProblem &p, const FwdWorkspace &ws, hipStream_t st);
hipError_t launch_build_cache(const void *k, const float *P2, void *kt, float *rc, int64_t B,
                              int64_t T, int64_t HQ, int64_t H, int64_t K, int dtype,
                              int cache_dtype, hipStream_t st);

// Backward pass of the prefill.
struct BwdProblem {
  FwdProblem f;                     // inputs and shapes as the forward
  const void *o, *dO;               // forward output and dL/do (dtype)
  const float *lse;                 // forward lse
  void *dq, *dk, *dv, *dg, *dgs;    // gradients (dtype); dgs NULL without g_scalar
  float *dsink;                     // [HQ] or NULL
};
struct BwdWorkspace {
  float *Dv, *psD;                  // [ntok, HQ] D_i, exp(sink - lse_i) D_i
  float *dq32, *dk_part, *dv_part;  // [ntok, HQ, K|V]: dq, each query head's dk and dv
  float *rows_ds, *cols_ds;         // [ntok, HQ] row and column sums of ds
  float *ctot;                      // [nseg*NCmax, HQ, K+4] chunk totals of dP (K) and dGs (at K), padded
  float *dsp;                       // [ceil(ntok/1024), HQ] partial sums of dsink
  void *qbh;                        // bf16 inputs: [HQ, ntok, K] half q_hat for the MFMA kernels
};
size_t bwd_workspace_layout(const FwdProblem &p, BwdWorkspace *bw, char *base);
hipError_t launch_attn_bwd(const BwdProblem &b, const FwdWorkspace &ws, const BwdWorkspace &bw,
                           hipStream_t st);
hipError_t launch_attn_bwd_mfma(const BwdProblem &b, const FwdWorkspace &ws,
                                const BwdWorkspace &bw, hipStream_t st);

// Element types (the values of the public WA_BF16 / WA_F32 / WA_F16).
enum { WA_DT_BF16 = 0, WA_DT_F32 = 1, WA_DT_F16 = 2 };

struct DecodeProblem {
  const void *q, *v, *kt;
  const float *p_curr, *rc, *sink;
  const float *gs_cache, *gs_curr;  // gate running sums (log2 units), or NULL
  const int32_t *seqlens;           // [B] cached tokens per row, or NULL (all T)
  const int32_t *block_table;       // [B, max_blocks] pages, or NULL (contiguous rows)
  void *o;
  float *lse;
  int64_t B, T, HQ, H, K, V;        // T: rows per batch row (contiguous) or max_blocks*page_size
  int64_t max_blocks, page_size, num_pages;
  int64_t window;                   // <= 0: none
  int64_t max_chunks;               // most chunks one row can visit (split planning)
  float scale;
  int dtype, cache_dtype;
};

// Kernel-side view of a decode call (passed by value).
struct DecodeParams {
  const void *q, *v, *kt;
  const float *p_curr, *rc, *gs_cache, *gs_curr;
  const int32_t *seqlens, *block_table;
  float *part_o, *part_ml;
  int64_t T, max_blocks;
  int page_size, num_pages, NC, HQ, H, nsplit, window;
  float qscale;
};

void decode_split_plan(int64_t B, int64_t nchunks, int64_t HQ, int64_t H, int *nsplit,
                       int *chunks_per_split);
size_t decode_workspace_size(int64_t B, int64_t nchunks, int64_t HQ, int64_t H, int64_t V);
hipError_t launch_decode(const DecodeProblem &p, void *ws, hipStream_t st);

// Streaming append of one token per batch row (decode cache).
struct AppendProblem {
  const void *k, *v;                // [B,1,H,K], [B,1,H,V] (dtype)
  const float *p_new;               // [B,1,HQ,K] P2 at the new token
  const float *gs_new;              // [B,1,HQ] gate running sum at the new token, or NULL
  void *kt, *vc;                    // cache k_tilde (cache_dtype), v cache (dtype)
  float *rc, *gs_cache;
  int32_t *seqlens;
  const int32_t *block_table;
  int64_t B, T, HQ, H, K, V, max_blocks, page_size, num_pages;
  int dtype, cache_dtype;
};
hipError_t launch_cache_append(const AppendProblem &p, hipStream_t st);

}  // namespace wa

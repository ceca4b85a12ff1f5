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
};

size_t fwd_workspace_layout(const FwdProblem &p, FwdWorkspace *ws, char *base);
size_t prefix_workspace_layout(int64_t nseg, int64_t maxlen, int64_t HQ, int64_t K, float **csum,
                               char *base);

hipError_t launch_prefix_phases(const FwdProblem &p, const FwdWorkspace &ws, hipStream_t st);
hipError_t launch_prefix_log2(const void *g, float *P2, const int32_t *cu, int64_t T, int64_t HQ,
                              int64_t K, int64_t nseg, int64_t maxlen, int dtype, float *csum,
                              hipStream_t st);
hipError_t launch_attn_fwd(const FwdProblem &p, const FwdWorkspace &ws, hipStream_t st);
hipError_t launch_build_cache(const void *k, const float *P2, void *kt, float *rc, int64_t B,
                              int64_t T, int64_t HQ, int64_t H, int64_t K, int dtype,
                              hipStream_t st);

struct DecodeProblem {
  const void *q, *v, *kt;
  const float *p_curr, *rc, *sink;
  void *o;
  float *lse;
  int64_t B, T, HQ, H, K, V;
  float scale;
  int dtype;
};
void decode_split_plan(int64_t B, int64_t T, int64_t HQ, int64_t H, int *nsplit,
                       int *chunks_per_split);
size_t decode_workspace_size(int64_t B, int64_t T, int64_t HQ, int64_t H, int64_t V);
hipError_t launch_decode(const DecodeProblem &p, void *ws, hipStream_t st);

}  // namespace wa

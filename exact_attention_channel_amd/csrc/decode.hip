// Single-step decode over the pre-rescaled cache (Wall Attention README,
// "Decode"): with k_tilde[j] = k[j] * 2^(R_c - P2[j]) already in the cache,
// the newest query only needs q_hat_c = q * 2^(p_curr - R_c) once per chunk
// and per head, and then plain dot products with k_tilde -- a bandwidth-bound
// GEMV over k_tilde and v instead of re-accumulating the prefix.
//
// Split-K layout (the split-KV decoding idea noted in the FlagAttention
// overview): workgroup (split, head group, b) streams the chunks of one
// split for NHB query heads that share one key/value head, so each v row is
// read once for all of them; it keeps an online softmax per head and writes
// (max, sum, partial output) per split.  A second kernel merges the splits
// and adds the sink logit.
//
// Options (all per call): per-row cache lengths (the query of row b sits at
// position len_b - 1), a sliding window over the newest keys (the
// FlexAttention article's window rule, as in the forward), the scalar gate
// through a cache of its running sums, and a paged cache whose 64-token
// chunks are found through a block table (the FlexAttention article's
// logical-to-physical page table; the FlagAttention overview's paged
// decoding).  Every chunk is addressed through its own buffer descriptor
// whose extent ends at the chunk's last valid row, so rows past a sequence's
// length read as zero and no address is formed outside the cache.
#include "decode_kernels.h"

namespace wa {

extern template hipError_t launch_decode_cache<bf16_t>(const DecodeParams &, int, int64_t, int64_t, const float *, void *, float *, int64_t, hipStream_t);
extern template hipError_t launch_decode_cache<_Float16>(const DecodeParams &, int, int64_t, int64_t, const float *, void *, float *, int64_t, hipStream_t);
extern template hipError_t launch_decode_cache<float>(const DecodeParams &, int, int64_t, int64_t, const float *, void *, float *, int64_t, hipStream_t);

// Splits of a call whose rows visit at most nchunks chunks: enough
// workgroups for about four full waves of three per CU (four measured a
// little faster than two, three, eight or sixteen on a 64-row 32K cache).
void decode_split_plan(int64_t B, int64_t nchunks, int64_t HQ, int64_t H, int *nsplit,
                       int *chunks_per_split) {
  const int64_t NC = nchunks < 1 ? 1 : nchunks;
  const int64_t units = B * (HQ / dec::heads_per_block(HQ, H));
  const int64_t target = 256 * 3 * 4;
  int64_t ns = (target + units - 1) / units;
  ns = ns < 1 ? 1 : (ns > NC ? NC : ns);
  const int64_t cps = (NC + ns - 1) / ns;
  ns = (NC + cps - 1) / cps;
  *nsplit = (int)ns;
  *chunks_per_split = (int)cps;
}

// Partial results for up to min(ceil(target / units), nchunks) splits: an
// upper bound of the split count of any call whose rows visit at most
// nchunks chunks (a window or shorter rows only lower it).
size_t decode_workspace_size(int64_t B, int64_t nchunks, int64_t HQ, int64_t H, int64_t V) {
  const int64_t NC = nchunks < 1 ? 1 : nchunks;
  const int64_t units = B * (HQ / dec::heads_per_block(HQ, H));
  const int64_t target = 256 * 3 * 4;
  int64_t ns = (target + units - 1) / units;
  ns = ns < 1 ? 1 : (ns > NC ? NC : ns);
  const size_t po = sizeof(float) * (size_t)(B * HQ * ns * V);
  const size_t pml = sizeof(float) * (size_t)(B * HQ * ns * 2);
  return ((po + 255) & ~size_t(255)) + ((pml + 255) & ~size_t(255));
}

hipError_t launch_decode(const DecodeProblem &dp, void *ws, hipStream_t st) {
  int ns, cps;
  decode_split_plan(dp.B, dp.max_chunks, dp.HQ, dp.H, &ns, &cps);
  DecodeParams p{};
  p.q = dp.q; p.v = dp.v; p.kt = dp.kt; p.p_curr = dp.p_curr; p.rc = dp.rc;
  p.gs_cache = dp.gs_cache; p.gs_curr = dp.gs_curr; p.seqlens = dp.seqlens;
  p.block_table = dp.block_table; p.max_blocks = dp.max_blocks; p.page_size = (int)dp.page_size;
  p.num_pages = (int)dp.num_pages;
  p.T = dp.T; p.NC = (int)((dp.T + CHUNK - 1) / CHUNK);
  p.HQ = (int)dp.HQ; p.H = (int)dp.H; p.nsplit = ns; p.window = (int)dp.window;
  p.qscale = dp.scale * LOG2E;
  p.part_o = static_cast<float *>(ws);
  const size_t pob = sizeof(float) * (size_t)(dp.B * dp.HQ * ns * dp.V);
  p.part_ml = reinterpret_cast<float *>(static_cast<char *>(ws) + ((pob + 255) & ~size_t(255)));
  switch (dp.cache_dtype) {
    case WA_DT_BF16: return launch_decode_cache<bf16_t>(p, dp.dtype, dp.K, dp.V, dp.sink, dp.o, dp.lse, dp.B, st);
    case WA_DT_F16: return launch_decode_cache<_Float16>(p, dp.dtype, dp.K, dp.V, dp.sink, dp.o, dp.lse, dp.B, st);
    default: return launch_decode_cache<float>(p, dp.dtype, dp.K, dp.V, dp.sink, dp.o, dp.lse, dp.B, st);
  }
}

}  // namespace wa

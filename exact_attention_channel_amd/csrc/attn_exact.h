// Exact prefill rows for (sequence, head) pairs whose decay leaves the range
// of the anchored operands.
//
// The factorised kernels (attn_fwd.hip) hold q_hat = q 2^(P2_i - RQ) and
// k_tilde = k 2^(R_J - P2_j), with one anchor per 64-token chunk, in IEEE
// half (bf16 inputs) or float (fp32 inputs).  A decay sum that changes by
// more than the operands' exponent range inside one chunk -- the Wall
// Attention README's claim that per-chunk anchors keep exp2 bounded holds
// only while a chunk's decay span is representable -- would overflow them.
// The pre-pass flags such (sequence, head) pairs; the attention kernels'
// workgroups of a flagged pair compute their rows with exact_chunk() instead,
// straight from the definition (README introduction): for each pair (i, j)
// and channel n the factor 2^(P2[i,n] - P2[j,n]) is formed on its own, so
// every factor of a causal pair is at most 1 for decaying channels whatever
// the decay rate, and the scores, masks, gate, online softmax (the
// FlashAttention papers' running max and sum) and sink follow as in the
// other kernels.  Float32 arithmetic, plain FMAs: a correctness path for
// inputs outside the fast path's range, not a tuned one.  It runs inside the
// attention kernels so that a forward with no flagged pair costs nothing.
//
// Layout: one 64-row query chunk per call, 256 threads = 64 query rows x 4,
// thread `sub` of a row owning channels n = 4e + sub; keys staged in blocks
// of 16 rows.  LDS: the caller's buffer of ExactLds<DK, DV>::BYTES bytes.
#pragma once

#include <math.h>

#include "common.h"

namespace wa {
namespace exact {

constexpr int XC = CHUNK;  // rows per query chunk and per key chunk
constexpr int XB = 16;     // key rows staged at a time

template <int DK, int DV> struct ExactLds {
  // Ks [XB][DK], Pk [XB][DK], Vs [XB][DV], Gj [XB], tot [256] (floats)
  static constexpr int BYTES = 4 * (XB * (2 * DK + DV) + XB + 256);
};

// Running decay sums in log2 units of rows XB hh .. XB hh + XB - 1 of one
// chunk into P2s (LDS, [XB][DK]): the chunk's exclusive offset (natural-log units,
// from the pre-pass) plus the inclusive in-chunk sum of g, times log2(e) --
// the same arithmetic for query and key rows, so the diagonal factor is
// exactly 1.  Starts and ends with every thread's LDS accesses done.
template <typename TE, int DK>
__device__ __forceinline__ void half_p2(const TE *__restrict__ g, const float *__restrict__ off_c,
                                        int64_t r0, int nrow, int HQ, int hq, int hh, float *P2s,
                                        float *tot) {
  constexpr int NSEG = 256 / DK, RPS = XC / NSEG;  // row segments per channel
  const int n = threadIdx.x % DK, sg = threadIdx.x / DK;
  const int lo = XB * hh;
  float acc = 0.f;
  for (int r = sg * RPS; r < sg * RPS + RPS; ++r) {
    acc += r < nrow ? Elem<TE>::ld(g + ((r0 + r) * HQ + hq) * DK + n) : 0.f;
    if (r >= lo && r < lo + XB) P2s[(r - lo) * DK + n] = acc;
  }
  tot[sg * DK + n] = acc;
  __syncthreads();
  float base = off_c[n];
  for (int q = 0; q < sg; ++q) base += tot[q * DK + n];
  const int r1 = sg * RPS + RPS < lo + XB ? sg * RPS + RPS : lo + XB;
  for (int r = sg * RPS > lo ? sg * RPS : lo; r < r1; ++r)
    P2s[(r - lo) * DK + n] = (base + P2s[(r - lo) * DK + n]) * LOG2E;
  __syncthreads();
}

// Rows of query chunk c of one (sequence, head): q, k, v, g in the input
// type TE, off_s the chunk offsets of the pair (chunk c at + c HQ DK), rows
// relative to bos, L the sequence length, window 0 for none.  Every thread
// of the workgroup calls it (it synchronises).
template <typename TE, int DK, int DV, bool HAS_GS>
__device__ __forceinline__ void exact_chunk(
    const TE *__restrict__ q, const TE *__restrict__ k, const TE *__restrict__ v,
    const TE *__restrict__ g, const float *__restrict__ off_s, const float *__restrict__ gsum,
    const float *__restrict__ sink, TE *__restrict__ o, float *__restrict__ lse, int64_t bos,
    int L, int hq, int HQ, int H, int window, float qscale, int c, unsigned char *smem) {
  constexpr int QPT = DK / 4, VPT = DV / 4;
  float *Ks = reinterpret_cast<float *>(smem);
  float *Pk = Ks + XB * DK;
  float *Vs = Pk + XB * DK;
  float *Gj = Vs + XB * DV;
  float *tot = Gj + XB;

  const int tid = threadIdx.x;
  const int h = hq / (HQ / H);
  const int row = tid >> 2, sub = tid & 3;
  const int i0 = c * XC;  // relative to bos
  const int nq = min(XC, L - i0);
  const int irel = i0 + row;
  const bool q_ok = row < nq;
  const int64_t qi = bos + irel;
  float qv[QPT], pq[QPT];
#pragma unroll
  for (int e = 0; e < QPT; ++e) {
    qv[e] = q_ok ? Elem<TE>::ld(q + (qi * HQ + hq) * DK + 4 * e + sub) * qscale : 0.f;
    pq[e] = 0.f;
  }
  // the query rows' running sums, one half of the chunk at a time
  for (int hh = 0; hh < XC / XB; ++hh) {
    half_p2<TE, DK>(g, off_s + (int64_t)c * HQ * DK, bos + i0, nq, HQ, hq, hh, Pk, tot);
    if (row / XB == hh)
#pragma unroll
      for (int e = 0; e < QPT; ++e) pq[e] = Pk[(row % XB) * DK + 4 * e + sub];
    __syncthreads();  // read before the next half overwrites them
  }
  const float g_i = (HAS_GS && q_ok) ? gsum[qi * HQ + hq] : 0.f;

  float m_run = -INFINITY, l_run = 0.f;
  float oacc[VPT];
#pragma unroll
  for (int e = 0; e < VPT; ++e) oacc[e] = 0.f;
  const int Jlo = window > 0 ? max(0, i0 - window + 1) / XC : 0;
  for (int J = Jlo; J <= c; ++J) {
    const int nkc = min(XC, L - J * XC);  // rows of key chunk J
    for (int hh = 0; hh < XC / XB; ++hh) {
      const int j0 = J * XC + XB * hh;
      const int nk = min(XB, L - j0);
      if (nk <= 0) break;
      half_p2<TE, DK>(g, off_s + (int64_t)J * HQ * DK, bos + J * XC, nkc, HQ, hq, hh, Pk, tot);
      for (int x = tid; x < XB * DK; x += 256) {
        const int r = x / DK, n = x % DK;
        Ks[x] = r < nk ? Elem<TE>::ld(k + ((bos + j0 + r) * H + h) * DK + n) : 0.f;
      }
      for (int x = tid; x < XB * DV; x += 256) {
        const int r = x / DV, n = x % DV;
        Vs[x] = r < nk ? Elem<TE>::ld(v + ((bos + j0 + r) * H + h) * DV + n) : 0.f;
      }
      if (HAS_GS && tid < XB) Gj[tid] = tid < nk ? gsum[(bos + j0 + tid) * HQ + hq] : 0.f;
      __syncthreads();
      // sub-blocks of KB keys, each with its own online-softmax update
      constexpr int KB = 16;
      for (int kb = 0; kb < XB; kb += KB) {
        float s[KB];
        float mx = -INFINITY;
#pragma unroll
        for (int u = 0; u < KB; ++u) {
          const int jj = kb + u;
          float part = 0.f;
#pragma unroll
          for (int e = 0; e < QPT; ++e) {
            const int n = 4 * e + sub;
            part = fmaf(qv[e] * Ks[jj * DK + n], fast_exp2(pq[e] - Pk[jj * DK + n]), part);
          }
          part += __shfl_xor(part, 1);
          part += __shfl_xor(part, 2);
          if (HAS_GS) part += g_i - Gj[jj];
          const int jrel = j0 + jj;
          if (jrel > irel || jj >= nk || (window > 0 && irel - jrel >= window)) part = -INFINITY;
          s[u] = part;
          mx = fmaxf(mx, part);
        }
        const float m_new = fmaxf(m_run, mx);
        const float m_use = m_new == -INFINITY ? 0.f : m_new;
        const float alpha = fast_exp2(m_run - m_use);
        float rs = 0.f;
#pragma unroll
        for (int u = 0; u < KB; ++u) {
          s[u] = fast_exp2(s[u] - m_use);
          rs += s[u];
        }
        l_run = l_run * alpha + rs;
        m_run = m_new;
#pragma unroll
        for (int e = 0; e < VPT; ++e) {
          float acc = oacc[e] * alpha;
#pragma unroll
          for (int u = 0; u < KB; ++u) acc = fmaf(s[u], Vs[(kb + u) * DV + 4 * e + sub], acc);
          oacc[e] = acc;
        }
      }
      __syncthreads();  // the block's LDS is read before the next one is staged
    }
  }
  if (q_ok) {
    float mf = m_run, Z = l_run;
    if (sink != nullptr) {
      const float s2 = sink[hq] * LOG2E;
      mf = fmaxf(m_run, s2);
      Z = l_run * fast_exp2(m_run - mf) + fast_exp2(s2 - mf);
    }
    const float inv = fast_exp2(m_run - mf) / Z;
#pragma unroll
    for (int e = 0; e < VPT; ++e) Elem<TE>::st(o + (qi * HQ + hq) * DV + 4 * e + sub, oacc[e] * inv);
    if (lse != nullptr && sub == 0) lse[qi * HQ + hq] = (mf + log2f(Z)) * LN2;
  }
}

}  // namespace exact
}  // namespace wa

// Exact prefill for (sequence, head) pairs whose decay leaves the range of
// the anchored operands.
//
// The factorised kernels (attn_fwd.hip) hold q_hat = q 2^(P2_i - RQ_I) and
// k_tilde = k 2^(R_J - P2_j), with one anchor per 64-token chunk, in IEEE
// half (bf16 inputs) or float (fp32 inputs).  A decay sum that changes by
// more than the operands' exponent range inside one chunk -- the Wall
// Attention README's "per-chunk anchors keep exp2 bounded" holds only while
// a chunk's decay span is representable -- would overflow them.  The
// pre-pass flags such (sequence, head) pairs; the factorised kernels skip
// them and this kernel computes their rows straight from the definition
// (README introduction): for each pair (i, j) and channel n the factor
// 2^(P2[i,n] - P2[j,n]) is formed on its own, so every factor of a causal
// pair is at most 1 for decaying channels whatever the decay rate, and the
// scores, masks, gate, online softmax (the FlashAttention papers' running
// max and sum) and sink follow as in the other kernels.  Float32 arithmetic,
// plain FMAs: this is a correctness path for inputs outside the fast path's
// range, not a tuned kernel.
//
// Layout: workgroup (segment x head, stride slot) walks the 64-row query
// chunks c = slot, slot + gridDim.y, ...; 256 threads = 64 query rows x 4,
// thread `sub` of a row owning channels n = 4e + sub.
#include <math.h>

#include "common.h"
#include "launch.h"

namespace wa {
namespace {

constexpr int XC = CHUNK;  // rows per query chunk and per key chunk

// Running decay sums in log2 units of the rows of one chunk into P2s
// (LDS, [XC][DK]): the chunk's exclusive offset (natural-log units, from the
// pre-pass) plus the inclusive in-chunk sum of g, times log2(e) -- the same
// arithmetic for query and key rows, so the diagonal factor is exactly 1.
template <typename TE, int DK>
__device__ void chunk_p2(const TE *__restrict__ g, const float *__restrict__ off_c, int64_t r0,
                         int nrow, int HQ, int hq, float *P2s, float *tot) {
  constexpr int NSEG = 256 / DK, RPS = XC / NSEG;  // row segments per channel
  const int n = threadIdx.x % DK, sg = threadIdx.x / DK;
  float acc = 0.f;
  for (int r = sg * RPS; r < sg * RPS + RPS; ++r) {
    acc += r < nrow ? Elem<TE>::ld(g + ((r0 + r) * HQ + hq) * DK + n) : 0.f;
    P2s[r * DK + n] = acc;
  }
  tot[sg * DK + n] = acc;
  __syncthreads();
  float base = off_c[n];
  for (int q = 0; q < sg; ++q) base += tot[q * DK + n];
  for (int r = sg * RPS; r < sg * RPS + RPS; ++r) P2s[r * DK + n] = (base + P2s[r * DK + n]) * LOG2E;
  __syncthreads();
}

template <typename TE, int DK, int DV, bool HAS_GS>
__global__ __launch_bounds__(256) void k_attn_exact(
    const TE *__restrict__ q, const TE *__restrict__ k, const TE *__restrict__ v,
    const TE *__restrict__ g, const float *__restrict__ off, const float *__restrict__ gsum,
    const float *__restrict__ sink, TE *__restrict__ o, float *__restrict__ lse,
    const int32_t *__restrict__ cu, const int *__restrict__ wide, int64_t T, int HQ, int H,
    int NCmax, int window, float qscale) {
  constexpr int QPT = DK / 4, VPT = DV / 4;
  __shared__ float Ks[XC * DK];
  __shared__ float Pk[XC * DK];
  __shared__ float Vs[XC * DV];
  __shared__ float Gj[XC];
  __shared__ float tot[256];

  const int tid = threadIdx.x;
  const int sh = blockIdx.x, seg = sh / HQ, hq = sh % HQ;
  if (__builtin_amdgcn_readfirstlane(wide[seg * HQ + hq]) == 0) return;
  int64_t bos, eos;
  segment_bounds(seg, T, cu, bos, eos);
  // the chunk slots the workspace holds for a segment (as the other kernels)
  const int L = (int)min(eos - bos, (int64_t)NCmax * XC);
  const int nch = (L + XC - 1) / XC;
  const int h = hq / (HQ / H);
  const int row = tid >> 2, sub = tid & 3;
  const float *off_s = off + ((int64_t)seg * NCmax * HQ + hq) * DK;  // chunk c: + c*HQ*DK

  for (int c = blockIdx.y; c < nch; c += gridDim.y) {
    const int i0 = c * XC;  // relative to bos
    const int nq = min(XC, L - i0);
    chunk_p2<TE, DK>(g, off_s + (int64_t)c * HQ * DK, bos + i0, nq, HQ, hq, Pk, tot);
    const int irel = i0 + row;
    const bool q_ok = row < nq;
    const int64_t qi = bos + irel;
    float qv[QPT], pq[QPT];
#pragma unroll
    for (int e = 0; e < QPT; ++e) {
      qv[e] = q_ok ? Elem<TE>::ld(q + (qi * HQ + hq) * DK + 4 * e + sub) * qscale : 0.f;
      pq[e] = Pk[row * DK + 4 * e + sub];
    }
    const float g_i = (HAS_GS && q_ok) ? gsum[qi * HQ + hq] : 0.f;
    __syncthreads();  // every row has read its sums before the key chunks overwrite them

    float m_run = -INFINITY, l_run = 0.f;
    float oacc[VPT];
#pragma unroll
    for (int e = 0; e < VPT; ++e) oacc[e] = 0.f;
    const int Jlo = window > 0 ? max(0, i0 - window + 1) / XC : 0;
    for (int J = Jlo; J <= c; ++J) {
      const int j0 = J * XC;
      const int nk = min(XC, L - j0);
      chunk_p2<TE, DK>(g, off_s + (int64_t)J * HQ * DK, bos + j0, nk, HQ, hq, Pk, tot);
      for (int x = tid; x < XC * DK; x += 256) {
        const int r = x / DK, n = x % DK;
        Ks[x] = r < nk ? Elem<TE>::ld(k + ((bos + j0 + r) * H + h) * DK + n) : 0.f;
      }
      for (int x = tid; x < XC * DV; x += 256) {
        const int r = x / DV, n = x % DV;
        Vs[x] = r < nk ? Elem<TE>::ld(v + ((bos + j0 + r) * H + h) * DV + n) : 0.f;
      }
      if (HAS_GS && tid < XC) Gj[tid] = tid < nk ? gsum[(bos + j0 + tid) * HQ + hq] : 0.f;
      __syncthreads();
      // sub-blocks of KB keys, each with its own online-softmax update
      constexpr int KB = 16;
      for (int kb = 0; kb < XC; kb += KB) {
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
      __syncthreads();  // the chunk's LDS is read before the next one is staged
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
}

template <typename TE, int DK, int DV>
hipError_t exact_t(const FwdProblem &p, const FwdWorkspace &ws, hipStream_t st) {
  const int NCmax = (int)((p.maxlen + CHUNK - 1) / CHUNK);
  // (segment, head) pairs along x; up to 16 workgroups stride over the query
  // chunks of a pair.  Unflagged pairs return at once.
  const dim3 grid((unsigned)(p.nseg * p.HQ), (unsigned)(NCmax < 16 ? NCmax : 16));
  auto args = [&](auto kern) {
    hipLaunchKernelGGL(kern, grid, dim3(256), 0, st, static_cast<const TE *>(p.q),
                       static_cast<const TE *>(p.k), static_cast<const TE *>(p.v),
                       static_cast<const TE *>(p.g), ws.csum, ws.gsum, p.sink,
                       static_cast<TE *>(p.o), p.lse, p.cu, ws.wide, p.T, (int)p.HQ, (int)p.H,
                       NCmax, (int)(p.window > 0 && p.window < p.maxlen ? p.window : 0),
                       p.scale * LOG2E);
  };
  if (p.g_scalar != nullptr)
    args(k_attn_exact<TE, DK, DV, true>);
  else
    args(k_attn_exact<TE, DK, DV, false>);
  return hipGetLastError();
}

template <typename TE>
hipError_t exact_te(const FwdProblem &p, const FwdWorkspace &ws, hipStream_t st) {
  if (p.K == 64) return p.V == 64 ? exact_t<TE, 64, 64>(p, ws, st) : exact_t<TE, 64, 128>(p, ws, st);
  return p.V == 64 ? exact_t<TE, 128, 64>(p, ws, st) : exact_t<TE, 128, 128>(p, ws, st);
}

}  // namespace

hipError_t launch_attn_exact(const FwdProblem &p, const FwdWorkspace &ws, hipStream_t st) {
  if (p.dtype == WA_DT_BF16) return exact_te<bf16_t>(p, ws, st);
  return exact_te<float>(p, ws, st);
}

}  // namespace wa

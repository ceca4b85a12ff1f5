// Backward pass on the matrix cores (bf16 inputs whose (sequence, head)
// stays within the anchored operands' range; the others go to the float32
// kernels of attn_bwd.hip).
//
// The forward's factorisation (Wall Attention README, "Decode": keys
// rescaled by per-chunk anchors) carries over to every product of the
// backward.  With q_hat_i = q_i 2^(P2_i - A_I) scale log2(e) (A_I the anchor
// of the query's own 64-token chunk), k_tilde_j = k_j 2^(R_J - P2_j) and the
// per-channel chunk factors d_IJ = 2^(A_I - R_J) (integer anchors: exact
// powers of two):
//   S_IJ  = (q_hat_I * d_IJ) k_tilde_J^T                (log2 units)
//   P     = 2^(S + Gs_i - Gs_j - lse_i log2(e)),   dP = dO_I V_J^T,
//   ds    = P * (dP - D_i)                               (FlashAttention's recomputation)
//   dV_J += P^T dO_I,
//   dk_j  = ln2 2^(R_J - P2_j) sum_I ds^T (q_hat_I * d_IJ),
//   dq_i  = scale 2^(P2_i - A_I) sum_J (ds k_tilde_J) * d_IJ.
// A factor d_IJ above 2^4 (a decay sum rising between key and query chunk)
// is rebalanced: the query operand takes d_IJ 2^-sigma, the scores and the
// key gradient's share 2^sigma.  Products are v_mfma_f32_32x32x16 (half for
// the rescaled q/k and ds, bf16 for P, V and dO) with operands staged in
// LDS; one workgroup per 64-key chunk walks the query chunks that see it
// (dk, dv, column sums of ds), one per 64-row query chunk walks its key
// chunks (dq, row sums).  The float32 finishing kernels of attn_bwd.hip
// (reverse running sums, sums over query heads) complete the gradients.
#include <math.h>

#include "common.h"
#include "launch.h"

namespace wa {
namespace {

constexpr int XC = CHUNK;  // 64 rows of a query chunk, keys of a key chunk

template <typename T> struct Mfma;
template <> struct Mfma<_Float16> {
  typedef f16x8 V;
  static __device__ __forceinline__ f32x16 run(V a, V b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
  }
};
template <> struct Mfma<bf16_t> {
  typedef bf16x8 V;
  static __device__ __forceinline__ f32x16 run(V a, V b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
  }
};

// C += A B over the 16 k's from k0, for a 32x32 block.  A is row-major
// [m][k] (row stride as elements, pointer at the block's first row), B is
// given as B^T row-major [n][k].  Lane l supplies A row l%32 and B column
// l%32, k's k0 + 8 (l/32) .. +7; element r of C sits at row
// 8 (r/4) + 4 (l/32) + r%4, column l%32.
template <typename T>
__device__ __forceinline__ f32x16 mma16(f32x16 c, const T *A, int as, const T *Bt, int bs, int k0,
                                        int lane) {
  typedef typename Mfma<T>::V V;
  const V a = *reinterpret_cast<const V *>(A + (lane & 31) * as + k0 + 8 * (lane >> 5));
  const V b = *reinterpret_cast<const V *>(Bt + (lane & 31) * bs + k0 + 8 * (lane >> 5));
  return Mfma<T>::run(a, b, c);
}
__device__ __forceinline__ int crow(int r, int lane) { return 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3); }

__device__ __forceinline__ _Float16 to_h(float x) { return (_Float16)x; }
__device__ __forceinline__ bf16_t to_b(float x) { return (bf16_t)f32_to_bf16_bits(x); }

// Running decay sums (log2 units) of one chunk's rows into P2s [XC][DK].
template <int DK>
__device__ void chunk_p2(const bf16_t *__restrict__ g, const float *__restrict__ off_c, int64_t r0,
                         int nrow, int HQ, int hq, float *P2s, float *tot) {
  constexpr int NSEG = 256 / DK, RPS = XC / NSEG;
  const int n = threadIdx.x % DK, sg = threadIdx.x / DK;
  float acc = 0.f;
  for (int r = sg * RPS; r < sg * RPS + RPS; ++r) {
    acc += r < nrow ? bf16_to_f32(g[((r0 + r) * HQ + hq) * DK + n]) : 0.f;
    P2s[r * DK + n] = acc;
  }
  tot[sg * DK + n] = acc;
  __syncthreads();
  float base = off_c[n];
  for (int q = 0; q < sg; ++q) base += tot[q * DK + n];
  for (int r = sg * RPS; r < sg * RPS + RPS; ++r) P2s[r * DK + n] = (base + P2s[r * DK + n]) * LOG2E;
  __syncthreads();
}

// 8 consecutive 16-bit elements (one 16-byte load); zeros past `valid`.
__device__ __forceinline__ u32x4 ld16(const void *p, bool valid) {
  return valid ? *reinterpret_cast<const u32x4 *>(p) : u32x4{0u, 0u, 0u, 0u};
}

// Chunk factors of a (query chunk, key chunk) pair: fac[n] = A_I[n] - R_J[n]
// (integers) and sigma = max(0, max_n fac - 4).  Threads 0..DK-1 take part;
// returns sigma to every thread.
template <int DK>
__device__ __forceinline__ int pair_factors(const float *aI, const float *rJ, float *fac, float *red) {
  const int tid = threadIdx.x;
  if (tid < DK) {
    const float e = aI[tid] - rJ[tid];
    fac[tid] = e;
    const float m = wave_max(e);
    if ((tid & 63) == 0) red[tid >> 6] = m;
  }
  __syncthreads();
  float emax = red[0];
  if (DK > 64) emax = fmaxf(emax, red[1]);
  return max(0, (int)emax - 4);
}

// dk, dv (each query head's share) and the column sums of ds.
// grid (NCmax*HQ, nseg): x = key chunk (longest first) * HQ + head, y = segment.
// Waves: w>>1 picks 32 keys; w&1 picks 32 query rows (scores) or half the
// channels (dv, dk).
template <int DK, int DV, bool HAS_GS>
__global__ __launch_bounds__(256) void k_bwd_dkdv_mfma(
    const _Float16 *__restrict__ kt, const _Float16 *__restrict__ qbh, const bf16_t *__restrict__ v,
    const bf16_t *__restrict__ dO, const bf16_t *__restrict__ g, const float *__restrict__ off,
    const float *__restrict__ anch, const float *__restrict__ gsum, const float *__restrict__ lse,
    const float *__restrict__ Dv, const int *__restrict__ wide, float *__restrict__ dk_part,
    float *__restrict__ dv_part, float *__restrict__ cols_ds, const int32_t *__restrict__ cu,
    int64_t T, int64_t ntok, int HQ, int H, int NCmax, int window) {
  constexpr int KS = DK + 8, VS = DV + 8, RS = XC + 8;  // padded LDS row strides (elements)
  constexpr int KX = DK + 16;                           // k_tilde row in the forward workspace
  constexpr int NBK = DK / 64, NBV = DV / 64;           // 32-column blocks per wave
  constexpr int O_KT = 0, O_VS = O_KT + XC * KS * 2, O_QP = O_VS + XC * VS * 2,
                O_QPT = O_QP + XC * KS * 2, O_OS = O_QPT + DK * RS * 2, O_OST = O_OS + XC * VS * 2,
                O_PT = O_OST + DV * RS * 2, O_DST = O_PT + XC * RS * 2, O_END = O_DST + XC * RS * 2;
  static_assert(O_OS - O_QP >= XC * DK * 4, "P2 scratch reuses Qp and QpT");
  __shared__ __attribute__((aligned(16))) unsigned char lds[O_END];
  __shared__ float Rj[DK], Ai[DK], Fac[DK], Li[XC], Di[XC], Gi[XC], Gj[XC], red[4], tot[256];
  __shared__ float csh[2][XC];
  _Float16 *Kt = reinterpret_cast<_Float16 *>(lds + O_KT);
  bf16_t *Vs = reinterpret_cast<bf16_t *>(lds + O_VS);
  _Float16 *Qp = reinterpret_cast<_Float16 *>(lds + O_QP);
  _Float16 *QpT = reinterpret_cast<_Float16 *>(lds + O_QPT);
  bf16_t *Os = reinterpret_cast<bf16_t *>(lds + O_OS);
  bf16_t *OsT = reinterpret_cast<bf16_t *>(lds + O_OST);
  bf16_t *PT = reinterpret_cast<bf16_t *>(lds + O_PT);
  _Float16 *DST = reinterpret_cast<_Float16 *>(lds + O_DST);

  const int hq = blockIdx.x % HQ, J = blockIdx.x / HQ, seg = blockIdx.y;
  if (__builtin_amdgcn_readfirstlane(wide[seg * HQ + hq]) != 0) return;
  int64_t bos, eos;
  segment_bounds(seg, T, cu, bos, eos);
  const int L = (int)min(eos - bos, (int64_t)NCmax * XC);
  const int nch = (L + XC - 1) / XC;
  if (J >= nch) return;
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int kb = w >> 1, wh = w & 1;
  const int h = hq / (HQ / H);
  const int j0 = J * XC, nk = min(XC, L - j0);
  const int64_t cbase = (int64_t)seg * NCmax;

  // the key chunk: k_tilde, v, anchors, gate sums
  for (int x = tid; x < XC * DK / 8; x += 256) {
    const int r = x / (DK / 8), p = x % (DK / 8);
    *reinterpret_cast<u32x4 *>(Kt + r * KS + 8 * p) =
        ld16(kt + ((int64_t)hq * ntok + bos + j0 + r) * KX + 8 * p, r < nk);
  }
  for (int x = tid; x < XC * DV / 8; x += 256) {
    const int r = x / (DV / 8), p = x % (DV / 8);
    *reinterpret_cast<u32x4 *>(Vs + r * VS + 8 * p) =
        ld16(v + ((bos + j0 + r) * H + h) * DV + 8 * p, r < nk);
  }
  if (tid < DK) Rj[tid] = anch[((cbase + J) * HQ + hq) * DK + tid];
  if (tid < XC) Gj[tid] = (HAS_GS && tid < nk) ? gsum[(bos + j0 + tid) * HQ + hq] : 0.f;

  f32x16 dVacc[NBV], dKacc[NBK];
#pragma unroll
  for (int b = 0; b < NBV; ++b) dVacc[b] = f32x16{};
#pragma unroll
  for (int b = 0; b < NBK; ++b) dKacc[b] = f32x16{};
  float csum[16];
#pragma unroll
  for (int r = 0; r < 16; ++r) csum[r] = 0.f;

  const int Ihi = window > 0 ? min(nch - 1, (j0 + XC - 1 + window - 1) / XC) : nch - 1;
  for (int I = J; I <= Ihi; ++I) {
    const int i0 = I * XC, nq = min(XC, L - i0);
    __syncthreads();  // the previous pair's operands are consumed; Rj/Gj are written
    if (tid < DK) Ai[tid] = anch[((cbase + I) * HQ + hq) * DK + tid];
    __syncthreads();
    const int sigma = pair_factors<DK>(Ai, Rj, Fac, red);
    // Q'' = q_hat * 2^(A_I - R_J - sigma): row-major and transposed
    for (int x = tid; x < XC * DK / 8; x += 256) {
      const int r = x / (DK / 8), p = x % (DK / 8);
      const u32x4 wq = ld16(qbh + ((int64_t)hq * ntok + bos + i0 + r) * DK + 8 * p, r < nq);
      u32x4 o;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int n = 8 * p + 2 * e;
        const float a = f16_lo(wq[e]) * __builtin_amdgcn_ldexpf(1.f, (int)Fac[n] - sigma);
        const float b = f16_hi(wq[e]) * __builtin_amdgcn_ldexpf(1.f, (int)Fac[n + 1] - sigma);
        o[e] = pack_f16x2(a, b);
        QpT[n * RS + r] = to_h(a);
        QpT[(n + 1) * RS + r] = to_h(b);
      }
      *reinterpret_cast<u32x4 *>(Qp + r * KS + 8 * p) = o;
    }
    for (int x = tid; x < XC * DV / 8; x += 256) {
      const int r = x / (DV / 8), p = x % (DV / 8);
      const u32x4 wo = ld16(dO + ((bos + i0 + r) * HQ + hq) * DV + 8 * p, r < nq);
      *reinterpret_cast<u32x4 *>(Os + r * VS + 8 * p) = wo;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        OsT[(8 * p + 2 * e) * RS + r] = (bf16_t)(wo[e] & 0xffffu);
        OsT[(8 * p + 2 * e + 1) * RS + r] = (bf16_t)(wo[e] >> 16);
      }
    }
    if (tid < XC) {
      const bool ok = tid < nq;
      const int64_t t = bos + i0 + tid;
      Li[tid] = ok ? lse[t * HQ + hq] * LOG2E : 0.f;
      Di[tid] = ok ? Dv[t * HQ + hq] : 0.f;
      Gi[tid] = (HAS_GS && ok) ? gsum[t * HQ + hq] : 0.f;
    }
    __syncthreads();
    // S^T (keys 32kb, rows 32wh) and dP^T = V dO^T
    f32x16 S = f32x16{}, dP = f32x16{};
#pragma unroll
    for (int ks = 0; ks < DK / 16; ++ks)
      S = mma16<_Float16>(S, Kt + 32 * kb * KS, KS, Qp + 32 * wh * KS, KS, 16 * ks, lane);
#pragma unroll
    for (int ks = 0; ks < DV / 16; ++ks)
      dP = mma16<bf16_t>(dP, Vs + 32 * kb * VS, VS, Os + 32 * wh * VS, VS, 16 * ks, lane);
    const float ssc = __builtin_amdgcn_ldexpf(1.f, sigma);
    const int n = 32 * wh + (lane & 31);  // query row in the chunk
    const int irel = i0 + n;
    const float Lr = Li[n], Dr = Di[n], Gr = Gi[n];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int m = 32 * kb + crow(r, lane);  // key in the chunk
      const int jrel = j0 + m;
      float s2 = S[r] * ssc;
      if (HAS_GS) s2 += Gr - Gj[m];
      const bool ok = n < nq && m < nk && jrel <= irel && !(window > 0 && irel - jrel >= window);
      const float p = ok ? fast_exp2(s2 - Lr) : 0.f;
      const float ds = p * (dP[r] - Dr);
      csum[r] += ds;
      PT[m * RS + n] = to_b(p);
      DST[m * RS + n] = to_h(ds);
    }
    __syncthreads();
    // dV += P^T dO and dK'' += ds^T Q'' over the chunk's 64 rows
#pragma unroll
    for (int b = 0; b < NBV; ++b) {
      const int c0 = (DV / 2) * wh + 32 * b;
#pragma unroll
      for (int ks = 0; ks < XC / 16; ++ks)
        dVacc[b] = mma16<bf16_t>(dVacc[b], PT + 32 * kb * RS, RS, OsT + c0 * RS, RS, 16 * ks, lane);
    }
#pragma unroll
    for (int b = 0; b < NBK; ++b) {
      const int n0 = (DK / 2) * wh + 32 * b;
      if (sigma == 0) {
#pragma unroll
        for (int ks = 0; ks < XC / 16; ++ks)
          dKacc[b] = mma16<_Float16>(dKacc[b], DST + 32 * kb * RS, RS, QpT + n0 * RS, RS, 16 * ks, lane);
      } else {
        f32x16 t = f32x16{};
#pragma unroll
        for (int ks = 0; ks < XC / 16; ++ks)
          t = mma16<_Float16>(t, DST + 32 * kb * RS, RS, QpT + n0 * RS, RS, 16 * ks, lane);
        dKacc[b] += t * ssc;
      }
    }
  }
  __syncthreads();
  // P2 of the key chunk (in the Qp/QpT space), then the outputs
  float *P2s = reinterpret_cast<float *>(lds + O_QP);
  chunk_p2<DK>(g, off + ((cbase + J) * HQ + hq) * DK, bos + j0, nk, HQ, hq, P2s, tot);
#pragma unroll
  for (int b = 0; b < NBK; ++b) {
    const int nc = (DK / 2) * wh + 32 * b + (lane & 31);
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int m = 32 * kb + crow(r, lane);
      if (m < nk)
        dk_part[((bos + j0 + m) * HQ + hq) * DK + nc] =
            LN2 * fast_exp2(Rj[nc] - P2s[m * DK + nc]) * dKacc[b][r];
    }
  }
#pragma unroll
  for (int b = 0; b < NBV; ++b) {
    const int c = (DV / 2) * wh + 32 * b + (lane & 31);
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int m = 32 * kb + crow(r, lane);
      if (m < nk) dv_part[((bos + j0 + m) * HQ + hq) * DV + c] = dVacc[b][r];
    }
  }
  // column sums: over the 32 lanes of a half-wave, then the two row halves
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    float x = csum[r];
#pragma unroll
    for (int o = 16; o >= 1; o >>= 1) x += __shfl_xor(x, o);
    csum[r] = x;
  }
  if ((lane & 31) == 0)
#pragma unroll
    for (int r = 0; r < 16; ++r) csh[wh][32 * kb + crow(r, lane)] = csum[r];
  __syncthreads();
  if (tid < nk) cols_ds[(bos + j0 + tid) * HQ + hq] = csh[0][tid] + csh[1][tid];
}

// dq and the row sums of ds.  grid (NCmax*HQ, nseg): x = query chunk
// (longest first) * HQ + head, y = segment.  Waves: w>>1 picks 32 query rows; w&1
// picks 32 keys (scores) or half the channels (dq).
template <int DK, int DV, bool HAS_GS>
__global__ __launch_bounds__(256) void k_bwd_dq_mfma(
    const _Float16 *__restrict__ kt, const _Float16 *__restrict__ qbh, const bf16_t *__restrict__ v,
    const bf16_t *__restrict__ dO, const bf16_t *__restrict__ g, const float *__restrict__ off,
    const float *__restrict__ anch, const float *__restrict__ gsum, const float *__restrict__ lse,
    const float *__restrict__ Dv, const int *__restrict__ wide, float *__restrict__ dq32,
    float *__restrict__ rows_ds, const int32_t *__restrict__ cu, int64_t T, int64_t ntok, int HQ,
    int H, int NCmax, int window, float scale) {
  constexpr int KS = DK + 8, VS = DV + 8, RS = XC + 8;
  constexpr int KX = DK + 16;
  constexpr int NBK = DK / 64;
  constexpr int O_QH = 0, O_QP = O_QH + XC * KS * 2, O_OS = O_QP + XC * KS * 2,
                O_KT = O_OS + XC * VS * 2, O_KTT = O_KT + XC * KS * 2, O_VS = O_KTT + DK * RS * 2,
                O_DS = O_VS + XC * VS * 2, O_END = O_DS + XC * RS * 2;
  static_assert(O_KTT - O_QP >= XC * DK * 4, "P2 scratch reuses Qp, Os and Kt");
  __shared__ __attribute__((aligned(16))) unsigned char lds[O_END];
  __shared__ float Aq[DK], Rj[DK], Fac[DK], Li[XC], Di[XC], Gi[XC], Gj[XC], red[4], tot[256];
  __shared__ float rsh[2][XC];
  _Float16 *Qh = reinterpret_cast<_Float16 *>(lds + O_QH);
  _Float16 *Qp = reinterpret_cast<_Float16 *>(lds + O_QP);
  bf16_t *Os = reinterpret_cast<bf16_t *>(lds + O_OS);
  _Float16 *Kt = reinterpret_cast<_Float16 *>(lds + O_KT);
  _Float16 *KtT = reinterpret_cast<_Float16 *>(lds + O_KTT);
  bf16_t *Vs = reinterpret_cast<bf16_t *>(lds + O_VS);
  _Float16 *DS = reinterpret_cast<_Float16 *>(lds + O_DS);

  const int hq = blockIdx.x % HQ, seg = blockIdx.y;
  if (__builtin_amdgcn_readfirstlane(wide[seg * HQ + hq]) != 0) return;
  int64_t bos, eos;
  segment_bounds(seg, T, cu, bos, eos);
  const int L = (int)min(eos - bos, (int64_t)NCmax * XC);
  const int nch = (L + XC - 1) / XC;
  const int I = NCmax - 1 - (int)(blockIdx.x / HQ);
  if (I >= nch) return;
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int rb = w >> 1, wk = w & 1;
  const int h = hq / (HQ / H);
  const int i0 = I * XC, nq = min(XC, L - i0);
  const int64_t cbase = (int64_t)seg * NCmax;

  // the query chunk: q_hat, dO, anchors, statistics
  for (int x = tid; x < XC * DK / 8; x += 256) {
    const int r = x / (DK / 8), p = x % (DK / 8);
    *reinterpret_cast<u32x4 *>(Qh + r * KS + 8 * p) =
        ld16(qbh + ((int64_t)hq * ntok + bos + i0 + r) * DK + 8 * p, r < nq);
  }
  for (int x = tid; x < XC * DV / 8; x += 256) {
    const int r = x / (DV / 8), p = x % (DV / 8);
    *reinterpret_cast<u32x4 *>(Os + r * VS + 8 * p) =
        ld16(dO + ((bos + i0 + r) * HQ + hq) * DV + 8 * p, r < nq);
  }
  if (tid < DK) Aq[tid] = anch[((cbase + I) * HQ + hq) * DK + tid];
  if (tid < XC) {
    const bool ok = tid < nq;
    const int64_t t = bos + i0 + tid;
    Li[tid] = ok ? lse[t * HQ + hq] * LOG2E : 0.f;
    Di[tid] = ok ? Dv[t * HQ + hq] : 0.f;
    Gi[tid] = (HAS_GS && ok) ? gsum[t * HQ + hq] : 0.f;
  }

  f32x16 dQacc[NBK];
#pragma unroll
  for (int b = 0; b < NBK; ++b) dQacc[b] = f32x16{};
  float rsum[16];
#pragma unroll
  for (int r = 0; r < 16; ++r) rsum[r] = 0.f;

  const int Jlo = window > 0 ? max(0, i0 - window + 1) / XC : 0;
  for (int J = Jlo; J <= I; ++J) {
    const int j0 = J * XC, nk = min(XC, L - j0);
    __syncthreads();  // the previous pair's operands are consumed
    if (tid < DK) Rj[tid] = anch[((cbase + J) * HQ + hq) * DK + tid];
    __syncthreads();
    const int sigma = pair_factors<DK>(Aq, Rj, Fac, red);
    for (int x = tid; x < XC * DK / 8; x += 256) {
      const int r = x / (DK / 8), p = x % (DK / 8);
      const u32x4 wk_ = ld16(kt + ((int64_t)hq * ntok + bos + j0 + r) * KX + 8 * p, r < nk);
      *reinterpret_cast<u32x4 *>(Kt + r * KS + 8 * p) = wk_;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        KtT[(8 * p + 2 * e) * RS + r] = __builtin_bit_cast(_Float16, (uint16_t)(wk_[e] & 0xffffu));
        KtT[(8 * p + 2 * e + 1) * RS + r] = __builtin_bit_cast(_Float16, (uint16_t)(wk_[e] >> 16));
      }
      // Q'' = q_hat * 2^(A_I - R_J - sigma)
      const u32x4 wq = *reinterpret_cast<const u32x4 *>(Qh + r * KS + 8 * p);
      u32x4 o;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int n = 8 * p + 2 * e;
        o[e] = pack_f16x2(f16_lo(wq[e]) * __builtin_amdgcn_ldexpf(1.f, (int)Fac[n] - sigma),
                          f16_hi(wq[e]) * __builtin_amdgcn_ldexpf(1.f, (int)Fac[n + 1] - sigma));
      }
      *reinterpret_cast<u32x4 *>(Qp + r * KS + 8 * p) = o;
    }
    for (int x = tid; x < XC * DV / 8; x += 256) {
      const int r = x / (DV / 8), p = x % (DV / 8);
      *reinterpret_cast<u32x4 *>(Vs + r * VS + 8 * p) =
          ld16(v + ((bos + j0 + r) * H + h) * DV + 8 * p, r < nk);
    }
    if (tid < XC) Gj[tid] = (HAS_GS && tid < nk) ? gsum[(bos + j0 + tid) * HQ + hq] : 0.f;
    __syncthreads();
    // S (rows 32rb, keys 32wk) and dP = dO V^T
    f32x16 S = f32x16{}, dP = f32x16{};
#pragma unroll
    for (int ks = 0; ks < DK / 16; ++ks)
      S = mma16<_Float16>(S, Qp + 32 * rb * KS, KS, Kt + 32 * wk * KS, KS, 16 * ks, lane);
#pragma unroll
    for (int ks = 0; ks < DV / 16; ++ks)
      dP = mma16<bf16_t>(dP, Os + 32 * rb * VS, VS, Vs + 32 * wk * VS, VS, 16 * ks, lane);
    const float ssc = __builtin_amdgcn_ldexpf(1.f, sigma);
    const int n = 32 * wk + (lane & 31);  // key in the chunk
    const int jrel = j0 + n;
    const float Gk = Gj[n];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int m = 32 * rb + crow(r, lane);  // query row in the chunk
      const int irel = i0 + m;
      float s2 = S[r] * ssc;
      if (HAS_GS) s2 += Gi[m] - Gk;
      const bool ok = m < nq && n < nk && jrel <= irel && !(window > 0 && irel - jrel >= window);
      const float p = ok ? fast_exp2(s2 - Li[m]) : 0.f;
      const float ds = p * (dP[r] - Di[m]);
      rsum[r] += ds;
      DS[m * RS + n] = to_h(ds);
    }
    __syncthreads();
    // dQ += (ds k_tilde) * d_IJ, the factor per channel (column)
#pragma unroll
    for (int b = 0; b < NBK; ++b) {
      const int n0 = (DK / 2) * wk + 32 * b;
      f32x16 t = f32x16{};
#pragma unroll
      for (int ks = 0; ks < XC / 16; ++ks)
        t = mma16<_Float16>(t, DS + 32 * rb * RS, RS, KtT + n0 * RS, RS, 16 * ks, lane);
      const float fq = __builtin_amdgcn_ldexpf(1.f, (int)Fac[n0 + (lane & 31)]);
      dQacc[b] += t * fq;
    }
  }
  __syncthreads();
  float *P2s = reinterpret_cast<float *>(lds + O_QP);
  chunk_p2<DK>(g, off + ((cbase + I) * HQ + hq) * DK, bos + i0, nq, HQ, hq, P2s, tot);
#pragma unroll
  for (int b = 0; b < NBK; ++b) {
    const int nc = (DK / 2) * wk + 32 * b + (lane & 31);
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int m = 32 * rb + crow(r, lane);
      if (m < nq)
        dq32[((bos + i0 + m) * HQ + hq) * DK + nc] =
            scale * fast_exp2(P2s[m * DK + nc] - Aq[nc]) * dQacc[b][r];
    }
  }
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    float x = rsum[r];
#pragma unroll
    for (int o = 16; o >= 1; o >>= 1) x += __shfl_xor(x, o);
    rsum[r] = x;
  }
  if ((lane & 31) == 0)
#pragma unroll
    for (int r = 0; r < 16; ++r) rsh[wk][32 * rb + crow(r, lane)] = rsum[r];
  __syncthreads();
  if (tid < nq) rows_ds[(bos + i0 + tid) * HQ + hq] = rsh[0][tid] + rsh[1][tid];
}

template <int DK, int DV>
hipError_t bwd_mfma_t(const BwdProblem &b, const FwdWorkspace &ws, const BwdWorkspace &bw,
                      hipStream_t st) {
  const FwdProblem &p = b.f;
  const int NCmax = (int)((p.maxlen + CHUNK - 1) / CHUNK);
  const int W = (int)(p.window > 0 && p.window < p.maxlen ? p.window : 0);
  const dim3 grid((unsigned)(NCmax * p.HQ), (unsigned)p.nseg);
  const bool gs = p.g_scalar != nullptr;
  auto kv = gs ? k_bwd_dkdv_mfma<DK, DV, true> : k_bwd_dkdv_mfma<DK, DV, false>;
  hipLaunchKernelGGL(kv, grid, dim3(256), 0, st, static_cast<const _Float16 *>(ws.kt),
                     static_cast<const _Float16 *>(bw.qbh), static_cast<const bf16_t *>(p.v),
                     static_cast<const bf16_t *>(b.dO), static_cast<const bf16_t *>(p.g), ws.csum,
                     ws.anch, ws.gsum, b.lse, bw.Dv, ws.wide, bw.dk_part, bw.dv_part, bw.cols_ds,
                     p.cu, p.T, p.ntok, (int)p.HQ, (int)p.H, NCmax, W);
  auto qk = gs ? k_bwd_dq_mfma<DK, DV, true> : k_bwd_dq_mfma<DK, DV, false>;
  hipLaunchKernelGGL(qk, grid, dim3(256), 0, st, static_cast<const _Float16 *>(ws.kt),
                     static_cast<const _Float16 *>(bw.qbh), static_cast<const bf16_t *>(p.v),
                     static_cast<const bf16_t *>(b.dO), static_cast<const bf16_t *>(p.g), ws.csum,
                     ws.anch, ws.gsum, b.lse, bw.Dv, ws.wide, bw.dq32, bw.rows_ds, p.cu, p.T,
                     p.ntok, (int)p.HQ, (int)p.H, NCmax, W, p.scale);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_attn_bwd_mfma(const BwdProblem &b, const FwdWorkspace &ws,
                                const BwdWorkspace &bw, hipStream_t st) {
  const FwdProblem &p = b.f;
  if (p.K == 64) return p.V == 64 ? bwd_mfma_t<64, 64>(b, ws, bw, st) : bwd_mfma_t<64, 128>(b, ws, bw, st);
  return p.V == 64 ? bwd_mfma_t<128, 64>(b, ws, bw, st) : bwd_mfma_t<128, 128>(b, ws, bw, st);
}

}  // namespace wa

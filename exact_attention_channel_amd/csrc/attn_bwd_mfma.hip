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
//   dq_i  = scale 2^(P2_i - A_I) sum_J ds (k_tilde_J * d_IJ).
// Decaying channels have d_IJ <= 1 (anchors are rounded chunk-end decay
// sums, which do not rise).  A pair of chunks with some d_IJ above 2^4 (a
// decay sum rising by more than 4 log2 units) would push the rescaled half
// operands towards overflow: the workgroup that meets one flags its
// (sequence, head) and stops, and the float32 kernels, which run after
// these and take every flagged pair, recompute that pair's gradients.
//
// Products are v_mfma_f32_32x32x16 (half for the rescaled q/k and ds, bf16
// for P, V and dO).  P and ds never leave registers: a 32x32 score tile
// holds, in lane l, column l%32 and the rows 8(r/4) + 4(l/32) + r%4 of its
// 16 values r, which is the B operand of a product contracting over those
// rows once the contraction index is taken in that order (two 16-row MFMAs
// per tile).  The matching A operand -- dO^T, the rescaled q^T or k^T --
// comes from row-major LDS tiles through ds_read_b64_tr_b16, which hands
// lane i of each 16-lane group column i of the 4 x 16 block its lanes
// address.  One workgroup per 64-key chunk walks the query chunks that see
// it (dk, dv, column sums of ds); one per 64-row query chunk walks its key
// chunks (dq, row sums).  Waves split a 64 x 64 block of pairs 2 x 2; the
// next block's tiles are fetched into registers while the current block's
// gradient products run.  The float32 finishing kernels of attn_bwd.hip (reverse
// running sums, sums over query heads) complete the gradients.
#include <math.h>

#include "common.h"
#include "launch.h"

namespace wa {
namespace {

constexpr int XC = CHUNK;  // 64 rows of a query chunk, keys of a key chunk

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef short s16x8 __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

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

// Row of element r of a 32x32 MFMA result tile in lane `lane` (its column is lane % 32).
__device__ __forceinline__ int crow(int r, int lane) { return 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3); }

// Operand (8 elements k = 8 (lane/32) .. +7 of row lane%32) of a row-major
// LDS matrix [32 rows][stride] at column k0.
template <typename T>
__device__ __forceinline__ typename Mfma<T>::V row_operand(const T *M, int stride, int k0, int lane) {
  return *reinterpret_cast<const typename Mfma<T>::V *>(M + (lane & 31) * stride + k0 + 8 * (lane >> 5));
}

__device__ __forceinline__ s16x4 tr16(const void *p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)(p));
}

// A operand of a product that contracts over the rows x of a row-major LDS
// matrix M [x][z] (stride in elements): output rows z0 .. z0+31, contraction
// rows x0 + 4 (lane/32) + {0..3, 8..11} -- the rows a result tile's values
// r = 0..7 hold (x0 = tile base + 16 m for its values 8m .. 8m+7).
template <typename T>
__device__ __forceinline__ typename Mfma<T>::V tr_operand(const T *M, int stride, int x0, int z0,
                                                         int lane) {
  const int row = x0 + 4 * (lane >> 5) + ((lane >> 2) & 3);
  const int col = z0 + 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
  const s16x4 lo = tr16(M + row * stride + col);
  const s16x4 hi = tr16(M + (row + 8) * stride + col);
  const s16x8 v = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
  return __builtin_bit_cast(typename Mfma<T>::V, v);
}

// B operand from a result tile's values 8m .. 8m+7, rounded to T.
__device__ __forceinline__ f16x8 pack_h(const float *x) {
  const u32x4 w = {pack_f16x2(x[0], x[1]), pack_f16x2(x[2], x[3]), pack_f16x2(x[4], x[5]),
                   pack_f16x2(x[6], x[7])};
  return __builtin_bit_cast(f16x8, w);
}
__device__ __forceinline__ bf16x8 pack_b(const float *x) {
  const u32x4 w = {pack_bf16x2(x[0], x[1]), pack_bf16x2(x[2], x[3]), pack_bf16x2(x[4], x[5]),
                   pack_bf16x2(x[6], x[7])};
  return __builtin_bit_cast(bf16x8, w);
}

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

// 8 half values times 2^e[i] (e: integer-valued chunk factors, at most 4).
__device__ __forceinline__ u32x4 rescale8(u32x4 w, const float *e) {
  u32x4 o;
#pragma unroll
  for (int i = 0; i < 4; ++i)
    o[i] = pack_f16x2(f16_lo(w[i]) * __builtin_amdgcn_ldexpf(1.f, (int)e[2 * i]),
                      f16_hi(w[i]) * __builtin_amdgcn_ldexpf(1.f, (int)e[2 * i + 1]));
  return o;
}

// Whether every chunk factor a[n] - b[n] of the DK channels is at most 4;
// every wave decides it from its own lanes' share (channel lane + 64 c), so
// all waves of a workgroup agree.
template <int DK>
__device__ __forceinline__ bool factors_in_range(const float *a, const float *b) {
  float m = -INFINITY;
#pragma unroll
  for (int c = 0; c < DK / 64; ++c) m = fmaxf(m, a[c] - b[c]);
  return wave_max(m) <= 4.f;
}

// ---------------------------------------------------------------------------
// dk, dv (each query head's share) and the column sums of ds.
// grid (NCmax*HQ, nseg): x = key chunk (longest first) * HQ + head, y = segment.
// Wave w: query rows 32 (w&1), keys 32 (w>>1) of each 64 x 64 block.
template <int DK, int DV, bool HAS_GS>
__global__ __launch_bounds__(256, 2) void k_bwd_dkdv_mfma(
    const _Float16 *__restrict__ kt, const _Float16 *__restrict__ qbh, const bf16_t *__restrict__ v,
    const bf16_t *__restrict__ dO, const bf16_t *__restrict__ g, const float *__restrict__ off,
    const float *__restrict__ anch, const float *__restrict__ gsum, const float *__restrict__ lse,
    const float *__restrict__ Dv, int *__restrict__ wide, float *__restrict__ dk_part,
    float *__restrict__ dv_part, float *__restrict__ cols_ds, const int32_t *__restrict__ cu,
    int64_t T, int64_t ntok, int HQ, int H, int NCmax, int window) {
  constexpr int KS = DK + 8, VS = DV + 8;  // padded LDS row strides (elements)
  constexpr int KX = DK + 16;              // k_tilde row in the forward workspace
  constexpr int TK = DK / 32, TV = DV / 32;
  constexpr int QI = XC * DK / 8 / 256, OI = XC * DV / 8 / 256;  // 16-byte items per thread
  constexpr int O_KT = 0, O_VS = O_KT + XC * KS * 2, O_QP = O_VS + XC * VS * 2,
                O_OS = O_QP + XC * KS * 2, O_LOOP = O_OS + XC * VS * 2;
  // epilogue: the two row halves' partial sums; P2 of the key chunk then
  // takes the place of dv's
  constexpr int XKS = DK + 1, XVS = DV + 1;
  constexpr int E_XV = XC * XKS * 4, E_P2 = E_XV;
  constexpr int E_END = E_XV + (XVS > DK ? XC * XVS * 4 : XC * DK * 4);
  constexpr int LDS_BYTES = O_LOOP > E_END ? O_LOOP : E_END;
  __shared__ __attribute__((aligned(16))) unsigned char lds[LDS_BYTES];
  __shared__ __attribute__((aligned(16))) float Rj[DK], Li[XC], Di[XC], Gi[XC], Gj[XC], csh[2][XC];
  __shared__ float tot[256];
  _Float16 *Kt = reinterpret_cast<_Float16 *>(lds + O_KT);
  bf16_t *Vs = reinterpret_cast<bf16_t *>(lds + O_VS);
  _Float16 *Qp = reinterpret_cast<_Float16 *>(lds + O_QP);
  bf16_t *Os = reinterpret_cast<bf16_t *>(lds + O_OS);

  const int hq = blockIdx.x % HQ, J = blockIdx.x / HQ, seg = blockIdx.y;
  if (__builtin_amdgcn_readfirstlane(wide[seg * HQ + hq]) != 0) return;
  int64_t bos, eos;
  segment_bounds(seg, T, cu, bos, eos);
  const int L = (int)min(eos - bos, (int64_t)NCmax * XC);
  const int nch = (L + XC - 1) / XC;
  if (J >= nch) return;
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int qb = w & 1, kb = w >> 1;
  const int h = hq / (HQ / H);
  const int j0 = J * XC, nk = min(XC, L - j0);
  const int64_t cbase = (int64_t)seg * NCmax;
  const float *anch_h = anch + (int64_t)hq * DK;  // chunk c: + c*HQ*DK

  // the key chunk: k_tilde, v, anchors, gate sums
#pragma unroll
  for (int u = 0; u < QI; ++u) {
    const int x = tid + 256 * u, r = x / (DK / 8), p = x % (DK / 8);
    *reinterpret_cast<u32x4 *>(Kt + r * KS + 8 * p) =
        ld16(kt + ((int64_t)hq * ntok + bos + j0 + r) * KX + 8 * p, r < nk);
  }
#pragma unroll
  for (int u = 0; u < OI; ++u) {
    const int x = tid + 256 * u, r = x / (DV / 8), p = x % (DV / 8);
    *reinterpret_cast<u32x4 *>(Vs + r * VS + 8 * p) =
        ld16(v + ((bos + j0 + r) * H + h) * DV + 8 * p, r < nk);
  }
  if (tid < DK) Rj[tid] = anch_h[(cbase + J) * HQ * DK + tid];
  if (tid < XC) Gj[tid] = (HAS_GS && tid < nk) ? gsum[(bos + j0 + tid) * HQ + hq] : 0.f;
  __syncthreads();

  // this thread's staging items: channels 8 pq .. 8 pq + 7 of rows rq + stride u
  const int pq = tid % (DK / 8), po = tid % (DV / 8);
  float rjw[DK / 64];
#pragma unroll
  for (int c = 0; c < DK / 64; ++c) rjw[c] = Rj[lane + 64 * c];

  // prefetch registers of the next query chunk
  u32x4 fq[QI], fo[OI];
  float fe8[8], faw[DK / 64], frow[3] = {0.f, 0.f, 0.f};
  auto fetch = [&](int I) {
    const int i0 = I * XC, nq = min(XC, L - i0);
#pragma unroll
    for (int u = 0; u < QI; ++u) {
      const int r = (tid + 256 * u) / (DK / 8);
      fq[u] = ld16(qbh + ((int64_t)hq * ntok + bos + i0 + r) * DK + 8 * pq, r < nq);
    }
#pragma unroll
    for (int u = 0; u < OI; ++u) {
      const int r = (tid + 256 * u) / (DV / 8);
      fo[u] = ld16(dO + ((bos + i0 + r) * HQ + hq) * DV + 8 * po, r < nq);
    }
    const float *aI = anch_h + (cbase + I) * HQ * DK;
    const f32x4 a0 = *reinterpret_cast<const f32x4 *>(aI + 8 * pq);
    const f32x4 a1 = *reinterpret_cast<const f32x4 *>(aI + 8 * pq + 4);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      fe8[e] = a0[e] - Rj[8 * pq + e];
      fe8[4 + e] = a1[e] - Rj[8 * pq + 4 + e];
    }
#pragma unroll
    for (int c = 0; c < DK / 64; ++c) faw[c] = aI[lane + 64 * c];
    if (tid < XC) {
      const bool ok = tid < nq;
      const int64_t t = bos + i0 + tid;
      frow[0] = ok ? lse[t * HQ + hq] * LOG2E : 0.f;
      frow[1] = ok ? Dv[t * HQ + hq] : 0.f;
      frow[2] = (HAS_GS && ok) ? gsum[t * HQ + hq] : 0.f;
    }
  };
  // registers -> LDS: Q'' = q_hat 2^(A_I - R_J), dO, row statistics; false
  // (nothing written) when a chunk factor is out of range
  auto commit = [&]() {
    if (!factors_in_range<DK>(faw, rjw)) return false;
#pragma unroll
    for (int u = 0; u < QI; ++u) {
      const int r = (tid + 256 * u) / (DK / 8);
      *reinterpret_cast<u32x4 *>(Qp + r * KS + 8 * pq) = rescale8(fq[u], fe8);
    }
#pragma unroll
    for (int u = 0; u < OI; ++u) {
      const int r = (tid + 256 * u) / (DV / 8);
      *reinterpret_cast<u32x4 *>(Os + r * VS + 8 * po) = fo[u];
    }
    if (tid < XC) { Li[tid] = frow[0]; Di[tid] = frow[1]; Gi[tid] = frow[2]; }
    return true;
  };

  f32x16 dVa[TV], dKa[TK];
#pragma unroll
  for (int t = 0; t < TV; ++t) dVa[t] = f32x16{};
#pragma unroll
  for (int t = 0; t < TK; ++t) dKa[t] = f32x16{};
  float csum = 0.f;

  const int Ihi = window > 0 ? min(nch - 1, (j0 + XC - 1 + window - 1) / XC) : nch - 1;
  fetch(J);
  if (!commit()) {
    if (tid == 0) wide[seg * HQ + hq] = 1;
    return;
  }
  __syncthreads();
  const int key = 32 * kb + (lane & 31);  // this lane's key in the chunk
  const int jrel = j0 + key;
  const float gk = Gj[key];
  for (int I = J; I <= Ihi; ++I) {
    const int i0 = I * XC, nq = min(XC, L - i0);
    // S = Q'' K^T, dP = dO V^T for rows 32 qb, keys 32 kb
    f32x16 S = f32x16{}, dP = f32x16{};
#pragma unroll
    for (int ks = 0; ks < DK / 16; ++ks)
      S = Mfma<_Float16>::run(row_operand(Qp + 32 * qb * KS, KS, 16 * ks, lane),
                              row_operand(Kt + 32 * kb * KS, KS, 16 * ks, lane), S);
#pragma unroll
    for (int ks = 0; ks < DV / 16; ++ks)
      dP = Mfma<bf16_t>::run(row_operand(Os + 32 * qb * VS, VS, 16 * ks, lane),
                             row_operand(Vs + 32 * kb * VS, VS, 16 * ks, lane), dP);
    // every pair of the block visible: full chunks, strictly below the
    // diagonal, inside the window
    const bool full = nq == XC && nk == XC && I > J && !(window > 0 && i0 + XC - 1 - j0 >= window);
    float pv[16], dsv[16];
#pragma unroll
    for (int a = 0; a < 4; ++a) {
      const int n0 = 32 * qb + 8 * a + 4 * (lane >> 5);  // rows n0 .. n0+3 (values 4a .. 4a+3)
      const f32x4 l4 = *reinterpret_cast<const f32x4 *>(Li + n0);
      const f32x4 d4 = *reinterpret_cast<const f32x4 *>(Di + n0);
      f32x4 g4 = f32x4{};
      if (HAS_GS) g4 = *reinterpret_cast<const f32x4 *>(Gi + n0);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int r = 4 * a + e;
        float s2 = S[r];
        if (HAS_GS) s2 += g4[e] - gk;
        bool ok = true;
        if (!full) {
          const int irel = i0 + n0 + e;
          ok = n0 + e < nq && key < nk && jrel <= irel && !(window > 0 && irel - jrel >= window);
        }
        const float p = ok ? fast_exp2(s2 - l4[e]) : 0.f;
        const float ds = p * (dP[r] - d4[e]);
        pv[r] = p;
        dsv[r] = ds;
        csum += ds;
      }
    }
    // dV^T += dO^T P and dK^T += Q''^T ds, contracting over the 32 rows
#pragma unroll
    for (int m = 0; m < 2; ++m) {
      const bf16x8 pb = pack_b(pv + 8 * m);
#pragma unroll
      for (int t = 0; t < TV; ++t)
        dVa[t] = Mfma<bf16_t>::run(tr_operand(Os, VS, 32 * qb + 16 * m, 32 * t, lane), pb, dVa[t]);
      const f16x8 db = pack_h(dsv + 8 * m);
#pragma unroll
      for (int t = 0; t < TK; ++t)
        dKa[t] = Mfma<_Float16>::run(tr_operand(Qp, KS, 32 * qb + 16 * m, 32 * t, lane), db, dKa[t]);
    }
    __syncthreads();  // the block's tiles are consumed
    if (I < Ihi) {
      fetch(I + 1);
      if (!commit()) {
        if (tid == 0) wide[seg * HQ + hq] = 1;
        return;
      }
      __syncthreads();
    }
  }

  // sum the two row halves' partials in LDS ([key][channel]), then write out
  float *Xk = reinterpret_cast<float *>(lds);
  float *Xv = reinterpret_cast<float *>(lds + E_XV);
  float *P2s = reinterpret_cast<float *>(lds + E_P2);
  const float cs = csum + __shfl_xor(csum, 32);
  if (lane < 32) csh[qb][key] = cs;
  if (qb == 1) {
#pragma unroll
    for (int t = 0; t < TV; ++t)
#pragma unroll
      for (int r = 0; r < 16; ++r) Xv[key * XVS + 32 * t + crow(r, lane)] = dVa[t][r];
#pragma unroll
    for (int t = 0; t < TK; ++t)
#pragma unroll
      for (int r = 0; r < 16; ++r) Xk[key * XKS + 32 * t + crow(r, lane)] = dKa[t][r];
  }
  __syncthreads();
  if (qb == 0) {
#pragma unroll
    for (int t = 0; t < TV; ++t)
#pragma unroll
      for (int r = 0; r < 16; ++r) Xv[key * XVS + 32 * t + crow(r, lane)] += dVa[t][r];
#pragma unroll
    for (int t = 0; t < TK; ++t)
#pragma unroll
      for (int r = 0; r < 16; ++r) Xk[key * XKS + 32 * t + crow(r, lane)] += dKa[t][r];
  }
  __syncthreads();
  for (int x = tid; x < nk * DV; x += 256) {
    const int m = x / DV, c = x % DV;
    dv_part[((bos + j0 + m) * HQ + hq) * DV + c] = Xv[m * XVS + c];
  }
  __syncthreads();  // dv is read out before P2s overwrites it
  chunk_p2<DK>(g, off + ((cbase + J) * HQ + hq) * DK, bos + j0, nk, HQ, hq, P2s, tot);
  for (int x = tid; x < nk * DK; x += 256) {
    const int m = x / DK, c = x % DK;
    dk_part[((bos + j0 + m) * HQ + hq) * DK + c] =
        LN2 * fast_exp2(Rj[c] - P2s[m * DK + c]) * Xk[m * XKS + c];
  }
  if (tid < nk) cols_ds[(bos + j0 + tid) * HQ + hq] = csh[0][tid] + csh[1][tid];
}

// ---------------------------------------------------------------------------
// dq and the row sums of ds.  grid (NCmax*HQ, nseg): x = query chunk
// (longest first) * HQ + head, y = segment.  Wave w: query rows 32 (w&1),
// keys 32 (w>>1) of each 64 x 64 block; its q_hat and dO rows stay in
// registers.
template <int DK, int DV, bool HAS_GS>
__global__ __launch_bounds__(256, 2) void k_bwd_dq_mfma(
    const _Float16 *__restrict__ kt, const _Float16 *__restrict__ qbh, const bf16_t *__restrict__ v,
    const bf16_t *__restrict__ dO, const bf16_t *__restrict__ g, const float *__restrict__ off,
    const float *__restrict__ anch, const float *__restrict__ gsum, const float *__restrict__ lse,
    const float *__restrict__ Dv, int *__restrict__ wide, float *__restrict__ dq32,
    float *__restrict__ rows_ds, const int32_t *__restrict__ cu, int64_t T, int64_t ntok, int HQ,
    int H, int NCmax, int window, float scale) {
  constexpr int KS = DK + 8, VS = DV + 8;
  constexpr int KX = DK + 16;
  constexpr int TK = DK / 32;
  constexpr int QI = XC * DK / 8 / 256, OI = XC * DV / 8 / 256;
  constexpr int O_KT = 0, O_VS = O_KT + XC * KS * 2, O_LOOP = O_VS + XC * VS * 2;
  constexpr int XQS = DK + 1;
  constexpr int E_P2 = XC * XQS * 4, E_END = E_P2 + XC * DK * 4;
  constexpr int LDS_BYTES = O_LOOP > E_END ? O_LOOP : E_END;
  __shared__ __attribute__((aligned(16))) unsigned char lds[LDS_BYTES];
  __shared__ __attribute__((aligned(16))) float Aq[DK], Gj[XC], rsh[2][XC];
  __shared__ float tot[256];
  _Float16 *Kt = reinterpret_cast<_Float16 *>(lds + O_KT);
  bf16_t *Vs = reinterpret_cast<bf16_t *>(lds + O_VS);

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
  const int qb = w & 1, kb = w >> 1;
  const int h = hq / (HQ / H);
  const int i0 = I * XC, nq = min(XC, L - i0);
  const int64_t cbase = (int64_t)seg * NCmax;
  const float *anch_h = anch + (int64_t)hq * DK;

  // this lane's query row: q_hat and dO as B operands, row statistics
  const int qrow = 32 * qb + (lane & 31);
  const bool qok = qrow < nq;
  const int64_t tq = bos + i0 + qrow;
  f16x8 qreg[DK / 16];
  bf16x8 oreg[DV / 16];
#pragma unroll
  for (int ks = 0; ks < DK / 16; ++ks)
    qreg[ks] = __builtin_bit_cast(
        f16x8, ld16(qbh + ((int64_t)hq * ntok + tq) * DK + 16 * ks + 8 * (lane >> 5), qok));
#pragma unroll
  for (int ks = 0; ks < DV / 16; ++ks)
    oreg[ks] = __builtin_bit_cast(bf16x8, ld16(dO + (tq * HQ + hq) * DV + 16 * ks + 8 * (lane >> 5), qok));
  const float Lr = qok ? lse[tq * HQ + hq] * LOG2E : 0.f;
  const float Dr = qok ? Dv[tq * HQ + hq] : 0.f;
  const float Gr = (HAS_GS && qok) ? gsum[tq * HQ + hq] : 0.f;
  if (tid < DK) Aq[tid] = anch_h[(cbase + I) * HQ * DK + tid];
  __syncthreads();

  const int pk = tid % (DK / 8), pv = tid % (DV / 8);
  float aqw[DK / 64];
#pragma unroll
  for (int c = 0; c < DK / 64; ++c) aqw[c] = Aq[lane + 64 * c];

  u32x4 fk[QI], fv[OI];
  float fe8[8], frw[DK / 64], fg = 0.f;
  auto fetch = [&](int J) {
    const int j0 = J * XC, nk = min(XC, L - j0);
#pragma unroll
    for (int u = 0; u < QI; ++u) {
      const int r = (tid + 256 * u) / (DK / 8);
      fk[u] = ld16(kt + ((int64_t)hq * ntok + bos + j0 + r) * KX + 8 * pk, r < nk);
    }
#pragma unroll
    for (int u = 0; u < OI; ++u) {
      const int r = (tid + 256 * u) / (DV / 8);
      fv[u] = ld16(v + ((bos + j0 + r) * H + h) * DV + 8 * pv, r < nk);
    }
    const float *rJ = anch_h + (cbase + J) * HQ * DK;
    const f32x4 a0 = *reinterpret_cast<const f32x4 *>(rJ + 8 * pk);
    const f32x4 a1 = *reinterpret_cast<const f32x4 *>(rJ + 8 * pk + 4);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      fe8[e] = Aq[8 * pk + e] - a0[e];
      fe8[4 + e] = Aq[8 * pk + 4 + e] - a1[e];
    }
#pragma unroll
    for (int c = 0; c < DK / 64; ++c) frw[c] = rJ[lane + 64 * c];
    if (tid < XC) fg = (HAS_GS && tid < nk) ? gsum[(bos + j0 + tid) * HQ + hq] : 0.f;
  };
  // registers -> LDS: K'' = k_tilde 2^(A_I - R_J), v, gate sums; false
  // (nothing written) when a chunk factor is out of range
  auto commit = [&]() {
    if (!factors_in_range<DK>(aqw, frw)) return false;
#pragma unroll
    for (int u = 0; u < QI; ++u) {
      const int r = (tid + 256 * u) / (DK / 8);
      *reinterpret_cast<u32x4 *>(Kt + r * KS + 8 * pk) = rescale8(fk[u], fe8);
    }
#pragma unroll
    for (int u = 0; u < OI; ++u) {
      const int r = (tid + 256 * u) / (DV / 8);
      *reinterpret_cast<u32x4 *>(Vs + r * VS + 8 * pv) = fv[u];
    }
    if (tid < XC) Gj[tid] = fg;
    return true;
  };

  f32x16 dQa[TK];
#pragma unroll
  for (int t = 0; t < TK; ++t) dQa[t] = f32x16{};
  float rsum = 0.f;

  const int Jlo = window > 0 ? max(0, i0 - window + 1) / XC : 0;
  const int irel = i0 + qrow;
  fetch(Jlo);
  if (!commit()) {
    if (tid == 0) wide[seg * HQ + hq] = 1;
    return;
  }
  __syncthreads();
  for (int J = Jlo; J <= I; ++J) {
    const int j0 = J * XC, nk = min(XC, L - j0);
    // S^T = K'' Q^T, dP^T = V dO^T for keys 32 kb, rows 32 qb
    f32x16 S = f32x16{}, dP = f32x16{};
#pragma unroll
    for (int ks = 0; ks < DK / 16; ++ks)
      S = Mfma<_Float16>::run(row_operand(Kt + 32 * kb * KS, KS, 16 * ks, lane), qreg[ks], S);
#pragma unroll
    for (int ks = 0; ks < DV / 16; ++ks)
      dP = Mfma<bf16_t>::run(row_operand(Vs + 32 * kb * VS, VS, 16 * ks, lane), oreg[ks], dP);
    const bool full = nq == XC && nk == XC && I > J && !(window > 0 && i0 + XC - 1 - j0 >= window);
    float dsv[16];
#pragma unroll
    for (int a = 0; a < 4; ++a) {
      const int m0 = 32 * kb + 8 * a + 4 * (lane >> 5);  // keys m0 .. m0+3 (values 4a .. 4a+3)
      f32x4 g4 = f32x4{};
      if (HAS_GS) g4 = *reinterpret_cast<const f32x4 *>(Gj + m0);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int r = 4 * a + e;
        float s2 = S[r];
        if (HAS_GS) s2 += Gr - g4[e];
        bool ok = true;
        if (!full) {
          const int jrel = j0 + m0 + e;
          ok = qok && m0 + e < nk && jrel <= irel && !(window > 0 && irel - jrel >= window);
        }
        const float p = ok ? fast_exp2(s2 - Lr) : 0.f;
        const float ds = p * (dP[r] - Dr);
        dsv[r] = ds;
        rsum += ds;
      }
    }
    // dQ^T += K''^T ds^T, contracting over the 32 keys
#pragma unroll
    for (int m = 0; m < 2; ++m) {
      const f16x8 db = pack_h(dsv + 8 * m);
#pragma unroll
      for (int t = 0; t < TK; ++t)
        dQa[t] = Mfma<_Float16>::run(tr_operand(Kt, KS, 32 * kb + 16 * m, 32 * t, lane), db, dQa[t]);
    }
    __syncthreads();
    if (J < I) {
      fetch(J + 1);
      if (!commit()) {
        if (tid == 0) wide[seg * HQ + hq] = 1;
        return;
      }
      __syncthreads();
    }
  }

  float *Xq = reinterpret_cast<float *>(lds);
  float *P2s = reinterpret_cast<float *>(lds + E_P2);
  const float rs = rsum + __shfl_xor(rsum, 32);
  if (lane < 32) rsh[kb][qrow] = rs;
  if (kb == 1) {
#pragma unroll
    for (int t = 0; t < TK; ++t)
#pragma unroll
      for (int r = 0; r < 16; ++r) Xq[qrow * XQS + 32 * t + crow(r, lane)] = dQa[t][r];
  }
  __syncthreads();
  if (kb == 0) {
#pragma unroll
    for (int t = 0; t < TK; ++t)
#pragma unroll
      for (int r = 0; r < 16; ++r) Xq[qrow * XQS + 32 * t + crow(r, lane)] += dQa[t][r];
  }
  chunk_p2<DK>(g, off + ((cbase + I) * HQ + hq) * DK, bos + i0, nq, HQ, hq, P2s, tot);
  for (int x = tid; x < nq * DK; x += 256) {
    const int m = x / DK, c = x % DK;
    dq32[((bos + i0 + m) * HQ + hq) * DK + c] = scale * fast_exp2(P2s[m * DK + c] - Aq[c]) * Xq[m * XQS + c];
  }
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

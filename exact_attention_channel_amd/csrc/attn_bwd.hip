// Backward pass of the prefill (Wall Attention README, introduction:
// analytic gradients for q, k, v, g, and the scalar gate; the FlashAttention
// papers' recomputation: the forward keeps only o and lse, and the backward
// recomputes the probabilities from them).
//
// For dL/do = dO, with p_ij = exp(s_ij - lse_i), dp_ij = dO_i . v_j,
// D_i = dO_i . o_i and ds_ij = p_ij (dp_ij - D_i):
//   dv_j  = sum_i p_ij dO_i,
//   dq_in = scale sum_j ds_ij k_jn e^(P_in - P_jn),
//   dk_jn = scale sum_i ds_ij q_in e^(P_in - P_jn),
//   dP_tn = q_tn dq_tn - k_tn dk(hq)_tn    (P_t enters as query and as key prefix;
//                                           dk(hq): this query head's share of dk),
//   dGs_t = sum_j ds_tj - sum_i ds_it,
//   dg = reverse running sum of dP within each sequence, dg_scalar likewise
//   of dGs, dsink = -sum_i exp(sink - lse_i) D_i.
// The pair products (dq, dk, dv and the row and column sums of ds) run on
// the matrix cores for bf16 inputs (attn_bwd_mfma.hip).  The kernels here
// take float32 inputs and the (sequence, head) pairs the pre-pass flags as
// outside the anchored operands' range: every (i, j) factor e^(P_in - P_jn)
// is formed on its own as 2^(P2_in - P2_jn) (one exp2 per channel and pair,
// the forward's exact path's arithmetic), so they hold for every decay rate; float32
// throughout, plain FMAs.
//
// Kernels: D and the sink terms per row; dq (a workgroup per query chunk,
// walking its key chunks); dk, dv (a workgroup per key chunk, walking the
// query chunks that see it), each head's share kept apart; then, for both
// paths, the sums over a key/value head's query heads and the reverse
// running sums.
#include <math.h>

#include <type_traits>

#include "common.h"
#include "launch.h"

namespace wa {
namespace {

constexpr int XC = CHUNK;

// Running decay sums (log2 units) of one chunk's rows into P2s [XC][DK] in
// LDS, as the exact forward kernel forms them.
template <typename TE, int DK>
__device__ void chunk_p2(const TE *__restrict__ g, const float *__restrict__ off_c, int64_t r0,
                         int nrow, int HQ, int hq, float *P2s, float *tot) {
  constexpr int NSEG = 256 / DK, RPS = XC / NSEG;
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

// D_i = dO_i . o_i and, with a sink, exp(sink - lse_i) D_i: a row of DV
// elements is read by DV * sizeof(TE) / 16 threads, 16 bytes each; grid
// ceil(ntok*HQ / rows per workgroup) x 256 threads.
template <typename TE, int DV>
__global__ __launch_bounds__(256) void k_bwd_rows(const TE *__restrict__ o, const TE *__restrict__ dO,
                                                  const float *__restrict__ lse,
                                                  const float *__restrict__ sink,
                                                  float *__restrict__ Dv, float *__restrict__ psD,
                                                  int64_t nrows, int HQ) {
  constexpr int EPT = 16 / (int)sizeof(TE), TPR = DV / EPT, RPB = 256 / TPR;
  const int64_t r = (int64_t)blockIdx.x * RPB + threadIdx.x / TPR;
  const int u = threadIdx.x % TPR;
  float acc = 0.f;
  if (r < nrows) {
    const u32x4 a = *reinterpret_cast<const u32x4 *>(o + r * DV + EPT * u);
    const u32x4 d = *reinterpret_cast<const u32x4 *>(dO + r * DV + EPT * u);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if (sizeof(TE) == 2)
        acc += bf16_lo(a[i]) * bf16_lo(d[i]) + bf16_hi(a[i]) * bf16_hi(d[i]);
      else
        acc += __uint_as_float(a[i]) * __uint_as_float(d[i]);
    }
  }
#pragma unroll
  for (int w = TPR / 2; w >= 1; w >>= 1) acc += __shfl_xor(acc, w, TPR);
  if (r < nrows && u == 0) {
    Dv[r] = acc;
    if (sink != nullptr) psD[r] = fast_exp2((sink[r % HQ] - lse[r]) * LOG2E) * acc;
  }
}

// dq, and the row sums of ds: workgroup (segment x head, slot) walks the
// 64-row query chunks slot, slot + gridDim.y, ...; 4 threads per row, thread
// `sub` owning channels 4e + sub.
template <typename TE, int DK, int DV, bool HAS_GS>
__global__ __launch_bounds__(256) void k_bwd_dq(
    const TE *__restrict__ q, const TE *__restrict__ k, const TE *__restrict__ v,
    const TE *__restrict__ g, const TE *__restrict__ dO, const float *__restrict__ off,
    const float *__restrict__ gsum, const float *__restrict__ lse, const float *__restrict__ Dv,
    float *__restrict__ dq32, float *__restrict__ rows_ds, const int32_t *__restrict__ cu,
    const int *__restrict__ wide, int64_t T, int HQ, int H, int NCmax, int window, float scale) {
  constexpr int QPT = DK / 4, VPT = DV / 4;
  __shared__ float Ks[XC * DK];
  __shared__ float Pk[XC * DK];
  __shared__ float Vs[XC * DV];
  __shared__ float Gj[XC];
  __shared__ float tot[256];
  const int tid = threadIdx.x;
  const int sh = blockIdx.x, seg = sh / HQ, hq = sh % HQ;
  // with flags given, only the flagged pairs (the matrix-core kernels take the rest)
  if (wide != nullptr && __builtin_amdgcn_readfirstlane(wide[seg * HQ + hq]) == 0) return;
  int64_t bos, eos;
  segment_bounds(seg, T, cu, bos, eos);
  const int L = (int)min(eos - bos, (int64_t)NCmax * XC);
  const int nch = (L + XC - 1) / XC;
  const int h = hq / (HQ / H);
  const int row = tid >> 2, sub = tid & 3;
  const float *off_s = off + ((int64_t)seg * NCmax * HQ + hq) * DK;
  const float sl2 = scale * LOG2E;
  for (int c = blockIdx.y; c < nch; c += gridDim.y) {
    const int i0 = c * XC, nq = min(XC, L - i0);
    chunk_p2<TE, DK>(g, off_s + (int64_t)c * HQ * DK, bos + i0, nq, HQ, hq, Pk, tot);
    const int irel = i0 + row;
    const bool q_ok = row < nq;
    const int64_t qi = bos + irel;
    float qs[QPT], pq[QPT], dq[QPT], dOr[VPT];
#pragma unroll
    for (int e = 0; e < QPT; ++e) {
      qs[e] = q_ok ? Elem<TE>::ld(q + (qi * HQ + hq) * DK + 4 * e + sub) * sl2 : 0.f;
      pq[e] = Pk[row * DK + 4 * e + sub];
      dq[e] = 0.f;
    }
#pragma unroll
    for (int e = 0; e < VPT; ++e) dOr[e] = q_ok ? Elem<TE>::ld(dO + (qi * HQ + hq) * DV + 4 * e + sub) : 0.f;
    const float lse2 = q_ok ? lse[qi * HQ + hq] * LOG2E : 0.f;
    const float Di = q_ok ? Dv[qi * HQ + hq] : 0.f;
    const float g_i = (HAS_GS && q_ok) ? gsum[qi * HQ + hq] : 0.f;
    float rsum = 0.f;
    __syncthreads();
    const int Jlo = window > 0 ? max(0, i0 - window + 1) / XC : 0;
    for (int J = Jlo; J <= c; ++J) {
      const int j0 = J * XC, nk = min(XC, L - j0);
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
      for (int jj = 0; jj < XC; ++jj) {
        float f[QPT];
        float s = 0.f, dp = 0.f;
#pragma unroll
        for (int e = 0; e < QPT; ++e) {
          const int n = 4 * e + sub;
          f[e] = fast_exp2(pq[e] - Pk[jj * DK + n]) * Ks[jj * DK + n];
          s = fmaf(qs[e], f[e], s);
        }
#pragma unroll
        for (int e = 0; e < VPT; ++e) dp = fmaf(dOr[e], Vs[jj * DV + 4 * e + sub], dp);
        s += __shfl_xor(s, 1);
        s += __shfl_xor(s, 2);
        dp += __shfl_xor(dp, 1);
        dp += __shfl_xor(dp, 2);
        if (HAS_GS) s += g_i - Gj[jj];
        const int jrel = j0 + jj;
        const bool ok = q_ok && jrel <= irel && jj < nk && !(window > 0 && irel - jrel >= window);
        const float p = ok ? fast_exp2(s - lse2) : 0.f;
        const float ds = p * (dp - Di);
        rsum += ds;
        // masked pairs stay out: their factor may be inf (a later key of a
        // fast-decaying channel) and 0 * inf is not 0
        if (ok) {
#pragma unroll
          for (int e = 0; e < QPT; ++e) dq[e] = fmaf(ds, f[e], dq[e]);
        }
      }
      __syncthreads();
    }
    if (q_ok) {
#pragma unroll
      for (int e = 0; e < QPT; ++e) dq32[(qi * HQ + hq) * DK + 4 * e + sub] = dq[e] * scale;
      if (sub == 0) rows_ds[qi * HQ + hq] = rsum;
    }
  }
}

// dk, dv (this query head's share) and the column sums of ds: workgroup
// (segment x head, slot) walks the 64-key chunks slot, slot + gridDim.y, ...;
// 4 threads per key, thread `sub` owning channels 4e + sub.
template <typename TE, int DK, int DV, bool HAS_GS>
__global__ __launch_bounds__(256) void k_bwd_dkdv(
    const TE *__restrict__ q, const TE *__restrict__ k, const TE *__restrict__ v,
    const TE *__restrict__ g, const TE *__restrict__ dO, const float *__restrict__ off,
    const float *__restrict__ gsum, const float *__restrict__ lse, const float *__restrict__ Dv,
    float *__restrict__ dk_part, float *__restrict__ dv_part, float *__restrict__ cols_ds,
    const int32_t *__restrict__ cu, const int *__restrict__ wide, int64_t T, int HQ, int H,
    int NCmax, int window, float scale) {
  constexpr int KPT = DK / 4, VPT = DV / 4;
  __shared__ float Qs[XC * DK];
  __shared__ float Pq[XC * DK];
  __shared__ float Os[XC * DV];
  __shared__ float Ls[XC], Ds[XC], Gi[XC];
  __shared__ float tot[256];
  const int tid = threadIdx.x;
  const int sh = blockIdx.x, seg = sh / HQ, hq = sh % HQ;
  // with flags given, only the flagged pairs (the matrix-core kernels take the rest)
  if (wide != nullptr && __builtin_amdgcn_readfirstlane(wide[seg * HQ + hq]) == 0) return;
  int64_t bos, eos;
  segment_bounds(seg, T, cu, bos, eos);
  const int L = (int)min(eos - bos, (int64_t)NCmax * XC);
  const int nch = (L + XC - 1) / XC;
  const int h = hq / (HQ / H);
  const int key = tid >> 2, sub = tid & 3;
  const float *off_s = off + ((int64_t)seg * NCmax * HQ + hq) * DK;
  const float sl2 = scale * LOG2E;
  for (int J = blockIdx.y; J < nch; J += gridDim.y) {
    const int j0 = J * XC, nk = min(XC, L - j0);
    chunk_p2<TE, DK>(g, off_s + (int64_t)J * HQ * DK, bos + j0, nk, HQ, hq, Pq, tot);
    const int jrel = j0 + key;
    const bool k_ok = key < nk;
    const int64_t kj = bos + jrel;
    float kr[KPT], pk[KPT], dk[KPT], vr[VPT], dv[VPT];
#pragma unroll
    for (int e = 0; e < KPT; ++e) {
      kr[e] = k_ok ? Elem<TE>::ld(k + (kj * H + h) * DK + 4 * e + sub) : 0.f;
      pk[e] = Pq[key * DK + 4 * e + sub];
      dk[e] = 0.f;
    }
#pragma unroll
    for (int e = 0; e < VPT; ++e) {
      vr[e] = k_ok ? Elem<TE>::ld(v + (kj * H + h) * DV + 4 * e + sub) : 0.f;
      dv[e] = 0.f;
    }
    const float g_j = (HAS_GS && k_ok) ? gsum[kj * HQ + hq] : 0.f;
    float csum = 0.f;
    __syncthreads();
    // query chunks that see this key chunk: J .. the last one within the window
    const int Ihi = window > 0 ? min(nch - 1, (j0 + XC - 1 + window - 1) / XC) : nch - 1;
    for (int I = J; I <= Ihi; ++I) {
      const int i0 = I * XC, nq = min(XC, L - i0);
      chunk_p2<TE, DK>(g, off_s + (int64_t)I * HQ * DK, bos + i0, nq, HQ, hq, Pq, tot);
      for (int x = tid; x < XC * DK; x += 256) {
        const int r = x / DK, n = x % DK;
        Qs[x] = r < nq ? Elem<TE>::ld(q + ((bos + i0 + r) * HQ + hq) * DK + n) : 0.f;
      }
      for (int x = tid; x < XC * DV; x += 256) {
        const int r = x / DV, n = x % DV;
        Os[x] = r < nq ? Elem<TE>::ld(dO + ((bos + i0 + r) * HQ + hq) * DV + n) : 0.f;
      }
      if (tid < XC) {
        const bool ok = tid < nq;
        const int64_t t = bos + i0 + tid;
        Ls[tid] = ok ? lse[t * HQ + hq] * LOG2E : 0.f;
        Ds[tid] = ok ? Dv[t * HQ + hq] : 0.f;
        Gi[tid] = (HAS_GS && ok) ? gsum[t * HQ + hq] : 0.f;
      }
      __syncthreads();
      for (int ii = 0; ii < XC; ++ii) {
        float f[KPT];
        float s = 0.f, dp = 0.f;
#pragma unroll
        for (int e = 0; e < KPT; ++e) {
          const int n = 4 * e + sub;
          f[e] = fast_exp2(Pq[ii * DK + n] - pk[e]) * Qs[ii * DK + n];
          s = fmaf(kr[e], f[e], s);
        }
#pragma unroll
        for (int e = 0; e < VPT; ++e) dp = fmaf(vr[e], Os[ii * DV + 4 * e + sub], dp);
        s += __shfl_xor(s, 1);
        s += __shfl_xor(s, 2);
        dp += __shfl_xor(dp, 1);
        dp += __shfl_xor(dp, 2);
        s = s * sl2;
        if (HAS_GS) s += Gi[ii] - g_j;
        const int irel = i0 + ii;
        const bool ok = k_ok && ii < nq && jrel <= irel && !(window > 0 && irel - jrel >= window);
        const float p = ok ? fast_exp2(s - Ls[ii]) : 0.f;
        const float ds = p * (dp - Ds[ii]);
        csum += ds;
        if (ok) {  // masked pairs stay out (their factor may be inf)
#pragma unroll
          for (int e = 0; e < KPT; ++e) dk[e] = fmaf(ds, f[e], dk[e]);
        }
#pragma unroll
        for (int e = 0; e < VPT; ++e) dv[e] = fmaf(p, Os[ii * DV + 4 * e + sub], dv[e]);
      }
      __syncthreads();
    }
    if (k_ok) {
#pragma unroll
      for (int e = 0; e < KPT; ++e) dk_part[(kj * HQ + hq) * DK + 4 * e + sub] = dk[e] * scale;
#pragma unroll
      for (int e = 0; e < VPT; ++e) dv_part[(kj * HQ + hq) * DV + 4 * e + sub] = dv[e];
      if (sub == 0) cols_ds[kj * HQ + hq] = csum;
    }
  }
}

// Four consecutive channels of a row as floats (8 bytes of bfloat16 or 16
// of float), and back in the input type (round to nearest even).
template <typename TE> __device__ __forceinline__ f32x4 ld4(const TE *p);
template <> __device__ __forceinline__ f32x4 ld4<bf16_t>(const bf16_t *p) {
  const u32x2 w = *reinterpret_cast<const u32x2 *>(p);
  return f32x4{bf16_lo(w[0]), bf16_hi(w[0]), bf16_lo(w[1]), bf16_hi(w[1])};
}
template <> __device__ __forceinline__ f32x4 ld4<float>(const float *p) {
  return *reinterpret_cast<const f32x4 *>(p);
}
__device__ __forceinline__ f32x4 ld4f(const float *p) { return *reinterpret_cast<const f32x4 *>(p); }
template <typename TE> __device__ __forceinline__ void st4(TE *p, f32x4 x);
template <> __device__ __forceinline__ void st4<bf16_t>(bf16_t *p, f32x4 x) {
  *reinterpret_cast<u32x2 *>(p) = u32x2{pack_bf16x2(x[0], x[1]), pack_bf16x2(x[2], x[3])};
}
template <> __device__ __forceinline__ void st4<float>(float *p, f32x4 x) { *reinterpret_cast<f32x4 *>(p) = x; }

// Row stride of the chunk totals: DK channel totals, the dGs total at DK,
// padding to a multiple of four floats (16-byte loads of any four channels).
template <int DK> constexpr int ctot_stride() { return DK + 4; }

// Thread layout of the two kernels below: a thread owns channels 4 cg ..
// 4 cg + 3 of RPG consecutive rows of the 64-row chunk, grp * RPG .. + RPG-1.
template <int DK> struct ChunkRows {
  static constexpr int NQ = DK / 4, NG = 256 / NQ, RPG = XC / NG;
};

// The same four channels kept raw (loaded early, converted where used).
template <typename TE> struct Raw4;
template <> struct Raw4<bf16_t> {
  typedef u32x2 T;
  static __device__ __forceinline__ T ld(const bf16_t *p) { return *reinterpret_cast<const u32x2 *>(p); }
  static __device__ __forceinline__ f32x4 cvt(T w) { return f32x4{bf16_lo(w[0]), bf16_hi(w[0]), bf16_lo(w[1]), bf16_hi(w[1])}; }
};
template <> struct Raw4<float> {
  typedef f32x4 T;
  static __device__ __forceinline__ T ld(const float *p) { return *reinterpret_cast<const f32x4 *>(p); }
  static __device__ __forceinline__ f32x4 cvt(T w) { return w; }
};

// dP_tn = q_tn dq_tn - k_tn dk(hq)_tn for the thread's rows (zero past the
// sequence), and the rows' dq.  Rows past the sequence load its last row
// (L > r0: the chunk holds at least one row), so that every load is
// unconditional and all of them go out before the first use.
template <typename TE, int DK>
__device__ __forceinline__ void chunk_dp(const TE *q, const TE *k, const float *dq32, const float *dk_part,
                                         int64_t bos, int r0, int L, int HQ, int H, int hq, f32x4 (&x)[ChunkRows<DK>::RPG],
                                         f32x4 (&dqv)[ChunkRows<DK>::RPG]) {
  typedef ChunkRows<DK> CR;
  typedef Raw4<TE> R;
  const int cg = threadIdx.x % CR::NQ, grp = threadIdx.x / CR::NQ, n = 4 * cg;
  const int h = hq / (HQ / H);
  typename R::T qv[CR::RPG], kv[CR::RPG];
  f32x4 dkv[CR::RPG];
#pragma unroll
  for (int i = 0; i < CR::RPG; ++i) {
    const int r = min(r0 + grp * CR::RPG + i, L - 1);
    const int64_t t = bos + r;
    qv[i] = R::ld(q + (t * HQ + hq) * DK + n);
    dqv[i] = ld4f(dq32 + (t * HQ + hq) * DK + n);
    kv[i] = R::ld(k + (t * H + h) * DK + n);
    dkv[i] = ld4f(dk_part + (t * HQ + hq) * DK + n);
  }
#pragma unroll
  for (int i = 0; i < CR::RPG; ++i) {
    const bool ok = r0 + grp * CR::RPG + i < L;
    x[i] = ok ? R::cvt(qv[i]) * dqv[i] - R::cvt(kv[i]) * dkv[i] : f32x4{};
  }
}

// Per (chunk, head, segment): totals of dP (per channel) and dGs over the
// chunk, dP_tn = q_tn dq_tn - k_tn dk(hq)_tn, dGs_t = rows_ds - cols_ds.
// grid (NCmax*HQ, nseg), 256 threads; the row groups' sums meet in LDS.
template <typename TE, int DK>
__global__ __launch_bounds__(256) void k_bwd_chunk_totals(
    const TE *__restrict__ q, const TE *__restrict__ k, const float *__restrict__ dq32,
    const float *__restrict__ dk_part, const float *__restrict__ rows_ds,
    const float *__restrict__ cols_ds, float *__restrict__ ctot, const int32_t *__restrict__ cu,
    int64_t T, int HQ, int H, int NCmax) {
  typedef ChunkRows<DK> CR;
  const int c = blockIdx.x % NCmax, hq = blockIdx.x / NCmax, s = blockIdx.y;
  int64_t bos, eos;
  segment_bounds(s, T, cu, bos, eos);
  const int L = (int)min(eos - bos, (int64_t)NCmax * XC);
  const int r0 = c * XC;
  float *out = ctot + (((int64_t)s * NCmax + c) * HQ + hq) * ctot_stride<DK>();
  const int cg = threadIdx.x % CR::NQ, grp = threadIdx.x / CR::NQ;
  if (r0 >= L) {  // a chunk slot past the sequence: zero totals (never read)
    if (threadIdx.x <= DK) out[threadIdx.x] = 0.f;
    return;
  }
  f32x4 x[CR::RPG], dqv[CR::RPG];
  chunk_dp<TE, DK>(q, k, dq32, dk_part, bos, r0, L, HQ, H, hq, x, dqv);
  f32x4 acc = x[0];
#pragma unroll
  for (int i = 1; i < CR::RPG; ++i) acc += x[i];
  __shared__ f32x4 red[CR::NG][CR::NQ];
  red[grp][cg] = acc;
  // dGs over the chunk's rows: the second wave, one row per lane
  if (threadIdx.x >= 64 && threadIdx.x < 128) {
    const int r = r0 + (int)threadIdx.x - 64;
    float y = r < L ? rows_ds[(bos + r) * HQ + hq] - cols_ds[(bos + r) * HQ + hq] : 0.f;
    y = wave_sum(y);
    if (threadIdx.x == 64) out[DK] = y;
  }
  __syncthreads();
  if (grp == 0) {
#pragma unroll
    for (int q2 = 1; q2 < CR::NG; ++q2) acc += red[q2][cg];
    *reinterpret_cast<f32x4 *>(out + 4 * cg) = acc;
  }
}

// Reverse running sums: dg (and dg_scalar) of chunk c = the totals of the
// later chunks plus the in-chunk reverse inclusive sums; dq in the output
// type.  grid (NCmax*HQ, nseg), 256 threads: each thread scans its own rows,
// the row groups' totals and the later chunks' totals meet in LDS.
template <typename TE, int DK>
__global__ __launch_bounds__(256) void k_bwd_scan(
    const TE *__restrict__ q, const TE *__restrict__ k, const float *__restrict__ dq32,
    const float *__restrict__ dk_part, const float *__restrict__ rows_ds,
    const float *__restrict__ cols_ds, const float *__restrict__ ctot, TE *__restrict__ dq,
    TE *__restrict__ dg, TE *__restrict__ dgs, const int32_t *__restrict__ cu, int64_t T, int HQ,
    int H, int NCmax) {
  typedef ChunkRows<DK> CR;
  constexpr int CS = ctot_stride<DK>();
  const int c = blockIdx.x % NCmax, hq = blockIdx.x / NCmax, s = blockIdx.y;
  int64_t bos, eos;
  segment_bounds(s, T, cu, bos, eos);
  const int L = (int)min(eos - bos, (int64_t)NCmax * XC);
  const int nch = (L + XC - 1) / XC;
  if (c >= nch) return;
  const int r0 = c * XC;
  const int cg = threadIdx.x % CR::NQ, grp = threadIdx.x / CR::NQ, n = 4 * cg;
  const float *tots = ctot + ((int64_t)s * NCmax * HQ + hq) * CS;  // chunk c2's row: + c2 * HQ * CS
  // totals of the later chunks, split over the row groups
  f32x4 later = f32x4{};
  for (int c2 = c + 1 + grp; c2 < nch; c2 += CR::NG) later += ld4f(tots + (int64_t)c2 * HQ * CS + n);
  f32x4 x[CR::RPG], dqv[CR::RPG];
  chunk_dp<TE, DK>(q, k, dq32, dk_part, bos, r0, L, HQ, H, hq, x, dqv);
#pragma unroll
  for (int i = CR::RPG - 2; i >= 0; --i) x[i] += x[i + 1];  // reverse inclusive, within the thread's rows
  __shared__ f32x4 red[CR::NG][CR::NQ], lat[CR::NG][CR::NQ];
  red[grp][cg] = x[0];
  lat[grp][cg] = later;
  // dg_scalar: the first wave, one row per lane
  if (dgs != nullptr && threadIdx.x < 64) {
    const int lane = threadIdx.x;
    const int r = r0 + lane;
    float y = r < L ? rows_ds[(bos + r) * HQ + hq] - cols_ds[(bos + r) * HQ + hq] : 0.f;
    float lt = 0.f;
    for (int c2 = c + 1 + lane; c2 < nch; c2 += 64) lt += tots[(int64_t)c2 * HQ * CS + DK];
    lt = wave_sum(lt);
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {  // reverse inclusive scan over the lanes
      const float v = __shfl_down(y, d);
      if (lane + d < 64) y += v;
    }
    if (r < L) Elem<TE>::st(dgs + (bos + r) * HQ + hq, y + lt);
  }
  __syncthreads();
  f32x4 add = f32x4{};
#pragma unroll
  for (int q2 = 0; q2 < CR::NG; ++q2) {
    add += lat[q2][cg];
    if (q2 > grp) add += red[q2][cg];
  }
#pragma unroll
  for (int i = 0; i < CR::RPG; ++i) {
    const int r = r0 + grp * CR::RPG + i;
    if (r < L) {
      const int64_t t = bos + r;
      st4<TE>(dg + (t * HQ + hq) * DK + n, x[i] + add);
      st4<TE>(dq + (t * HQ + hq) * DK + n, dqv[i]);
    }
  }
}

// dk, dv: sums over each key/value head's query heads.  grid over
// ntok*H*max(DK,DV) elements.
template <typename TE, int DK, int DV>
__global__ __launch_bounds__(256) void k_bwd_kv_sum(const float *__restrict__ dk_part,
                                                    const float *__restrict__ dv_part,
                                                    TE *__restrict__ dk, TE *__restrict__ dv,
                                                    int64_t ntok, int HQ, int H) {
  // four channels per thread: 16-byte loads of each query head's share
  constexpr int DM = DK > DV ? DK : DV, Q = DM / 4;
  const int64_t x = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (x >= ntok * H * Q) return;
  const int n = 4 * (int)(x % Q);
  const int64_t th = x / Q;
  const int h = (int)(th % H);
  const int64_t t = th / H;
  const int G = HQ / H;
  auto sum4 = [&](const float *part, int D, TE *out) {
    f32x4 a = f32x4{};
    for (int u = 0; u < G; ++u) a += *reinterpret_cast<const f32x4 *>(part + (t * HQ + h * G + u) * D + n);
#pragma unroll
    for (int e = 0; e < 4; ++e) Elem<TE>::st(out + (t * H + h) * D + n + e, a[e]);
  };
  if (n < DK) sum4(dk_part, DK, dk);
  if (n < DV) sum4(dv_part, DV, dv);
}

// dsink[hq] = -sum over tokens of exp(sink - lse) D, in two fixed-order
// passes: partial sums over blocks of DS_TOK tokens (grid blocks x HQ), then
// their sum per head (one workgroup per head).
constexpr int DS_TOK = 1024;
__global__ __launch_bounds__(256) void k_bwd_dsink_part(const float *__restrict__ psD,
                                                        float *__restrict__ part, int64_t ntok,
                                                        int HQ) {
  const int blk = blockIdx.x, hq = blockIdx.y;
  const int64_t t0 = (int64_t)blk * DS_TOK;
  const int64_t t1 = ntok - t0 < DS_TOK ? ntok : t0 + DS_TOK;
  float acc = 0.f;
  for (int64_t t = t0 + threadIdx.x; t < t1; t += 256) acc += psD[t * HQ + hq];
  acc = wave_sum(acc);
  __shared__ float w4[4];
  if ((threadIdx.x & 63) == 0) w4[threadIdx.x >> 6] = acc;
  __syncthreads();
  if (threadIdx.x == 0) part[(int64_t)blk * HQ + hq] = w4[0] + w4[1] + w4[2] + w4[3];
}

__global__ __launch_bounds__(256) void k_bwd_dsink(const float *__restrict__ part,
                                                   float *__restrict__ dsink, int nblk, int HQ) {
  const int hq = blockIdx.x;
  float acc = 0.f;
  for (int b = threadIdx.x; b < nblk; b += 256) acc += part[(int64_t)b * HQ + hq];
  acc = wave_sum(acc);
  __shared__ float w4[4];
  if ((threadIdx.x & 63) == 0) w4[threadIdx.x >> 6] = acc;
  __syncthreads();
  if (threadIdx.x == 0) dsink[hq] = -(w4[0] + w4[1] + w4[2] + w4[3]);
}

template <typename TE, int DK, int DV>
hipError_t bwd_t(const BwdProblem &b, const FwdWorkspace &ws, const BwdWorkspace &bw,
                 hipStream_t st) {
  const FwdProblem &p = b.f;
  const int NCmax = (int)((p.maxlen + CHUNK - 1) / CHUNK);
  const int64_t nrows = p.ntok * p.HQ;
  const int W = (int)(p.window > 0 && p.window < p.maxlen ? p.window : 0);
  const TE *q = static_cast<const TE *>(p.q), *k = static_cast<const TE *>(p.k);
  const TE *v = static_cast<const TE *>(p.v), *g = static_cast<const TE *>(p.g);
  const TE *dO = static_cast<const TE *>(b.dO);
  constexpr int RPB = 256 / (DV * (int)sizeof(TE) / 16);  // rows per workgroup of k_bwd_rows
  hipLaunchKernelGGL((k_bwd_rows<TE, DV>), dim3((unsigned)((nrows + RPB - 1) / RPB)), dim3(256), 0, st,
                     static_cast<const TE *>(b.o), dO, b.lse, p.sink, bw.Dv, bw.psD, nrows,
                     (int)p.HQ);
  // half-operand inputs: the matrix-core kernels take the pairs within the
  // anchored operands' range, these float32 kernels the flagged ones
  const bool mfma = std::is_same<TE, bf16_t>::value;
  const int *fl = mfma ? ws.wide : nullptr;
  if (mfma) {
    const hipError_t e = launch_attn_bwd_mfma(b, ws, bw, st);
    if (e != hipSuccess) return e;
  }
  const dim3 grid((unsigned)(p.nseg * p.HQ), (unsigned)(NCmax < 16 ? NCmax : 16));
  auto dq_k = p.g_scalar != nullptr ? k_bwd_dq<TE, DK, DV, true> : k_bwd_dq<TE, DK, DV, false>;
  hipLaunchKernelGGL(dq_k, grid, dim3(256), 0, st, q, k, v, g, dO, ws.csum, ws.gsum, b.lse, bw.Dv,
                     bw.dq32, bw.rows_ds, p.cu, fl, p.T, (int)p.HQ, (int)p.H, NCmax, W, p.scale);
  auto kv_k = p.g_scalar != nullptr ? k_bwd_dkdv<TE, DK, DV, true> : k_bwd_dkdv<TE, DK, DV, false>;
  hipLaunchKernelGGL(kv_k, grid, dim3(256), 0, st, q, k, v, g, dO, ws.csum, ws.gsum, b.lse, bw.Dv,
                     bw.dk_part, bw.dv_part, bw.cols_ds, p.cu, fl, p.T, (int)p.HQ, (int)p.H, NCmax,
                     W, p.scale);
  const dim3 gridc((unsigned)(NCmax * p.HQ), (unsigned)p.nseg);
  hipLaunchKernelGGL((k_bwd_chunk_totals<TE, DK>), gridc, dim3(256), 0, st, q, k, bw.dq32,
                     bw.dk_part, bw.rows_ds, bw.cols_ds, bw.ctot, p.cu, p.T, (int)p.HQ, (int)p.H,
                     NCmax);
  hipLaunchKernelGGL((k_bwd_scan<TE, DK>), gridc, dim3(256), 0, st, q, k, bw.dq32, bw.dk_part,
                     bw.rows_ds, bw.cols_ds, bw.ctot, static_cast<TE *>(b.dq),
                     static_cast<TE *>(b.dg), static_cast<TE *>(b.dgs), p.cu, p.T, (int)p.HQ,
                     (int)p.H, NCmax);
  constexpr int DM = DK > DV ? DK : DV;
  const int64_t nkv = p.ntok * p.H * (DM / 4);
  hipLaunchKernelGGL((k_bwd_kv_sum<TE, DK, DV>), dim3((unsigned)((nkv + 255) / 256)), dim3(256), 0,
                     st, bw.dk_part, bw.dv_part, static_cast<TE *>(b.dk), static_cast<TE *>(b.dv),
                     p.ntok, (int)p.HQ, (int)p.H);
  if (b.dsink != nullptr) {
    const int nblk = (int)((p.ntok + DS_TOK - 1) / DS_TOK);
    hipLaunchKernelGGL(k_bwd_dsink_part, dim3((unsigned)nblk, (unsigned)p.HQ), dim3(256), 0, st,
                       bw.psD, bw.dsp, p.ntok, (int)p.HQ);
    hipLaunchKernelGGL(k_bwd_dsink, dim3((unsigned)p.HQ), dim3(256), 0, st, bw.dsp, b.dsink, nblk,
                       (int)p.HQ);
  }
  return hipGetLastError();
}

template <typename TE>
hipError_t bwd_te(const BwdProblem &b, const FwdWorkspace &ws, const BwdWorkspace &bw,
                  hipStream_t st) {
  const FwdProblem &p = b.f;
  if (p.K == 64) return p.V == 64 ? bwd_t<TE, 64, 64>(b, ws, bw, st) : bwd_t<TE, 64, 128>(b, ws, bw, st);
  return p.V == 64 ? bwd_t<TE, 128, 64>(b, ws, bw, st) : bwd_t<TE, 128, 128>(b, ws, bw, st);
}

}  // namespace

static inline size_t al256(size_t x) { return (x + 255) & ~size_t(255); }

size_t bwd_workspace_layout(const FwdProblem &p, BwdWorkspace *bw, char *base) {
  const int64_t NCmax = (p.maxlen + CHUNK - 1) / CHUNK;
  const int64_t nrows = p.ntok * p.HQ;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    char *ptr = base ? base + off : nullptr;
    off += al256(bytes);
    return reinterpret_cast<float *>(ptr);
  };
  float *Dv = take(sizeof(float) * nrows);
  float *psD = take(sizeof(float) * nrows);
  float *dq32 = take(sizeof(float) * nrows * p.K);
  float *dk_part = take(sizeof(float) * nrows * p.K);
  float *dv_part = take(sizeof(float) * nrows * p.V);
  float *rows_ds = take(sizeof(float) * nrows);
  float *cols_ds = take(sizeof(float) * nrows);
  float *ctot = take(sizeof(float) * p.nseg * NCmax * p.HQ * (p.K + 4));
  float *dsp = take(sizeof(float) * ((p.ntok + DS_TOK - 1) / DS_TOK) * p.HQ);
  float *qbh = take(p.dtype == WA_DT_BF16 ? sizeof(uint16_t) * nrows * p.K : 0);
  if (bw) {
    bw->Dv = Dv; bw->psD = psD; bw->dq32 = dq32; bw->dk_part = dk_part; bw->dv_part = dv_part;
    bw->rows_ds = rows_ds; bw->cols_ds = cols_ds; bw->ctot = ctot; bw->dsp = dsp;
    bw->qbh = p.dtype == WA_DT_BF16 ? qbh : nullptr;
  }
  return off;
}

hipError_t launch_attn_bwd(const BwdProblem &b, const FwdWorkspace &ws, const BwdWorkspace &bw,
                           hipStream_t st) {
  if (b.f.dtype == WA_DT_BF16) return bwd_te<bf16_t>(b, ws, bw, st);
  return bwd_te<float>(b, ws, bw, st);
}

}  // namespace wa

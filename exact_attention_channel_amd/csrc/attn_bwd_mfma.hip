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
// Products run on the matrix cores (half for the rescaled q/k and ds, bf16
// for P, V and dO).  P and ds never leave registers: a score tile holds, in
// lane l, one column and a set of rows of its values, which is the B
// operand of a product contracting over those rows once the contraction
// index is taken in that order.  The matching A operand -- dO^T, the
// rescaled q^T or k^T -- comes from row-major LDS tiles through
// ds_read_b64_tr_b16, which hands lane i of each 16-lane group column i of
// the 4 x 16 block its lanes address.  One workgroup per 64-key chunk walks
// the query chunks that see it (dk, dv, column sums of ds); one per 64-row
// query chunk walks its key chunks (dq, row sums).  Both use waves of 16
// keys (16 rows) on v_mfma_f32_16x16x32, keep the wave's own rows in
// registers, and double-buffer the walked blocks in LDS through LDS-direct
// loads.  The float32 finishing kernels of attn_bwd.hip (reverse running
// sums, sums over query heads) complete the gradients.
#include <math.h>

#include <type_traits>

#include "common.h"
#include "launch.h"

namespace wa {
namespace {

constexpr int XC = CHUNK;  // 64 rows of a query chunk, keys of a key chunk

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

__device__ __forceinline__ s16x4 tr16(const void *p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)(p));
}

// B operand from 8 result values, rounded to half / bfloat16.
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

// 8 consecutive 16-bit elements (one 16-byte load); zeros past `valid`.
__device__ __forceinline__ u32x4 ld16(const void *p, bool valid) {
  return valid ? *reinterpret_cast<const u32x4 *>(p) : u32x4{0u, 0u, 0u, 0u};
}

// ---------------------------------------------------------------------------
// dk, dv (each query head's share) and the column sums of ds, with waves of
// 16 keys.  grid (NCmax*HQ, nseg): x = key chunk (longest first) * HQ + head,
// y = segment.  Wave w owns keys 16 w .. 16 w + 15 of the chunk over all 64
// rows of each query block, on v_mfma_f32_16x16x32 (A lane l: row l%16,
// k 8(l/16)..+7; B lane l: column l%16, same k; result lane l: column l%16,
// rows 4(l/16) + r):
//   S[q, key]  = Q''[q] . k_tilde[key],   Q'' = q_hat 2^(A_I - R_J)
//   dP[q, key] = dO . v
//   dV^T[ch, key] += dO^T P,  dK^T[ch, key] += Q''^T ds
// The last two contract over the block's rows in the order of the result
// tiles' values (two 16-row tiles per 32-row step), their A operands read
// transposed from LDS.  The q_hat and dO blocks and the rows' statistics go
// to LDS through LDS-direct loads, double-buffered: the next block loads
// while the current one is computed.  Each thread then scales the q_hat
// pieces it loaded by their channels' factors (one 8-channel group per
// thread, whose anchors it loads itself), so no extra barrier is needed.
// Half the accumulators of 32-key waves, no reduction over row halves.
template <int D> __device__ __forceinline__ int qswz(int r) {
  // 16-byte piece p of row r of an unpadded [64][D] tile sits at p ^ qswz(r):
  // the 16-byte row reads (16 consecutive rows, one piece) and the transposed
  // reads (8 consecutive rows from a multiple of 8, two pieces) hit distinct
  // banks
  return D == 128 ? ((r & 7) << 1) | ((r >> 3) & 1) : (((r >> 1) & 3) << 1) | ((r >> 3) & 1);
}
template <int D> __device__ __forceinline__ int qpiece(int r, int p) { return r * D + 8 * (p ^ qswz<D>(r)); }

template <typename T> struct Mfma16;
template <> struct Mfma16<_Float16> {
  typedef f16x8 V;
  static __device__ __forceinline__ f32x4 run(V a, V b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
  }
};
template <> struct Mfma16<bf16_t> {
  typedef bf16x8 V;
  static __device__ __forceinline__ f32x4 run(V a, V b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
  }
};
// A operand of a 16x16x32 product that contracts over the rows of a swizzled
// LDS tile M [64][D]: output rows (channels) c0 .. c0+15, contraction rows
// x0 + 4 (lane/16) + {0..3} and x0 + 16 + 4 (lane/16) + {0..3}.
template <typename T, int D>
__device__ __forceinline__ typename Mfma16<T>::V tr16_operand(const T *M, int x0, int c0, int lane) {
  const int row = x0 + 4 * (lane >> 4) + ((lane >> 2) & 3);
  const int col = c0 + 4 * (lane & 3);
  const s16x4 lo = tr16(M + qpiece<D>(row, col >> 3) + (col & 7));
  const s16x4 hi = tr16(M + qpiece<D>(row + 16, col >> 3) + (col & 7));
  return __builtin_bit_cast(typename Mfma16<T>::V, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
}

typedef __attribute__((address_space(3))) void lds_void;
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *p, int64_t bytes) {
  const int n = bytes > 0x7fffffff ? 0x7fffffff : (bytes < 0 ? 0 : (int)bytes);
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(p), 0, n, 0x00020000);
}
// LDS-direct loads: lane l writes LDS bytes dst + 16 l .. + 15 (dst + 4 l .. + 3) from its
// buffer offset (zeros past the resource's extent); counted by vmcnt.
__device__ __forceinline__ void dma16(__amdgpu_buffer_rsrc_t rs, void *dst, int voff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(
      rs, (lds_void *)(__attribute__((address_space(3))) unsigned char *)dst, 16, voff, 0, 0, 0);
}
__device__ __forceinline__ void dma4(__amdgpu_buffer_rsrc_t rs, void *dst, int voff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(
      rs, (lds_void *)(__attribute__((address_space(3))) unsigned char *)dst, 4, voff, 0, 0, 0);
}
__device__ __forceinline__ void vm_wait0() { __builtin_amdgcn_s_waitcnt(0x0F70); }  // vmcnt(0) only

// Running decay sums (log2 units) of channels c0 .. c0 + NCP - 1 of one
// chunk's rows into P2s [XC][NCP].
template <int NCP>
__device__ void part_p2(const bf16_t *__restrict__ g, const float *__restrict__ off_c, int64_t r0,
                        int nrow, int HQ, int hq, int DKg, int c0, float *P2s, float *tot) {
  constexpr int NSEG = 256 / NCP, RPS = XC / NSEG;
  const int n = threadIdx.x % NCP, sg = threadIdx.x / NCP;
  float x[RPS];  // the segment's rows, loaded together
#pragma unroll
  for (int i = 0; i < RPS; ++i) {
    const int r = sg * RPS + i;
    x[i] = r < nrow ? bf16_to_f32(g[((r0 + r) * HQ + hq) * DKg + c0 + n]) : 0.f;
  }
  float acc = 0.f;
#pragma unroll
  for (int i = 0; i < RPS; ++i) {
    acc += x[i];
    P2s[(sg * RPS + i) * NCP + n] = acc;
  }
  tot[sg * NCP + n] = acc;
  __syncthreads();
  float base = off_c[c0 + n];
  for (int q = 0; q < sg; ++q) base += tot[q * NCP + n];
  for (int r = sg * RPS; r < sg * RPS + RPS; ++r) P2s[r * NCP + n] = (base + P2s[r * NCP + n]) * LOG2E;
  __syncthreads();
}

template <int DK, int DV, bool HAS_GS>
__global__ __launch_bounds__(256, 2) void k_bwd_dkdv_w16(
    const _Float16 *__restrict__ kt, const _Float16 *__restrict__ qbh, const bf16_t *__restrict__ v,
    const bf16_t *__restrict__ dO, const bf16_t *__restrict__ g, const float *__restrict__ off,
    const float *__restrict__ anch, const float *__restrict__ gsum, const float *__restrict__ lse,
    const float *__restrict__ Dv, int *__restrict__ wide, float *__restrict__ dk_part,
    float *__restrict__ dv_part, float *__restrict__ cols_ds, const int32_t *__restrict__ cu,
    int64_t T, int64_t ntok, int HQ, int H, int NCmax, int window) {
  constexpr int KX = DK + 16;                       // k_tilde row in the forward workspace
  constexpr int QB = XC * DK * 2, OB = XC * DV * 2;  // bytes of a q_hat / dO block
  constexpr int NQD = QB / 1024, NOD = OB / 1024;    // 1-KiB LDS-direct loads per block
  constexpr int NSK = DK / 32, NSV = DV / 32;        // 32-channel steps of S and dP
  constexpr int NCK = DK / 16, NCV = DV / 16;        // 16-channel blocks of dK^T and dV^T
  constexpr int SA = 3 * XC;                         // statistics: L, D, G of the rows
  constexpr int NCP = QB / (XC * 4) < 64 ? QB / (XC * 4) : 64;  // channels per epilogue pass
  constexpr int RA = 4;                              // products an LDS operand is read ahead
  static_assert(NQD % 4 == 0 && NOD % 4 == 0, "a block is a multiple of 4 KiB");
  __shared__ __attribute__((aligned(16))) unsigned char Qb0[QB], Qb1[QB];
  __shared__ __attribute__((aligned(16))) unsigned char Ob0[OB], Ob1[OB];
  __shared__ __attribute__((aligned(16))) float St0[SA], St1[SA];
  __shared__ __attribute__((aligned(16))) float Rj[DK], Gj[XC];
  __shared__ float tot[256];

  const int hq = blockIdx.x % HQ, J = blockIdx.x / HQ, seg = blockIdx.y;
  if (__builtin_amdgcn_readfirstlane(wide[seg * HQ + hq]) != 0) return;
  int64_t bos, eos;
  segment_bounds(seg, T, cu, bos, eos);
  const int L = (int)min(eos - bos, (int64_t)NCmax * XC);
  const int nch = (L + XC - 1) / XC;
  if (J >= nch) return;
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int c16 = lane & 15, gq = lane >> 4;
  const int h = hq / (HQ / H);
  const int j0 = J * XC, nk = min(XC, L - j0);
  const int64_t cbase = (int64_t)seg * NCmax;
  const int kw = 16 * w + c16;  // this lane's key in the chunk
  const bool kok = kw < nk;

  // the wave's keys and values as B operands (channels 32 s + 8 (lane/16) ..)
  f16x8 kr[NSK];
  bf16x8 vr[NSV];
#pragma unroll
  for (int s = 0; s < NSK; ++s)
    kr[s] = __builtin_bit_cast(f16x8, ld16(kt + ((int64_t)hq * ntok + bos + j0 + kw) * KX + 32 * s + 8 * gq, kok));
#pragma unroll
  for (int s = 0; s < NSV; ++s)
    vr[s] = __builtin_bit_cast(bf16x8, ld16(v + ((bos + j0 + kw) * H + h) * DV + 32 * s + 8 * gq, kok));
  if (tid < DK) Rj[tid] = anch[((cbase + J) * HQ + hq) * DK + tid];
  if (tid < XC) Gj[tid] = (HAS_GS && tid < nk) ? gsum[(bos + j0 + tid) * HQ + hq] : 0.f;
  __syncthreads();  // Rj and Gj are read by every wave from the first block on

  // sources of the query blocks (rows relative to bos; rows past L read zero)
  const __amdgpu_buffer_rsrc_t q_rs =
      make_rsrc(qbh + uniform64(((int64_t)hq * ntok + bos) * DK), uniform64((int64_t)L * DK * 2));
  const __amdgpu_buffer_rsrc_t o_rs =
      make_rsrc(dO + uniform64((bos * HQ + hq) * DV), uniform64(((int64_t)(L - 1) * HQ * DV + DV) * 2));
  const int64_t srow = ((int64_t)(L - 1) * HQ + 1) * 4;
  const __amdgpu_buffer_rsrc_t l_rs = make_rsrc(lse + uniform64(bos * HQ + hq), uniform64(srow));
  const __amdgpu_buffer_rsrc_t d_rs = make_rsrc(Dv + uniform64(bos * HQ + hq), uniform64(srow));
  const __amdgpu_buffer_rsrc_t g_rs = make_rsrc(gsum + uniform64(bos * HQ + hq), uniform64(HAS_GS ? srow : 0));
  // block I into a buffer: load m of a tile by wave m % 4, lane l filling
  // LDS piece 64 m + l (row r, piece pp) from piece pp ^ qswz(r) of row r;
  // the statistics by one wave each (4 bytes a lane)
  auto issue = [&](int I, unsigned char *Qb, unsigned char *Ob, float *St) {
    const int i0 = I * XC;
#pragma unroll
    for (int mm = 0; mm < NQD / 4; ++mm) {
      const int m = w + 4 * mm, gi = 64 * m + lane, r = gi / (DK / 8), pp = gi % (DK / 8);
      dma16(q_rs, Qb + 1024 * m, ((i0 + r) * DK + 8 * (pp ^ qswz<DK>(r))) * 2);
    }
#pragma unroll
    for (int mm = 0; mm < NOD / 4; ++mm) {
      const int m = w + 4 * mm, gi = 64 * m + lane, r = gi / (DV / 8), pp = gi % (DV / 8);
      dma16(o_rs, Ob + 1024 * m, ((i0 + r) * HQ * DV + 8 * (pp ^ qswz<DV>(r))) * 2);
    }
    if (w == 0) dma4(l_rs, St, (i0 + lane) * HQ * 4);
    if (w == 1) dma4(d_rs, St + XC, (i0 + lane) * HQ * 4);
    if (HAS_GS && w == 2) dma4(g_rs, St + 2 * XC, (i0 + lane) * HQ * 4);
  };
  // This thread's q_hat pieces (loads m = w + 4 mm) all hold one 8-channel
  // group: their rows agree mod 16, so the swizzle maps them to one piece
  // index.  Its anchors are loaded with each block, the key chunk's kept.
  const int lpq = (lane % (DK / 8)) ^ qswz<DK>((64 * w + lane) / (DK / 8));
  f32x4 aq0, aq1;
  float ac[DK / 64];
  auto load_anchors = [&](int I) {
    const float *aI = anch + ((cbase + I) * HQ + hq) * DK;
    aq0 = *reinterpret_cast<const f32x4 *>(aI + 8 * lpq);
    aq1 = *reinterpret_cast<const f32x4 *>(aI + 8 * lpq + 4);
#pragma unroll
    for (int c = 0; c < DK / 64; ++c) ac[c] = aI[lane + 64 * c];
  };
  // once the block's loads are complete: whether every chunk factor is in
  // range (the same answer in every wave), and this thread's q_hat pieces
  // times 2^(A_I - R_J)
  auto scale_own = [&](unsigned char *Qb) -> bool {
    float mx = -INFINITY;
#pragma unroll
    for (int c = 0; c < DK / 64; ++c) mx = fmaxf(mx, ac[c] - Rj[lane + 64 * c]);
    if (wave_max(mx) > 4.f) return false;
    const f32x4 r0 = *reinterpret_cast<const f32x4 *>(Rj + 8 * lpq);
    const f32x4 r1 = *reinterpret_cast<const f32x4 *>(Rj + 8 * lpq + 4);
    f16x8 fac;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      fac[e] = (_Float16)__builtin_amdgcn_ldexpf(1.f, (int)(aq0[e] - r0[e]));
      fac[4 + e] = (_Float16)__builtin_amdgcn_ldexpf(1.f, (int)(aq1[e] - r1[e]));
    }
#pragma unroll
    for (int mm = 0; mm < NQD / 4; ++mm) {
      f16x8 *pc = reinterpret_cast<f16x8 *>(Qb + 1024 * (w + 4 * mm) + 16 * lane);
      *pc = *pc * fac;
    }
    return true;
  };

  f32x4 dVa[NCV], dKa[NCK];
#pragma unroll
  for (int t = 0; t < NCV; ++t) dVa[t] = f32x4{};
#pragma unroll
  for (int t = 0; t < NCK; ++t) dKa[t] = f32x4{};
  float csum = 0.f;
  const int Ihi = window > 0 ? min(nch - 1, (j0 + XC - 1 + window - 1) / XC) : nch - 1;
  const int jrel = j0 + kw;

  // one query block from buffer P; false (nothing issued) when a chunk
  // factor is out of range -- every wave reads the same anchors and agrees
  auto block = [&](auto par_c, int I) {
    constexpr int P = decltype(par_c)::value;
    const unsigned char *const Qb = P ? Qb1 : Qb0;
    const unsigned char *const Ob = P ? Ob1 : Ob0;
    const float *const St = P ? St1 : St0;
    if (I < Ihi) {
      issue(I + 1, P ? Qb0 : Qb1, P ? Ob0 : Ob1, P ? St0 : St1);
      load_anchors(I + 1);
    }
    const _Float16 *Qh = reinterpret_cast<const _Float16 *>(Qb);
    const bf16_t *Oh = reinterpret_cast<const bf16_t *>(Ob);
    // S = Q'' k_tilde^T and dP = dO v^T: four 16-row tiles, one sequence of
    // products whose LDS operands are read RA products ahead (sched_barrier
    // keeps each step's read and product together, so the compiler does not
    // pull every read down to the product that uses it)
    f32x4 S[4], dPt[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) S[t] = dPt[t] = f32x4{};
    {
      constexpr int NS1 = 4 * NSK, NS2 = NS1 + 4 * NSV;
      u32x4 op[NS2];
      auto rd = [&](int i) {
        if (i < NS1)
          op[i] = *reinterpret_cast<const u32x4 *>(Qh + qpiece<DK>(16 * (i % 4) + c16, 4 * (i / 4) + gq));
        else
          op[i] = *reinterpret_cast<const u32x4 *>(Oh + qpiece<DV>(16 * (i % 4) + c16, 4 * ((i - NS1) / 4) + gq));
      };
#pragma unroll
      for (int i = 0; i < RA; ++i) rd(i);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int i = 0; i < NS2; ++i) {
        if (i + RA < NS2) rd(i + RA);
        if (i < NS1)
          S[i % 4] = Mfma16<_Float16>::run(__builtin_bit_cast(f16x8, op[i]), kr[i / 4], S[i % 4]);
        else
          dPt[i % 4] = Mfma16<bf16_t>::run(__builtin_bit_cast(bf16x8, op[i]), vr[(i - NS1) / 4], dPt[i % 4]);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    // probabilities and ds: lane's key kw, rows 16 t + 4 (lane/16) + e
    const int i0 = I * XC, nq = min(XC, L - i0);
    const bool full = nq == XC && nk == XC && I > J && !(window > 0 && i0 + XC - 1 - j0 >= window);
    const float gk = Gj[kw];
    float pv[16], dsv[16];
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const int n0 = 16 * t + 4 * gq;
      const f32x4 l4 = *reinterpret_cast<const f32x4 *>(St + n0);
      const f32x4 d4 = *reinterpret_cast<const f32x4 *>(St + XC + n0);
      f32x4 g4 = f32x4{};
      if (HAS_GS) g4 = *reinterpret_cast<const f32x4 *>(St + 2 * XC + n0);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        float s2 = S[t][e];
        if (HAS_GS) s2 += g4[e] - gk;
        bool ok = true;
        if (!full) {
          const int irel = i0 + n0 + e;
          ok = n0 + e < nq && kok && jrel <= irel && !(window > 0 && irel - jrel >= window);
        }
        const float p = ok ? fast_exp2(s2 - l4[e] * LOG2E) : 0.f;
        const float ds = p * (dPt[t][e] - d4[e]);
        pv[4 * t + e] = p;
        dsv[4 * t + e] = ds;
        csum += ds;
      }
    }
    // dV^T += dO^T P, dK^T += Q''^T ds over two 32-row steps, the
    // transposed operands read RA products ahead as above
    {
      const bf16x8 pb[2] = {pack_b(pv), pack_b(pv + 8)};
      const f16x8 db[2] = {pack_h(dsv), pack_h(dsv + 8)};
      constexpr int NT = NCV + NCK, NT2 = 2 * NT;
      u32x4 op[NT2];
      auto rd = [&](int i) {
        const int u = i / NT, k = i % NT;
        if (k < NCV)
          op[i] = __builtin_bit_cast(u32x4, tr16_operand<bf16_t, DV>(Oh, 32 * u, 16 * k, lane));
        else
          op[i] = __builtin_bit_cast(u32x4, tr16_operand<_Float16, DK>(Qh, 32 * u, 16 * (k - NCV), lane));
      };
#pragma unroll
      for (int i = 0; i < RA; ++i) rd(i);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int i = 0; i < NT2; ++i) {
        if (i + RA < NT2) rd(i + RA);
        const int u = i / NT, k = i % NT;
        if (k < NCV)
          dVa[k] = Mfma16<bf16_t>::run(__builtin_bit_cast(bf16x8, op[i]), pb[u], dVa[k]);
        else
          dKa[k - NCV] = Mfma16<_Float16>::run(__builtin_bit_cast(f16x8, op[i]), db[u], dKa[k - NCV]);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    return true;
  };

  // blocks alternate between the two buffers; after each block, its
  // successor's loads are waited for and scaled, then one barrier
  issue(J, Qb0, Ob0, St0);
  load_anchors(J);
  vm_wait0();
  bool in_range = scale_own(Qb0);
  __syncthreads();
  for (int I = J; in_range;) {
    block(std::integral_constant<int, 0>{}, I);
    if (I == Ihi) break;
    ++I;
    vm_wait0();
    in_range = scale_own(Qb1);
    __syncthreads();
    if (!in_range) break;
    block(std::integral_constant<int, 1>{}, I);
    if (I == Ihi) break;
    ++I;
    vm_wait0();
    in_range = scale_own(Qb0);
    __syncthreads();
  }
  if (!in_range) {  // a chunk factor above 2^4: the float32 kernels take the pair
    if (tid == 0) wide[seg * HQ + hq] = 1;
    return;
  }

  // dv: lane's key kw, channels 16 cb + 4 (lane/16) .. +3
  if (kok)
#pragma unroll
    for (int cb = 0; cb < NCV; ++cb)
      *reinterpret_cast<f32x4 *>(dv_part + ((bos + j0 + kw) * HQ + hq) * DV + 16 * cb + 4 * gq) = dVa[cb];
  float cs = csum + __shfl_xor(csum, 16);
  cs += __shfl_xor(cs, 32);
  if (gq == 0 && kok) cols_ds[(bos + j0 + kw) * HQ + hq] = cs;
  // dk = ln2 2^(R_J - P2_j) dK, the chunk's running sums NCP channels at a time
  __syncthreads();  // the LDS blocks are read
  float *P2s = reinterpret_cast<float *>(Qb0);
#pragma unroll
  for (int c0 = 0; c0 < DK; c0 += NCP) {
    part_p2<NCP>(g, off + ((cbase + J) * HQ + hq) * DK, bos + j0, nk, HQ, hq, DK, c0, P2s, tot);
    if (kok)
#pragma unroll
      for (int cb = c0 / 16; cb < (c0 + NCP) / 16; ++cb) {
        f32x4 o;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int ch = 16 * cb + 4 * gq + r;
          o[r] = LN2 * fast_exp2(Rj[ch] - P2s[kw * NCP + ch - c0]) * dKa[cb][r];
        }
        *reinterpret_cast<f32x4 *>(dk_part + ((bos + j0 + kw) * HQ + hq) * DK + 16 * cb + 4 * gq) = o;
      }
    __syncthreads();  // P2s is read before the next pass overwrites it
  }
}

// ---------------------------------------------------------------------------
// dq and the row sums of ds, with waves of 16 query rows.  grid
// (NCmax*HQ, nseg): x = query chunk (longest first) * HQ + head, y = segment.
// Wave w owns rows 16 w .. 16 w + 15 of the chunk against all 64 keys of
// each key chunk, on v_mfma_f32_16x16x32:
//   S^T[key, q]  = K''[key] . q_hat[q],   K'' = k_tilde 2^(A_I - R_J)
//   dP^T[key, q] = v[key] . dO[q]
//   dQ^T[ch, q] += K''^T ds^T
// The wave's q_hat and dO rows stay in registers (B operands); a lane holds
// one query row, whose lse, D and gate sum are scalars.  The key chunks' K''
// and v and the keys' gate sums arrive by LDS-direct loads into two
// buffers; each thread scales the k_tilde pieces it loaded by their
// channels' factors (its anchors R_J loaded beside them).
template <int DK, int DV, bool HAS_GS>
__global__ __launch_bounds__(256, 2) void k_bwd_dq_w16(
    const _Float16 *__restrict__ kt, const _Float16 *__restrict__ qbh, const bf16_t *__restrict__ v,
    const bf16_t *__restrict__ dO, const bf16_t *__restrict__ g, const float *__restrict__ off,
    const float *__restrict__ anch, const float *__restrict__ gsum, const float *__restrict__ lse,
    const float *__restrict__ Dv, int *__restrict__ wide, float *__restrict__ dq32,
    float *__restrict__ rows_ds, const int32_t *__restrict__ cu, int64_t T, int64_t ntok, int HQ,
    int H, int NCmax, int window, float scale) {
  constexpr int KX = DK + 16;                       // k_tilde row in the forward workspace
  constexpr int KB = XC * DK * 2, VB = XC * DV * 2;  // bytes of a key / value chunk
  constexpr int NKD = KB / 1024, NVD = VB / 1024;    // 1-KiB LDS-direct loads per chunk
  constexpr int NSK = DK / 32, NSV = DV / 32;        // 32-channel steps of S^T and dP^T
  constexpr int NCK = DK / 16;                       // 16-channel blocks of dQ^T
  constexpr int NCP = KB / (XC * 4) < 64 ? KB / (XC * 4) : 64;  // channels per epilogue pass
  static_assert(NKD % 4 == 0 && NVD % 4 == 0, "a chunk is a multiple of 4 KiB");
  __shared__ __attribute__((aligned(16))) unsigned char Kb0[KB], Kb1[KB];
  __shared__ __attribute__((aligned(16))) unsigned char Vb0[VB], Vb1[VB];
  __shared__ __attribute__((aligned(16))) float Gb0[XC], Gb1[XC];
  __shared__ __attribute__((aligned(16))) float Aq[DK];
  __shared__ float tot[256];

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
  const int c16 = lane & 15, gq = lane >> 4;
  const int h = hq / (HQ / H);
  const int i0 = I * XC, nq = min(XC, L - i0);
  const int64_t cbase = (int64_t)seg * NCmax;
  const int qw = 16 * w + c16;  // this lane's query row in the chunk
  const bool qok = qw < nq;
  const int64_t tq = bos + i0 + qw;

  // the wave's rows as B operands (channels 32 s + 8 (lane/16) ..), the lane's row statistics
  f16x8 qr[NSK];
  bf16x8 orr[NSV];
#pragma unroll
  for (int s = 0; s < NSK; ++s)
    qr[s] = __builtin_bit_cast(f16x8, ld16(qbh + ((int64_t)hq * ntok + tq) * DK + 32 * s + 8 * gq, qok));
#pragma unroll
  for (int s = 0; s < NSV; ++s)
    orr[s] = __builtin_bit_cast(bf16x8, ld16(dO + (tq * HQ + hq) * DV + 32 * s + 8 * gq, qok));
  const float Lr = qok ? lse[tq * HQ + hq] * LOG2E : 0.f;
  const float Dr = qok ? Dv[tq * HQ + hq] : 0.f;
  const float Gr = (HAS_GS && qok) ? gsum[tq * HQ + hq] : 0.f;
  if (tid < DK) Aq[tid] = anch[((cbase + I) * HQ + hq) * DK + tid];
  __syncthreads();  // Aq is read by every wave

  // sources of the key chunks (rows relative to bos; rows past L read zero)
  const __amdgpu_buffer_rsrc_t k_rs =
      make_rsrc(kt + uniform64(((int64_t)hq * ntok + bos) * KX), uniform64(((int64_t)(L - 1) * KX + DK) * 2));
  const __amdgpu_buffer_rsrc_t v_rs =
      make_rsrc(v + uniform64((bos * H + h) * DV), uniform64(((int64_t)(L - 1) * H * DV + DV) * 2));
  const __amdgpu_buffer_rsrc_t g_rs =
      make_rsrc(gsum + uniform64(bos * HQ + hq), uniform64(HAS_GS ? ((int64_t)(L - 1) * HQ + 1) * 4 : 0));
  // key chunk J into a buffer: load m of a tile by wave m % 4, lane l filling
  // LDS piece 64 m + l (row r, piece pp) from piece pp ^ qswz(r) of row r
  auto issue = [&](int J, unsigned char *Kb, unsigned char *Vb, float *Gb) {
    const int j0 = J * XC;
#pragma unroll
    for (int mm = 0; mm < NKD / 4; ++mm) {
      const int m = w + 4 * mm, gi = 64 * m + lane, r = gi / (DK / 8), pp = gi % (DK / 8);
      dma16(k_rs, Kb + 1024 * m, ((j0 + r) * KX + 8 * (pp ^ qswz<DK>(r))) * 2);
    }
#pragma unroll
    for (int mm = 0; mm < NVD / 4; ++mm) {
      const int m = w + 4 * mm, gi = 64 * m + lane, r = gi / (DV / 8), pp = gi % (DV / 8);
      dma16(v_rs, Vb + 1024 * m, ((j0 + r) * H * DV + 8 * (pp ^ qswz<DV>(r))) * 2);
    }
    if (HAS_GS && w == 0) dma4(g_rs, Gb, (j0 + lane) * HQ * 4);
  };
  // This thread's k_tilde pieces share one 8-channel group (their rows agree
  // mod 16); the chunk's anchors for it and for the range check load with
  // each chunk.
  const int lpk = (lane % (DK / 8)) ^ qswz<DK>((64 * w + lane) / (DK / 8));
  f32x4 ar0, ar1;
  float arc[DK / 64];
  auto load_anchors = [&](int J) {
    const float *aJ = anch + ((cbase + J) * HQ + hq) * DK;
    ar0 = *reinterpret_cast<const f32x4 *>(aJ + 8 * lpk);
    ar1 = *reinterpret_cast<const f32x4 *>(aJ + 8 * lpk + 4);
#pragma unroll
    for (int c = 0; c < DK / 64; ++c) arc[c] = aJ[lane + 64 * c];
  };
  auto scale_own = [&](unsigned char *Kb) -> bool {
    float mx = -INFINITY;
#pragma unroll
    for (int c = 0; c < DK / 64; ++c) mx = fmaxf(mx, Aq[lane + 64 * c] - arc[c]);
    if (wave_max(mx) > 4.f) return false;
    const f32x4 q0 = *reinterpret_cast<const f32x4 *>(Aq + 8 * lpk);
    const f32x4 q1 = *reinterpret_cast<const f32x4 *>(Aq + 8 * lpk + 4);
    f16x8 fac;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      fac[e] = (_Float16)__builtin_amdgcn_ldexpf(1.f, (int)(q0[e] - ar0[e]));
      fac[4 + e] = (_Float16)__builtin_amdgcn_ldexpf(1.f, (int)(q1[e] - ar1[e]));
    }
#pragma unroll
    for (int mm = 0; mm < NKD / 4; ++mm) {
      f16x8 *pc = reinterpret_cast<f16x8 *>(Kb + 1024 * (w + 4 * mm) + 16 * lane);
      *pc = *pc * fac;
    }
    return true;
  };

  f32x4 dQa[NCK];
#pragma unroll
  for (int t = 0; t < NCK; ++t) dQa[t] = f32x4{};
  float rsum = 0.f;
  const int Jlo = window > 0 ? max(0, i0 - window + 1) / XC : 0;
  const int irel = i0 + qw;

  auto block = [&](auto par_c, int J) {
    constexpr int P = decltype(par_c)::value;
    const unsigned char *const Kb = P ? Kb1 : Kb0;
    const unsigned char *const Vb = P ? Vb1 : Vb0;
    const float *const Gb = P ? Gb1 : Gb0;
    if (J < I) {
      issue(J + 1, P ? Kb0 : Kb1, P ? Vb0 : Vb1, P ? Gb0 : Gb1);
      load_anchors(J + 1);
    }
    const _Float16 *Kh = reinterpret_cast<const _Float16 *>(Kb);
    const bf16_t *Vh = reinterpret_cast<const bf16_t *>(Vb);
    // S^T = K'' q_hat^T and dP^T = v dO^T: four 16-key tiles
    f32x4 S[4], dPt[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) S[t] = dPt[t] = f32x4{};
#pragma unroll
    for (int s = 0; s < NSK; ++s)
#pragma unroll
      for (int t = 0; t < 4; ++t)
        S[t] = Mfma16<_Float16>::run(
            *reinterpret_cast<const f16x8 *>(Kh + qpiece<DK>(16 * t + c16, 4 * s + gq)), qr[s], S[t]);
#pragma unroll
    for (int s = 0; s < NSV; ++s)
#pragma unroll
      for (int t = 0; t < 4; ++t)
        dPt[t] = Mfma16<bf16_t>::run(
            *reinterpret_cast<const bf16x8 *>(Vh + qpiece<DV>(16 * t + c16, 4 * s + gq)), orr[s], dPt[t]);
    // ds: lane's row qw, keys 16 t + 4 (lane/16) + e
    const int j0 = J * XC, nk = min(XC, L - j0);
    const bool full = nq == XC && nk == XC && I > J && !(window > 0 && i0 + XC - 1 - j0 >= window);
    float dsv[16];
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const int m0 = 16 * t + 4 * gq;
      f32x4 g4 = f32x4{};
      if (HAS_GS) g4 = *reinterpret_cast<const f32x4 *>(Gb + m0);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        float s2 = S[t][e];
        if (HAS_GS) s2 += Gr - g4[e];
        bool ok = true;
        if (!full) {
          const int jrel = j0 + m0 + e;
          ok = qok && m0 + e < nk && jrel <= irel && !(window > 0 && irel - jrel >= window);
        }
        const float p = ok ? fast_exp2(s2 - Lr) : 0.f;
        const float ds = p * (dPt[t][e] - Dr);
        dsv[4 * t + e] = ds;
        rsum += ds;
      }
    }
    // dQ^T += K''^T ds^T over two 32-key steps
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const f16x8 db = pack_h(dsv + 8 * u);
#pragma unroll
      for (int cb = 0; cb < NCK; ++cb)
        dQa[cb] = Mfma16<_Float16>::run(tr16_operand<_Float16, DK>(Kh, 32 * u, 16 * cb, lane), db, dQa[cb]);
    }
  };

  issue(Jlo, Kb0, Vb0, Gb0);
  load_anchors(Jlo);
  vm_wait0();
  bool in_range = scale_own(Kb0);
  __syncthreads();
  for (int J = Jlo; in_range;) {
    block(std::integral_constant<int, 0>{}, J);
    if (J == I) break;
    ++J;
    vm_wait0();
    in_range = scale_own(Kb1);
    __syncthreads();
    if (!in_range) break;
    block(std::integral_constant<int, 1>{}, J);
    if (J == I) break;
    ++J;
    vm_wait0();
    in_range = scale_own(Kb0);
    __syncthreads();
  }
  if (!in_range) {  // a chunk factor above 2^4: the float32 kernels take the pair
    if (tid == 0) wide[seg * HQ + hq] = 1;
    return;
  }

  float rs = rsum + __shfl_xor(rsum, 16);
  rs += __shfl_xor(rs, 32);
  if (gq == 0 && qok) rows_ds[tq * HQ + hq] = rs;
  // dq = scale 2^(P2_i - A_I) dQ, the chunk's running sums NCP channels at a time
  __syncthreads();  // the LDS chunks are read
  float *P2s = reinterpret_cast<float *>(Kb0);
#pragma unroll
  for (int c0 = 0; c0 < DK; c0 += NCP) {
    part_p2<NCP>(g, off + ((cbase + I) * HQ + hq) * DK, bos + i0, nq, HQ, hq, DK, c0, P2s, tot);
    if (qok)
#pragma unroll
      for (int cb = c0 / 16; cb < (c0 + NCP) / 16; ++cb) {
        f32x4 o;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int ch = 16 * cb + 4 * gq + r;
          o[r] = scale * fast_exp2(P2s[qw * NCP + ch - c0] - Aq[ch]) * dQa[cb][r];
        }
        *reinterpret_cast<f32x4 *>(dq32 + (tq * HQ + hq) * DK + 16 * cb + 4 * gq) = o;
      }
    __syncthreads();  // P2s is read before the next pass overwrites it
  }
}

template <int DK, int DV>
hipError_t bwd_mfma_t(const BwdProblem &b, const FwdWorkspace &ws, const BwdWorkspace &bw,
                      hipStream_t st) {
  const FwdProblem &p = b.f;
  const int NCmax = (int)((p.maxlen + CHUNK - 1) / CHUNK);
  const int W = (int)(p.window > 0 && p.window < p.maxlen ? p.window : 0);
  const dim3 grid((unsigned)(NCmax * p.HQ), (unsigned)p.nseg);
  const bool gs = p.g_scalar != nullptr;
  auto kv = gs ? k_bwd_dkdv_w16<DK, DV, true> : k_bwd_dkdv_w16<DK, DV, false>;
  hipLaunchKernelGGL(kv, grid, dim3(256), 0, st, static_cast<const _Float16 *>(ws.kt),
                     static_cast<const _Float16 *>(bw.qbh), static_cast<const bf16_t *>(p.v),
                     static_cast<const bf16_t *>(b.dO), static_cast<const bf16_t *>(p.g), ws.csum,
                     ws.anch, ws.gsum, b.lse, bw.Dv, ws.wide, bw.dk_part, bw.dv_part, bw.cols_ds,
                     p.cu, p.T, p.ntok, (int)p.HQ, (int)p.H, NCmax, W);
  auto qk = gs ? k_bwd_dq_w16<DK, DV, true> : k_bwd_dq_w16<DK, DV, false>;
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

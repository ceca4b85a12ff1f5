// Prefill attention with the Wall Attention per-channel decay (gfx950).
//
// Wall Attention README, introduction: the score of query i and key j weights
// channel n of q_i . k_j by exp(P[i,n] - P[j,n]), P the running sum of the
// learned decay g; "Usage" adds GQA, the scalar gate g_scalar, sink_bias,
// window_size and cu_seqlens.  The pre-pass (prefix.hip) has already written
//   q_hat_i   = q_i * 2^(P2_i - RQ_I) * scale * log2(e)     (query tile anchor RQ_I)
//   k_tilde_j = k_j * 2^(R_J - P2_j)                        (key chunk anchor R_J)
// so for a query tile I and a 64-key tile J the decayed scores are one dense
// product: S = q_hat . (k_tilde * d_IJ)^T with d_IJ[n] = 2^(RQ_I[n] - R_J[n]),
// K exponentials per tile pair instead of K per (i, j) pair.  Scores are in
// log2 units, so the online softmax (FlashAttention's running max and sum,
// see the FlashAttention papers' tiling with rescaled partial outputs) uses
// exp2 directly.
//
// bf16 inputs: the rescaled q/k operands are IEEE half (3 more mantissa bits
// than bfloat16, which keeps the rounding of large decayed scores within
// tolerance); P and V stay bfloat16.  If a key tile's inter-tile factor
// d_IJ exceeds 2^8 (the decay sum grew between the key tile and the query
// tile) the tile is staged as d_IJ * 2^-sigma with an integer sigma and the
// scores are multiplied back by 2^sigma, so the half operands cannot
// overflow; a channel pushed below the half range that way is smaller than
// the dominant one by more than 2^20 and does not change the score.
//
// Kernel layout: 256 threads = 4 waves x 32 query rows; per tile the workgroup
// stages the decayed key tile (row-major) and the value tile (transposed) in
// LDS.  Each wave computes S^T = K_hat Q_hat^T with v_mfma_f32_32x32x16_f16
// so that a lane holds one query column: the row max and sum are in-lane
// plus one swap between the two half-waves, and the probabilities feed the
// next MFMA (O^T += V^T P^T, bf16) as its B operand without leaving registers.
// Tiles outside the causal / window / sequence range are never visited and
// only boundary tiles are masked element by element (the block-sparse idea
// of FlexAttention's BlockMask, computed from indices instead of stored).
#include <math.h>

#include "common.h"
#include "launch.h"

namespace wa {
namespace {

constexpr int BN = CHUNK;  // keys per tile
constexpr int WROWS = 32;  // query rows per wave

// Bounds-checked 16-byte load through a buffer resource: offsets past the
// resource's extent read as zero, and the per-tile offset is a scalar.
__device__ __forceinline__ u32x4 buf_load16(__amdgpu_buffer_rsrc_t rs, int voff, int soff) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, voff, soff, 0));
}
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *p, int64_t bytes) {
  // integer select: HIP's min() on 64-bit integers goes through f64 VALU code,
  // which would make the descriptor a vector value (and each load a loop)
  const int n = bytes > 0x7fffffff ? 0x7fffffff : (int)bytes;
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(p), 0, n, 0x00020000);
}
// Values of lanes l and l^32 combined: v_permlane32_swap exchanges the two
// half-waves without going through LDS.
__device__ __forceinline__ float half_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float half_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

template <int DK, int DV, bool HAS_GS>
__global__ __launch_bounds__(256, 2) void k_attn_fwd_bf16(
    const _Float16 *__restrict__ qh, const _Float16 *__restrict__ kt, const bf16_t *__restrict__ v,
    const float *__restrict__ anch, const float *__restrict__ gsum,
    const float *__restrict__ sink, bf16_t *__restrict__ o, float *__restrict__ lse,
    const int32_t *__restrict__ cu, int64_t T, int HQ, int H, int nseg, int NCmax, int NQT,
    int window) {
  // Key tile rows hold DK decayed channels plus one extra 16-channel block
  // that folds the softmax shift and the gate into the same MFMA:
  //   extra channels of key j:   [2^-s, 2^-s, -Gs_j hi * 2^-s, -Gs_j lo * 2^-s, 0 ...]
  //   extra channels of query i: [-m_i hi, -m_i lo, 1, 1, 0 ...]
  // so the MFMA returns (score - running max) / 2^s directly (s = sigma of
  // the tile, almost always 0) and the common path needs only the exp2.
  constexpr int KX = DK + 16;      // channels per staged key row
  constexpr int KS = KX + 8;       // LDS row stride (elements) of the key tile
  constexpr int VS = BN + 8;       // LDS row stride (elements) of the transposed value tile
  constexpr int NKS = KX / 16;     // MFMA k-steps of the score product
  __shared__ __attribute__((aligned(16))) uint16_t Ks[2][BN * KS];  // half bits
  __shared__ __attribute__((aligned(16))) bf16_t Vt[2][DV * VS];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int hq = blockIdx.x % HQ;
  const int rest = blockIdx.x / HQ;
  const int seg = rest % nseg;
  const int I = NQT - 1 - rest / nseg;  // longest query tiles first
  int64_t bos64, eos64;
  segment_bounds(seg, T, cu, bos64, eos64);
  const int L = (int)(eos64 - bos64);  // sequence length; positions below are relative to bos
  const int nqt = (L + QTILE - 1) / QTILE;
  if (I >= nqt) return;
  const int h = hq / (HQ / H);
  const int i0 = I * QTILE;
  const int i_last = min(i0 + QTILE, L) - 1;
  const int jlo_blk = window > 0 ? max(0, i0 - window + 1) : 0;
  const int Jlo = jlo_blk / BN, Jhi = i_last / BN;

  const int qw0 = i0 + wave * WROWS;
  const bool wave_live = qw0 < L;
  const int qw_last = min(qw0 + WROWS, L) - 1;
  const int jw_lo = window > 0 ? max(0, qw0 - window + 1) : 0;

  const int col = lane & 31, half = lane >> 5;
  const int qi = qw0 + col;
  const bool q_ok = qi < L;

  // per-sequence, per-head buffer resources (byte offsets; rows past L read 0)
  const int qrow = HQ * DK, vrow = H * DV;
  const __amdgpu_buffer_rsrc_t kt_rs = make_rsrc(kt + (bos64 * HQ + hq) * DK, (int64_t)L * qrow * 2);
  const __amdgpu_buffer_rsrc_t v_rs = make_rsrc(v + (bos64 * H + h) * DV, (int64_t)L * vrow * 2);
  const float *gs_b = HAS_GS ? gsum + bos64 * HQ + hq : nullptr;

  f16x8 qB[NKS];
  {
    const _Float16 *qh_b = qh + (bos64 * HQ + hq) * DK;
    const int r = q_ok ? qi : L - 1;
#pragma unroll
    for (int ks = 0; ks < DK / 16; ++ks)
      qB[ks] = *reinterpret_cast<const f16x8 *>(qh_b + r * qrow + ks * 16 + half * 8);
  }
  const float g_i = (HAS_GS && q_ok) ? gs_b[qi * HQ] : 0.f;
  // running max of (score - Gs_i) in log2 units; 0 until the first visible key
  float m_run = 0.f;
  bool m_unset = true;
  auto set_qx = [&]() {
    const _Float16 mh = (_Float16)(-m_run);
    const _Float16 ml = (_Float16)(-m_run - (float)mh);
    f16x8 x = f16x8{};
    if (half == 0) {
      x[0] = mh;
      x[1] = ml;
      x[2] = (_Float16)1.f;
      x[3] = (_Float16)1.f;
    }
    qB[NKS - 1] = x;
  };
  set_qx();

  // staging roles
  constexpr int KCP = DK / 8;      // 16-byte pieces per key row
  constexpr int KRP = 256 / KCP;   // key rows per pass
  constexpr int KNP = BN / KRP;    // passes
  const int cp = tid % KCP, kr = tid / KCP;
  const int koff = (kr * qrow + cp * 8) * 2;  // byte offset of this thread's first piece
  constexpr int VNB = (DV / 8) * 16;  // 4-key x 8-channel blocks of the value tile
  const int kq = tid % 16, cg = tid / 16;
  const bool v_role = tid < VNB;
  const int voff = (4 * kq * vrow + cg * 8) * 2;
  const int sq = kq & 3;
  const int vpos = 16 * (kq >> 2) + 4 * (sq >> 1) + 8 * (sq & 1);

  const int64_t cbase = (int64_t)seg * NCmax;
  const int cq = 2 * I;  // the query tile's anchor: its first chunk

  // Tile-pair decay factors d_IJ = 2^(RQ_I - R_J): the prefill anchors are
  // integers, so the exponents are exact integers and the factors exact powers
  // of two.  Wave 0 computes them for the tile two steps ahead (lane l: the
  // channel pair 2l, 2l+1) and publishes packed half pairs in LDS together
  // with 2^sigma; sigma > 0 only if some factor exceeds 2^8 (the decay sum
  // rose between key tile and query tile), and then the staged operand is
  // scaled by 2^-sigma and the scores by 2^sigma.
  __shared__ __attribute__((aligned(16))) uint32_t Dsh[2][DK / 2];
  __shared__ float Csh[2];
  constexpr int DPAIRS = DK / 2;
  const int dl = lane % DPAIRS;  // wave 0: channel pair of this lane
  float2 rq2 = make_float2(0.f, 0.f), an2 = make_float2(0.f, 0.f);
  const float *anch_b = anch + (cbase * HQ + hq) * DK + 2 * dl;
  if (wave == 0) rq2 = *reinterpret_cast<const float2 *>(anch_b + (int64_t)cq * HQ * DK);
  auto publish_d = [&](int slot) {  // wave 0 only
    const float e0 = rq2.x - an2.x, e1 = rq2.y - an2.y;
    const float emax = wave_max(fmaxf(e0, e1));
    const int sigma = emax > 8.f ? (int)emax - 8 : 0;
    const int x0 = max((int)e0 - sigma, -30), x1 = max((int)e1 - sigma, -30);
    const uint32_t w = pack_f16x2(__builtin_amdgcn_ldexpf(1.f, x0), __builtin_amdgcn_ldexpf(1.f, x1));
    if (lane < DPAIRS) Dsh[slot][lane] = w;
    if (lane == 0) Csh[slot] = __builtin_amdgcn_ldexpf(1.f, sigma);
  };

  u32x4 kreg[KNP];
  u32x4 vreg[4];
  float gj_reg = 0.f;

  auto load_tile = [&](int J) {
    const int kj0 = J * BN;
#pragma unroll
    for (int p = 0; p < KNP; ++p) kreg[p] = buf_load16(kt_rs, koff + p * KRP * qrow * 2, kj0 * qrow * 2);
    if (v_role) {
#pragma unroll
      for (int r = 0; r < 4; ++r) vreg[r] = buf_load16(v_rs, voff + r * vrow * 2, kj0 * vrow * 2);
    }
    if (HAS_GS && tid < BN) gj_reg = gs_b[min(kj0 + tid, L - 1) * HQ];
    if (wave == 0) an2 = *reinterpret_cast<const float2 *>(anch_b + (int64_t)J * HQ * DK);
  };

  auto store_tile = [&](int buf) {
    const u32x4 dpk = *reinterpret_cast<const u32x4 *>(&Dsh[buf][cp * 4]);
    const float csg = Csh[buf];
#pragma unroll
    for (int p = 0; p < KNP; ++p) {
      u32x4 out;
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        // copy the vector elements to scalars first: bit-casting an element
        // expression directly has been seen to read element 0
        const uint32_t kw = kreg[p][w], dw = dpk[w];
        const f16x2 prod = __builtin_bit_cast(f16x2, kw) * __builtin_bit_cast(f16x2, dw);
        out[w] = __builtin_bit_cast(uint32_t, prod);
      }
      *reinterpret_cast<u32x4 *>(&Ks[buf][(kr + p * KRP) * KS + cp * 8]) = out;
    }
    if (tid < BN) {  // the extra channels of key row tid
      const float inv = 1.f / csg;  // exact: a power of two
      u32x4 x = u32x4{0, 0, 0, 0};
      x[0] = pack_f16x2(inv, inv);
      if (HAS_GS) {
        const float gsc = -gj_reg * inv;
        const _Float16 gh = (_Float16)gsc;
        x[1] = pack_f16x2((float)gh, gsc - (float)gh);
      }
      *reinterpret_cast<u32x4 *>(&Ks[buf][tid * KS + DK]) = x;
      *reinterpret_cast<u32x4 *>(&Ks[buf][tid * KS + DK + 8]) = u32x4{0, 0, 0, 0};
    }
    if (v_role) {
#pragma unroll
      for (int c = 0; c < 8; ++c) {
        const int wi = c >> 1;
        u32x2 out;
        if (c & 1) {
          out.x = (vreg[0][wi] >> 16) | (vreg[1][wi] & 0xffff0000u);
          out.y = (vreg[2][wi] >> 16) | (vreg[3][wi] & 0xffff0000u);
        } else {
          out.x = (vreg[0][wi] & 0xffffu) | (vreg[1][wi] << 16);
          out.y = (vreg[2][wi] & 0xffffu) | (vreg[3][wi] << 16);
        }
        *reinterpret_cast<u32x2 *>(&Vt[buf][(cg * 8 + c) * VS + vpos]) = out;
      }
    }
    return csg;
  };

  // Online softmax.  The running max is raised only when a tile's max exceeds
  // it by more than 2^8 (exp2 of the shifted scores stays below 256, far
  // inside fp32 and bf16 range), so the output accumulators and the query's
  // shift channels change rarely.
  constexpr float TAU = 8.f;
  float l_run = 0.f;
  f32x16 oacc[DV / 32];
#pragma unroll
  for (int mb = 0; mb < DV / 32; ++mb) oacc[mb] = f32x16{};

  // Pipeline: tile J computes from LDS buffer J&1 while tile J+1 is staged
  // into the other buffer and tile J+2 is being loaded into registers.  The
  // schedule is unconditional (tiles past Jhi repeat Jhi; their buffers are
  // never read) so registers need no copies between iterations.
  load_tile(Jlo);
  if (wave == 0) publish_d(Jlo & 1);
  __syncthreads();
  float csig_cur = store_tile(Jlo & 1);
  load_tile(min(Jlo + 1, Jhi));
  if (wave == 0) publish_d((Jlo + 1) & 1);
  const int rel0 = qi - 4 * half;  // query position minus this lane's key sub-offset

  for (int J = Jlo; J <= Jhi; ++J) {
    const int buf = J & 1;
    __syncthreads();  // tile J is in LDS; every wave has finished reading the other buffer
    const float csig_stg = store_tile(buf ^ 1);
    load_tile(min(J + 2, Jhi));
    const int kj0 = J * BN;
    const bool need = wave_live && kj0 <= qw_last && kj0 + BN - 1 >= jw_lo;
    if (need) {
      f32x16 S[2];
#pragma unroll
      for (int sb = 0; sb < 2; ++sb) {
        S[sb] = f32x16{};
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) {
          const f16x8 a =
              *reinterpret_cast<const f16x8 *>(&Ks[buf][(sb * 32 + col) * KS + ks * 16 + half * 8]);
          S[sb] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, qB[ks], S[sb], 0, 0, 0);
        }
      }
      const float cs = csig_cur;  // scores are S * cs
      const bool masked = (kj0 + BN - 1 > qw0) || (window > 0 && qw0 + WROWS - 1 - kj0 >= window);
      if (masked) {
        const int rel = rel0 - kj0;  // allowed key offsets kk (without the 4*half part): kk <= rel
#pragma unroll
        for (int sb = 0; sb < 2; ++sb)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int kk = sb * 32 + 8 * (r >> 2) + (r & 3);
            bool ok = kk <= rel;
            if (window > 0) ok = ok && (rel - kk < window);
            S[sb][r] = ok ? S[sb][r] : -INFINITY;
          }
      }
      float mx = -INFINITY;
#pragma unroll
      for (int sb = 0; sb < 2; ++sb)
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, S[sb][r]);
      mx = half_max(mx) * cs;  // tile max minus the running max
      const bool raise = m_unset ? mx > -INFINITY : mx > TAU;
      const bool any_raise = __ballot(raise) != 0;
      if (any_raise || cs != 1.f) {
        // rare: a lane raises its max, or the tile was staged with 2^-sigma
        __asm__ volatile("s_nop 0");  // keep this a branch
        const float shift = raise ? mx : 0.f;
        if (any_raise) {
          // lanes that keep their max scale by exactly 1; a lane's first
          // visible tile has nothing accumulated yet
          const float alpha = raise ? (m_unset ? 0.f : fast_exp2(-mx)) : 1.f;
          l_run *= alpha;
#pragma unroll
          for (int mb = 0; mb < DV / 32; ++mb) oacc[mb] *= alpha;
          m_run += shift;
          m_unset = m_unset && !raise;
          set_qx();
        }
#pragma unroll
        for (int sb = 0; sb < 2; ++sb)
#pragma unroll
          for (int r = 0; r < 16; ++r) S[sb][r] = fmaf(S[sb][r], cs, -shift);
      }
      float rs = 0.f;
#pragma unroll
      for (int sb = 0; sb < 2; ++sb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float p = fast_exp2(S[sb][r]);
          S[sb][r] = p;
          rs += p;
        }
      l_run += half_sum(rs);
      bf16x8 pB[4];
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const f32x16 &src = S[s >> 1];
        const f32x8 p8 = (s & 1) ? __builtin_shufflevector(src, src, 8, 9, 10, 11, 12, 13, 14, 15)
                                 : __builtin_shufflevector(src, src, 0, 1, 2, 3, 4, 5, 6, 7);
        pB[s] = __builtin_convertvector(p8, bf16x8);
      }
#pragma unroll
      for (int mb = 0; mb < DV / 32; ++mb) {
#pragma unroll
        for (int s = 0; s < 4; ++s) {
          const bf16x8 a =
              *reinterpret_cast<const bf16x8 *>(&Vt[buf][(mb * 32 + col) * VS + s * 16 + half * 8]);
          oacc[mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pB[s], oacc[mb], 0, 0, 0);
        }
      }
    }
    if (wave == 0) publish_d(buf);  // factors of tile min(J+2, Jhi), staged next iteration
    csig_cur = csig_stg;
  }

  if (!q_ok) return;
  // scores above are relative to the row term Gs[i] (g_i); restore it here
  float mf = m_run, Z = l_run;
  if (sink != nullptr) {
    const float s2 = sink[hq] * LOG2E - g_i;
    mf = fmaxf(m_run, s2);
    Z = l_run * fast_exp2(m_run - mf) + fast_exp2(s2 - mf);
  }
  const float inv = fast_exp2(m_run - mf) / Z;
  bf16_t *orow = o + ((bos64 + qi) * HQ + hq) * DV;
#pragma unroll
  for (int mb = 0; mb < DV / 32; ++mb)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      u32x2 w;
      w.x = pack_bf16x2(oacc[mb][4 * j] * inv, oacc[mb][4 * j + 1] * inv);
      w.y = pack_bf16x2(oacc[mb][4 * j + 2] * inv, oacc[mb][4 * j + 3] * inv);
      *reinterpret_cast<u32x2 *>(orow + mb * 32 + 8 * j + 4 * half) = w;
    }
  if (lse != nullptr && half == 0) lse[(bos64 + qi) * HQ + hq] = (mf + g_i + log2f(Z)) * LN2;
}

// fp32 kernel: plain FMA arithmetic, one 64-row chunk of queries per
// workgroup, 4 threads per query row; thread `sub` owns channels n = 4e + sub.
template <int DK, int DV, bool HAS_GS>
__global__ __launch_bounds__(256) void k_attn_fwd_f32(
    const float *__restrict__ qh, const float *__restrict__ kt, const float *__restrict__ v,
    const float *__restrict__ anch, const float *__restrict__ gsum,
    const float *__restrict__ sink, float *__restrict__ o, float *__restrict__ lse,
    const int32_t *__restrict__ cu, int64_t T, int HQ, int H, int nseg, int NCmax, int NCH,
    int64_t window) {
  constexpr int QPT = DK / 4, VPT = DV / 4;
  __shared__ float Ks[BN * DK];
  __shared__ float Vs[BN * DV];
  __shared__ float dL[DK];
  __shared__ float Gj[BN];

  const int tid = threadIdx.x;
  const int hq = blockIdx.x % HQ;
  const int rest = blockIdx.x / HQ;
  const int seg = rest % nseg;
  const int c = NCH - 1 - rest / nseg;
  int64_t bos, eos;
  segment_bounds(seg, T, cu, bos, eos);
  const int64_t L = eos - bos;
  const int nch = (int)((L + CHUNK - 1) / CHUNK);
  if (c >= nch) return;
  const int h = hq / (HQ / H);
  const int64_t i0 = bos + (int64_t)c * CHUNK;
  const int64_t i_last = min(i0 + CHUNK, eos) - 1;
  const int64_t jlo_blk = window > 0 ? max(bos, i0 - window + 1) : bos;
  const int Jlo = (int)((jlo_blk - bos) / BN), Jhi = c;

  const int row = tid >> 2, sub = tid & 3;
  const int64_t qi = i0 + row;
  const bool q_ok = qi < eos;
  float qv[QPT];
#pragma unroll
  for (int e = 0; e < QPT; ++e) qv[e] = q_ok ? qh[(qi * HQ + hq) * DK + 4 * e + sub] : 0.f;
  const float g_i = (HAS_GS && q_ok) ? gsum[qi * HQ + hq] : 0.f;
  const int64_t cbase = (int64_t)seg * NCmax;
  const int cq = c & ~1;  // anchor of the first chunk of the 128-row query tile
  const float RQ = tid < DK ? anch[((cbase + cq) * HQ + hq) * DK + tid] : 0.f;

  float m_run = -INFINITY, l_run = 0.f;
  float oacc[VPT];
#pragma unroll
  for (int e = 0; e < VPT; ++e) oacc[e] = 0.f;

  for (int J = Jlo; J <= Jhi; ++J) {
    const int64_t kj0 = bos + (int64_t)J * BN;
    __syncthreads();
    if (tid < DK) dL[tid] = fast_exp2(RQ - anch[((cbase + J) * HQ + hq) * DK + tid]);
    if (HAS_GS && tid < BN) Gj[tid] = kj0 + tid < eos ? gsum[(kj0 + tid) * HQ + hq] : 0.f;
    __syncthreads();
    for (int x = tid; x < BN * DK; x += 256) {
      const int r = x / DK, n = x % DK;
      Ks[x] = kj0 + r < eos ? kt[((kj0 + r) * HQ + hq) * DK + n] * dL[n] : 0.f;
    }
    for (int x = tid; x < BN * DV; x += 256) {
      const int r = x / DV, n = x % DV;
      Vs[x] = kj0 + r < eos ? v[((kj0 + r) * H + h) * DV + n] : 0.f;
    }
    __syncthreads();
    float s[BN];
    float mx = -INFINITY;
#pragma unroll
    for (int jj = 0; jj < BN; ++jj) {
      float part = 0.f;
#pragma unroll
      for (int e = 0; e < QPT; ++e) part = fmaf(qv[e], Ks[jj * DK + 4 * e + sub], part);
      part += __shfl_xor(part, 1);
      part += __shfl_xor(part, 2);
      const int64_t j = kj0 + jj;
      if (HAS_GS) part += g_i - Gj[jj];
      if (j > qi || j >= eos || (window > 0 && qi - j >= window)) part = -INFINITY;
      s[jj] = part;
      mx = fmaxf(mx, part);
    }
    const float m_new = fmaxf(m_run, mx);
    const float m_use = m_new == -INFINITY ? 0.f : m_new;
    const float alpha = fast_exp2(m_run - m_use);
    float rs = 0.f;
#pragma unroll
    for (int jj = 0; jj < BN; ++jj) {
      s[jj] = fast_exp2(s[jj] - m_use);
      rs += s[jj];
    }
    l_run = l_run * alpha + rs;
    m_run = m_new;
#pragma unroll
    for (int e = 0; e < VPT; ++e) {
      float acc = oacc[e] * alpha;
#pragma unroll
      for (int jj = 0; jj < BN; ++jj) acc = fmaf(s[jj], Vs[jj * DV + 4 * e + sub], acc);
      oacc[e] = acc;
    }
  }
  (void)i_last;
  if (!q_ok) return;
  float mf = m_run, Z = l_run;
  if (sink != nullptr) {
    const float s2 = sink[hq] * LOG2E;
    mf = fmaxf(m_run, s2);
    Z = l_run * fast_exp2(m_run - mf) + fast_exp2(s2 - mf);
  }
  const float inv = fast_exp2(m_run - mf) / Z;
#pragma unroll
  for (int e = 0; e < VPT; ++e) o[(qi * HQ + hq) * DV + 4 * e + sub] = oacc[e] * inv;
  if (lse != nullptr && sub == 0) lse[qi * HQ + hq] = (mf + log2f(Z)) * LN2;
}

template <int DK, int DV>
hipError_t attn_bf16_t(const FwdProblem &p, const FwdWorkspace &ws, hipStream_t st) {
  const int NCmax = (int)((p.maxlen + CHUNK - 1) / CHUNK);
  const int NQT = (int)((p.maxlen + QTILE - 1) / QTILE);
  const dim3 grid((unsigned)(NQT * p.nseg * p.HQ));
  auto args = [&](auto kern) {
    hipLaunchKernelGGL(kern, grid, dim3(256), 0, st, static_cast<const _Float16 *>(ws.qh),
                       static_cast<const _Float16 *>(ws.kt), static_cast<const bf16_t *>(p.v),
                       ws.anch, ws.gsum, p.sink, static_cast<bf16_t *>(p.o), p.lse, p.cu, p.T,
                       (int)p.HQ, (int)p.H, (int)p.nseg, NCmax, NQT,
                       (int)(p.window > 0 && p.window < p.maxlen ? p.window : 0));
  };
  if (p.g_scalar != nullptr)
    args(k_attn_fwd_bf16<DK, DV, true>);
  else
    args(k_attn_fwd_bf16<DK, DV, false>);
  return hipGetLastError();
}

template <int DK, int DV>
hipError_t attn_f32_t(const FwdProblem &p, const FwdWorkspace &ws, hipStream_t st) {
  const int NCmax = (int)((p.maxlen + CHUNK - 1) / CHUNK);
  const dim3 grid((unsigned)(NCmax * p.nseg * p.HQ));
  auto args = [&](auto kern) {
    hipLaunchKernelGGL(kern, grid, dim3(256), 0, st, static_cast<const float *>(ws.qh),
                       static_cast<const float *>(ws.kt), static_cast<const float *>(p.v),
                       ws.anch, ws.gsum, p.sink, static_cast<float *>(p.o), p.lse, p.cu, p.T,
                       (int)p.HQ, (int)p.H, (int)p.nseg, NCmax, NCmax, p.window);
  };
  if (p.g_scalar != nullptr)
    args(k_attn_fwd_f32<DK, DV, true>);
  else
    args(k_attn_fwd_f32<DK, DV, false>);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_attn_fwd(const FwdProblem &p, const FwdWorkspace &ws, hipStream_t st) {
  if (p.dtype == 0) {
    if (p.K == 64) return p.V == 64 ? attn_bf16_t<64, 64>(p, ws, st) : attn_bf16_t<64, 128>(p, ws, st);
    return p.V == 64 ? attn_bf16_t<128, 64>(p, ws, st) : attn_bf16_t<128, 128>(p, ws, st);
  }
  if (p.K == 64) return p.V == 64 ? attn_f32_t<64, 64>(p, ws, st) : attn_f32_t<64, 128>(p, ws, st);
  return p.V == 64 ? attn_f32_t<128, 64>(p, ws, st) : attn_f32_t<128, 128>(p, ws, st);
}

}  // namespace wa

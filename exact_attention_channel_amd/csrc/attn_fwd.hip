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

#include <type_traits>

#include "common.h"
#include "launch.h"

namespace wa {
namespace {

constexpr int BN = CHUNK;          // keys per tile of the fp32 kernel
constexpr int BK = 32;             // keys per tile of the bf16 kernel (half an anchor chunk)

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

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
// LDS transpose read (ds_read_b64_tr_b16).  Within each group of 16 lanes,
// lane i receives element i%4 of the four 8-byte pieces addressed by lanes
// i/4, 4 + i/4, 8 + i/4 and 12 + i/4 of its group.  With lane j of a group
// addressing row r0 + j/4, columns c0 + 4(j%4) .. +3 of a row-major tile,
// lane i receives column c0 + i of rows r0 .. r0+3: a column slice, which is
// what a matrix-core operand wants from a tile stored the other way round.
__device__ __forceinline__ s16x4 lds_read_tr4(const unsigned char *p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (lds_s16x4 *)((__attribute__((address_space(3))) unsigned char *)const_cast<unsigned char *>(p)));
}

// Issue order of the steady-state block of a wave: NS score slots (one
// dependent chain per query block) and NP value slots (NP/2 independent
// chains per 16-key step); a slot issues one MFMA per query block from the
// same LDS operand.  The first SA score slots run alone while the
// exponentials of the previous tile are computed; after that score and value
// slots alternate, so consecutive MFMAs rarely depend on each other.
// Operands are read from LDS a few slots ahead of their use.
template <int NS, int NP, int SA> struct FusedOrder {
  static constexpr int N = NS + NP;
  static constexpr int S_ALONE = NS < SA ? NS : SA;
  int kind[N];  // 0: score MFMA, 1: value MFMA
  int idx[N];   // k-step of the score MFMA / index of the value MFMA
  int slot_s[NS], slot_p[NP];
  constexpr FusedOrder() : kind(), idx(), slot_s(), slot_p() {
    int n = 0, i = 0, j = 0;
    for (; i < S_ALONE; ++i, ++n) { kind[n] = 0; idx[n] = i; slot_s[i] = n; }
    while (i < NS || j < NP) {
      if (j < NP) { kind[n] = 1; idx[n] = j; slot_p[j] = n; ++j; ++n; }
      if (i < NS) { kind[n] = 0; idx[n] = i; slot_s[i] = n; ++i; ++n; }
    }
  }
};

// NQB = 32-row query blocks per wave: 1 -> four waves of 32 rows, two waves
// per SIMD (register budget 256); 2 -> two waves of 64 rows sharing every
// staged operand between two blocks, one wave per SIMD (budget 512).
template <int NQB> struct BfShape {
  static constexpr int WQ = 32 * NQB;       // query rows per wave
  static constexpr int NWV = QTILE / WQ;    // waves per workgroup
  static constexpr int NTH = 64 * NWV;      // threads per workgroup
  static constexpr int OCC = NQB == 1 ? 2 : 1;  // waves per SIMD
};

template <int DK, int DV, bool HAS_GS, int NQB>
__global__ __launch_bounds__(BfShape<NQB>::NTH, BfShape<NQB>::OCC) void k_attn_fwd_bf16(
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
  constexpr int WQ = BfShape<NQB>::WQ, NWV = BfShape<NQB>::NWV, NTH = BfShape<NQB>::NTH;
  constexpr int KX = DK + 16;            // channels per staged key row
  constexpr int KSB = 2 * (KX + 8);      // LDS row stride of the key tile (bytes)
  // LDS row stride of the value tile (bytes): 64 bytes of padding put the
  // four rows of one transpose read, and the two 16-lane groups reading
  // neighbouring columns, on disjoint banks
  constexpr int VSB = 2 * DV + 64;
  constexpr int NKS = KX / 16;           // MFMA k-steps of the score product
  constexpr int NMB = DV / 32;           // 32-channel blocks of the output
  constexpr int KP = DK / 8, KRP = NTH / KP, KNP = BK / KRP;  // key staging: pieces, rows/pass, passes
  constexpr int VP = DV / 8, VRP = NTH / VP, VNP = BK / VRP;  // value staging
  constexpr int KS1 = 2;                 // score k-steps issued before the running-max check
  __shared__ __attribute__((aligned(16))) unsigned char Ksm[2][BK * KSB];  // half
  __shared__ __attribute__((aligned(16))) unsigned char Vsm[2][BK * VSB];  // bfloat16, row-major
  __shared__ __attribute__((aligned(16))) uint16_t Dsh[2][DK];  // 2^e_n as half bits
  __shared__ __attribute__((aligned(16))) float Esh[2][DK];     // e_n
  __shared__ int Fsh[2][NWV];                                   // some e_n > 8 (per wave)

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int col = lane & 31, half = lane >> 5;
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
  const int Jlo = (window > 0 ? max(0, i0 - window + 1) : 0) / BK;
  const int Jhi = i_last / BK;

  // this wave's rows qw0 .. qw0 + 63 and the key tiles they see
  const int qw0 = i0 + wave * WQ;
  const bool wave_live = qw0 < L;
  const int qw_last = min(qw0 + WQ, L) - 1;
  const int Jlo_w = (window > 0 ? max(0, qw0 - window + 1) : 0) / BK;
  const int Jhi_w = wave_live ? qw_last / BK : -1;

  const int qrow = HQ * DK, vrow = H * DV;
  const __amdgpu_buffer_rsrc_t kt_rs = make_rsrc(kt + (bos64 * HQ + hq) * DK, (int64_t)L * qrow * 2);
  const __amdgpu_buffer_rsrc_t v_rs = make_rsrc(v + (bos64 * H + h) * DV, (int64_t)L * vrow * 2);
  const float *gs_b = HAS_GS ? gsum + bos64 * HQ + hq : nullptr;

  // query operands: block qb holds rows qw0 + 32 qb + col
  f16x8 qB[NQB][NKS];
  float g_i[NQB];
  {
    const _Float16 *qh_b = qh + (bos64 * HQ + hq) * DK;
#pragma unroll
    for (int qb = 0; qb < NQB; ++qb) {
      const int r = qw0 + 32 * qb + col;
      const int rr = r < L ? r : L - 1;
      g_i[qb] = 0.f;
#pragma unroll
      for (int ks = 0; ks < DK / 16; ++ks)
        qB[qb][ks] = *reinterpret_cast<const f16x8 *>(qh_b + (int64_t)rr * qrow + ks * 16 + half * 8);
      if (HAS_GS && r < L) g_i[qb] = gs_b[(int64_t)r * HQ];
    }
  }
  // the query's extra channels carry minus the row's reference max (log2
  // units, relative to the row term Gs_i), split into two halves
  auto set_qx = [&](int qb, float m) {
    const _Float16 mh = (_Float16)(-m);
    const _Float16 ml = (_Float16)(-m - (float)mh);
    f16x8 x = f16x8{};
    if (half == 0) {
      x[0] = mh;
      x[1] = ml;
      x[2] = (_Float16)1.f;
      x[3] = (_Float16)1.f;
    }
    qB[qb][NKS - 1] = x;
  };

  // ---- staging roles (all threads) ----
  const int kcp = tid % KP, kr0 = tid / KP;
  const int kgoff = (kr0 * qrow + kcp * 8) * 2;
  const int kloff = kr0 * KSB + kcp * 16;
  const int vcp = tid % VP, vr0 = tid / VP;
  const int vgoff = (vr0 * vrow + vcp * 8) * 2;
  const int vloff = vr0 * VSB + vcp * 16;
  constexpr int XPW = BK / NWV;                  // key rows whose extra channels each wave writes
  const bool x_role = (tid & 63) < XPW;
  const int xr = (tid >> 6) * XPW + (tid & 63);

  // Tile-pair decay factors d_IJ[n] = 2^(RQ_I[n] - R_J[n]): the prefill
  // anchors are integers, so the exponents are exact integers and the factors
  // exact powers of two.  Thread n computes channel n of the tile two steps
  // ahead; a flag per wave records an exponent above 8 (the decay sum rose
  // between key tile and query tile), in which case the staging threads
  // rebalance with an integer sigma = max_n e_n - 8: the staged operand is
  // scaled by 2^-sigma and the scores by 2^sigma.
  const int64_t cbase = (int64_t)seg * NCmax;
  const float *anch_b = anch + (cbase * HQ + hq) * DK;
  constexpr int DPW = DK / NWV;                  // channels whose factor each wave computes
  const bool d_role = lane < DPW;
  const int dn = wave * DPW + lane;              // this thread's channel
  const float rq = d_role ? anch_b[(int64_t)(2 * I) * HQ * DK + dn] : 0.f;  // query tile anchor

  u32x4 kraw[KNP], vraw[VNP];
  float graw = 0.f, araw = 0.f;
  // per-tile scalars through buffer resources: lane offset plus a scalar tile
  // offset, rows past the sequence read zero (such keys are always masked)
  const __amdgpu_buffer_rsrc_t gs_rs = make_rsrc(HAS_GS ? gs_b : gsum, HAS_GS ? (int64_t)L * HQ * 4 : 0);
  const int nch = (L + CHUNK - 1) / CHUNK;
  const __amdgpu_buffer_rsrc_t an_rs = make_rsrc(anch_b, (int64_t)nch * HQ * DK * 4);
  auto load_k = [&](int J) {
    const int soff = J * BK * qrow * 2;
#pragma unroll
    for (int p = 0; p < KNP; ++p) kraw[p] = buf_load16(kt_rs, kgoff + p * KRP * qrow * 2, soff);
    if (HAS_GS && x_role)
      graw = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(gs_rs, xr * HQ * 4, J * BK * HQ * 4, 0));
  };
  auto load_v = [&](int J) {
    const int soff = J * BK * vrow * 2;
#pragma unroll
    for (int p = 0; p < VNP; ++p) vraw[p] = buf_load16(v_rs, vgoff + p * VRP * vrow * 2, soff);
  };
  auto load_a = [&](int J) {  // anchor of the chunk holding key tile J
    if (d_role)
      araw = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(an_rs, dn * 4, (J * BK / CHUNK) * HQ * DK * 4, 0));
  };
  auto produce_d = [&](int t, int J) {  // araw holds the anchor of tile J, the t-th visited
    const int slot = t & 1;
    (void)J;
    const float e = rq - araw;
    if (d_role) {
      const int ei = max((int)e, -30);
      Dsh[slot][dn] = __builtin_bit_cast(uint16_t, (_Float16)__builtin_amdgcn_ldexpf(1.f, ei));
      Esh[slot][dn] = e;
    }
    const bool big = __ballot(d_role && e > 8.f) != 0;
    if (lane == 0) Fsh[slot][wave] = big ? 1 : 0;
  };
  // K_hat = k_tilde * d_IJ of the t-th visited tile into key buffer kbuf;
  // returns 2^sigma of the tile.  Two 32-key tiles of one anchor chunk share
  // their factors: the second reuses them from registers (the factors of a
  // tile are published only when its chunk differs from the previous tile's).
  u32x4 dpk_keep = u32x4{0, 0, 0, 0};
  float csg_keep = 1.f, inv_keep = 1.f;
  int chunk_keep = -1;
  auto stage_k = [&](int t, int kbuf, int chunk) -> float {
    const int slot = t & 1;
    u32x4 dpk = dpk_keep;
    float csg = csg_keep, inv = inv_keep;
    if (chunk != chunk_keep) {
      int big = 0;
#pragma unroll
      for (int w = 0; w < NWV; ++w) big |= Fsh[slot][w];
      csg = 1.f;
      inv = 1.f;
      if (!big) {
        dpk = *reinterpret_cast<const u32x4 *>(&Dsh[slot][kcp * 8]);
      } else {
        float em = -INFINITY;
        for (int n = 0; n < DK; ++n) em = fmaxf(em, Esh[slot][n]);
        const int sigma = (int)em - 8;
        csg = __builtin_amdgcn_ldexpf(1.f, sigma);
        inv = __builtin_amdgcn_ldexpf(1.f, -sigma);
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          const int e0 = max((int)Esh[slot][kcp * 8 + 2 * w] - sigma, -30);
          const int e1 = max((int)Esh[slot][kcp * 8 + 2 * w + 1] - sigma, -30);
          dpk[w] = pack_f16x2(__builtin_amdgcn_ldexpf(1.f, e0), __builtin_amdgcn_ldexpf(1.f, e1));
        }
      }
      dpk_keep = dpk;
      csg_keep = csg;
      inv_keep = inv;
      chunk_keep = chunk;
    }
    unsigned char *kb = Ksm[kbuf];
#pragma unroll
    for (int p = 0; p < KNP; ++p) {
      u32x4 out;
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        // copy the vector elements to scalars first: bit-casting an element
        // expression directly has been seen to read element 0
        const uint32_t kw = kraw[p][w], dw = dpk[w];
        const f16x2 prod = __builtin_bit_cast(f16x2, kw) * __builtin_bit_cast(f16x2, dw);
        out[w] = __builtin_bit_cast(uint32_t, prod);
      }
      *reinterpret_cast<u32x4 *>(kb + kloff + p * KRP * KSB) = out;
    }
    if (x_role) {
      u32x4 x = u32x4{0, 0, 0, 0};
      x[0] = pack_f16x2(inv, inv);
      if (HAS_GS) {
        const float gsc = -graw * inv;
        const _Float16 gh = (_Float16)gsc;
        x[1] = pack_f16x2((float)gh, gsc - (float)gh);
      }
      *reinterpret_cast<u32x4 *>(kb + xr * KSB + DK * 2) = x;
    }
    return csg;
  };
  auto stage_v = [&](int vbuf) {
    unsigned char *vb = Vsm[vbuf];
#pragma unroll
    for (int p = 0; p < VNP; ++p) *reinterpret_cast<u32x4 *>(vb + vloff + p * VRP * VSB) = vraw[p];
  };

  // ---- compute pieces ----
  // score A operand: key row col of the tile, channels 16 ks + 8 half .. +7
  const int sa_off = col * KSB + half * 16;
  auto s_mfma = [&](f32x16 (&S)[NQB], int kbuf, int ks) {
    const f16x8 a = *reinterpret_cast<const f16x8 *>(&Ksm[kbuf][sa_off + ks * 32]);
#pragma unroll
    for (int qb = 0; qb < NQB; ++qb)
      S[qb] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, qB[qb][ks], S[qb], 0, 0, 0);
  };
  // The S^T accumulator holds, in lane (col, half), keys 8 (r/4) + 4 half + r%4
  // (r = 0..15) of query column col.  Its elements r = 8t..8t+7 are directly
  // the B operand (k = 16 keys) of the value product, with the keys in the
  // order k -> 8(k/4 % 2) + 4 half + k%4 within the 16-key step; the value
  // operand is read in the same order with two transpose reads (rows
  // key0 .. key0+3 each).
  const int j16 = lane & 15;
  const int tr_off = (4 * half + (j16 >> 2)) * VSB + 2 * (16 * ((lane >> 4) & 1) + 4 * (j16 & 3));
  f32x16 oacc[NQB][NMB];
  auto pv = [&](int vbuf, const bf16x8 (&pB)[NQB][2]) {
#pragma unroll
    for (int mb = 0; mb < NMB; ++mb)
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        const unsigned char *base = &Vsm[vbuf][tr_off + 16 * s * VSB + 64 * mb];
        const s16x4 a0 = lds_read_tr4(base), a1 = lds_read_tr4(base + 8 * VSB);
        const bf16x8 a = __builtin_bit_cast(bf16x8, __builtin_shufflevector(a0, a1, 0, 1, 2, 3, 4, 5, 6, 7));
#pragma unroll
        for (int qb = 0; qb < NQB; ++qb)
          oacc[qb][mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pB[qb][s], oacc[qb][mb], 0, 0, 0);
      }
  };
  auto mask = [&](f32x16 (&S)[NQB], int kj0) {
#pragma unroll
    for (int qb = 0; qb < NQB; ++qb) {
      const int rel = qw0 + 32 * qb + col - kj0 - 4 * half;  // allowed: kk <= rel
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int kk = 8 * (r >> 2) + (r & 3);
        bool ok = kk <= rel;
        if (window > 0) ok = ok && (rel - kk < window);
        S[qb][r] = ok ? S[qb][r] : -INFINITY;
      }
    }
  };
  auto tile_max = [&](const f32x16 &S) {
    float m = -INFINITY;
#pragma unroll
    for (int r = 0; r < 16; ++r) m = fmaxf(m, S[r]);
    return half_max(m);
  };

  // Softmax with a per-row reference max instead of a running one.  The
  // query tile's own key tiles are visited first, newest first, so a row's
  // reference is the max over its diagonal tile (with decaying channels and a
  // forget gate the newest keys carry the largest scores); every later tile
  // is summed against that fixed reference and the output accumulators are
  // never rescaled.  A tile
  // whose probabilities could exceed 2^64 against the reference (scores far
  // above the diagonal's) sets a flag; the workgroup then recomputes its rows
  // with the exact row max from a max-only sweep, which cannot overflow.
  constexpr float PBIG = 0x1p64f;
  float m_ref[NQB], l_part[NQB];  // l_part: this lane's half of each row's key sum
  bool m_set[NQB];
  bool all_set = false, ovf = false;
  float m_true[NQB];
#pragma unroll
  for (int qb = 0; qb < NQB; ++qb) m_true[qb] = -INFINITY;
  auto tail = [&](f32x16 (&S)[NQB], bf16x8 (&pB)[NQB][2]) {
#pragma unroll
    for (int qb = 0; qb < NQB; ++qb) {
      float rs = 0.f;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float p = fast_exp2(S[qb][r]);
        S[qb][r] = p;
        rs += p;
      }
      l_part[qb] += rs;
      ovf = ovf || !(rs <= PBIG);
      pB[qb][0] = __builtin_convertvector(__builtin_shufflevector(S[qb], S[qb], 0, 1, 2, 3, 4, 5, 6, 7), bf16x8);
      pB[qb][1] = __builtin_convertvector(__builtin_shufflevector(S[qb], S[qb], 8, 9, 10, 11, 12, 13, 14, 15), bf16x8);
    }
  };
  // rows without a reference yet take this tile's max (nothing is
  // accumulated for them, so nothing needs rescaling)
  auto set_rows = [&](f32x16 (&S)[NQB]) {
#pragma unroll
    for (int qb = 0; qb < NQB; ++qb) {
      const float mx = tile_max(S[qb]);
      const bool take = !m_set[qb] && mx > -INFINITY;
      const float shift = take ? mx : 0.f;
      if (take) {
        m_ref[qb] = mx;
        m_set[qb] = true;
      }
#pragma unroll
      for (int r = 0; r < 16; ++r) S[qb][r] -= shift;
      set_qx(qb, m_ref[qb]);
    }
    bool mine = true;
#pragma unroll
    for (int qb = 0; qb < NQB; ++qb) mine = mine && m_set[qb];
    all_set = __ballot(!mine) == 0;
  };

  // Steady-state tile in a fixed issue order (FusedOrder): scores of the next
  // tile, exponentials of this tile, value MFMAs of this tile.
  // sched_barrier(0) keeps each slot's instructions together; the wave runs
  // its MFMA-dense part at raised priority so that the other wave on the SIMD
  // fills the gaps with its own VALU and LDS work.
  auto fused = [&](f32x16 (&Sc)[NQB], f32x16 (&Sn)[NQB], int vbuf, int kbuf) {
    constexpr int NP = 2 * NMB;
    constexpr int SA = NQB == 1 ? 4 : 6;  // score slots before the first value slot
    constexpr FusedOrder<NKS, NP, SA> FO{};
    constexpr int KAHEAD = 4, VAHEAD = 3;
    constexpr int E = 16 * NQB;           // exponentials of the tile
    f16x8 ka[NKS];
    bf16x8 va[NP];
    auto kread = [&](int ks) {
      ka[ks] = *reinterpret_cast<const f16x8 *>(&Ksm[kbuf][sa_off + ks * 32]);
    };
    auto vread = [&](int j) {  // value slot j: block mb = j % NMB, 16-key step st = j / NMB
      const int mb = j % NMB, st = j / NMB;
      const unsigned char *base = &Vsm[vbuf][tr_off + 16 * st * VSB + 64 * mb];
      const s16x4 a0 = lds_read_tr4(base), a1 = lds_read_tr4(base + 8 * VSB);
      va[j] = __builtin_bit_cast(bf16x8, __builtin_shufflevector(a0, a1, 0, 1, 2, 3, 4, 5, 6, 7));
    };
    // exponential e: 16-key step st = e / (8 NQB), block qb = e / 8 % NQB, element 8 st + e % 8
    float pr[NQB][16];
    bf16x8 pb[NQB][2];
    float rs[NQB][2];
#pragma unroll
    for (int qb = 0; qb < NQB; ++qb) rs[qb][0] = rs[qb][1] = 0.f;
#pragma unroll
    for (int i = 0; i < NKS; ++i)
      if (FO.slot_s[i] < KAHEAD) kread(i);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int n = 0; n < FO.N; ++n) {
#pragma unroll
      for (int i = 0; i < NKS; ++i)
        if (FO.slot_s[i] >= KAHEAD && FO.slot_s[i] - KAHEAD == n) kread(i);
#pragma unroll
      for (int j = 0; j < NP; ++j)
        if (FO.slot_p[j] - VAHEAD == n || (FO.slot_p[j] < VAHEAD && n == 0)) vread(j);
      if (n == FO.S_ALONE) __builtin_amdgcn_s_setprio(1);
      if (FO.kind[n] == 0) {
        const int ks = FO.idx[n];
#pragma unroll
        for (int qb = 0; qb < NQB; ++qb)
          Sn[qb] = __builtin_amdgcn_mfma_f32_32x32x16_f16(ka[ks], qB[qb][ks], ks == 0 ? f32x16{} : Sn[qb], 0, 0, 0);
      } else {
        const int j = FO.idx[n], mb = j % NMB, st = j / NMB;
#pragma unroll
        for (int qb = 0; qb < NQB; ++qb)
          oacc[qb][mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va[j], pb[qb][st], oacc[qb][mb], 0, 0, 0);
      }
      if (n < FO.S_ALONE) {
        const int e0 = n * E / FO.S_ALONE, e1 = (n + 1) * E / FO.S_ALONE;
#pragma unroll
        for (int e = 0; e < E; ++e) {
          if (e < e0 || e >= e1) continue;
          const int st = e / (8 * NQB), qb = e / 8 % NQB, r = 8 * st + e % 8;
          pr[qb][r] = fast_exp2(Sc[qb][r]);
          rs[qb][r & 1] += pr[qb][r];
        }
#pragma unroll
        for (int st = 0; st < 2; ++st)
          if (e0 < E / 2 * (st + 1) && e1 >= E / 2 * (st + 1)) {
#pragma unroll
            for (int qb = 0; qb < NQB; ++qb) {
              f32x8 p8;
#pragma unroll
              for (int r = 0; r < 8; ++r) p8[r] = pr[qb][8 * st + r];
              pb[qb][st] = __builtin_convertvector(p8, bf16x8);
            }
          }
        if (e1 == E) {
#pragma unroll
          for (int qb = 0; qb < NQB; ++qb) {
            const float t = rs[qb][0] + rs[qb][1];
            l_part[qb] += t;
            ovf = ovf || !(t <= PBIG);
          }
        }
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    __builtin_amdgcn_s_setprio(0);
  };

  // ---- pipeline ----
  // Visiting order: the query tile's own QTILE/BK key tiles newest first,
  // then the older tiles from the oldest up, so that workgroups running
  // side by side walk the same key tiles together and find them in L2.
  // Iteration t: scores of
  // tile t+1 (key buffer (t+1)&1) are accumulated while the softmax of tile t
  // runs, then tile t's probabilities meet its values (value buffer t&1).
  // Staging in the same iteration writes K_hat(t+2) into key buffer t&1 and
  // V(t+1) into value buffer (t+1)&1 from registers loaded one iteration
  // earlier; one barrier per iteration orders it all.
  if (x_role) {  // the unused half of the extra block stays zero
    *reinterpret_cast<u32x4 *>(&Ksm[0][xr * KSB + DK * 2 + 16]) = u32x4{0, 0, 0, 0};
    *reinterpret_cast<u32x4 *>(&Ksm[1][xr * KSB + DK * 2 + 16]) = u32x4{0, 0, 0, 0};
  }
  __shared__ int wg_ovf;
  if (tid == 0) wg_ovf = 0;
  const int NTL = Jhi - Jlo + 1;  // tiles of this workgroup
  // mode 0: reference max from the diagonal tiles; 1: max-only sweep; 2: exact row max known
  auto sweep = [&](auto mode_c) {
    constexpr int MODE = decltype(mode_c)::value;
    constexpr bool VAL = MODE != 1;  // the pass needs values
    const int ND = NTL < QTILE / BK ? NTL : QTILE / BK;  // diagonal tiles, visited first
    auto tileJ = [&](int t) { return t < ND ? Jhi - t : Jlo + (t - ND); };
    auto chunkOf = [&](int t) { return tileJ(t) * BK / CHUNK; };
    // factors are published for a tile only when its chunk differs from the
    // previous visited tile's (the staging reuses them otherwise)
    auto new_chunk = [&](int t) { return t == 0 || chunkOf(t) != chunkOf(t - 1); };
    chunk_keep = -1;
    auto stage_v_if = [&](int vbuf) {
      if (VAL) stage_v(vbuf);
    };
    auto load_v_if = [&](int t) {
      if (VAL) load_v(tileJ(t));
    };
    load_k(tileJ(0));
    load_v_if(0);
    load_a(tileJ(0));
    produce_d(0, tileJ(0));
    if (1 < NTL) load_a(tileJ(1));
    __syncthreads();
    float cs_cur = stage_k(0, 0, chunkOf(0));
    stage_v_if(0);
    if (1 < NTL) {
      if (new_chunk(1)) produce_d(1, tileJ(1));
      load_k(tileJ(1));
      load_v_if(1);
    }
    if (2 < NTL) load_a(tileJ(2));
    __syncthreads();
    f32x16 Sa[NQB], Sb[NQB];
    {
      const int J = tileJ(0);
      if (J >= Jlo_w && J <= Jhi_w) {
#pragma unroll
        for (int qb = 0; qb < NQB; ++qb) Sa[qb] = f32x16{};
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) s_mfma(Sa, 0, ks);
      }
    }
    float cs_next = 1.f;
    if (1 < NTL) cs_next = stage_k(1, 1, chunkOf(1));
    if (2 < NTL) {
      if (new_chunk(2)) produce_d(2, tileJ(2));
      load_k(tileJ(2));
    }
    if (3 < NTL) load_a(tileJ(3));

    auto body = [&](int t, f32x16 (&Sc)[NQB], f32x16 (&Sn)[NQB]) {
      __syncthreads();
      const int buf = t & 1, nbuf = buf ^ 1;
      const int J = tileJ(t), Jn = tileJ(t + 1);
      const bool need_cur = J >= Jlo_w && J <= Jhi_w;
      const bool need_next = t + 1 < NTL && Jn >= Jlo_w && Jn <= Jhi_w;
      const int kj0 = J * BK;
      const bool masked = kj0 + BK - 1 > qw0 || (window > 0 && qw0 + WQ - 1 - kj0 >= window);
      bf16x8 pB[NQB][2];
      const bool general = masked || cs_cur != 1.f || (MODE == 0 && !all_set);
      if (MODE != 1 && need_cur && need_next && !general) {
        // steady state: one block of score MFMAs, exponentials and value MFMAs
        fused(Sc, Sn, buf, nbuf);
      } else {
        if (need_next) {
#pragma unroll
        for (int qb = 0; qb < NQB; ++qb) Sn[qb] = f32x16{};
#pragma unroll
          for (int ks = 0; ks < NKS - 1; ++ks) s_mfma(Sn, nbuf, ks);
        }
        if (need_cur) {
          __asm__ volatile("s_nop 0");  // keep this a branch
          if (masked) mask(Sc, kj0);
          if (cs_cur != 1.f) {
#pragma unroll
            for (int qb = 0; qb < NQB; ++qb) Sc[qb] *= cs_cur;
          }
          if (MODE == 1) {
#pragma unroll
            for (int qb = 0; qb < NQB; ++qb) m_true[qb] = fmaxf(m_true[qb], tile_max(Sc[qb]));
          } else {
            if (MODE == 0 && !all_set) set_rows(Sc);
            tail(Sc, pB);
            pv(buf, pB);
          }
        }
        if (need_next) s_mfma(Sn, nbuf, NKS - 1);  // after any change of the row reference
      }
      float cs_stage = 1.f;
      if (t + 2 < NTL) cs_stage = stage_k(t + 2, buf, chunkOf(t + 2));
      if (t + 1 < NTL) stage_v_if(nbuf);
      if (t + 3 < NTL) {
        if (new_chunk(t + 3)) produce_d(t + 3, tileJ(t + 3));
        load_k(tileJ(t + 3));
      }
      if (t + 2 < NTL) load_v_if(t + 2);
      if (t + 4 < NTL) load_a(tileJ(t + 4));
      cs_cur = cs_next;
      cs_next = cs_stage;
    };
    for (int t = 0; t < NTL; t += 2) {
      body(t, Sa, Sb);
      if (t + 1 >= NTL) break;
      body(t + 1, Sb, Sa);
    }
  };
  auto reset = [&](bool known) {
#pragma unroll
    for (int qb = 0; qb < NQB; ++qb) {
      m_ref[qb] = known ? (m_true[qb] > -INFINITY ? m_true[qb] : 0.f) : 0.f;
      m_set[qb] = known;
      l_part[qb] = 0.f;
      set_qx(qb, m_ref[qb]);
#pragma unroll
      for (int mb = 0; mb < NMB; ++mb) oacc[qb][mb] = f32x16{};
    }
    all_set = known;
    ovf = false;
  };
  reset(false);
  sweep(std::integral_constant<int, 0>{});
  if (__ballot(ovf) != 0 && lane == 0) wg_ovf = 1;
  __syncthreads();
  if (wg_ovf) {
    // rare: recompute with the exact row max (a sweep for the max, then the
    // sum against it), so no tile can overflow
#pragma unroll
    for (int qb = 0; qb < NQB; ++qb) set_qx(qb, 0.f);
    sweep(std::integral_constant<int, 1>{});
    reset(true);
    sweep(std::integral_constant<int, 2>{});
  }

  // ---- epilogue ----
  // scores above are relative to the row term Gs[i] (g_i); restore it here
#pragma unroll
  for (int qb = 0; qb < NQB; ++qb) {
    const int qi = qw0 + 32 * qb + col;
    const float Zl = half_sum(l_part[qb]);
    if (qi < L) {
      float mf = m_ref[qb], Z = Zl;
      if (sink != nullptr) {
        const float s2 = sink[hq] * LOG2E - g_i[qb];
        mf = fmaxf(m_ref[qb], s2);
        Z = Zl * fast_exp2(m_ref[qb] - mf) + fast_exp2(s2 - mf);
      }
      const float inv = fast_exp2(m_ref[qb] - mf) / Z;
      bf16_t *orow = o + ((bos64 + qi) * HQ + hq) * DV;
#pragma unroll
      for (int mb = 0; mb < NMB; ++mb)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          u32x2 w;
          w.x = pack_bf16x2(oacc[qb][mb][4 * j] * inv, oacc[qb][mb][4 * j + 1] * inv);
          w.y = pack_bf16x2(oacc[qb][mb][4 * j + 2] * inv, oacc[qb][mb][4 * j + 3] * inv);
          *reinterpret_cast<u32x2 *>(orow + mb * 32 + 8 * j + 4 * half) = w;
        }
      if (lse != nullptr && half == 0)
        lse[(bos64 + qi) * HQ + hq] = (mf + g_i[qb] + log2f(Z)) * LN2;
    }
  }
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
  constexpr int NQB = 1;
  auto args = [&](auto kern) {
    hipLaunchKernelGGL(kern, grid, dim3(BfShape<NQB>::NTH), 0, st, static_cast<const _Float16 *>(ws.qh),
                       static_cast<const _Float16 *>(ws.kt), static_cast<const bf16_t *>(p.v),
                       ws.anch, ws.gsum, p.sink, static_cast<bf16_t *>(p.o), p.lse, p.cu, p.T,
                       (int)p.HQ, (int)p.H, (int)p.nseg, NCmax, NQT,
                       (int)(p.window > 0 && p.window < p.maxlen ? p.window : 0));
  };
  if (p.g_scalar != nullptr)
    args(k_attn_fwd_bf16<DK, DV, true, NQB>);
  else
    args(k_attn_fwd_bf16<DK, DV, false, NQB>);
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

// Prefill attention with the Wall Attention per-channel decay (gfx950).
//
// Wall Attention README, introduction: the score of query i and key j weights
// channel n of q_i . k_j by exp(P[i,n] - P[j,n]), P the running sum of the
// learned decay g; "Usage" adds GQA, the scalar gate g_scalar, sink_bias,
// window_size and cu_seqlens.  With the operands
//   q_hat_i   = q_i * 2^(P2_i - RQ_I) * scale * log2(e)     (query tile anchor RQ_I)
//   k_tilde_j = k_j * 2^(R_J - P2_j)                        (key chunk anchor R_J)
// (k_tilde written by the pre-pass, prefix.hip; q_hat formed per query tile
// here from q, g and the pre-pass's chunk offsets, or written by the
// pre-pass for fp32 inputs) the decayed scores of a query tile I and a
// 64-key chunk J are one dense product: S = (q_hat * d_IJ) . k_tilde^T with
// d_IJ[n] = 2^(RQ_I[n] - R_J[n]), K exponentials per tile pair instead of K
// per (i, j) pair.  Scores are in log2 units, so the softmax uses exp2
// directly: the fp32 kernel keeps FlashAttention's running max and sum (the
// FlashAttention papers' tiling with rescaled partial outputs), the bf16
// kernel a fixed per-row reference max (see its sweep below).
//
// bf16 inputs: the rescaled q/k operands are IEEE half (3 more mantissa bits
// than bfloat16, which keeps the rounding of large decayed scores within
// tolerance); P and V stay bfloat16.  If a chunk's factor d_IJ exceeds 2^8
// (the decay sum grew between the key chunk and the query tile) the query
// operand takes d_IJ * 2^-sigma with an integer sigma and the scores are
// multiplied back by 2^sigma, so the half operands cannot overflow; a
// channel pushed below the half range that way is smaller than the dominant
// one by more than 2^20 and does not change the score.
//
// Kernel layout: 256 threads = 4 waves x 32 query rows.  Key and value tiles
// of 32 rows go from global memory straight into LDS (LDS-direct buffer
// loads, no register staging); the decay factors sit on the query side, so
// each wave rebuilds its half-precision query operand once per anchor chunk
// from q_hat kept in LDS.  Each wave computes S^T = K_tilde Q'^T with
// v_mfma_f32_32x32x16_f16 so that a lane holds one query column: the row max
// and sum are in-lane plus one swap between the two half-waves, and the
// probabilities feed the next MFMA (O^T += V^T P^T, bf16) as its B operand
// without leaving registers; the value operand comes from transpose reads.
// Tiles outside the causal / window / sequence range are never visited and
// only boundary tiles are masked element by element (the block-sparse idea
// of FlexAttention's BlockMask, computed from indices instead of stored).
// The workgroups of a (sequence, head) that the pre-pass flagged as outside
// the anchored operands' range compute their rows with the exact path
// (attn_exact.h) in the same LDS.
#include <math.h>

#include <type_traits>

#include "attn_exact.h"
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

// Tile geometry of the bf16 kernel for head sizes DK (scores) and DV (values).
template <int DK, int DV> struct BfTile {
  static constexpr int NWV = QTILE / 32;       // waves, 32 query rows each
  static constexpr int NTH = 64 * NWV;         // threads per workgroup
  static constexpr int KX = DK + 16;           // channels of a key row: decayed + one extra block
  static constexpr int KRB = 2 * KX;           // bytes of a key row (global and LDS)
  static constexpr int KPR = KRB / 16;         // 16-byte pieces per key row
  // bytes of a value row in LDS: 64 bytes of padding after the 2 DV data
  // bytes.  A transpose read serves 32 lanes per pass, four consecutive rows
  // x 64 bytes; with the row stride at 64 mod 256 bytes those four 64-byte
  // pieces fall on disjoint banks (measured: no bank conflicts; a 32-byte
  // pad left 24% of the LDS cycles in conflicts, unpadded rows ran at 60%)
  static constexpr int VRB = 2 * DV + 64;
  static constexpr int VPR = VRB / 16;         // 16-byte pieces per value row (the last four padding)
  static constexpr int QSB = 2 * DK + 16;      // LDS row stride of the query tile (bytes)
  static constexpr int NKI = BK * KRB / 1024;  // LDS-direct loads per key tile
  static constexpr int NVI = BK * VRB / 1024;  // LDS-direct loads per value tile
  static_assert(NKI * 1024 == BK * KRB && NVI * 1024 == BK * VRB, "tiles must be whole KiB");
  static_assert(KPR % 2 == 0, "key row swizzle pairs 16-byte pieces");
};

typedef __attribute__((address_space(3))) void lds_void;
// LDS-direct 16-byte load: lane l of the wave writes LDS bytes dst + 16 l ..
// dst + 16 l + 15 (one contiguous KiB per instruction) from its own buffer
// offset; offsets outside the resource's extent write zeros.  Completion is
// counted by vmcnt, so the issuing wave waits for it before the barrier that
// hands the tile to the other waves.
__device__ __forceinline__ void dma16(__amdgpu_buffer_rsrc_t rs, unsigned char *dst, int voff, int soff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void *)(__attribute__((address_space(3))) unsigned char *)dst,
                                           16, voff, soff, 0, 0);
}
__device__ __forceinline__ void vm_wait0() { __builtin_amdgcn_s_waitcnt(0x0F70); }  // vmcnt(0) only

// Sum of the eight bfloat16 probabilities of a value-product operand, added
// to acc: four v_dot2c_f32_bf16 against (1, 1).  The row sum is thus taken
// over the same rounded probabilities that meet the values.  The empty asm
// ties the result to this point of the instruction stream, so the compiler
// cannot sink the additions past the matrix-core block they are issued in.
__device__ __forceinline__ float bf16x8_sum(const bf16x8 &p, float acc) {
  const bf16x2 one = __builtin_bit_cast(bf16x2, 0x3f803f80u);
  // (pairs taken with constant shuffles: a bit cast of the vector's 32-bit
  // words to bfloat16 pairs compiled to the first word four times)
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(p, p, 0, 1), one, acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(p, p, 2, 3), one, acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(p, p, 4, 5), one, acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(p, p, 6, 7), one, acc, false);
  __asm__ volatile("" : "+v"(acc));
  return acc;
}

template <int DK, int DV, bool HAS_GS>
__global__ __launch_bounds__(64 * QTILE / 32, 2) void k_attn_fwd_bf16(
    const bf16_t *__restrict__ q, const bf16_t *__restrict__ k, const bf16_t *__restrict__ g,
    const float *__restrict__ off, const _Float16 *__restrict__ kt, const bf16_t *__restrict__ v,
    const float *__restrict__ anch, const float *__restrict__ gsum,
    const float *__restrict__ sink, bf16_t *__restrict__ o, float *__restrict__ lse,
    const int32_t *__restrict__ cu, int64_t T, int64_t ntok, int HQ, int H, int nseg, int NCmax,
    int NQT, int window, float qscale, const int *__restrict__ wide, const float *__restrict__ mid) {
  // Score product per 32-key tile and wave: S^T = K_tilde Q'^T over DK + 16
  // channels.  The key rows come from the pre-pass with their extra block
  // [1, 1, -Gs_j hi, -Gs_j lo, 0 ...]; the wave's query operand Q' holds
  // q_hat * d_IJ * 2^-s for the tile's anchor chunk and the extra block
  // [-m_i hi * 2^-s, -m_i lo * 2^-s, 2^-s, 2^-s, 0 ...], so the MFMA returns
  // (score - m_i - Gs_j) / 2^s directly (s = sigma of the chunk, almost
  // always 0) and the common path needs only the exp2.
  typedef BfTile<DK, DV> BT;
  constexpr int NWV = BT::NWV, KRB = BT::KRB, VRB = BT::VRB, QSB = BT::QSB;
  constexpr int NKS = BT::KX / 16;       // MFMA k-steps of the score product (last: extra block)
  constexpr int NMB = DV / 32;           // 32-channel blocks of the output
  constexpr int CPL = DK / 64;           // channels per lane in the factor computation
  // key tiles: rows of KRB bytes, 16-byte piece p of row r stored at piece
  // p ^ ((r >> 3) & 1) (rows r and r + 8 then read disjoint banks);
  // value tiles: rows of VRB bytes (2 DV data bytes, then padding)
  // (separate LDS objects: the compiler tracks the LDS-direct loads per
  // object, so a read of one buffer does not wait for loads into another)
  __shared__ __attribute__((aligned(16))) unsigned char K0[BK * KRB], K1[BK * KRB];
  __shared__ __attribute__((aligned(16))) unsigned char V0[BK * VRB], V1[BK * VRB];
  __shared__ __attribute__((aligned(16))) unsigned char Qs[QTILE * QSB];  // q_hat of the tile, half
  __shared__ __attribute__((aligned(16))) uint16_t Fq[NWV][DK];           // each wave's factors, half bits
  __shared__ int wg_ovf;
  static_assert(QTILE * QSB >= exact::ExactLds<DK, DV>::BYTES, "the exact path fits in Qs");

  const int tid = threadIdx.x, lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave index
  const int col = lane & 31, half = lane >> 5;
  // Workgroups go to the 8 XCDs round robin; with HQ a multiple of 8, XCD x
  // serves query heads x*HQ/8 .. (x+1)*HQ/8 - 1, neighbours that share
  // key/value heads, so the value tiles they read meet in one L2 (packed
  // varlen workload: 2-4% faster; neutral at HQ = 16).
  const int hq = HQ % 8 == 0 ? (int)(blockIdx.x % 8) * (HQ / 8) + (int)((blockIdx.x % HQ) / 8)
                             : (int)(blockIdx.x % HQ);
  const int rest = blockIdx.x / HQ;
  // Without a window, longest query tiles first over all segments (balance:
  // a tile's key count grows with I).  With a window every tile sees about
  // the same number of keys, so segments go one after the other and the
  // workgroups running side by side are neighbouring query tiles of one
  // sequence, sharing most of their key and value tiles in L2.
  const int seg = window > 0 ? rest / NQT : rest % nseg;
  const int I = NQT - 1 - (window > 0 ? rest % NQT : rest / nseg);
  const bool pair_wide = __builtin_amdgcn_readfirstlane(wide[seg * HQ + hq]) != 0;
  int64_t bos64, eos64;
  segment_bounds(seg, T, cu, bos64, eos64);
  // sequence length (positions below are relative to bos), clamped to the
  // NCmax chunks per segment that the workspace holds: with an understated
  // max_seqlen the rows past it are left unwritten, never read out of bounds
  const int L = (int)min(eos64 - bos64, (int64_t)NCmax * CHUNK);
  const int nqt = (L + QTILE - 1) / QTILE;
  if (I >= nqt) return;
  if (pair_wide) {  // the decay leaves the half operands' range: exact rows
    const float *off_s = off + ((int64_t)seg * NCmax * HQ + hq) * DK;
    for (int c = I * (QTILE / CHUNK); c < min((I + 1) * (QTILE / CHUNK), (L + CHUNK - 1) / CHUNK); ++c)
      exact::exact_chunk<bf16_t, DK, DV, HAS_GS>(q, k, v, g, off_s, gsum, sink, o, lse, bos64, L, hq, HQ, H,
                                                 window, qscale, c, Qs);
    return;
  }
  const int h = hq / (HQ / H);
  const int i0 = I * QTILE;
  const int i_last = min(i0 + QTILE, L) - 1;
  // rounded down to the start of an anchor chunk, so that the older tiles
  // pair up with chunks (see the steady pairs below); the tile this may add
  // lies below every row's window, and each wave skips it
  const int Jlo = ((window > 0 ? max(0, i0 - window + 1) : 0) / BK) & ~1;
  const int Jhi = i_last / BK;

  // this wave's rows qw0 .. qw0 + 31 and the key tiles they see
  const int qw0 = i0 + wv * 32;
  const bool wave_live = qw0 < L;
  const int qw_last = min(qw0 + 32, L) - 1;
  const int Jlo_w = (window > 0 ? max(0, qw0 - window + 1) : 0) / BK;
  const int Jhi_w = wave_live ? qw_last / BK : -1;

  const int qrow = HQ * DK, vrow = H * DV;
  const __amdgpu_buffer_rsrc_t kt_rs = make_rsrc(kt + ((int64_t)hq * ntok + bos64) * BT::KX, (int64_t)L * KRB);
  const __amdgpu_buffer_rsrc_t v_rs = make_rsrc(v + (bos64 * H + h) * DV, (int64_t)L * vrow * 2);

  float g_i = 0.f;
  if (HAS_GS && qw0 + col < L) g_i = gsum[(bos64 + qw0 + col) * HQ + hq];

  // Chunk decay factors d_IJ[n] = 2^(RQ_I[n] - R_J[n]): the prefill anchors
  // are integers, so the exponents are exact integers and the factors exact
  // powers of two.  Each wave computes all DK of them for its own use (CPL
  // channels per lane).  If some exponent exceeds 8 (the decay sum rose
  // between key chunk and query tile) the wave rebalances with an integer
  // sigma = max_n e_n - 8: its query operand is scaled by 2^-sigma and the
  // scores by 2^sigma, so the half operands cannot overflow.
  const int64_t cbase = (int64_t)seg * NCmax;
  const float *anch_b = anch + (cbase * HQ + hq) * DK;
  const int nch = (L + CHUNK - 1) / CHUNK;
  // built from explicitly uniform values: left to the compiler, the
  // descriptor can land in vector registers and every anchor load becomes a
  // loop over lanes
  const __amdgpu_buffer_rsrc_t an_rs =
      make_rsrc(anch + uniform64((cbase * HQ + hq) * DK), uniform64((int64_t)nch * HQ * DK * 4));
  float rq[CPL], araw[CPL];
#pragma unroll
  for (int c = 0; c < CPL; ++c) {
    rq[c] = anch_b[(int64_t)(2 * I) * HQ * DK + CPL * lane + c];  // query tile anchor
    araw[c] = 0.f;
  }

  // q_hat of the wave's 32 rows into LDS (read back once per anchor chunk):
  // the running decay sum of each channel is the chunk's offset plus the sum
  // of g over the chunk's rows up to the row (the pre-pass forms the keys'
  // the same way), and q_hat = q * 2^(P2 - RQ_I) * scale * log2(e).  Lane
  // owns channels CPL*lane .. +CPL-1, so every row is one coalesced read.
  // All of a wave's loads (g over the chunk up to its last row, q over its
  // rows) go out together, one memory round trip, right after the first tile
  // loads are issued.
  // exponent bound of this wave's q_hat (max |q_hat| < 2^qexp), folded into
  // the chunk factors' rebalancing so that Q' = q_hat * d_IJ stays below 2^12
  int qexp = 0;
  auto make_qhat = [&]() {
    if (!wave_live) return;
    float qmx = 0.f;
    const int cw = qw0 / CHUNK, r0 = cw * CHUNK;  // the rows' chunk and its first row
    const bool second = qw0 > r0;                 // the wave's rows are the chunk's second half
    // acc: the exponent of q_hat's factor in log2 units, with log2(qscale)
    // folded in, so that each row costs one fma, one exp2 and one multiply
    // per channel: acc = P2 - RQ_I + log2(qscale), P2 = (offset + g sum) log2(e)
    // A wave of the chunk's second 32 rows starts from the pre-pass's
    // running sum at row 31 (log2 units), the others from the chunk offset.
    const float lq = __builtin_amdgcn_logf(qscale);
    const float a_scale = second ? 1.f : LOG2E;
    // buffer loads: the row offset is a scalar, and rows past the sequence
    // read as zero without a branch per row
    const int64_t ext = ((int64_t)(L - 1) * qrow + DK) * 2;
    const __amdgpu_buffer_rsrc_t g_rs = make_rsrc(g + uniform64((bos64 * HQ + hq) * DK), uniform64(ext));
    const __amdgpu_buffer_rsrc_t q_rs = make_rsrc(q + uniform64((bos64 * HQ + hq) * DK), uniform64(ext));
    if constexpr (DK == 64) {
      // 64 channels: a lane takes two channels (4-byte loads), the lower
      // half-wave rows 0..15 of the wave and the upper half rows 16..31;
      // the upper half starts from the lower half's sum over its rows
      const int cl = lane & 31, hr = lane >> 5;
      const float *a0 = (second ? mid : off) + ((cbase + cw) * HQ + hq) * DK + 2 * cl;
      const float *rq2 = anch_b + (int64_t)(2 * I) * HQ * DK + 2 * cl;
      float acc2[2] = {a0[0] * a_scale - rq2[0] + lq, a0[1] * a_scale - rq2[1] + lq};
      uint32_t gw[16], qw[16];
#pragma unroll
      for (int u = 0; u < 16; ++u) {
        const int voff = 4 * cl + hr * 16 * qrow * 2, soff = (qw0 + u) * qrow * 2;
        gw[u] = __builtin_amdgcn_raw_buffer_load_b32(g_rs, voff, soff, 0);
        qw[u] = __builtin_amdgcn_raw_buffer_load_b32(q_rs, voff, soff, 0);
      }
      float hs[2] = {0.f, 0.f};
#pragma unroll
      for (int u = 0; u < 16; ++u) {
        hs[0] += bf16_lo(gw[u]);
        hs[1] += bf16_hi(gw[u]);
      }
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        const float other = __shfl_xor(hs[c], 32);
        if (hr == 1) acc2[c] = fmaf(other, LOG2E, acc2[c]);
      }
#pragma unroll
      for (int u = 0; u < 16; ++u) {
        acc2[0] = fmaf(bf16_lo(gw[u]), LOG2E, acc2[0]);
        acc2[1] = fmaf(bf16_hi(gw[u]), LOG2E, acc2[1]);
        const float q0 = bf16_lo(qw[u]) * fast_exp2(acc2[0]), q1 = bf16_hi(qw[u]) * fast_exp2(acc2[1]);
        qmx = fmaxf(qmx, fmaxf(fabsf(q0), fabsf(q1)));
        *reinterpret_cast<uint32_t *>(&Qs[(wv * 32 + 16 * hr + u) * QSB + 4 * cl]) = pack_f16x2(q0, q1);
      }
      qmx = wave_max(qmx);
      int ex = 0;
      (void)frexpf(qmx, &ex);  // qmx < 2^ex
      qexp = __builtin_amdgcn_readfirstlane(max(ex, -8));
      return;
    }
    const float *a0 = (second ? mid : off) + ((cbase + cw) * HQ + hq) * DK + CPL * lane;
    float acc[CPL];
#pragma unroll
    for (int c = 0; c < CPL; ++c) acc[c] = a0[c] * a_scale - rq[c] + lq;
    const __amdgpu_buffer_rsrc_t *g_b = &g_rs, *q_b = &q_rs;
    auto ld = [&](const __amdgpu_buffer_rsrc_t *rs, int r) -> uint32_t {
      if (CPL == 2) return __builtin_amdgcn_raw_buffer_load_b32(*rs, 4 * lane, r * qrow * 2, 0);
      return __builtin_amdgcn_raw_buffer_load_b16(*rs, 2 * lane, r * qrow * 2, 0);
    };
    uint32_t gw[32], qw[32];  // g and q of the rows
#pragma unroll
    for (int u = 0; u < 32; ++u) {
      gw[u] = ld(g_b, qw0 + u);
      qw[u] = ld(q_b, qw0 + u);
    }
#pragma unroll
    for (int u = 0; u < 32; ++u) {
      float qv[CPL];
      acc[0] = fmaf(bf16_lo(gw[u]), LOG2E, acc[0]);
      qv[0] = bf16_lo(qw[u]);
      if (CPL == 2) {
        acc[CPL - 1] = fmaf(bf16_hi(gw[u]), LOG2E, acc[CPL - 1]);
        qv[CPL - 1] = bf16_hi(qw[u]);
      }
      float qo[CPL];
#pragma unroll
      for (int c = 0; c < CPL; ++c) {
        qo[c] = qv[c] * fast_exp2(acc[c]);
        qmx = fmaxf(qmx, fabsf(qo[c]));
      }
      unsigned char *dst = &Qs[(wv * 32 + u) * QSB + 2 * CPL * lane];
      if (CPL == 2)
        *reinterpret_cast<uint32_t *>(dst) = pack_f16x2(qo[0], qo[CPL - 1]);
      else
        *reinterpret_cast<uint16_t *>(dst) = __builtin_bit_cast(uint16_t, (_Float16)qo[0]);
    }
    qmx = wave_max(qmx);
    int ex = 0;
    (void)frexpf(qmx, &ex);  // qmx < 2^ex
    qexp = __builtin_amdgcn_readfirstlane(max(ex, -8));
  };
  auto load_anch = [&](int chunk, float (&a)[CPL]) {  // anchors of a key chunk, this lane's channels
    const int soff = chunk * HQ * DK * 4;
    if (CPL == 2) {
      const u32x2 x = __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(an_rs, lane * 8, soff, 0));
      a[0] = __uint_as_float(x[0]);
      a[CPL - 1] = __uint_as_float(x[1]);
    } else {
      a[0] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(an_rs, lane * 4, soff, 0));
    }
  };
  auto load_a = [&](int chunk) { load_anch(chunk, araw); };

  // ---- query operand ----
  f16x8 qB[NKS];
  float inv_q = 1.f;  // 2^-sigma of the chunk whose factors qB holds
  float m_ref = 0.f;  // the row's reference max (log2 units, relative to Gs_i)
  // the query's extra channels carry minus the reference max, split into two
  // halves, and the chunk's 2^-sigma for the key's 1 and gate channels
  auto set_qx = [&]() {
    const _Float16 mh = (_Float16)(-m_ref);
    const _Float16 ml = (_Float16)(-m_ref - (float)mh);
    f16x8 x = f16x8{};
    if (half == 0) {
      x[0] = (_Float16)((float)mh * inv_q);
      x[1] = (_Float16)((float)ml * inv_q);
      x[2] = (_Float16)inv_q;
      x[3] = (_Float16)inv_q;
    }
    qB[NKS - 1] = x;
  };
  // Publish the factors of the chunk whose anchors araw holds into the
  // wave's Fq row (with the chunk's 2^-sigma in inv_pend); returns 2^sigma.
  float inv_pend = 1.f;
  auto factors = [&]() -> float {
    float e[CPL];
    bool big = false;
    // largest factor exponent kept without rebalancing: the half factor
    // itself below 2^15 and q_hat * factor below 2^12
    const int cap = min(15, 12 - qexp);
#pragma unroll
    for (int c = 0; c < CPL; ++c) {
      e[c] = rq[c] - araw[c];
      big = big || e[c] > (float)cap;
    }
    int sigma = 0;
    float csg = 1.f;
    inv_pend = 1.f;
    if (__ballot(big) != 0) {
      float em = e[0];
      if (CPL == 2) em = fmaxf(em, e[CPL - 1]);
#pragma unroll
      for (int d = 32; d >= 1; d >>= 1) em = fmaxf(em, __shfl_xor(em, d));
      sigma = (int)em - cap;
      csg = __builtin_amdgcn_ldexpf(1.f, sigma);
      inv_pend = __builtin_amdgcn_ldexpf(1.f, -sigma);
    }
    if (CPL == 2) {
      const int e0 = max((int)e[0] - sigma, -30), e1 = max((int)e[CPL - 1] - sigma, -30);
      *reinterpret_cast<uint32_t *>(&Fq[wv][2 * lane]) =
          pack_f16x2(__builtin_amdgcn_ldexpf(1.f, e0), __builtin_amdgcn_ldexpf(1.f, e1));
    } else {
      const int e0 = max((int)e[0] - sigma, -30);
      Fq[wv][lane] = __builtin_bit_cast(uint16_t, (_Float16)__builtin_amdgcn_ldexpf(1.f, e0));
    }
    return csg;
  };
  // k-step ks of Q' from q_hat and the published factors
  auto q_read = [&](int ks) {
    return *reinterpret_cast<const f16x8 *>(&Qs[(wv * 32 + col) * QSB + 32 * ks + 16 * half]);
  };
  auto f_read = [&](int ks) { return *reinterpret_cast<const f16x8 *>(&Fq[wv][16 * ks + 8 * half]); };
  auto rebuild = [&]() {
#pragma unroll
    for (int ks = 0; ks < NKS - 1; ++ks) qB[ks] = q_read(ks) * f_read(ks);
    inv_q = inv_pend;
    set_qx();
  };

  // ---- LDS-direct staging: instruction i of a tile is issued by wave i % NWV ----
  constexpr int NKM = (BT::NKI + NWV - 1) / NWV, NVM = (BT::NVI + NWV - 1) / NWV;
  int koff[NKM], voff[NVM];
#pragma unroll
  for (int m = 0; m < NKM; ++m) {
    const int g = 64 * (wv + NWV * m) + lane, r = g / BT::KPR, pp = g % BT::KPR;
    koff[m] = r * KRB + 16 * (pp ^ ((r >> 3) & 1));
  }
#pragma unroll
  for (int m = 0; m < NVM; ++m) {
    // padding pieces load the row's first piece again (in range, never read)
    const int g = 64 * (wv + NWV * m) + lane, r = g / BT::VPR, pp = g % BT::VPR;
    voff[m] = r * vrow * 2 + (pp < DV / 8 ? 16 * pp : 0);
  }
  auto dma_k = [&](int J, unsigned char *buf) {
#pragma unroll
    for (int m = 0; m < NKM; ++m) {
      const int i = wv + NWV * m;
      if ((m + 1) * NWV <= BT::NKI || i < BT::NKI) dma16(kt_rs, buf + 1024 * i, koff[m], J * BK * KRB);
    }
  };
  auto dma_v = [&](int J, unsigned char *buf) {
#pragma unroll
    for (int m = 0; m < NVM; ++m) {
      const int i = wv + NWV * m;
      if ((m + 1) * NWV <= BT::NVI || i < BT::NVI) dma16(v_rs, buf + 1024 * i, voff[m], J * BK * vrow * 2);
    }
  };
  // the wave's d-th load of an iteration: key loads first, then value loads
  constexpr int NDM = NKM + NVM;
  // a tile of 9 (or 5) KiB leaves a last load for the first wave(s) only;
  // the steady-state block issues that one right at its start, so that the
  // block itself has no branch on the wave index
  constexpr int KR = (BT::NKI % NWV) ? NKM - 1 : -1, VR = (BT::NVI % NWV) ? NVM - 1 : -1;
  auto dma_one = [&](int d, int Jk, unsigned char *kbuf, int Jv, unsigned char *vbuf, bool kdo, bool vdo) {
    if (d < NKM) {
      const int i = wv + NWV * d;
      if (kdo && ((d + 1) * NWV <= BT::NKI || i < BT::NKI)) dma16(kt_rs, kbuf + 1024 * i, koff[d], Jk * BK * KRB);
    } else {
      const int m = d - NKM, i = wv + NWV * m;
      if (vdo && ((m + 1) * NWV <= BT::NVI || i < BT::NVI)) dma16(v_rs, vbuf + 1024 * i, voff[m], Jv * BK * vrow * 2);
    }
  };

  // ---- compute pieces ----
  // score A operand: key row col of the tile, channels 16 ks + 8 half .. +7
  const int sa_off = col * KRB + 16 * (half ^ ((col >> 3) & 1));
  auto s_mfma = [&](f32x16 &S, const unsigned char *Kb, int ks) {
    const f16x8 a = *reinterpret_cast<const f16x8 *>(Kb + sa_off + ks * 32);
    S = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, qB[ks], S, 0, 0, 0);
  };
  // k-steps 0 .. n-1 of a tile's scores into a fresh accumulator, every
  // operand read issued before the first MFMA (one LDS round trip, not n)
  auto s_batch = [&](auto n_c, f32x16 &S, const unsigned char *Kb) {
    constexpr int N = decltype(n_c)::value;
    f16x8 a[N];
#pragma unroll
    for (int ks = 0; ks < N; ++ks) a[ks] = *reinterpret_cast<const f16x8 *>(Kb + sa_off + ks * 32);
    __builtin_amdgcn_sched_barrier(0);
    S = f32x16{};
#pragma unroll
    for (int ks = 0; ks < N; ++ks) S = __builtin_amdgcn_mfma_f32_32x32x16_f16(a[ks], qB[ks], S, 0, 0, 0);
  };
  // The S^T accumulator holds, in lane (col, half), keys 8 (r/4) + 4 half + r%4
  // (r = 0..15) of query column col.  Its elements r = 8t..8t+7 are directly
  // the B operand (k = 16 keys) of the value product, with the keys in the
  // order k -> 8(k/4 % 2) + 4 half + k%4 within the 16-key step; the value
  // operand is read in the same order with two transpose reads (rows
  // key0 .. key0+3 each).  tr_off: this lane's piece of the first of those
  // reads (row 4 half + j16/4) for output block 0.
  const int j16 = lane & 15;
  const int tr_off = (4 * half + (j16 >> 2)) * VRB + 32 * ((lane >> 4) & 1) + 8 * (j16 & 3);
  f32x16 oacc[NMB];
  auto vread8 = [&](const unsigned char *Vb, int mb, int st) {
    const unsigned char *base = Vb + tr_off + 64 * mb + 16 * st * VRB;
    const s16x4 a0 = lds_read_tr4(base), a1 = lds_read_tr4(base + 8 * VRB);
    return __builtin_bit_cast(bf16x8, __builtin_shufflevector(a0, a1, 0, 1, 2, 3, 4, 5, 6, 7));
  };
  // value operands of a whole tile, read ahead of the softmax that feeds them
  auto vload = [&](const unsigned char *Vb, bf16x8 (&va)[2 * NMB]) {
#pragma unroll
    for (int mb = 0; mb < NMB; ++mb)
#pragma unroll
      for (int s = 0; s < 2; ++s) va[2 * mb + s] = vread8(Vb, mb, s);
    __builtin_amdgcn_sched_barrier(0);
  };
  auto pv = [&](const bf16x8 (&va)[2 * NMB], const bf16x8 (&pB)[2]) {
#pragma unroll
    for (int mb = 0; mb < NMB; ++mb)
#pragma unroll
      for (int s = 0; s < 2; ++s)
        oacc[mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va[2 * mb + s], pB[s], oacc[mb], 0, 0, 0);
  };
  auto mask = [&](f32x16 &S, int kj0) {
    const int rel = qw0 + col - kj0 - 4 * half;  // allowed: kk <= rel
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int kk = 8 * (r >> 2) + (r & 3);
      bool ok = kk <= rel;
      if (window > 0) ok = ok && (rel - kk < window);
      S[r] = ok ? S[r] : -INFINITY;
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
  // never rescaled.  A tile whose probabilities could exceed 2^64 against
  // the reference (scores far above the diagonal's) sets a flag; the
  // workgroup then recomputes its rows with the exact row max from a
  // max-only sweep, which cannot overflow.
  constexpr float PBIG = 0x1p64f;
  float l_part = 0.f;  // this lane's half of the row's key sum
  bool m_set = false, all_set = false, ovf = false;
  float m_true = -INFINITY;
  auto tail = [&](f32x16 &S, bf16x8 (&pB)[2]) {
#pragma unroll
    for (int r = 0; r < 16; ++r) S[r] = fast_exp2(S[r]);
    pB[0] = __builtin_convertvector(__builtin_shufflevector(S, S, 0, 1, 2, 3, 4, 5, 6, 7), bf16x8);
    pB[1] = __builtin_convertvector(__builtin_shufflevector(S, S, 8, 9, 10, 11, 12, 13, 14, 15), bf16x8);
    const float rs = bf16x8_sum(pB[1], bf16x8_sum(pB[0], 0.f));
    l_part += rs;
    ovf = ovf || !(rs <= PBIG);
  };
  // rows without a reference yet take this tile's max (nothing is
  // accumulated for them, so nothing needs rescaling)
  auto set_rows = [&](f32x16 &S) {
    const float mx = tile_max(S);
    const bool take = !m_set && mx > -INFINITY;
    const float shift = take ? mx : 0.f;
    if (take) {
      m_ref = mx;
      m_set = true;
    }
#pragma unroll
    for (int r = 0; r < 16; ++r) S[r] -= shift;
    set_qx();
    all_set = __ballot(!m_set) == 0;
  };

  // Steady-state tile in a fixed issue order (FusedOrder): scores of the next
  // tile, exponentials of this tile, value MFMAs of this tile.
  // sched_barrier(0) keeps each slot's instructions together; the wave runs
  // its MFMA-dense part at raised priority so that the other wave on the SIMD
  // fills the gaps with its own VALU and LDS work.
  // The block also issues the wave's LDS-direct loads of the next tiles (one
  // per slot from slot DSLOT on; a tile's ragged last load just before the
  // block) and, with RB, rebuilds each k-step of the query operand for the
  // tile after next right after the score MFMA that last reads it, from the
  // factors last published (the first block of a steady pair, whose tile
  // after next starts a chunk).  A tile that crosses the window edge of the
  // wave's rows (mk: its first key, else -1) is masked before its
  // exponentials.
  auto fused = [&](auto rb_c, f32x16 &Sc, f32x16 &Sn, const unsigned char *Vb, const unsigned char *Kb,
                   int Jk, unsigned char *kbuf, int Jv, unsigned char *vbuf, bool kdo, int mk) {
    constexpr bool RB = decltype(rb_c)::value;
    constexpr int NP = 2 * NMB;
    constexpr FusedOrder<NKS, NP, 4> FO{};
    constexpr int KAHEAD = 4, VAHEAD = 4, RAHEAD = 1, DSLOT = 4;
    constexpr int E = 16;                 // exponentials of the tile
    static_assert(DSLOT + NDM <= FO.N, "every load needs a slot");
    f16x8 ka[NKS];
    bf16x8 va[NP];
    f16x8 qr[NKS], fr[NKS];
    auto kread = [&](int ks) { ka[ks] = *reinterpret_cast<const f16x8 *>(Kb + sa_off + ks * 32); };
    auto vread = [&](int j) { va[j] = vread8(Vb, j % NMB, j / NMB); };  // block j % NMB, 16-key step j / NMB
    auto rread = [&](int ks) {
      if (RB && ks < NKS - 1) {
        qr[ks] = q_read(ks);
        fr[ks] = f_read(ks);
      }
    };
    if (KR >= 0 && kdo && wv + NWV * KR < BT::NKI) dma16(kt_rs, kbuf + 1024 * (wv + NWV * KR), koff[KR], Jk * BK * KRB);
    if (VR >= 0 && wv + NWV * VR < BT::NVI) dma16(v_rs, vbuf + 1024 * (wv + NWV * VR), voff[VR], Jv * BK * vrow * 2);
    if (mk >= 0) mask(Sc, mk);
    float pr[16];
    bf16x8 pb[2];
    float rs = 0.f;
#pragma unroll
    for (int i = 0; i < NKS; ++i) {
      if (FO.slot_s[i] < KAHEAD) kread(i);
      if (FO.slot_s[i] < RAHEAD) rread(i);
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int n = 0; n < FO.N; ++n) {
#pragma unroll
      for (int i = 0; i < NKS; ++i) {
        if (FO.slot_s[i] >= KAHEAD && FO.slot_s[i] - KAHEAD == n) kread(i);
        if (FO.slot_s[i] >= RAHEAD && FO.slot_s[i] - RAHEAD == n) rread(i);
      }
#pragma unroll
      for (int j = 0; j < NP; ++j)
        if (FO.slot_p[j] - VAHEAD == n || (FO.slot_p[j] < VAHEAD && n == 0)) vread(j);
      if (n == FO.S_ALONE) __builtin_amdgcn_s_setprio(1);
      if (FO.kind[n] == 0) {
        const int ks = FO.idx[n];
        Sn = __builtin_amdgcn_mfma_f32_32x32x16_f16(ka[ks], qB[ks], ks == 0 ? f32x16{} : Sn, 0, 0, 0);
        if (RB && ks < NKS - 1) qB[ks] = qr[ks] * fr[ks];
      } else {
        const int j = FO.idx[n], mb = j % NMB, st = j / NMB;
        oacc[mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va[j], pb[st], oacc[mb], 0, 0, 0);
      }
      if (n >= DSLOT && n - DSLOT < NDM && n - DSLOT != KR && n - DSLOT != NKM + VR)
        dma_one(n - DSLOT, Jk, kbuf, Jv, vbuf, kdo, true);
      // exponentials: the first half (probabilities of the first 16-key
      // step) in the score-only slots, the second half spread over the slots
      // up to the first value MFMA that needs them
      constexpr int XS = FO.slot_p[NMB] - FO.S_ALONE;
      if (n < FO.S_ALONE + XS) {
        const int e0 = n < FO.S_ALONE ? n * (E / 2) / FO.S_ALONE : E / 2 + (n - FO.S_ALONE) * (E / 2) / XS;
        const int e1 = n < FO.S_ALONE ? (n + 1) * (E / 2) / FO.S_ALONE : E / 2 + (n - FO.S_ALONE + 1) * (E / 2) / XS;
#pragma unroll
        for (int e = 0; e < E; ++e) {
          if (e < e0 || e >= e1) continue;
          pr[e] = fast_exp2(Sc[e]);
        }
#pragma unroll
        for (int st = 0; st < 2; ++st)
          if (e0 < E / 2 * (st + 1) && e1 >= E / 2 * (st + 1)) {
            f32x8 p8;
#pragma unroll
            for (int r = 0; r < 8; ++r) p8[r] = pr[8 * st + r];
            pb[st] = __builtin_convertvector(p8, bf16x8);
            rs = bf16x8_sum(pb[st], rs);
          }
        if (e1 == E) {
          l_part += rs;
          ovf = ovf || !(rs <= PBIG);
        }
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    __builtin_amdgcn_s_setprio(0);
    if (RB) {
      inv_q = inv_pend;
      set_qx();
    }
  };

  // ---- pipeline ----
  // Visiting order: the query tile's own QTILE/BK key tiles newest first,
  // then the older tiles from the oldest up, so that workgroups running
  // side by side walk the same key tiles together and find them in L2.
  // Iteration t: scores of tile t+1 (key buffer (t+1)&1) are accumulated
  // while the softmax of tile t runs, then tile t's probabilities meet its
  // values (value buffer t&1).  After the iteration's barrier each wave
  // issues its share of the LDS-direct loads of key tile t+2 (into key
  // buffer t&1, free once tile t's scores are done) and value tile t+1 (into
  // value buffer (t+1)&1), and the anchors of tile t+3's chunk; if tile t+2
  // starts a new chunk, its factors (anchors from the previous iteration)
  // are published first and the query operand is rebuilt as soon as tile
  // t+1's scores no longer need it.  The wave's loads are waited for before
  // the next barrier.
  if (tid == 0) wg_ovf = 0;
  const int NTL = Jhi - Jlo + 1;  // tiles of this workgroup
  // mode 0: reference max from the diagonal tiles; 1: max-only sweep; 2: exact row max known
  auto sweep = [&](auto mode_c) {
    constexpr int MODE = decltype(mode_c)::value;
    constexpr bool VAL = MODE != 1;  // the pass needs values
    const int ND = NTL < QTILE / BK ? NTL : QTILE / BK;  // diagonal tiles, visited first
    auto tileJ = [&](int t) { return t < ND ? Jhi - t : Jlo + (t - ND); };
    static_assert(CHUNK == 2 * BK, "a chunk is two key tiles");
    auto chunkOf = [&](int t) { return tileJ(t) >> 1; };  // tile indices are never negative
    auto new_chunk = [&](int t) { return t == 0 || chunkOf(t) != chunkOf(t - 1); };
    if (MODE != 0) __syncthreads();  // the previous sweep's reads of the tile buffers are done
    // the anchors of the first three tiles' chunks load together, ahead of
    // the tile loads and q_hat
    const bool nc1 = 1 < NTL && new_chunk(1);
    const bool nc2p = 2 < NTL && new_chunk(2);
    float a1[CPL], a2[CPL];
    load_a(chunkOf(0));
    if (nc1) load_anch(chunkOf(1), a1);
    if (nc2p) load_anch(chunkOf(2), a2);
    dma_k(tileJ(0), K0);
    if (VAL) dma_v(tileJ(0), V0);
    if (1 < NTL) dma_k(tileJ(1), K1);
    if (MODE == 0) make_qhat();  // overlaps the first tile loads
    float cs_cur = factors();
    rebuild();
    float cs_next = cs_cur;
    if (nc1) {
#pragma unroll
      for (int c = 0; c < CPL; ++c) araw[c] = a1[c];
      cs_next = factors();
    }
    if (nc2p) {
#pragma unroll
      for (int c = 0; c < CPL; ++c) araw[c] = a2[c];
    }
    vm_wait0();
    __syncthreads();
    f32x16 Sa, Sb;
    {
      const int J = tileJ(0);
      if (J >= Jlo_w && J <= Jhi_w) s_batch(std::integral_constant<int, NKS>{}, Sa, K0);
    }
    if (nc1) rebuild();
    float cs_next2 = cs_next;  // 2^sigma of the tile after next
    if (nc2p) cs_next2 = factors();

    auto body = [&](auto par_c, int t, f32x16 &Sc, f32x16 &Sn) {
      constexpr int P = decltype(par_c)::value;  // t & 1
      unsigned char *const Kc = P ? K1 : K0;     // key buffer of tiles t and t+2
      unsigned char *const Kn = P ? K0 : K1;     // key buffer of tile t+1
      unsigned char *const Vc = P ? V1 : V0;     // value buffer of tile t
      unsigned char *const Vn = P ? V0 : V1;     // value buffer of tile t+1
      __syncthreads();
      // tile t+2's chunk factors were published at the end of the previous
      // iteration; they reach the query operand once tile t+1's scores are
      // issued.  The anchors of tile t+3's chunk load now and are published
      // at the end of this iteration, while the tile loads complete.
      const bool nc2 = t + 2 < NTL && new_chunk(t + 2);
      const bool nc3 = t + 3 < NTL && new_chunk(t + 3);
      if (nc3) load_a(chunkOf(t + 3));
      const int J = tileJ(t), Jn = tileJ(t + 1);
      const bool need_cur = J >= Jlo_w && J <= Jhi_w;
      const bool need_next = t + 1 < NTL && Jn >= Jlo_w && Jn <= Jhi_w;
      const int kj0 = J * BK;
      const bool masked = kj0 + BK - 1 > qw0 || (window > 0 && qw0 + 31 - kj0 >= window);
      bf16x8 pB[2];
      {
        if (t + 2 < NTL) dma_k(tileJ(t + 2), Kc);
        if (VAL && t + 1 < NTL) dma_v(Jn, Vn);
        if (need_next) s_batch(std::integral_constant<int, NKS - 1>{}, Sn, Kn);
        if (need_cur) {
          __asm__ volatile("s_nop 0");  // keep this a branch
          bf16x8 va[2 * NMB];
          if (VAL) vload(Vc, va);
          if (masked) mask(Sc, kj0);
          if (cs_cur != 1.f) Sc *= cs_cur;
          if (MODE == 1) {
            m_true = fmaxf(m_true, tile_max(Sc));
          } else {
            if (MODE == 0 && !all_set) set_rows(Sc);
            tail(Sc, pB);
            pv(va, pB);
          }
        }
        if (need_next) s_mfma(Sn, Kn, NKS - 1);  // after any change of the row reference
        if (nc2) rebuild();
      }
      float cs3 = cs_next2;
      if (nc3) cs3 = factors();
      cs_cur = cs_next;
      cs_next = cs_next2;
      cs_next2 = cs3;
      vm_wait0();
    };
    // A pair of tiles t (even, the first of an anchor chunk) and t + 1, both
    // older than the query tile's own key tiles, with every row's reference
    // set and sigma = 0 for their chunk, with tiles up to t + 4 still to
    // come: body() would take its steady-state block for both, rebuild
    // inside the first one and publish the factors of chunk(t + 4) after the
    // second one.  The same work with every condition known in advance.  A
    // tile at the window edge is masked inside the block; a tile that lies
    // wholly below the wave's window then adds nothing (body() would skip
    // it for this wave).
    auto pair_ok = [&](int t) -> bool {
      if (MODE == 1 || t < ND || t + 2 >= NTL) return false;
      if (tileJ(t) & 1) return false;
      return __ballot(!(all_set && cs_cur == 1.f && cs_next == 1.f)) == 0;
    };
    // first key of tile J when it crosses the window edge of the wave's rows
    auto edge = [&](int J) { return window > 0 && qw0 + 31 - J * BK >= window ? J * BK : -1; };
    auto steady_pair = [&](int t) {
      const int J = tileJ(t);  // tiles t .. t + 3 are J .. J + 3
      __syncthreads();
      fused(std::true_type{}, Sa, Sb, V0, K1, J + 2, K0, J + 1, V1, true, edge(J));
      cs_cur = cs_next;
      cs_next = cs_next2;
      vm_wait0();
      __syncthreads();
      const bool nc4 = t + 4 < NTL;  // tile t + 4 exists (and starts a chunk)
      if (nc4) load_a((J + 4) >> 1);
      fused(std::false_type{}, Sb, Sa, V1, K0, J + 3, K1, J + 2, V0, t + 3 < NTL, edge(J + 1));
      float cs3 = cs_next2;
      if (nc4) cs3 = factors();
      cs_cur = cs_next;
      cs_next = cs_next2;
      cs_next2 = cs3;
      vm_wait0();
    };
    int t = 0;
    while (t < NTL) {
      for (; t < NTL && !pair_ok(t); t += 2) {
        body(std::integral_constant<int, 0>{}, t, Sa, Sb);
        if (t + 1 < NTL) body(std::integral_constant<int, 1>{}, t + 1, Sb, Sa);
      }
      for (; t < NTL && pair_ok(t); t += 2) steady_pair(t);
    }
  };
  auto reset = [&](bool known) {
    m_ref = known ? (m_true > -INFINITY ? m_true : 0.f) : 0.f;
    m_set = known;
    l_part = 0.f;
#pragma unroll
    for (int mb = 0; mb < NMB; ++mb) oacc[mb] = f32x16{};
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
    m_ref = 0.f;
    sweep(std::integral_constant<int, 1>{});
    reset(true);
    sweep(std::integral_constant<int, 2>{});
  }

  // ---- epilogue ----
  // scores above are relative to the row term Gs[i] (g_i); restore it here
  {
    const int qi = qw0 + col;
    const float Zl = half_sum(l_part);
    if (qi < L) {
      float mf = m_ref, Z = Zl;
      if (sink != nullptr) {
        const float s2 = sink[hq] * LOG2E - g_i;
        mf = fmaxf(m_ref, s2);
        Z = Zl * fast_exp2(m_ref - mf) + fast_exp2(s2 - mf);
      }
      const float inv = fast_exp2(m_ref - mf) / Z;
      bf16_t *orow = o + ((bos64 + qi) * HQ + hq) * DV;
#pragma unroll
      for (int mb = 0; mb < NMB; ++mb)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          u32x2 w;
          w.x = pack_bf16x2(oacc[mb][4 * j] * inv, oacc[mb][4 * j + 1] * inv);
          w.y = pack_bf16x2(oacc[mb][4 * j + 2] * inv, oacc[mb][4 * j + 3] * inv);
          *reinterpret_cast<u32x2 *>(orow + mb * 32 + 8 * j + 4 * half) = w;
        }
      if (lse != nullptr && half == 0)
        lse[(bos64 + qi) * HQ + hq] = (mf + g_i + log2f(Z)) * LN2;
    }
  }
}

// fp32 kernel: plain FMA arithmetic, one 64-row chunk of queries per
// workgroup, 4 threads per query row; thread `sub` owns channels n = 4e + sub.
template <int DK, int DV, bool HAS_GS>
__global__ __launch_bounds__(256) void k_attn_fwd_f32(
    const float *__restrict__ q, const float *__restrict__ k, const float *__restrict__ g,
    const float *__restrict__ off, const float *__restrict__ qh, const float *__restrict__ kt,
    const float *__restrict__ v, const float *__restrict__ anch, const float *__restrict__ gsum,
    const float *__restrict__ sink, float *__restrict__ o, float *__restrict__ lse,
    const int32_t *__restrict__ cu, int64_t T, int HQ, int H, int nseg, int NCmax, int NCH,
    int64_t window, float qscale, const int *__restrict__ wide) {
  constexpr int QPT = DK / 4, VPT = DV / 4;
  // keys then values; the exact path reuses the block
  static_assert(4 * BN * (DK + DV) >= exact::ExactLds<DK, DV>::BYTES, "the exact path fits in the LDS block");
  __shared__ __attribute__((aligned(16))) float KVs[BN * (DK + DV)];
  float *const Ks = KVs, *const Vs = KVs + BN * DK;
  __shared__ float dL[DK];
  __shared__ float Gj[BN];

  const int tid = threadIdx.x;
  const int hq = blockIdx.x % HQ;
  const int rest = blockIdx.x / HQ;
  const int seg = rest % nseg;
  const int c = NCH - 1 - rest / nseg;
  const bool pair_wide = __builtin_amdgcn_readfirstlane(wide[seg * HQ + hq]) != 0;
  int64_t bos, eos;
  segment_bounds(seg, T, cu, bos, eos);
  const int64_t L = eos - bos;
  const int nch = (int)((L + CHUNK - 1) / CHUNK);
  if (c >= nch) return;
  if (pair_wide) {  // the decay leaves the float operands' range: exact rows
    exact::exact_chunk<float, DK, DV, HAS_GS>(q, k, v, g, off + ((int64_t)seg * NCmax * HQ + hq) * DK, gsum,
                                              sink, o, lse, bos, (int)L, hq, HQ, H,
                                              window > 0 && window < L ? (int)window : 0, qscale, c,
                                              reinterpret_cast<unsigned char *>(KVs));
    return;
  }
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
    hipLaunchKernelGGL(kern, grid, dim3(BfTile<DK, DV>::NTH), 0, st,
                       static_cast<const bf16_t *>(p.q), static_cast<const bf16_t *>(p.k),
                       static_cast<const bf16_t *>(p.g), ws.csum, static_cast<const _Float16 *>(ws.kt),
                       static_cast<const bf16_t *>(p.v),
                       ws.anch, ws.gsum, p.sink, static_cast<bf16_t *>(p.o), p.lse, p.cu, p.T,
                       p.ntok, (int)p.HQ, (int)p.H, (int)p.nseg, NCmax, NQT,
                       (int)(p.window > 0 && p.window < p.maxlen ? p.window : 0), p.scale * LOG2E,
                       ws.wide, ws.mid);
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
    hipLaunchKernelGGL(kern, grid, dim3(256), 0, st, static_cast<const float *>(p.q),
                       static_cast<const float *>(p.k), static_cast<const float *>(p.g), ws.csum,
                       static_cast<const float *>(ws.qh), static_cast<const float *>(ws.kt),
                       static_cast<const float *>(p.v), ws.anch, ws.gsum, p.sink,
                       static_cast<float *>(p.o), p.lse, p.cu, p.T, (int)p.HQ, (int)p.H,
                       (int)p.nseg, NCmax, NCmax, p.window, p.scale * LOG2E, ws.wide);
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

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
#pragma once
#include <math.h>

#include "common.h"
#include "launch.h"

namespace wa {
namespace dec {
// internal linkage: every translation unit keeps its own kernels
namespace {

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *p, int64_t bytes) {
  // integer select: HIP's min() on 64-bit integers goes through f64 VALU code
  const int n = bytes > 0x7fffffff ? 0x7fffffff : (int)bytes;
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(p), 0, n, 0x00020000);
}
// k_tilde and v are read once per call: streaming (non-temporal) loads,
// cache policy 2, which a plain read-only stream measured at 7.2 TB/s
// against 6.3 TB/s for default-policy loads on MI355X.
__device__ __forceinline__ u32x4 buf_load16(__amdgpu_buffer_rsrc_t rs, int voff, int soff) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, voff, soff, 2));
}

// Eight elements of one lane in registers.  16-bit types hold 8 consecutive
// elements (one 16-byte load); float holds two runs of 4, the second `far`
// bytes after the first (one 16-byte load each).
template <typename TE>
struct Vec8;
template <>
struct Vec8<bf16_t> {
  u32x4 w;
  __device__ __forceinline__ void load(__amdgpu_buffer_rsrc_t rs, int voff, int soff, int) {
    w = buf_load16(rs, voff, soff);
  }
  __device__ __forceinline__ float operator[](int e) const {
    return (e & 1) ? bf16_hi(w[e >> 1]) : bf16_lo(w[e >> 1]);
  }
};
template <>
struct Vec8<_Float16> {
  u32x4 w;
  __device__ __forceinline__ void load(__amdgpu_buffer_rsrc_t rs, int voff, int soff, int) {
    w = buf_load16(rs, voff, soff);
  }
  __device__ __forceinline__ float operator[](int e) const {
    return (e & 1) ? f16_hi(w[e >> 1]) : f16_lo(w[e >> 1]);
  }
};
template <>
struct Vec8<float> {
  u32x4 a, b;
  __device__ __forceinline__ void load(__amdgpu_buffer_rsrc_t rs, int voff, int soff, int far) {
    a = buf_load16(rs, voff, soff);
    b = buf_load16(rs, voff + far, soff);
  }
  __device__ __forceinline__ float operator[](int e) const {
    return __uint_as_float(e < 4 ? a[e & 3] : b[e & 3]);
  }
};

// Sum of x over groups of N consecutive lanes (N = 8 or 16) with DPP row
// rotations; every lane of a group gets the group's sum.
template <int N>
__device__ __forceinline__ float row_sum(float x) {
  static_assert(N == 8 || N == 16, "groups of 8 or 16 lanes");
  // row_ror:n has DPP control 0x120 + n; rotations stay inside 16-lane rows
  if (N == 16) x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x128, 0xf, 0xf, false));
  if (N == 8) {
    // rotations by 4, 2, 1 inside a 16-lane row mix the two 8-lane halves;
    // use xor shuffles within 8 lanes instead
    x += __shfl_xor(x, 4, 8);
    x += __shfl_xor(x, 2, 8);
    x += __shfl_xor(x, 1, 8);
    return x;
  }
  x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x124, 0xf, 0xf, false));
  x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x122, 0xf, 0xf, false));
  x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x121, 0xf, 0xf, false));
  return x;
}

// Where chunk c of batch row b lives: the pool row of its first token (rows
// of k_tilde / v / the gate cache) and its anchor row in r_cache.
struct ChunkAddr {
  int64_t row, anchor;
};
__device__ __forceinline__ ChunkAddr chunk_addr(const DecodeParams &p, int b, int c) {
  ChunkAddr a;
  a.row = cache_row(p.block_table, p.max_blocks, p.page_size, p.num_pages, p.T, b, c * CHUNK);
  // contiguous rows: r_cache has ceil(T/C) anchors per batch row; pages hold
  // whole chunks, so a page row's anchor is its row / C
  a.anchor = p.block_table != nullptr ? a.row / CHUNK : (int64_t)b * p.NC + c;
  a.row = uniform64(a.row);
  a.anchor = uniform64(a.anchor);
  return a;
}

// grid (nsplit, HQ/NHB, B), 256 threads.  TE: type of q and v; TK: type of
// the cache k_tilde.
//
// Memory-level parallelism: every 16-byte piece of the next chunk's keys and
// values is requested as soon as the same piece of the current chunk has been
// consumed, so one register set holds both the data in use and the data in
// flight (about one chunk ahead).
// Three workgroups per CU where the registers allow it (16-bit caches and
// values, no gate), else two.
template <typename TE, typename TK, int DK, int DV, int NHB, bool GATE>
__global__ __launch_bounds__(256, (sizeof(TK) == 2 && sizeof(TE) == 2 && !GATE) ? 3 : 2) void k_decode_split(
    DecodeParams p) {
  constexpr int C = CHUNK;
  constexpr int VCG = DV / 8;         // 8-channel groups of a value row
  constexpr int KL = 256 / VCG;       // key lanes in the PV phase
  constexpr int KPL = C / KL;         // keys per key lane
  constexpr int QN = NHB * DK;        // rescaled query values per chunk
  constexpr int QPT = (QN + 255) / 256;

  __shared__ __attribute__((aligned(16))) float Qs[2][NHB][DK];
  __shared__ __attribute__((aligned(16))) float Ps[2][C][NHB];
  __shared__ float Al[2][NHB];
  __shared__ float red[KL][NHB][DV];

  const TE *__restrict__ q = static_cast<const TE *>(p.q);
  const TE *__restrict__ v = static_cast<const TE *>(p.v);
  const TK *__restrict__ kt = static_cast<const TK *>(p.kt);
  const int HQ = p.HQ, H = p.H;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: keeps descriptors scalar
  const int split = blockIdx.x, hq0 = blockIdx.y * NHB, b = blockIdx.z;
  const int h = hq0 / (HQ / H);
  const int64_t pbase = ((int64_t)b * HQ + hq0) * p.nsplit + split;

  // this row's visible keys [j_lo, L) and its share of their chunks
  // lengths outside [0, T] are clamped into it (no access leaves the cache)
  const int L = __builtin_amdgcn_readfirstlane(
      p.seqlens != nullptr ? min(max(p.seqlens[b], 0), (int)p.T) : (int)p.T);
  const int j_lo = p.window > 0 ? max(0, L - p.window) : 0;
  const int c_lo = j_lo / C, nch = L > 0 ? (L - 1) / C - c_lo + 1 : 0;
  const int cps = (nch + p.nsplit - 1) / p.nsplit;
  const int c_begin = c_lo + split * cps, c_end = min(c_lo + nch, c_begin + cps);
  if (c_begin >= c_end) {  // nothing to do: an empty partial result
    for (int x = tid; x < NHB * DV; x += 256)
      p.part_o[(pbase + (int64_t)(x / DV) * p.nsplit) * DV + x % DV] = 0.f;
    if (tid < NHB) {
      p.part_ml[(pbase + (int64_t)tid * p.nsplit) * 2 + 0] = -INFINITY;
      p.part_ml[(pbase + (int64_t)tid * p.nsplit) * 2 + 1] = 0.f;
    }
    return;
  }
  auto nvalid = [&](int c) { return min(C, L - c * C); };

  // rescaling inputs: q and p_curr per (head, channel) owned by this thread
  float qreg[QPT], preg[QPT], rreg[QPT];
#pragma unroll
  for (int i = 0; i < QPT; ++i) {
    const int x = tid + 256 * i;
    const int hh = x / DK, n = x % DK;
    qreg[i] = x < QN ? Elem<TE>::ld(q + ((int64_t)b * HQ + hq0 + hh) * DK + n) : 0.f;
    preg[i] = x < QN ? p.p_curr[((int64_t)b * HQ + hq0 + hh) * DK + n] : 0.f;
  }
  auto load_r = [&](int64_t anchor) {
#pragma unroll
    for (int i = 0; i < QPT; ++i) {
      const int x = tid + 256 * i;
      const int hh = x / DK, n = x % DK;
      rreg[i] = x < QN ? p.rc[(anchor * HQ + hq0 + hh) * DK + n] : 0.f;
    }
  };

  // score role: head sh = wave.  Load i of a chunk brings keys RPI i + r
  // (r = lane / LPR), lane u = lane % LPR holding 8 channels of its key
  // (channels 8u .. 8u+7 for 16-bit caches; 4u .. 4u+3 and DK/2 + 4u .. +3
  // for float caches, so that each load instruction still covers whole
  // 16-byte-per-lane runs of consecutive channels).  The partial dot
  // products are summed over the LPR lanes of a row, and lane (r, u) then
  // owns key kk = RPI u + r.
  static_assert(DK == 128 || DK == 64, "key rows of 16 or 8 lanes");
  constexpr bool KF32 = sizeof(TK) == 4;
  constexpr int LPR = DK / 8;         // lanes per key row
  constexpr int RPI = 64 / LPR;       // key rows per load instruction
  constexpr int NKI = C / RPI;        // loads per chunk
  constexpr int KROW = DK * (int)sizeof(TK);
  const int sh = wave, kr = lane / LPR, ku = lane % LPR;
  const int kk = RPI * ku + kr;       // the key whose score this lane keeps (NKI == LPR)
  static_assert(NKI == LPR, "one reduced score per lane");
  const bool s_role = sh < NHB;
  const int hs = hq0 + (s_role ? sh : 0);  // this wave's head
  const int k_voff = kr * HQ * KROW + 16 * ku;
  const int q_a = KF32 ? 4 * ku : 8 * ku, q_b = KF32 ? DK / 2 + 4 * ku : 8 * ku + 4;
  auto k_rsrc = [&](const ChunkAddr &a, int c) {
    return make_rsrc(kt + (a.row * HQ + hs) * DK, (int64_t)nvalid(c) * HQ * KROW);
  };
  auto kload = [&](Vec8<TK> &r, __amdgpu_buffer_rsrc_t rs, int i) {
    r.load(rs, k_voff, RPI * i * HQ * KROW, DK * 2);
  };
  Vec8<TK> kreg[NKI];
  // gate: the running gate sum (log2 units) of this lane's key
  constexpr bool gate = GATE;  // p.gs_cache != nullptr
  const float g_cur = gate && s_role ? p.gs_curr[(int64_t)b * HQ + hs] : 0.f;
  auto g_rsrc = [&](const ChunkAddr &a, int c) {
    return make_rsrc(p.gs_cache + a.row * HQ + hs, (int64_t)nvalid(c) * HQ * 4);
  };
  auto gload = [&](__amdgpu_buffer_rsrc_t rs) {
    return __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rs, kk * HQ * 4, 0, 0));
  };

  // PV role: channel group cg, key lane kl
  const int cg = tid % VCG, kl = tid / VCG;
  auto v_rsrc = [&](const ChunkAddr &a, int c) {
    return make_rsrc(v + (a.row * H + h) * DV, (int64_t)nvalid(c) * H * DV * (int)sizeof(TE));
  };
  const int v_voff = (kl * H * DV + cg * 8) * (int)sizeof(TE);
  auto vload = [&](Vec8<TE> &r, __amdgpu_buffer_rsrc_t rs, int i) {
    r.load(rs, v_voff, KL * i * H * DV * (int)sizeof(TE), 16);
  };
  Vec8<TE> vreg[KPL];

  float m_run = -INFINITY, l_run = 0.f;  // per score wave (its head)
  float oacc[NHB][8];
#pragma unroll
  for (int hh = 0; hh < NHB; ++hh)
#pragma unroll
    for (int e = 0; e < 8; ++e) oacc[hh][e] = 0.f;

  ChunkAddr acur = chunk_addr(p, b, c_begin);
  load_r(acur.anchor);
  __amdgpu_buffer_rsrc_t krs = k_rsrc(acur, c_begin), vrs = v_rsrc(acur, c_begin);
  __amdgpu_buffer_rsrc_t grs = krs;
  float gval = 0.f;
  if (s_role) {
#pragma unroll
    for (int i = 0; i < NKI; ++i) kload(kreg[i], krs, i);
    if (gate) {
      grs = g_rsrc(acur, c_begin);
      gval = gload(grs);
    }
  }
#pragma unroll
  for (int i = 0; i < KPL; ++i) vload(vreg[i], vrs, i);

  for (int c = c_begin; c < c_end; ++c) {
    const int buf = c & 1;
    const int cn = min(c + 1, c_end - 1);  // next chunk (the last one repeats)
    const ChunkAddr anext = chunk_addr(p, b, cn);
#pragma unroll
    for (int i = 0; i < QPT; ++i) {
      const int x = tid + 256 * i;
      if (x < QN) Qs[buf][x / DK][x % DK] = qreg[i] * fast_exp2(preg[i] - rreg[i]) * p.qscale;
    }
    load_r(anext.anchor);
    __syncthreads();
    if (s_role) {
      const __amdgpu_buffer_rsrc_t krn = k_rsrc(anext, cn);
      const float4 qa = *reinterpret_cast<const float4 *>(&Qs[buf][sh][q_a]);
      const float4 qb = *reinterpret_cast<const float4 *>(&Qs[buf][sh][q_b]);
      float part[NKI];
#pragma unroll
      for (int i = 0; i < NKI; ++i) {
        float t = qa.x * kreg[i][0];
        t = fmaf(qa.y, kreg[i][1], t);
        t = fmaf(qa.z, kreg[i][2], t);
        t = fmaf(qa.w, kreg[i][3], t);
        t = fmaf(qb.x, kreg[i][4], t);
        t = fmaf(qb.y, kreg[i][5], t);
        t = fmaf(qb.z, kreg[i][6], t);
        t = fmaf(qb.w, kreg[i][7], t);
        part[i] = t;
        kload(kreg[i], krn, i);  // same piece of the next chunk
      }
      // sum each partial over the LPR lanes of its key row (rotations within
      // a 16-lane row; for 8-lane rows the rotation by 8 is skipped and the
      // two halves of a 16-lane row hold different keys)
#pragma unroll
      for (int i = 0; i < NKI; ++i) part[i] = row_sum<LPR>(part[i]);
      float s = part[0];
#pragma unroll
      for (int i = 1; i < NKI; ++i) s = ku == i ? part[i] : s;
      if (gate) {
        s += g_cur - gval;
        grs = g_rsrc(anext, cn);
        gval = gload(grs);
      }
      const int j = c * C + kk;
      if (j >= L || j < j_lo) s = -INFINITY;
      const float cm = wave_max(s);
      const float m_new = fmaxf(m_run, cm);  // finite: every visited chunk has a visible key
      const float pj = fast_exp2(s - m_new);
      const float alpha = fast_exp2(m_run - m_new);
      l_run = l_run * alpha + wave_sum(pj);
      m_run = m_new;
      Ps[buf][kk][sh] = pj;
      if (lane == 0) Al[buf][sh] = alpha;
    }
    __syncthreads();
    float al[NHB];
#pragma unroll
    for (int hh = 0; hh < NHB; ++hh) al[hh] = Al[buf][hh];
#pragma unroll
    for (int hh = 0; hh < NHB; ++hh)
#pragma unroll
      for (int e = 0; e < 8; ++e) oacc[hh][e] *= al[hh];
    const __amdgpu_buffer_rsrc_t vrn = v_rsrc(anext, cn);
#pragma unroll
    for (int i = 0; i < KPL; ++i) {
      const int key = kl + KL * i;
      float pp[NHB];
      if (NHB == 4) {
        const float4 p4 = *reinterpret_cast<const float4 *>(&Ps[buf][key][0]);
        pp[0] = p4.x; pp[1 % NHB] = p4.y; pp[2 % NHB] = p4.z; pp[3 % NHB] = p4.w;
      } else {
#pragma unroll
        for (int hh = 0; hh < NHB; ++hh) pp[hh] = Ps[buf][key][hh];
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float ve = vreg[i][e];
#pragma unroll
        for (int hh = 0; hh < NHB; ++hh) oacc[hh][e] = fmaf(pp[hh], ve, oacc[hh][e]);
      }
      vload(vreg[i], vrn, i);  // same piece of the next chunk
    }
  }

  // reduce partial outputs across key lanes
#pragma unroll
  for (int hh = 0; hh < NHB; ++hh)
#pragma unroll
    for (int e = 0; e < 8; ++e) red[kl][hh][cg * 8 + e] = oacc[hh][e];
  __syncthreads();
  for (int x = tid; x < NHB * DV; x += 256) {
    const int hh = x / DV, ch = x % DV;
    float acc = 0.f;
#pragma unroll
    for (int q2 = 0; q2 < KL; ++q2) acc += red[q2][hh][ch];
    p.part_o[(pbase + (int64_t)hh * p.nsplit) * DV + ch] = acc;
  }
  if (s_role && lane == 0) {
    p.part_ml[(pbase + (int64_t)sh * p.nsplit) * 2 + 0] = m_run;
    p.part_ml[(pbase + (int64_t)sh * p.nsplit) * 2 + 1] = l_run;
  }
}

// grid (B*HQ), DV threads: merge the splits, add the sink, normalise.  A row
// with no visible key (length 0) gets o = 0 and lse = the sink logit, or
// -inf without a sink.
template <typename TE, int DV>
__global__ __launch_bounds__(128) void k_decode_combine(const float *__restrict__ part_o,
                                                        const float *__restrict__ part_ml,
                                                        const float *__restrict__ sink,
                                                        TE *__restrict__ o,
                                                        float *__restrict__ lse, int HQ,
                                                        int nsplit) {
  const int bh = blockIdx.x, hq = bh % HQ, ch = threadIdx.x;
  const float *ml = part_ml + (int64_t)bh * nsplit * 2;
  float M = -INFINITY;
  for (int s = 0; s < nsplit; ++s) M = fmaxf(M, ml[2 * s]);
  float s2 = 0.f;
  if (sink != nullptr) {
    s2 = sink[hq] * LOG2E;
    M = fmaxf(M, s2);
  }
  if (M == -INFINITY) {
    if (ch < DV) Elem<TE>::st(o + (int64_t)bh * DV + ch, 0.f);
    if (lse != nullptr && ch == 0) lse[bh] = -INFINITY;
    return;
  }
  float Z = sink != nullptr ? fast_exp2(s2 - M) : 0.f;
  float acc = 0.f;
  const float *po = part_o + (int64_t)bh * nsplit * DV + ch;
  for (int s = 0; s < nsplit; ++s) {
    const float w = fast_exp2(ml[2 * s] - M);
    Z += ml[2 * s + 1] * w;
    acc += po[(int64_t)s * DV] * w;
  }
  if (ch < DV) Elem<TE>::st(o + (int64_t)bh * DV + ch, acc / Z);
  if (lse != nullptr && ch == 0) lse[bh] = (M + log2f(Z)) * LN2;
}

int heads_per_block(int64_t HQ, int64_t H) {
  const int64_t group = HQ / H;
  return group % 4 == 0 ? 4 : group % 2 == 0 ? 2 : 1;
}

template <typename TE, typename TK, int DK, int DV, int NHB>
hipError_t decode_t(const DecodeParams &p, const float *sink, void *o, float *lse, int64_t B,
                    hipStream_t st) {
  const dim3 grid((unsigned)p.nsplit, (unsigned)(p.HQ / NHB), (unsigned)B);
  if (p.gs_cache != nullptr)
    hipLaunchKernelGGL((k_decode_split<TE, TK, DK, DV, NHB, true>), grid, dim3(256), 0, st, p);
  else
    hipLaunchKernelGGL((k_decode_split<TE, TK, DK, DV, NHB, false>), grid, dim3(256), 0, st, p);
  hipLaunchKernelGGL((k_decode_combine<TE, DV>), dim3((unsigned)(B * p.HQ)), dim3(DV), 0, st,
                     p.part_o, p.part_ml, sink, static_cast<TE *>(o), lse, p.HQ, p.nsplit);
  return hipGetLastError();
}

template <typename TE, typename TK, int DK, int DV>
hipError_t decode_heads(const DecodeParams &p, const float *sink, void *o, float *lse, int64_t B,
                        hipStream_t st) {
  switch (heads_per_block(p.HQ, p.H)) {
    case 4: return decode_t<TE, TK, DK, DV, 4>(p, sink, o, lse, B, st);
    case 2: return decode_t<TE, TK, DK, DV, 2>(p, sink, o, lse, B, st);
    default: return decode_t<TE, TK, DK, DV, 1>(p, sink, o, lse, B, st);
  }
}

template <typename TE, typename TK>
hipError_t decode_dims(const DecodeParams &p, int64_t K, int64_t V, const float *sink, void *o,
                       float *lse, int64_t B, hipStream_t st) {
  if (K == 64) return V == 64 ? decode_heads<TE, TK, 64, 64>(p, sink, o, lse, B, st)
                              : decode_heads<TE, TK, 64, 128>(p, sink, o, lse, B, st);
  return V == 64 ? decode_heads<TE, TK, 128, 64>(p, sink, o, lse, B, st)
                 : decode_heads<TE, TK, 128, 128>(p, sink, o, lse, B, st);
}

}  // namespace
}  // namespace dec

// Launch of the split and combine kernels for one cache element type
// (instantiated in decode_cache_<type>.hip).
template <typename TK>
hipError_t launch_decode_cache(const DecodeParams &p, int dtype, int64_t K, int64_t V,
                               const float *sink, void *o, float *lse, int64_t B, hipStream_t st) {
  if (dtype == WA_DT_BF16) return dec::decode_dims<bf16_t, TK>(p, K, V, sink, o, lse, B, st);
  return dec::decode_dims<float, TK>(p, K, V, sink, o, lse, B, st);
}

}  // namespace wa

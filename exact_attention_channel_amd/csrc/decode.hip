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
#include <math.h>

#include "common.h"
#include "launch.h"

namespace wa {
namespace {

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *p, int64_t bytes) {
  // integer select: HIP's min() on 64-bit integers goes through f64 VALU code
  const int n = bytes > 0x7fffffff ? 0x7fffffff : (int)bytes;
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(p), 0, n, 0x00020000);
}
__device__ __forceinline__ u32x4 buf_load16(__amdgpu_buffer_rsrc_t rs, int voff, int soff) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, voff, soff, 0));
}

template <typename TE>
struct Vec8;  // 8 consecutive elements in registers
template <>
struct Vec8<bf16_t> {
  u32x4 w;
  __device__ __forceinline__ void load(const bf16_t *p) { w = *reinterpret_cast<const u32x4 *>(p); }
  __device__ __forceinline__ void zero() { w = u32x4{0, 0, 0, 0}; }
  __device__ __forceinline__ float operator[](int e) const {
    return (e & 1) ? bf16_hi(w[e >> 1]) : bf16_lo(w[e >> 1]);
  }
};
template <>
struct Vec8<_Float16> {
  u32x4 w;
  __device__ __forceinline__ void load(const _Float16 *p) { w = *reinterpret_cast<const u32x4 *>(p); }
  __device__ __forceinline__ void load(__amdgpu_buffer_rsrc_t rs, int voff, int soff) {
    w = buf_load16(rs, voff, soff);
  }
  __device__ __forceinline__ void zero() { w = u32x4{0, 0, 0, 0}; }
  __device__ __forceinline__ float operator[](int e) const {
    return (e & 1) ? f16_hi(w[e >> 1]) : f16_lo(w[e >> 1]);
  }
};
template <>
struct Vec8<float> {
  float4 a, b;
  __device__ __forceinline__ void load(const float *p) {
    a = *reinterpret_cast<const float4 *>(p);
    b = *reinterpret_cast<const float4 *>(p + 4);
  }
  __device__ __forceinline__ void load(__amdgpu_buffer_rsrc_t rs, int voff, int soff) {
    a = __builtin_bit_cast(float4, buf_load16(rs, voff, soff));
    b = __builtin_bit_cast(float4, buf_load16(rs, voff + 16, soff));
  }
  __device__ __forceinline__ void zero() { a = b = make_float4(0.f, 0.f, 0.f, 0.f); }
  __device__ __forceinline__ float operator[](int e) const {
    const float4 &x = e < 4 ? a : b;
    const int i = e & 3;
    return i == 0 ? x.x : i == 1 ? x.y : i == 2 ? x.z : x.w;
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

// grid (nsplit, HQ/NHB, B), 256 threads.  The cache holds k_tilde in the
// operand type TK (IEEE half for bf16 inputs).
//
// Memory-level parallelism: every 16-byte piece of the next chunk's keys and
// values is requested as soon as the same piece of the current chunk has been
// consumed, so one register set holds both the data in use and the data in
// flight (about one chunk ahead) and the kernel runs three workgroups per CU.
template <typename TE, int DK, int DV, int NHB, typename TK = typename OperandOf<TE>::type>
__global__ __launch_bounds__(256, 3) void k_decode_split(
    const TE *__restrict__ q, const TE *__restrict__ v, const float *__restrict__ p_curr,
    const TK *__restrict__ kt, const float *__restrict__ rc, float *__restrict__ part_o,
    float *__restrict__ part_ml, int64_t T, int HQ, int H, int NC, int nsplit, int cps,
    float qscale) {
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

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int split = blockIdx.x, hq0 = blockIdx.y * NHB, b = blockIdx.z;
  const int h = hq0 / (HQ / H);
  const int c_begin = split * cps, c_end = min(NC, c_begin + cps);
  const int64_t tb = (int64_t)b * T;

  // rescaling inputs: q and p_curr per (head, channel) owned by this thread
  float qreg[QPT], preg[QPT], rreg[QPT];
#pragma unroll
  for (int i = 0; i < QPT; ++i) {
    const int x = tid + 256 * i;
    const int hh = x / DK, n = x % DK;
    qreg[i] = x < QN ? Elem<TE>::ld(q + ((int64_t)b * HQ + hq0 + hh) * DK + n) : 0.f;
    preg[i] = x < QN ? p_curr[((int64_t)b * HQ + hq0 + hh) * DK + n] : 0.f;
  }
  auto load_r = [&](int c) {
#pragma unroll
    for (int i = 0; i < QPT; ++i) {
      const int x = tid + 256 * i;
      const int hh = x / DK, n = x % DK;
      rreg[i] = x < QN ? rc[(((int64_t)b * NC + c) * HQ + hq0 + hh) * DK + n] : 0.f;
    }
  };

  // score role: head sh = wave.  Load i of a chunk brings keys 4 i + r
  // (r = lane / 16), lane u = lane % 16 holding channels 8u .. 8u+7 of its
  // key: each load instruction covers four whole 256-byte key rows.  The
  // partial dot products are summed over the 16 lanes of a row, and lane
  // (r, u) then owns key kk = 4u + r.  Key rows come through a buffer
  // resource over this batch row and head (lane offset plus a scalar row
  // offset per load); rows past T_kv read zero and are masked.
  static_assert(DK == 128 || DK == 64, "key rows of 16 or 8 pieces");
  constexpr int LPR = DK / 8;         // lanes per key row
  constexpr int RPI = 64 / LPR;       // key rows per load instruction
  constexpr int NKI = C / RPI;        // load instructions per chunk
  const int sh = wave, kr = lane / LPR, ku = lane % LPR;
  const int kk = RPI * ku + kr;       // the key whose score this lane keeps (NKI == LPR)
  static_assert(NKI == LPR, "one reduced score per lane");
  const bool s_role = sh < NHB;
  const __amdgpu_buffer_rsrc_t kt_rs =
      make_rsrc(kt + (tb * HQ + hq0 + (s_role ? sh : 0)) * DK, T * HQ * DK * (int64_t)sizeof(TK));
  const int k_voff = (kr * HQ * DK + 8 * ku) * (int)sizeof(TK);
  auto kload = [&](Vec8<TK> &r, int c, int i) {
    r.load(kt_rs, k_voff, (c * C + RPI * i) * HQ * DK * (int)sizeof(TK));
  };
  Vec8<TK> kreg[NKI];

  // PV role: channel group cg, key lane kl
  const int cg = tid % VCG, kl = tid / VCG;
  const TE *v_row = v + (tb * H + h) * DV + cg * 8;
  auto vptr = [&](int c, int i) {
    const int64_t j = min((int64_t)c * C + kl + KL * i, T - 1);
    return v_row + j * H * DV;
  };
  Vec8<TE> vreg[KPL];

  float m_run = -INFINITY, l_run = 0.f;  // per score wave (its head)
  float oacc[NHB][8];
#pragma unroll
  for (int hh = 0; hh < NHB; ++hh)
#pragma unroll
    for (int e = 0; e < 8; ++e) oacc[hh][e] = 0.f;

  load_r(c_begin);
  if (s_role) {
#pragma unroll
    for (int i = 0; i < NKI; ++i) kload(kreg[i], c_begin, i);
  }
#pragma unroll
  for (int i = 0; i < KPL; ++i) vreg[i].load(vptr(c_begin, i));

  for (int c = c_begin; c < c_end; ++c) {
    const int buf = c & 1;
    const int cn = min(c + 1, c_end - 1);  // next chunk (the last one repeats)
#pragma unroll
    for (int i = 0; i < QPT; ++i) {
      const int x = tid + 256 * i;
      if (x < QN) Qs[buf][x / DK][x % DK] = qreg[i] * fast_exp2(preg[i] - rreg[i]) * qscale;
    }
    load_r(cn);
    __syncthreads();
    if (s_role) {
      const float4 qa = *reinterpret_cast<const float4 *>(&Qs[buf][sh][8 * ku]);
      const float4 qb = *reinterpret_cast<const float4 *>(&Qs[buf][sh][8 * ku + 4]);
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
        kload(kreg[i], cn, i);  // same piece of the next chunk
      }
      // sum each partial over the LPR lanes of its key row (rotations within
      // a 16-lane row; for 8-lane rows the rotation by 8 is skipped and the
      // two halves of a 16-lane row hold different keys)
#pragma unroll
      for (int i = 0; i < NKI; ++i) part[i] = row_sum<LPR>(part[i]);
      float s = part[0];
#pragma unroll
      for (int i = 1; i < NKI; ++i) s = ku == i ? part[i] : s;
      if ((int64_t)c * C + kk >= T) s = -INFINITY;
      const float cm = wave_max(s);
      const float m_new = fmaxf(m_run, cm);  // finite: every chunk has a valid key
      const float p = fast_exp2(s - m_new);
      const float alpha = fast_exp2(m_run - m_new);
      l_run = l_run * alpha + wave_sum(p);
      m_run = m_new;
      Ps[buf][kk][sh] = p;
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
      vreg[i].load(vptr(cn, i));  // same piece of the next chunk
    }
  }

  // reduce partial outputs across key lanes
#pragma unroll
  for (int hh = 0; hh < NHB; ++hh)
#pragma unroll
    for (int e = 0; e < 8; ++e) red[kl][hh][cg * 8 + e] = oacc[hh][e];
  __syncthreads();
  const int64_t pbase = ((int64_t)b * HQ + hq0) * nsplit + split;
  for (int x = tid; x < NHB * DV; x += 256) {
    const int hh = x / DV, ch = x % DV;
    float acc = 0.f;
#pragma unroll
    for (int q2 = 0; q2 < KL; ++q2) acc += red[q2][hh][ch];
    part_o[(pbase + (int64_t)hh * nsplit) * DV + ch] = acc;
  }
  if (s_role && lane == 0) {
    part_ml[(pbase + (int64_t)sh * nsplit) * 2 + 0] = m_run;
    part_ml[(pbase + (int64_t)sh * nsplit) * 2 + 1] = l_run;
  }
}

// grid (B*HQ), DV threads: merge the splits, add the sink, normalise.
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

template <typename TE, int DK, int DV, int NHB>
hipError_t decode_t(const DecodeProblem &p, float *part_o, float *part_ml, int nsplit, int cps,
                    hipStream_t st) {
  const int NC = (int)((p.T + CHUNK - 1) / CHUNK);
  const dim3 grid((unsigned)nsplit, (unsigned)(p.HQ / NHB), (unsigned)p.B);
  hipLaunchKernelGGL((k_decode_split<TE, DK, DV, NHB>), grid, dim3(256), 0, st,
                     static_cast<const TE *>(p.q), static_cast<const TE *>(p.v), p.p_curr,
                     static_cast<const typename OperandOf<TE>::type *>(p.kt), p.rc, part_o,
                     part_ml, p.T, (int)p.HQ,
                     (int)p.H, NC, nsplit, cps, p.scale * LOG2E);
  hipLaunchKernelGGL((k_decode_combine<TE, DV>), dim3((unsigned)(p.B * p.HQ)), dim3(DV), 0, st,
                     part_o, part_ml, p.sink, static_cast<TE *>(p.o), p.lse, (int)p.HQ, nsplit);
  return hipGetLastError();
}

template <typename TE, int DK, int DV>
hipError_t decode_heads(const DecodeProblem &p, float *po, float *pml, int ns, int cps,
                        hipStream_t st) {
  switch (heads_per_block(p.HQ, p.H)) {
    case 4: return decode_t<TE, DK, DV, 4>(p, po, pml, ns, cps, st);
    case 2: return decode_t<TE, DK, DV, 2>(p, po, pml, ns, cps, st);
    default: return decode_t<TE, DK, DV, 1>(p, po, pml, ns, cps, st);
  }
}

template <typename TE>
hipError_t decode_dims(const DecodeProblem &p, float *po, float *pml, int ns, int cps,
                       hipStream_t st) {
  if (p.K == 64) return p.V == 64 ? decode_heads<TE, 64, 64>(p, po, pml, ns, cps, st)
                                  : decode_heads<TE, 64, 128>(p, po, pml, ns, cps, st);
  return p.V == 64 ? decode_heads<TE, 128, 64>(p, po, pml, ns, cps, st)
                   : decode_heads<TE, 128, 128>(p, po, pml, ns, cps, st);
}

}  // namespace

void decode_split_plan(int64_t B, int64_t T, int64_t HQ, int64_t H, int *nsplit,
                       int *chunks_per_split) {
  const int64_t NC = (T + CHUNK - 1) / CHUNK;
  const int64_t units = B * (HQ / heads_per_block(HQ, H));
  const int64_t target = 256 * 3 * 8;  // eight full waves of 3 resident workgroups per CU
  int64_t ns = (target + units - 1) / units;
  ns = ns < 1 ? 1 : (ns > NC ? NC : ns);
  const int64_t cps = (NC + ns - 1) / ns;
  ns = (NC + cps - 1) / cps;
  *nsplit = (int)ns;
  *chunks_per_split = (int)cps;
}

size_t decode_workspace_size(int64_t B, int64_t T, int64_t HQ, int64_t H, int64_t V) {
  int ns, cps;
  decode_split_plan(B, T, HQ, H, &ns, &cps);
  const size_t po = sizeof(float) * (size_t)(B * HQ * ns * V);
  const size_t pml = sizeof(float) * (size_t)(B * HQ * ns * 2);
  return ((po + 255) & ~size_t(255)) + ((pml + 255) & ~size_t(255));
}

hipError_t launch_decode(const DecodeProblem &p, void *ws, hipStream_t st) {
  int ns, cps;
  decode_split_plan(p.B, p.T, p.HQ, p.H, &ns, &cps);
  float *po = static_cast<float *>(ws);
  const size_t pob = sizeof(float) * (size_t)(p.B * p.HQ * ns * p.V);
  float *pml = reinterpret_cast<float *>(static_cast<char *>(ws) + ((pob + 255) & ~size_t(255)));
  if (p.dtype == 0) return decode_dims<bf16_t>(p, po, pml, ns, cps, st);
  return decode_dims<float>(p, po, pml, ns, cps, st);
}

}  // namespace wa

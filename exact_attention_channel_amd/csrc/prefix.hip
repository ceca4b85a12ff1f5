// Running decay sums, chunk anchors and rescaled operands (the pre-pass of
// the prefill and the decode-cache build).
//
// Wall Attention README, "Decode": the prefix P of g is taken in log2 units
// (scale 1/ln 2), and per-chunk anchors R_c fold the decay into the keys,
// k_tilde[j] = k[j] * 2^(R_c - P[j]), keeping every exp2 argument bounded
// ("Features": numerically stable long context).  The same factorisation
// serves the prefill: for query i in query tile I and key j in key chunk J,
//   exp(P_i - P_j) = 2^(P2_i - RQ_I) * 2^(RQ_I - R_J) * 2^(R_J - P2_j)
// exactly, so this pass writes q_hat_i = q_i * 2^(P2_i - RQ_I) * scale/ln2 and
// k_tilde_j = k_j * 2^(R_J - P2_j) once per token, and the attention kernel
// applies the K factors 2^(RQ_I - R_J) once per (query tile, key chunk) pair.
//
// The running sum along time is a three-phase chunked scan:
//   A: per-chunk channel sums,  B: exclusive scan over chunks,  C: in-chunk
//   inclusive sums plus the operand rescaling.
#include <type_traits>

#include "common.h"
#include "launch.h"

namespace wa {

namespace {

// N consecutive channels as floats; the pre-pass moves 16 bytes of its input
// type per access (CPT = 8 bfloat16 or 4 float channels per thread).
template <typename TE> constexpr int cpt() { return 16 / (int)sizeof(TE); }
template <int N> struct FV {
  float v[N];
};
template <int N> __device__ __forceinline__ FV<N> zerov() {
  FV<N> r;
#pragma unroll
  for (int j = 0; j < N; ++j) r.v[j] = 0.f;
  return r;
}
template <typename TE, int N> __device__ __forceinline__ FV<N> loadv(const TE *p);
template <> __device__ __forceinline__ FV<8> loadv<bf16_t, 8>(const bf16_t *p) {
  const u32x4 w = *reinterpret_cast<const u32x4 *>(p);
  FV<8> r;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    r.v[2 * j] = bf16_lo(w[j]);
    r.v[2 * j + 1] = bf16_hi(w[j]);
  }
  return r;
}
template <> __device__ __forceinline__ FV<4> loadv<float, 4>(const float *p) {
  const float4 x = *reinterpret_cast<const float4 *>(p);
  return FV<4>{{x.x, x.y, x.z, x.w}};
}
template <> __device__ __forceinline__ FV<8> loadv<float, 8>(const float *p) {
  const float4 x = reinterpret_cast<const float4 *>(p)[0], y = reinterpret_cast<const float4 *>(p)[1];
  return FV<8>{{x.x, x.y, x.z, x.w, y.x, y.y, y.z, y.w}};
}
template <typename TO, int N> __device__ __forceinline__ void storev(TO *p, const FV<N> &x);
template <> __device__ __forceinline__ void storev<_Float16, 8>(_Float16 *p, const FV<8> &x) {
  u32x4 w;
#pragma unroll
  for (int j = 0; j < 4; ++j) w[j] = pack_f16x2(x.v[2 * j], x.v[2 * j + 1]);
  *reinterpret_cast<u32x4 *>(p) = w;
}
template <> __device__ __forceinline__ void storev<float, 4>(float *p, const FV<4> &x) {
  *reinterpret_cast<float4 *>(p) = make_float4(x.v[0], x.v[1], x.v[2], x.v[3]);
}
template <> __device__ __forceinline__ void storev<float, 8>(float *p, const FV<8> &x) {
  reinterpret_cast<float4 *>(p)[0] = make_float4(x.v[0], x.v[1], x.v[2], x.v[3]);
  reinterpret_cast<float4 *>(p)[1] = make_float4(x.v[4], x.v[5], x.v[6], x.v[7]);
}

// Workgroup x of a per-(chunk, query head) grid -> (hq, c); false for the
// padding workgroups.  Two orders, chosen on the host by grid size:
//  * chunk order (c fastest): for a grid the GPU holds at once; whole chunks
//    of every head then share an XCD (workgroups go to the 8 XCDs round
//    robin), which measured fastest for one 8K-token sequence;
//  * pair order: pairs p = (key/value head h, chunk c) with h fastest, the
//    G query heads of a pair on one XCD (they read the pair's key rows
//    through one L2), so that a grid that runs in many waves keeps the rows
//    in flight together (16 packed sequences: phase C 222 -> 194 us).
struct ChunkGrid {
  int H, G, NC, pair;
  __device__ __forceinline__ bool map(int x, int &hq, int &c) const {
    if (!pair) {
      c = x % NC;
      hq = x / NC;
      return true;
    }
    const int r = x >> 3, g = r % G, pr = 8 * (r / G) + (x & 7);
    c = pr / H;
    hq = (pr % H) * G + g;
    return c < NC;
  }
  unsigned size() const {
    return (unsigned)(pair ? 8 * (int64_t)G * (((int64_t)H * NC + 7) / 8) : (int64_t)H * G * NC);
  }
};
// nrep: the grid's second dimension (segments or batch rows)
inline ChunkGrid chunk_grid(int64_t H, int64_t G, int64_t NC, int64_t nrep) {
  constexpr int64_t RESIDENT = 256 * 8;  // 256-thread workgroups the GPU holds at once
  return ChunkGrid{(int)H, (int)G, (int)NC, H * G * NC * nrep > 2 * RESIDENT ? 1 : 0};
}

__device__ __forceinline__ float wave_inclusive_scan(float x) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    float y = __shfl_up(x, d);
    if (lane >= d) x += y;
  }
  return x;
}

// Phase A: sum of g (per channel) and of g_scalar over each chunk.
// grid (cg.size(), nseg), 256 threads; a thread owns CPT channels.
template <typename TE, int KD>
__global__ __launch_bounds__(256) void k_chunk_sums(const TE *__restrict__ g,
                                                    const TE *__restrict__ gs,
                                                    float *__restrict__ csum,
                                                    float *__restrict__ csum_s,
                                                    const int32_t *__restrict__ cu, int64_t T,
                                                    int HQ, int NCmax, ChunkGrid cg) {
  int hq, c;
  if (!cg.map(blockIdx.x, hq, c)) return;
  const int s = blockIdx.y;
  int64_t bos, eos;
  segment_bounds(s, T, cu, bos, eos);
  const int64_t r0 = bos + (int64_t)c * CHUNK;
  if (r0 >= eos) return;
  const int nrow = (eos - r0) < CHUNK ? (int)(eos - r0) : CHUNK;
  constexpr int CPT = cpt<TE>(), NQ = KD / CPT, NG = 256 / NQ;
  const int cgi = threadIdx.x % NQ, grp = threadIdx.x / NQ;
  // compile-time row count with a guard: the thread's loads go out together
  FV<CPT> xs[CHUNK / NG];
#pragma unroll
  for (int i = 0; i < CHUNK / NG; ++i) {
    const int r = grp + i * NG;
    xs[i] = r < nrow ? loadv<TE, CPT>(g + ((r0 + r) * HQ + hq) * KD + CPT * cgi) : zerov<CPT>();
  }
  FV<CPT> acc = zerov<CPT>();
#pragma unroll
  for (int i = 0; i < CHUNK / NG; ++i)
#pragma unroll
    for (int j = 0; j < CPT; ++j) acc.v[j] += xs[i].v[j];
  __shared__ FV<CPT> red[NG][NQ];
  red[grp][cgi] = acc;
  __syncthreads();
  const int64_t cidx = (int64_t)s * NCmax + c;
  if (grp == 0) {
#pragma unroll
    for (int q = 1; q < NG; ++q)
#pragma unroll
      for (int j = 0; j < CPT; ++j) acc.v[j] += red[q][cgi].v[j];
    storev<float, CPT>(csum + (cidx * HQ + hq) * KD + CPT * cgi, acc);
  }
  if (gs != nullptr && threadIdx.x < 64) {
    float a = (int)threadIdx.x < nrow ? Elem<TE>::ld(gs + (r0 + threadIdx.x) * HQ + hq) : 0.f;
    a = wave_sum(a);
    if (threadIdx.x == 0) csum_s[cidx * HQ + hq] = a;
  }
}

// Phase B: exclusive scan of the chunk sums along time (in place), and the
// chunk anchors anch[c] = the integer nearest to P2 at the chunk's last token,
// (offset + sum of chunk c) * log2(e).  Any anchor cancels in the score; an
// integer one makes every tile-pair factor 2^(RQ_I - R_J) an exact power of
// two, applied without rounding.  Channel index KD stands for g_scalar.
// grid (HQ, nseg, ceil((KD+1)/32)), 256 threads = 32 channels x 8 chunk groups.
template <int KD>
__global__ __launch_bounds__(256) void k_chunk_scan(float *__restrict__ csum,
                                                    float *__restrict__ anch,
                                                    float *__restrict__ csum_s,
                                                    const int32_t *__restrict__ cu, int64_t T,
                                                    int HQ, int NCmax, int with_gs) {
  const int hq = blockIdx.x, s = blockIdx.y;
  const int ch = blockIdx.z * 32 + (threadIdx.x & 31);
  const int grp = threadIdx.x >> 5;
  int64_t bos, eos;
  segment_bounds(s, T, cu, bos, eos);
  const int nch = (int)((eos - bos + CHUNK - 1) / CHUNK);
  const bool active = ch < KD || (ch == KD && with_gs);
  const int span = (nch + 7) / 8;
  const int cb = grp * span, ce = min(nch, cb + span);
  float *p;
  int64_t stride;
  const int64_t c0 = (int64_t)s * NCmax;
  if (ch < KD) {
    p = csum + (c0 * HQ + hq) * KD + ch;
    stride = (int64_t)HQ * KD;
  } else {
    p = csum_s + c0 * HQ + hq;
    stride = HQ;
  }
  // the chunk sums are read in batches of 8 independent loads: one memory
  // round trip per batch instead of one per chunk; up to MAXS chunks per
  // thread (sequences up to 8192 tokens) stay in registers for the second
  // pass, so the whole scan is one round trip
  constexpr int MAXS = 16;
  const bool in_regs = span <= MAXS;
  float xs[MAXS];
  float tot = 0.f;
  if (active) {
    if (in_regs) {
#pragma unroll
      for (int u = 0; u < MAXS; ++u) xs[u] = cb + u < ce ? p[(int64_t)(cb + u) * stride] : 0.f;
#pragma unroll
      for (int u = 0; u < MAXS; ++u) tot += xs[u];
    } else {
      for (int c = cb; c < ce; c += 8) {
        float x[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) x[u] = c + u < ce ? p[(int64_t)(c + u) * stride] : 0.f;
#pragma unroll
        for (int u = 0; u < 8; ++u) tot += x[u];
      }
    }
  }
  __shared__ float part[8][32];
  part[grp][threadIdx.x & 31] = tot;
  __syncthreads();
  if (!active) return;
  float run = 0.f;
  for (int q = 0; q < grp; ++q) run += part[q][threadIdx.x & 31];
  float *a = anch + (c0 * HQ + hq) * KD + ch;
  if (in_regs) {
#pragma unroll
    for (int u = 0; u < MAXS; ++u) {
      if (cb + u < ce) {
        p[(int64_t)(cb + u) * stride] = run;
        if (ch < KD) a[(int64_t)(cb + u) * stride] = rintf((run + xs[u]) * LOG2E);
      }
      run += xs[u];
    }
    return;
  }
  for (int c = cb; c < ce; c += 8) {
    float x[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) x[u] = c + u < ce ? p[(int64_t)(c + u) * stride] : 0.f;
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      if (c + u < ce) {
        p[(int64_t)(c + u) * stride] = run;
        if (ch < KD) a[(int64_t)(c + u) * stride] = rintf((run + x[u]) * LOG2E);
      }
      run += x[u];
    }
  }
}

// In-chunk running sums of g for CPT channels of one chunk (shared by the two
// phase-C kernels): rows are split into NG groups of RPG consecutive rows;
// each thread scans its group, the group totals go through LDS.  Returns in
// p2[i] the running sum at row grp*RPG + i in log2 units (offset included).
template <typename TE, int KD>
struct ChunkScan {
  static constexpr int CPT = cpt<TE>(), NQ = KD / CPT, NG = 256 / NQ, RPG = CHUNK / NG;
  __device__ __forceinline__ static void run(const TE *g, int64_t r0, int nrow, int HQ, int hq,
                                             int cgi, int grp, FV<CPT> base, FV<CPT> (&p2)[RPG]) {
    __shared__ FV<CPT> tot[NG][NQ];
#pragma unroll
    for (int i = 0; i < RPG; ++i) {
      const int r = grp * RPG + i;
      p2[i] = r < nrow ? loadv<TE, CPT>(g + ((r0 + r) * HQ + hq) * KD + CPT * cgi) : zerov<CPT>();
      if (i > 0)
#pragma unroll
        for (int j = 0; j < CPT; ++j) p2[i].v[j] += p2[i - 1].v[j];
    }
    tot[grp][cgi] = p2[RPG - 1];
    __syncthreads();
    for (int q = 0; q < grp; ++q)
#pragma unroll
      for (int j = 0; j < CPT; ++j) base.v[j] += tot[q][cgi].v[j];
#pragma unroll
    for (int i = 0; i < RPG; ++i)
#pragma unroll
      for (int j = 0; j < CPT; ++j) p2[i].v[j] = (base.v[j] + p2[i].v[j]) * LOG2E;
  }
};

// Phase C for the prefill: in-chunk running sums, then
//   q_hat = q * 2^(P2 - RQ) * qscale   (RQ: anchor of the first chunk of the
//                                       128-row query tile, so |P2 - RQ| is
//                                       at most one chunk's decay span;
//                                       float operands only: for half
//                                       operands the attention kernel forms
//                                       q_hat from q, g and the chunk offsets)
//   k_tilde = k * 2^(R_c - P2)         (R_c: anchor of this 64-token chunk)
// written in the operand type (IEEE half for bf16 inputs, float for fp32).
//   gsum = running sum of g_scalar in log2 units.
// Half operands (bf16 inputs): k_tilde is stored head-major, [HQ, ntok, KD+16],
// each row followed by 16 extra channels [1, 1, -G hi, -G lo, 0 ...] (G =
// gsum of the token split into two halves, 0 without a gate), so a key tile
// is one contiguous block and the attention kernel's score product also
// subtracts the row shift and the gate.  Float operands keep [ntok, HQ, KD].
// grid (cg.size(), nseg), 256 threads; a thread owns CPT channels.
template <typename TE, int KD, typename TO = typename OperandOf<TE>::type>
__global__ __launch_bounds__(256) void k_prefill_operands(
    const TE *__restrict__ q, const TE *__restrict__ k, const TE *__restrict__ g,
    const TE *__restrict__ gs, const float *__restrict__ off, const float *__restrict__ anch,
    const float *__restrict__ off_s, TO *__restrict__ qh, TO *__restrict__ kt,
    float *__restrict__ gsum, const int32_t *__restrict__ cu, int64_t T, int64_t ntok, int HQ,
    int H, int NCmax, float qscale, ChunkGrid cg) {
  constexpr bool HM = std::is_same<TO, _Float16>::value;  // head-major rows with extras
  constexpr int KX = HM ? KD + 16 : KD;
  int hq, c;
  if (!cg.map(blockIdx.x, hq, c)) return;
  const int s = blockIdx.y;
  int64_t bos, eos;
  segment_bounds(s, T, cu, bos, eos);
  const int64_t r0 = bos + (int64_t)c * CHUNK;
  if (r0 >= eos) return;
  const int nrow = (eos - r0) < CHUNK ? (int)(eos - r0) : CHUNK;
  const int h = hq / (HQ / H);
  typedef ChunkScan<TE, KD> CS;
  constexpr int CPT = CS::CPT;
  const int cgi = threadIdx.x % CS::NQ, grp = threadIdx.x / CS::NQ;
  const int64_t cidx = (int64_t)s * NCmax + c;
  const FV<CPT> base = loadv<float, CPT>(off + (cidx * HQ + hq) * KD + CPT * cgi);
  const FV<CPT> A = loadv<float, CPT>(anch + (cidx * HQ + hq) * KD + CPT * cgi);
  FV<CPT> p2[CS::RPG];
  CS::run(g, r0, nrow, HQ, hq, cgi, grp, base, p2);
#pragma unroll
  for (int i = 0; i < CS::RPG; ++i) {
    const int r = grp * CS::RPG + i;
    if (r < nrow) {
      const int64_t t = r0 + r;
      if (!HM) {  // half operands: the attention kernel forms q_hat itself
        const int64_t cq = (int64_t)s * NCmax + (c & ~1);
        const FV<CPT> RQ = loadv<float, CPT>(anch + (cq * HQ + hq) * KD + CPT * cgi);
        const FV<CPT> qv = loadv<TE, CPT>(q + (t * HQ + hq) * KD + CPT * cgi);
        FV<CPT> qo;
#pragma unroll
        for (int j = 0; j < CPT; ++j) qo.v[j] = qv.v[j] * fast_exp2(p2[i].v[j] - RQ.v[j]) * qscale;
        storev<TO, CPT>(qh + (t * HQ + hq) * KD + CPT * cgi, qo);
      }
      const FV<CPT> kv = loadv<TE, CPT>(k + (t * H + h) * KD + CPT * cgi);
      FV<CPT> ko;
#pragma unroll
      for (int j = 0; j < CPT; ++j) ko.v[j] = kv.v[j] * fast_exp2(A.v[j] - p2[i].v[j]);
      storev<TO, CPT>(kt + (HM ? (hq * ntok + t) : (t * HQ + hq)) * KX + CPT * cgi, ko);
    }
  }
  if (threadIdx.x < 64) {
    const int r = threadIdx.x;
    float G = 0.f;
    if (gs != nullptr) {
      float x = r < nrow ? Elem<TE>::ld(gs + (r0 + r) * HQ + hq) : 0.f;
      x = wave_inclusive_scan(x);
      G = (off_s[cidx * HQ + hq] + x) * LOG2E;
      if (r < nrow) gsum[(r0 + r) * HQ + hq] = G;
    }
    if (HM && r < nrow) {
      const _Float16 gh = (_Float16)(-G);
      u32x4 x0 = u32x4{pack_f16x2(1.f, 1.f), pack_f16x2((float)gh, -G - (float)gh), 0u, 0u};
      u32x4 *dst = reinterpret_cast<u32x4 *>(kt + (hq * ntok + r0 + r) * KX + KD);
      dst[0] = x0;
      dst[1] = u32x4{0u, 0u, 0u, 0u};
    }
  }
}

// Phase C for the stand-alone prefix: P2 = (offset + in-chunk sum) * log2(e).
template <typename TE, int KD>
__global__ __launch_bounds__(256) void k_prefix_write(const TE *__restrict__ g,
                                                      const float *__restrict__ off,
                                                      float *__restrict__ P2,
                                                      const int32_t *__restrict__ cu, int64_t T,
                                                      int HQ, int NCmax, ChunkGrid cg) {
  int hq, c;
  if (!cg.map(blockIdx.x, hq, c)) return;
  const int s = blockIdx.y;
  int64_t bos, eos;
  segment_bounds(s, T, cu, bos, eos);
  const int64_t r0 = bos + (int64_t)c * CHUNK;
  if (r0 >= eos) return;
  const int nrow = (eos - r0) < CHUNK ? (int)(eos - r0) : CHUNK;
  typedef ChunkScan<TE, KD> CS;
  constexpr int CPT = CS::CPT;
  const int cgi = threadIdx.x % CS::NQ, grp = threadIdx.x / CS::NQ;
  const int64_t cidx = (int64_t)s * NCmax + c;
  const FV<CPT> base = loadv<float, CPT>(off + (cidx * HQ + hq) * KD + CPT * cgi);
  FV<CPT> p2[CS::RPG];
  CS::run(g, r0, nrow, HQ, hq, cgi, grp, base, p2);
#pragma unroll
  for (int i = 0; i < CS::RPG; ++i) {
    const int r = grp * CS::RPG + i;
    if (r < nrow) storev<float, CPT>(P2 + ((r0 + r) * HQ + hq) * KD + CPT * cgi, p2[i]);
  }
}

// Decode cache: r_cache[c] = P2 at the chunk's last token (copied), and
// k_tilde = k * 2^(r_cache[c] - P2) in the operand type.
// grid (cg.size(), B), 256 threads; each thread owns CPT channels.
template <typename TE, int KD, typename TO = typename OperandOf<TE>::type>
__global__ __launch_bounds__(256) void k_build_cache(const TE *__restrict__ k,
                                                     const float *__restrict__ P2,
                                                     TO *__restrict__ kt, float *__restrict__ rc,
                                                     int64_t T, int HQ, int H, int NC, ChunkGrid cg) {
  int hq, c;
  if (!cg.map(blockIdx.x, hq, c)) return;
  const int b = blockIdx.y;
  const int64_t r0 = (int64_t)c * CHUNK;
  const int nrow = (T - r0) < CHUNK ? (int)(T - r0) : CHUNK;
  const int h = hq / (HQ / H);
  constexpr int CPT = cpt<TE>(), NQ = KD / CPT, NRG = 256 / NQ, RPT = CHUNK / NRG;
  const int n0 = (threadIdx.x % NQ) * CPT, rg = threadIdx.x / NQ;
  const int64_t tb = (int64_t)b * T;
  const FV<CPT> R = loadv<float, CPT>(P2 + ((tb + r0 + nrow - 1) * HQ + hq) * KD + n0);
  if (rg == 0) storev<float, CPT>(rc + (((int64_t)b * NC + c) * HQ + hq) * KD + n0, R);
  // compile-time row count with a guard: the thread's loads go out together
  FV<CPT> p[RPT], kv[RPT];
#pragma unroll
  for (int i = 0; i < RPT; ++i) {
    const int r = rg + i * NRG;
    const int64_t t = tb + r0 + r;
    p[i] = r < nrow ? loadv<float, CPT>(P2 + (t * HQ + hq) * KD + n0) : zerov<CPT>();
    kv[i] = r < nrow ? loadv<TE, CPT>(k + (t * H + h) * KD + n0) : zerov<CPT>();
  }
#pragma unroll
  for (int i = 0; i < RPT; ++i) {
    const int r = rg + i * NRG;
    if (r < nrow) {
      FV<CPT> out;
#pragma unroll
      for (int j = 0; j < CPT; ++j) out.v[j] = kv[i].v[j] * fast_exp2(R.v[j] - p[i].v[j]);
      storev<TO, CPT>(kt + ((tb + r0 + r) * HQ + hq) * KD + n0, out);
    }
  }
}

template <typename TE, int KD>
hipError_t prefix_phases_t(const FwdProblem &p, const FwdWorkspace &ws, hipStream_t st) {
  typedef typename OperandOf<TE>::type TO;
  const int NCmax = (int)((p.maxlen + CHUNK - 1) / CHUNK);
  const ChunkGrid cgA = chunk_grid(p.HQ, 1, NCmax, p.nseg), cgC = chunk_grid(p.H, p.HQ / p.H, NCmax, p.nseg);
  const dim3 gridA(cgA.size(), (unsigned)p.nseg), gridC(cgC.size(), (unsigned)p.nseg);
  const TE *gs = static_cast<const TE *>(p.g_scalar);
  hipLaunchKernelGGL((k_chunk_sums<TE, KD>), gridA, dim3(256), 0, st,
                     static_cast<const TE *>(p.g), gs, ws.csum, ws.csum_s, p.cu, p.T, (int)p.HQ,
                     NCmax, cgA);
  const dim3 gridB((unsigned)p.HQ, (unsigned)p.nseg, (KD + 1 + 31) / 32);
  hipLaunchKernelGGL((k_chunk_scan<KD>), gridB, dim3(256), 0, st, ws.csum, ws.anch, ws.csum_s,
                     p.cu, p.T, (int)p.HQ, NCmax, gs != nullptr ? 1 : 0);
  const float qscale = p.scale * LOG2E;
  hipLaunchKernelGGL((k_prefill_operands<TE, KD>), gridC, dim3(256), 0, st,
                     static_cast<const TE *>(p.q), static_cast<const TE *>(p.k),
                     static_cast<const TE *>(p.g), gs, ws.csum, ws.anch, ws.csum_s,
                     static_cast<TO *>(ws.qh), static_cast<TO *>(ws.kt), ws.gsum, p.cu, p.T,
                     p.ntok, (int)p.HQ, (int)p.H, NCmax, qscale, cgC);
  return hipGetLastError();
}

template <typename TE, int KD>
hipError_t prefix_log2_t(const void *g, float *P2, const int32_t *cu, int64_t T, int64_t HQ,
                         int64_t nseg, int64_t maxlen, float *csum, hipStream_t st) {
  const int NCmax = (int)((maxlen + CHUNK - 1) / CHUNK);
  const ChunkGrid cgA = chunk_grid(HQ, 1, NCmax, nseg);
  const dim3 gridA(cgA.size(), (unsigned)nseg);
  hipLaunchKernelGGL((k_chunk_sums<TE, KD>), gridA, dim3(256), 0, st,
                     static_cast<const TE *>(g), (const TE *)nullptr, csum, (float *)nullptr, cu,
                     T, (int)HQ, NCmax, cgA);
  // The anchors of phase B are not needed here; they go to the upper half of
  // the workspace, which prefix_workspace_layout reserves for them.
  float *anch = csum + (int64_t)nseg * NCmax * HQ * KD;
  const dim3 gridB((unsigned)HQ, (unsigned)nseg, KD / 32);
  hipLaunchKernelGGL((k_chunk_scan<KD>), gridB, dim3(256), 0, st, csum, anch, (float *)nullptr,
                     cu, T, (int)HQ, NCmax, 0);
  hipLaunchKernelGGL((k_prefix_write<TE, KD>), gridA, dim3(256), 0, st,
                     static_cast<const TE *>(g), csum, P2, cu, T, (int)HQ, NCmax, cgA);
  return hipGetLastError();
}

}  // namespace

static inline size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

size_t fwd_workspace_layout(const FwdProblem &p, FwdWorkspace *ws, char *base) {
  const int64_t NCmax = (p.maxlen + CHUNK - 1) / CHUNK;
  const int64_t nchunk = p.nseg * NCmax;
  const size_t esz = p.dtype == 0 ? 2 : 4;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    char *ptr = base ? base + off : nullptr;
    off += align256(bytes);
    return ptr;
  };
  char *csum = take(sizeof(float) * nchunk * p.HQ * p.K);
  char *anch = take(sizeof(float) * nchunk * p.HQ * p.K);
  char *csum_s = take(sizeof(float) * nchunk * p.HQ);
  char *qh = take(p.dtype == 0 ? 0 : esz * p.ntok * p.HQ * p.K);  // bf16: q_hat formed in the attention kernel
  char *kt = take(esz * p.ntok * p.HQ * (p.dtype == 0 ? p.K + 16 : p.K));
  char *gsum = take(sizeof(float) * p.ntok * p.HQ);
  if (ws) {
    ws->csum = reinterpret_cast<float *>(csum);
    ws->anch = reinterpret_cast<float *>(anch);
    ws->csum_s = reinterpret_cast<float *>(csum_s);
    ws->qh = qh;
    ws->kt = kt;
    ws->gsum = reinterpret_cast<float *>(gsum);
  }
  return off;
}

size_t prefix_workspace_layout(int64_t nseg, int64_t maxlen, int64_t HQ, int64_t K, float **csum,
                               char *base) {
  const int64_t NCmax = (maxlen + CHUNK - 1) / CHUNK;
  if (csum) *csum = reinterpret_cast<float *>(base);
  return align256(2 * sizeof(float) * nseg * NCmax * HQ * K);
}

hipError_t launch_prefix_phases(const FwdProblem &p, const FwdWorkspace &ws, hipStream_t st) {
  if (p.dtype == 0) {
    return p.K == 64 ? prefix_phases_t<bf16_t, 64>(p, ws, st) : prefix_phases_t<bf16_t, 128>(p, ws, st);
  }
  return p.K == 64 ? prefix_phases_t<float, 64>(p, ws, st) : prefix_phases_t<float, 128>(p, ws, st);
}

hipError_t launch_prefix_log2(const void *g, float *P2, const int32_t *cu, int64_t T, int64_t HQ,
                              int64_t K, int64_t nseg, int64_t maxlen, int dtype, float *csum,
                              hipStream_t st) {
  if (dtype == 0)
    return K == 64 ? prefix_log2_t<bf16_t, 64>(g, P2, cu, T, HQ, nseg, maxlen, csum, st)
                   : prefix_log2_t<bf16_t, 128>(g, P2, cu, T, HQ, nseg, maxlen, csum, st);
  return K == 64 ? prefix_log2_t<float, 64>(g, P2, cu, T, HQ, nseg, maxlen, csum, st)
                 : prefix_log2_t<float, 128>(g, P2, cu, T, HQ, nseg, maxlen, csum, st);
}

hipError_t launch_build_cache(const void *k, const float *P2, void *kt, float *rc, int64_t B,
                              int64_t T, int64_t HQ, int64_t H, int64_t K, int dtype,
                              hipStream_t st) {
  const int NC = (int)((T + CHUNK - 1) / CHUNK);
  const ChunkGrid cg = chunk_grid(H, HQ / H, NC, B);
  const dim3 grid(cg.size(), (unsigned)B);
  if (dtype == 0) {
    if (K == 64)
      hipLaunchKernelGGL((k_build_cache<bf16_t, 64>), grid, dim3(256), 0, st,
                         static_cast<const bf16_t *>(k), P2, static_cast<_Float16 *>(kt), rc, T,
                         (int)HQ, (int)H, NC, cg);
    else
      hipLaunchKernelGGL((k_build_cache<bf16_t, 128>), grid, dim3(256), 0, st,
                         static_cast<const bf16_t *>(k), P2, static_cast<_Float16 *>(kt), rc, T,
                         (int)HQ, (int)H, NC, cg);
  } else {
    if (K == 64)
      hipLaunchKernelGGL((k_build_cache<float, 64>), grid, dim3(256), 0, st,
                         static_cast<const float *>(k), P2, static_cast<float *>(kt), rc, T,
                         (int)HQ, (int)H, NC, cg);
    else
      hipLaunchKernelGGL((k_build_cache<float, 128>), grid, dim3(256), 0, st,
                         static_cast<const float *>(k), P2, static_cast<float *>(kt), rc, T,
                         (int)HQ, (int)H, NC, cg);
  }
  return hipGetLastError();
}

}  // namespace wa

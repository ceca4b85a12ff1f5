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
// A row past the chunk's last one: its channels read as zero.  Loads of
// such rows fetch the chunk's last row instead (every load unconditional),
// so that the compiler issues a thread's loads together instead of waiting
// for each one inside its own branch.
template <int N> __device__ __forceinline__ FV<N> keep_if(bool ok, FV<N> x) {
#pragma unroll
  for (int j = 0; j < N; ++j) x.v[j] = ok ? x.v[j] : 0.f;
  return x;
}
// One element kept as raw bits (loaded early, converted where used).
template <typename TE> struct RawElem;
template <> struct RawElem<bf16_t> {
  static __device__ __forceinline__ uint32_t ld(const bf16_t *p) { return *p; }
  static __device__ __forceinline__ float cvt(uint32_t b) { return __uint_as_float(b << 16); }
};
template <> struct RawElem<float> {
  static __device__ __forceinline__ uint32_t ld(const float *p) { return __float_as_uint(*p); }
  static __device__ __forceinline__ float cvt(uint32_t b) { return __uint_as_float(b); }
};
// The same 16 bytes kept raw (loaded early, converted where used).
__device__ __forceinline__ u32x4 load16(const void *p) { return *reinterpret_cast<const u32x4 *>(p); }
template <typename TE, int N> __device__ __forceinline__ FV<N> fromraw(u32x4 w);
template <> __device__ __forceinline__ FV<8> fromraw<bf16_t, 8>(u32x4 w) {
  FV<8> r;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    r.v[2 * j] = bf16_lo(w[j]);
    r.v[2 * j + 1] = bf16_hi(w[j]);
  }
  return r;
}
template <> __device__ __forceinline__ FV<4> fromraw<float, 4>(u32x4 w) {
  return FV<4>{{__uint_as_float(w[0]), __uint_as_float(w[1]), __uint_as_float(w[2]), __uint_as_float(w[3])}};
}

// N consecutive floats stored as N elements of TO (round to nearest even):
// 16-bit types pack two per word, N = 8 is one 16-byte store, N = 4 one
// 8-byte store.
template <typename TO> __device__ __forceinline__ uint32_t pack2(float lo, float hi);
template <> __device__ __forceinline__ uint32_t pack2<_Float16>(float lo, float hi) { return pack_f16x2(lo, hi); }
template <> __device__ __forceinline__ uint32_t pack2<bf16_t>(float lo, float hi) { return pack_bf16x2(lo, hi); }
template <typename TO, int N> __device__ __forceinline__ void storev(TO *p, const FV<N> &x) {
  if constexpr (std::is_same<TO, float>::value) {
#pragma unroll
    for (int j = 0; j < N / 4; ++j)
      reinterpret_cast<float4 *>(p)[j] = make_float4(x.v[4 * j], x.v[4 * j + 1], x.v[4 * j + 2], x.v[4 * j + 3]);
  } else if constexpr (N == 8) {
    u32x4 w;
#pragma unroll
    for (int j = 0; j < 4; ++j) w[j] = pack2<TO>(x.v[2 * j], x.v[2 * j + 1]);
    *reinterpret_cast<u32x4 *>(p) = w;
  } else {
    static_assert(N == 4, "4 or 8 elements");
    *reinterpret_cast<u32x2 *>(p) = u32x2{pack2<TO>(x.v[0], x.v[1]), pack2<TO>(x.v[2], x.v[3])};
  }
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
                                                    int HQ, int NCmax, ChunkGrid cg,
                                                    int *__restrict__ wide) {
  int hq, c;
  if (!cg.map(blockIdx.x, hq, c)) return;
  const int s = blockIdx.y;
  // the range flags of this call start clear (phase C sets them)
  if (wide != nullptr && c == 0 && threadIdx.x == 0) wide[s * HQ + hq] = 0;
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
    const int r = min(grp + i * NG, nrow - 1);
    xs[i] = loadv<TE, CPT>(g + ((r0 + r) * HQ + hq) * KD + CPT * cgi);
  }
  // this row's g_scalar (first wave), loaded with the rest (raw bits; a valid
  // dummy address without a gate)
  const uint32_t gs_bits =
      RawElem<TE>::ld(gs != nullptr ? gs + (r0 + min((int)(threadIdx.x & 63), nrow - 1)) * HQ + hq : g);
  FV<CPT> acc = zerov<CPT>();
#pragma unroll
  for (int i = 0; i < CHUNK / NG; ++i) {
    const FV<CPT> x = keep_if<CPT>(grp + i * NG < nrow, xs[i]);
#pragma unroll
    for (int j = 0; j < CPT; ++j) acc.v[j] += x.v[j];
  }
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
    float a = (int)threadIdx.x < nrow ? RawElem<TE>::cvt(gs_bits) : 0.f;
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
  // at most NCmax chunks per segment have workspace slots (a max_seqlen below
  // the true length leaves the rest of the segment unprocessed, never out of
  // bounds)
  const int nch = min((int)((eos - bos + CHUNK - 1) / CHUNK), NCmax);
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
      const int r = min(grp * RPG + i, nrow - 1);
      p2[i] = loadv<TE, CPT>(g + ((r0 + r) * HQ + hq) * KD + CPT * cgi);
    }
#pragma unroll
    for (int i = 0; i < RPG; ++i) {
      p2[i] = keep_if<CPT>(grp * RPG + i < nrow, p2[i]);
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
template <typename TE, int KD, bool QBH, typename TO = typename OperandOf<TE>::type>
__global__ __launch_bounds__(256) void k_prefill_operands(
    const TE *__restrict__ q, const TE *__restrict__ k, const TE *__restrict__ g,
    const TE *__restrict__ gs, const float *__restrict__ off, const float *__restrict__ anch,
    const float *__restrict__ off_s, TO *__restrict__ qh, TO *__restrict__ kt,
    float *__restrict__ gsum, const int32_t *__restrict__ cu, int64_t T, int64_t ntok, int HQ,
    int H, int NCmax, float qscale, ChunkGrid cg, int *__restrict__ wide,
    _Float16 *__restrict__ qbh, float *__restrict__ mid) {
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
  // anchor of the query tile (its first chunk): q_hat = q 2^(P2 - RQ)
  const int64_t cq = (int64_t)s * NCmax + (c & ~1);
  const FV<CPT> RQ = loadv<float, CPT>(anch + (cq * HQ + hq) * KD + CPT * cgi);
  // the rows' keys (and queries, where this pass rescales them) load
  // together with g, ahead of the in-chunk scan: every load of the
  // workgroup goes out in one memory round trip
  constexpr bool QL = !HM || QBH;  // queries needed below
  u32x4 kin[CS::RPG], qin[CS::RPG];
#pragma unroll
  for (int i = 0; i < CS::RPG; ++i) {
    // rows past the chunk load its last row (unconditional loads; never stored)
    const int64_t t = r0 + min(grp * CS::RPG + i, nrow - 1);
    kin[i] = load16(k + (t * H + h) * KD + CPT * cgi);
    if (QL) qin[i] = load16(q + (t * HQ + hq) * KD + CPT * cgi);
  }
  // the gate's chunk offset and this row's g_scalar (used by the first
  // wave), kept as raw bits until used; every thread loads (the same 64 rows
  // per wave), and without a gate a valid dummy address is read, so that no
  // branch holds a wait
  const TE *gsp = gs != nullptr ? gs + (r0 + min((int)(threadIdx.x & 63), nrow - 1)) * HQ + hq : g;
  const uint32_t gs_bits = RawElem<TE>::ld(gsp);
  const float gs_off = gs != nullptr ? off_s[cidx * HQ + hq] : 0.f;
  FV<CPT> p2[CS::RPG];
  CS::run(g, r0, nrow, HQ, hq, cgi, grp, base, p2);
  // half operands: the running sum at row 31, from which the attention
  // kernel's waves for the chunk's second 32 rows start their own sums
  if (HM && grp == 31 / CS::RPG && nrow > 32)
    storev<float, CPT>(mid + (cidx * HQ + hq) * KD + CPT * cgi, p2[31 % CS::RPG]);
  // Range of the anchored operands: the exponents of q_hat and k_tilde stay
  // within EMAX (and the half keys and gate sums below their limits), else
  // the (segment, head) goes to the exact path.  The benchmark workloads
  // stay below 5.6; a decay sum changing by more than ~8 log2 units inside
  // one 64-token chunk does not.
  constexpr float EMAX = HM ? 8.f : 60.f;
  bool out_of_range = false;
#pragma unroll
  for (int i = 0; i < CS::RPG; ++i) {
    const int r = grp * CS::RPG + i;
    if (r < nrow) {
      const int64_t t = r0 + r;
#pragma unroll
      for (int j = 0; j < CPT; ++j)
        out_of_range = out_of_range || !(fabsf(A.v[j] - p2[i].v[j]) <= EMAX) ||
                       !(fabsf(p2[i].v[j] - RQ.v[j]) <= EMAX);
      if (!HM) {  // half operands: the attention kernel forms q_hat itself
        const FV<CPT> qv = fromraw<TE, CPT>(qin[i]);
        FV<CPT> qo;
#pragma unroll
        for (int j = 0; j < CPT; ++j) qo.v[j] = qv.v[j] * fast_exp2(p2[i].v[j] - RQ.v[j]) * qscale;
        storev<TO, CPT>(qh + (t * HQ + hq) * KD + CPT * cgi, qo);
      }
      if (HM && QBH) {
        // the backward's query operand: half, head-major [HQ, ntok, KD],
        // anchored at the token's own chunk, q 2^(P2 - R_c) scale log2(e)
        const FV<CPT> qv = fromraw<TE, CPT>(qin[i]);
        FV<CPT> qo;
#pragma unroll
        for (int j = 0; j < CPT; ++j) {
          qo.v[j] = qv.v[j] * fast_exp2(p2[i].v[j] - A.v[j]) * qscale;
          // room for the backward's factor of up to 2^4 on q_hat in half
          out_of_range = out_of_range || !(fabsf(qo.v[j]) < 4096.f);
        }
        storev<_Float16, CPT>(qbh + ((int64_t)hq * ntok + t) * KD + CPT * cgi, qo);
      }
      const FV<CPT> kv = fromraw<TE, CPT>(kin[i]);
      FV<CPT> ko;
#pragma unroll
      for (int j = 0; j < CPT; ++j) {
        ko.v[j] = kv.v[j] * fast_exp2(A.v[j] - p2[i].v[j]);
        // the backward's key operand also takes chunk factors of up to 2^4
        if (HM) out_of_range = out_of_range || !(fabsf(ko.v[j]) < (QBH ? 4096.f : 32768.f));
      }
      storev<TO, CPT>(kt + (HM ? (hq * ntok + t) : (t * HQ + hq)) * KX + CPT * cgi, ko);
    }
  }
  if (out_of_range) wide[s * HQ + hq] = 1;
  if (threadIdx.x < 64) {
    const int r = threadIdx.x;
    float G = 0.f;
    if (gs != nullptr) {
      const float x = wave_inclusive_scan(r < nrow ? RawElem<TE>::cvt(gs_bits) : 0.f);
      G = (gs_off + x) * LOG2E;
      if (r < nrow) gsum[(r0 + r) * HQ + hq] = G;
      // the half keys carry -G split into two halves
      if (HM && r < nrow && !(fabsf(G) < 16384.f)) wide[s * HQ + hq] = 1;
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

// Stand-alone prefix (the decode path's P2 and gate sums G2), accumulated
// in double so that each stored float is the running sum rounded once:
// decode scores reach ~1e5 on long random-walk decays, where the float error
// of a float-accumulated scan would show in the lse.
// Phase A in double: the per-chunk sums of g (per channel) and of g_scalar.
// grid (cg.size(), nseg), 256 threads; a thread owns CPT channels.
template <typename TE, int KD>
__global__ __launch_bounds__(256) void k_chunk_sums_f64(const TE *__restrict__ g,
                                                        const TE *__restrict__ gs,
                                                        double *__restrict__ csum,
                                                        double *__restrict__ csum_s,
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
  FV<CPT> xs[CHUNK / NG];
#pragma unroll
  for (int i = 0; i < CHUNK / NG; ++i) {
    const int r = min(grp + i * NG, nrow - 1);
    xs[i] = loadv<TE, CPT>(g + ((r0 + r) * HQ + hq) * KD + CPT * cgi);
  }
  const uint32_t gs_bits =
      RawElem<TE>::ld(gs != nullptr ? gs + (r0 + min((int)(threadIdx.x & 63), nrow - 1)) * HQ + hq : g);
  double acc[CPT];
#pragma unroll
  for (int j = 0; j < CPT; ++j) acc[j] = 0.0;
#pragma unroll
  for (int i = 0; i < CHUNK / NG; ++i) {
    const FV<CPT> x = keep_if<CPT>(grp + i * NG < nrow, xs[i]);
#pragma unroll
    for (int j = 0; j < CPT; ++j) acc[j] += (double)x.v[j];
  }
  __shared__ double red[NG][KD];
#pragma unroll
  for (int j = 0; j < CPT; ++j) red[grp][CPT * cgi + j] = acc[j];
  __syncthreads();
  const int64_t cidx = (int64_t)s * NCmax + c;
  for (int ch = threadIdx.x; ch < KD; ch += 256) {
    double t = 0.0;
    for (int q = 0; q < NG; ++q) t += red[q][ch];
    csum[(cidx * HQ + hq) * KD + ch] = t;
  }
  if (gs != nullptr && threadIdx.x < 64) {
    double a = (int)threadIdx.x < nrow ? (double)RawElem<TE>::cvt(gs_bits) : 0.0;
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) a += __shfl_xor(a, o);
    if (threadIdx.x == 0) csum_s[cidx * HQ + hq] = a;
  }
}

// Phase B in double: exclusive offsets of the chunk sums (channel KD stands
// for g_scalar).  grid (HQ, nseg, ceil((KD+1)/32)), 256 threads = 32
// channels x 8 chunk groups.
template <int KD>
__global__ __launch_bounds__(256) void k_scan_offsets_f64(const double *__restrict__ csum,
                                                          const double *__restrict__ csum_s,
                                                          double *__restrict__ off,
                                                          double *__restrict__ off_s,
                                                          const int32_t *__restrict__ cu,
                                                          int64_t T, int HQ, int NCmax,
                                                          int with_gs) {
  const int hq = blockIdx.x, s = blockIdx.y;
  const int ch = blockIdx.z * 32 + (threadIdx.x & 31);
  const int grp = threadIdx.x >> 5;
  int64_t bos, eos;
  segment_bounds(s, T, cu, bos, eos);
  const int nch = min((int)((eos - bos + CHUNK - 1) / CHUNK), NCmax);
  const bool active = ch < KD || (ch == KD && with_gs);
  const int span = (nch + 7) / 8;
  const int cb = grp * span, ce = min(nch, cb + span);
  const int64_t c0 = (int64_t)s * NCmax;
  const double *src;
  double *dst;
  int64_t stride;
  if (ch < KD) {
    src = csum + (c0 * HQ + hq) * KD + ch;
    dst = off + (c0 * HQ + hq) * KD + ch;
    stride = (int64_t)HQ * KD;
  } else {
    src = csum_s + c0 * HQ + hq;
    dst = off_s + c0 * HQ + hq;
    stride = HQ;
  }
  double tot = 0.0;
  if (active)
    for (int c = cb; c < ce; c += 8) {
      double x[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) x[u] = c + u < ce ? src[(int64_t)(c + u) * stride] : 0.0;
#pragma unroll
      for (int u = 0; u < 8; ++u) tot += x[u];
    }
  __shared__ double part[8][32];
  part[grp][threadIdx.x & 31] = tot;
  __syncthreads();
  if (!active) return;
  double run = 0.0;
  for (int q = 0; q < grp; ++q) run += part[q][threadIdx.x & 31];
  for (int c = cb; c < ce; c += 8) {
    double x[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) x[u] = c + u < ce ? src[(int64_t)(c + u) * stride] : 0.0;
#pragma unroll
    for (int u = 0; u < 8; ++u)
      if (c + u < ce) {
        dst[(int64_t)(c + u) * stride] = run;
        run += x[u];
      }
  }
}

// Phase C in double: P2 = round_to_float((offset + in-chunk sum) * log2(e)),
// and G2 likewise for g_scalar.  grid (cg.size(), nseg), 256 threads; a
// thread owns CPT channels of RPG consecutive rows.
template <typename TE, int KD>
__global__ __launch_bounds__(256) void k_prefix_write_f64(const TE *__restrict__ g,
                                                          const TE *__restrict__ gs,
                                                          const double *__restrict__ off,
                                                          const double *__restrict__ off_s,
                                                          float *__restrict__ P2,
                                                          float *__restrict__ G2,
                                                          const int32_t *__restrict__ cu,
                                                          int64_t T, int HQ, int NCmax,
                                                          ChunkGrid cg) {
  int hq, c;
  if (!cg.map(blockIdx.x, hq, c)) return;
  const int s = blockIdx.y;
  int64_t bos, eos;
  segment_bounds(s, T, cu, bos, eos);
  const int64_t r0 = bos + (int64_t)c * CHUNK;
  if (r0 >= eos) return;
  const int nrow = (eos - r0) < CHUNK ? (int)(eos - r0) : CHUNK;
  constexpr int CPT = cpt<TE>(), NQ = KD / CPT, NG = 256 / NQ, RPG = CHUNK / NG;
  const int cgi = threadIdx.x % NQ, grp = threadIdx.x / NQ;
  const int64_t cidx = (int64_t)s * NCmax + c;
  const double L2E = 1.4426950408889634074;
  FV<CPT> xs[RPG];
#pragma unroll
  for (int i = 0; i < RPG; ++i) {
    const int r = min(grp * RPG + i, nrow - 1);
    xs[i] = loadv<TE, CPT>(g + ((r0 + r) * HQ + hq) * KD + CPT * cgi);
  }
  // the chunk offsets and this row's g_scalar load with the rows
  double base[CPT];
#pragma unroll
  for (int j = 0; j < CPT; ++j) base[j] = off[(cidx * HQ + hq) * KD + CPT * cgi + j];
  const uint32_t gs_bits =
      RawElem<TE>::ld(gs != nullptr ? gs + (r0 + min((int)(threadIdx.x & 63), nrow - 1)) * HQ + hq : g);
  double acc[CPT];
#pragma unroll
  for (int j = 0; j < CPT; ++j) acc[j] = 0.0;
#pragma unroll
  for (int i = 0; i < RPG; ++i) {
    xs[i] = keep_if<CPT>(grp * RPG + i < nrow, xs[i]);
#pragma unroll
    for (int j = 0; j < CPT; ++j) acc[j] += (double)xs[i].v[j];
  }
  __shared__ double tot[NG][KD];
#pragma unroll
  for (int j = 0; j < CPT; ++j) tot[grp][CPT * cgi + j] = acc[j];
  __syncthreads();
  for (int q = 0; q < grp; ++q)
#pragma unroll
    for (int j = 0; j < CPT; ++j) base[j] += tot[q][CPT * cgi + j];
#pragma unroll
  for (int i = 0; i < RPG; ++i) {
    FV<CPT> out;
#pragma unroll
    for (int j = 0; j < CPT; ++j) {
      base[j] += (double)xs[i].v[j];
      out.v[j] = (float)(base[j] * L2E);
    }
    const int r = grp * RPG + i;
    if (r < nrow) storev<float, CPT>(P2 + ((r0 + r) * HQ + hq) * KD + CPT * cgi, out);
  }
  if (gs != nullptr && threadIdx.x < 64) {
    const int r = threadIdx.x;
    double x = r < nrow ? (double)RawElem<TE>::cvt(gs_bits) : 0.0;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
      const double y = __shfl_up(x, d);
      if (r >= d) x += y;
    }
    if (r < nrow) G2[(r0 + r) * HQ + hq] = (float)((off_s[cidx * HQ + hq] + x) * L2E);
  }
}

// Decode cache: r_cache[c] = P2 at the chunk's last token (copied), and
// k_tilde = k * 2^(r_cache[c] - P2) rounded to the cache type TO.
// grid (cg.size(), B), 256 threads; each thread owns CPT channels.
template <typename TE, int KD, typename TO>
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

// Streaming append (one token per batch row) to a decode cache of any
// layout.  Token t = len_b goes to chunk c = t / C.  The open chunk keeps its
// anchor at its newest token, rounded to an integer: R_new = rint(p_new),
// k_tilde_t = k_t * 2^(R_new - p_new), and the rows already in the chunk are
// re-anchored by 2^(R_new - R_old) -- an exact power of two when R_old is an
// integer too (always, except for a chunk left open by the cache build,
// whose anchor is a copied P2: one rounding at its first append).  Rows of
// a full cache (len_b >= T) are left alone.
// grid (HQ, B), 256 threads.
template <typename TE, typename TK, int KD>
__global__ __launch_bounds__(256) void k_cache_append(AppendProblem p) {
  const int hq = blockIdx.x, b = blockIdx.y, HQ = (int)p.HQ, H = (int)p.H;
  const int h = hq / (HQ / H);
  const int t = __builtin_amdgcn_readfirstlane(max(p.seqlens[b], 0));
  if (t >= p.T) return;
  const int tc = t - t % CHUNK;  // first token of the open chunk
  const int nold = t - tc;
  const int64_t row0 = uniform64(cache_row(p.block_table, p.max_blocks, (int)p.page_size,
                                           (int)p.num_pages, p.T, b, tc));
  const int64_t anchor = p.block_table != nullptr ? row0 / CHUNK
                                                  : (int64_t)b * ((p.T + CHUNK - 1) / CHUNK) + tc / CHUNK;
  __shared__ float fac[KD];
  const float *pn = p.p_new + ((int64_t)b * HQ + hq) * KD;
  float *rcp = p.rc + (anchor * HQ + hq) * KD;
  TK *kt = static_cast<TK *>(p.kt);
  for (int n = threadIdx.x; n < KD; n += 256) {
    const float rn = rintf(pn[n]);
    float f = 1.f;
    if (nold > 0) {
      const float d = rn - rcp[n];
      f = d == rintf(d) ? __builtin_amdgcn_ldexpf(1.f, (int)d) : exp2f(d);
    }
    fac[n] = f;
    const float kn = Elem<TE>::ld(static_cast<const TE *>(p.k) + ((int64_t)b * H + h) * KD + n);
    Elem<TK>::st(kt + ((row0 + nold) * HQ + hq) * KD + n, kn * exp2f(rn - pn[n]));
  }
  __syncthreads();
  for (int x = threadIdx.x; x < nold * KD; x += 256) {
    const int r = x / KD, n = x % KD;
    TK *e = kt + ((row0 + r) * HQ + hq) * KD + n;
    Elem<TK>::st(e, Elem<TK>::ld(e) * fac[n]);
  }
  __syncthreads();  // every thread has read its old anchors
  for (int n = threadIdx.x; n < KD; n += 256) rcp[n] = rintf(pn[n]);
  if (p.gs_cache != nullptr && threadIdx.x == 0)
    p.gs_cache[(row0 + nold) * HQ + hq] = p.gs_new[(int64_t)b * HQ + hq];
  if (hq % (HQ / H) == 0)
    for (int n = threadIdx.x; n < p.V; n += 256)
      static_cast<TE *>(p.vc)[((row0 + nold) * H + h) * p.V + n] =
          static_cast<const TE *>(p.v)[((int64_t)b * H + h) * p.V + n];
}

// After an append: every row that had room holds one more token.
__global__ __launch_bounds__(256) void k_seqlens_advance(int32_t *__restrict__ seqlens,
                                                         int64_t B, int64_t T) {
  for (int64_t b = blockIdx.x * 256 + threadIdx.x; b < B; b += (int64_t)gridDim.x * 256) {
    const int L = max(seqlens[b], 0);
    seqlens[b] = L < T ? L + 1 : L;
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
                     NCmax, cgA, ws.wide);
  const dim3 gridB((unsigned)p.HQ, (unsigned)p.nseg, (KD + 1 + 31) / 32);
  hipLaunchKernelGGL((k_chunk_scan<KD>), gridB, dim3(256), 0, st, ws.csum, ws.anch, ws.csum_s,
                     p.cu, p.T, (int)p.HQ, NCmax, gs != nullptr ? 1 : 0);
  const float qscale = p.scale * LOG2E;
  auto args = [&](auto kern) {
    hipLaunchKernelGGL(kern, gridC, dim3(256), 0, st, static_cast<const TE *>(p.q),
                       static_cast<const TE *>(p.k), static_cast<const TE *>(p.g), gs, ws.csum,
                       ws.anch, ws.csum_s, static_cast<TO *>(ws.qh), static_cast<TO *>(ws.kt),
                       ws.gsum, p.cu, p.T, p.ntok, (int)p.HQ, (int)p.H, NCmax, qscale, cgC,
                       ws.wide, static_cast<_Float16 *>(ws.qbh), ws.mid);
  };
  // the backward's half q_hat (bf16 inputs only) comes from its own instance
  if constexpr (std::is_same<TE, bf16_t>::value) {
    if (ws.qbh != nullptr) {
      args(k_prefill_operands<TE, KD, true>);
      return hipGetLastError();
    }
  }
  args(k_prefill_operands<TE, KD, false>);
  return hipGetLastError();
}

template <typename TE, int KD>
hipError_t prefix_log2_t(const void *g, const void *gs, float *P2, float *G2, const int32_t *cu,
                         int64_t T, int64_t HQ, int64_t nseg, int64_t maxlen, void *ws,
                         hipStream_t st) {
  const int NCmax = (int)((maxlen + CHUNK - 1) / CHUNK);
  const int64_t n = nseg * NCmax;
  // workspace: double chunk sums [n, HQ, K] and [n, HQ], then double offsets
  double *csum = static_cast<double *>(ws);
  double *csum_s = csum + n * HQ * KD;
  double *off = reinterpret_cast<double *>(static_cast<char *>(ws) + ((sizeof(double) * n * HQ * (KD + 1) + 255) & ~size_t(255)));
  double *off_s = off + n * HQ * KD;
  const ChunkGrid cgA = chunk_grid(HQ, 1, NCmax, nseg);
  const dim3 gridA(cgA.size(), (unsigned)nseg);
  const TE *gsp = static_cast<const TE *>(gs);
  hipLaunchKernelGGL((k_chunk_sums_f64<TE, KD>), gridA, dim3(256), 0, st,
                     static_cast<const TE *>(g), gsp, csum, csum_s, cu, T, (int)HQ, NCmax, cgA);
  const dim3 gridB((unsigned)HQ, (unsigned)nseg, (KD + 1 + 31) / 32);
  hipLaunchKernelGGL((k_scan_offsets_f64<KD>), gridB, dim3(256), 0, st, csum, csum_s, off, off_s,
                     cu, T, (int)HQ, NCmax, gs != nullptr ? 1 : 0);
  hipLaunchKernelGGL((k_prefix_write_f64<TE, KD>), gridA, dim3(256), 0, st,
                     static_cast<const TE *>(g), gsp, off, off_s, P2, G2, cu, T, (int)HQ, NCmax,
                     cgA);
  return hipGetLastError();
}

template <typename TE, typename TK, int KD>
hipError_t build_cache_t(const void *k, const float *P2, void *kt, float *rc, int64_t B, int64_t T,
                         int64_t HQ, int64_t H, hipStream_t st) {
  const int NC = (int)((T + CHUNK - 1) / CHUNK);
  const ChunkGrid cg = chunk_grid(H, HQ / H, NC, B);
  const dim3 grid(cg.size(), (unsigned)B);
  hipLaunchKernelGGL((k_build_cache<TE, KD, TK>), grid, dim3(256), 0, st,
                     static_cast<const TE *>(k), P2, static_cast<TK *>(kt), rc, T, (int)HQ,
                     (int)H, NC, cg);
  return hipGetLastError();
}

template <typename TE, typename TK>
hipError_t append_t(const AppendProblem &p, hipStream_t st) {
  if (p.K == 64)
    hipLaunchKernelGGL((k_cache_append<TE, TK, 64>), dim3((unsigned)p.HQ, (unsigned)p.B), dim3(256), 0, st, p);
  else
    hipLaunchKernelGGL((k_cache_append<TE, TK, 128>), dim3((unsigned)p.HQ, (unsigned)p.B), dim3(256), 0, st, p);
  const unsigned nb = (unsigned)((p.B + 255) / 256 < 1024 ? (p.B + 255) / 256 : 1024);
  hipLaunchKernelGGL(k_seqlens_advance, dim3(nb), dim3(256), 0, st, p.seqlens, p.B, p.T);
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
  char *wide = take(sizeof(int) * p.nseg * p.HQ);
  char *mid = take(p.dtype == 0 ? sizeof(float) * nchunk * p.HQ * p.K : 0);
  if (ws) {
    ws->csum = reinterpret_cast<float *>(csum);
    ws->anch = reinterpret_cast<float *>(anch);
    ws->csum_s = reinterpret_cast<float *>(csum_s);
    ws->qh = qh;
    ws->kt = kt;
    ws->gsum = reinterpret_cast<float *>(gsum);
    ws->wide = reinterpret_cast<int *>(wide);
    ws->qbh = nullptr;  // the backward sets it to its own buffer
    ws->mid = reinterpret_cast<float *>(mid);
  }
  return off;
}

size_t prefix_workspace_layout(int64_t nseg, int64_t maxlen, int64_t HQ, int64_t K) {
  const int64_t n = nseg * ((maxlen + CHUNK - 1) / CHUNK);
  return 2 * align256(sizeof(double) * n * HQ * (K + 1));
}

hipError_t launch_prefix_phases(const FwdProblem &p, const FwdWorkspace &ws, hipStream_t st) {
  if (p.dtype == 0) {
    return p.K == 64 ? prefix_phases_t<bf16_t, 64>(p, ws, st) : prefix_phases_t<bf16_t, 128>(p, ws, st);
  }
  return p.K == 64 ? prefix_phases_t<float, 64>(p, ws, st) : prefix_phases_t<float, 128>(p, ws, st);
}

hipError_t launch_prefix_log2(const void *g, const void *gs, float *P2, float *G2,
                              const int32_t *cu, int64_t T, int64_t HQ, int64_t K, int64_t nseg,
                              int64_t maxlen, int dtype, void *ws, hipStream_t st) {
  if (dtype == WA_DT_BF16)
    return K == 64 ? prefix_log2_t<bf16_t, 64>(g, gs, P2, G2, cu, T, HQ, nseg, maxlen, ws, st)
                   : prefix_log2_t<bf16_t, 128>(g, gs, P2, G2, cu, T, HQ, nseg, maxlen, ws, st);
  return K == 64 ? prefix_log2_t<float, 64>(g, gs, P2, G2, cu, T, HQ, nseg, maxlen, ws, st)
                 : prefix_log2_t<float, 128>(g, gs, P2, G2, cu, T, HQ, nseg, maxlen, ws, st);
}

template <typename TE>
static hipError_t build_cache_te(const void *k, const float *P2, void *kt, float *rc, int64_t B,
                                 int64_t T, int64_t HQ, int64_t H, int64_t K, int cache_dtype,
                                 hipStream_t st) {
  if (K == 64) {
    if (cache_dtype == WA_DT_BF16) return build_cache_t<TE, bf16_t, 64>(k, P2, kt, rc, B, T, HQ, H, st);
    if (cache_dtype == WA_DT_F16) return build_cache_t<TE, _Float16, 64>(k, P2, kt, rc, B, T, HQ, H, st);
    return build_cache_t<TE, float, 64>(k, P2, kt, rc, B, T, HQ, H, st);
  }
  if (cache_dtype == WA_DT_BF16) return build_cache_t<TE, bf16_t, 128>(k, P2, kt, rc, B, T, HQ, H, st);
  if (cache_dtype == WA_DT_F16) return build_cache_t<TE, _Float16, 128>(k, P2, kt, rc, B, T, HQ, H, st);
  return build_cache_t<TE, float, 128>(k, P2, kt, rc, B, T, HQ, H, st);
}

hipError_t launch_build_cache(const void *k, const float *P2, void *kt, float *rc, int64_t B,
                              int64_t T, int64_t HQ, int64_t H, int64_t K, int dtype,
                              int cache_dtype, hipStream_t st) {
  if (dtype == WA_DT_BF16) return build_cache_te<bf16_t>(k, P2, kt, rc, B, T, HQ, H, K, cache_dtype, st);
  return build_cache_te<float>(k, P2, kt, rc, B, T, HQ, H, K, cache_dtype, st);
}

hipError_t launch_cache_append(const AppendProblem &p, hipStream_t st) {
  if (p.dtype == WA_DT_BF16) {
    if (p.cache_dtype == WA_DT_BF16) return append_t<bf16_t, bf16_t>(p, st);
    if (p.cache_dtype == WA_DT_F16) return append_t<bf16_t, _Float16>(p, st);
    return append_t<bf16_t, float>(p, st);
  }
  if (p.cache_dtype == WA_DT_BF16) return append_t<float, bf16_t>(p, st);
  if (p.cache_dtype == WA_DT_F16) return append_t<float, _Float16>(p, st);
  return append_t<float, float>(p, st);
}

}  // namespace wa

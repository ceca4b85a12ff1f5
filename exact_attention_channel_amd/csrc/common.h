// Shared device helpers for libwallattn (gfx950 / CDNA4).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace wa {

// Chunk length of the anchors (Wall Attention README, "Decode": C = 64 is the
// anchor granularity).  The prefill kernels use the same length for key tiles,
// so a key tile's anchor is its chunk's anchor.
constexpr int CHUNK = 64;
// Query rows per prefill workgroup (4 waves x 32 rows); the query-side anchor
// is shared by these rows.
constexpr int QTILE = 128;

constexpr float LOG2E = 1.4426950408889634f;
constexpr float LN2 = 0.6931471805599453f;

typedef uint16_t bf16_t;  // raw bfloat16 bits in memory
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
__device__ __forceinline__ float bf16_to_f32(bf16_t h) { return __uint_as_float((uint32_t)h << 16); }

// Round-to-nearest-even float -> bfloat16 bits, NaN kept quiet.
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
  __bf16 b = (__bf16)f;
  return (uint32_t)__builtin_bit_cast(uint16_t, b);
}
// Two floats -> packed bf16 pair (lo in bits 0..15), one v_cvt_pk_bf16_f32.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2){lo, hi}, bf16x2));
}

// IEEE half helpers.  Rescaled q/k operands of the bf16 path are held in
// half precision: 3 more mantissa bits than bfloat16, and their range is
// bounded by one chunk's decay span (see prefix.hip).
__device__ __forceinline__ float f16_lo(uint32_t w) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)(w & 0xffffu));
}
__device__ __forceinline__ float f16_hi(uint32_t w) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)(w >> 16));
}
__device__ __forceinline__ uint32_t pack_f16x2(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2){lo, hi}, f16x2));
}

// 2^x on the transcendental unit (v_exp_f32).
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float fast_log2(float x) { return __builtin_amdgcn_logf(x); }

// Element loads/stores for the two supported storage types.
template <typename TE> struct Elem;
template <> struct Elem<bf16_t> {
  static __device__ __forceinline__ float ld(const bf16_t *p) { return bf16_to_f32(*p); }
  static __device__ __forceinline__ void st(bf16_t *p, float x) { *p = (bf16_t)f32_to_bf16_bits(x); }
};
template <> struct Elem<_Float16> {
  static __device__ __forceinline__ float ld(const _Float16 *p) { return (float)*p; }
  static __device__ __forceinline__ void st(_Float16 *p, float x) { *p = (_Float16)x; }
};
template <> struct Elem<float> {
  static __device__ __forceinline__ float ld(const float *p) { return *p; }
  static __device__ __forceinline__ void st(float *p, float x) { *p = x; }
};

// Storage type of the rescaled operands (q_hat, k_tilde) for an input type.
template <typename TE> struct OperandOf;
template <> struct OperandOf<bf16_t> { typedef _Float16 type; };
template <> struct OperandOf<float> { typedef float type; };

// A workgroup-uniform value moved into scalar registers, so that everything
// derived from it (addresses, buffer descriptors, loop bounds) stays scalar.
__device__ __forceinline__ int64_t uniform64(int64_t x) {
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)x);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)((uint64_t)x >> 32));
  return (int64_t)(((uint64_t)hi << 32) | lo);
}

// Token range [bos, eos) of segment s: batch row s of length T, or the packed
// sequence s of cu_seqlens.  s must be uniform across the workgroup.
__device__ __forceinline__ void segment_bounds(int s, int64_t T, const int32_t *cu, int64_t &bos,
                                               int64_t &eos) {
  if (cu) {
    bos = cu[s];
    eos = cu[s + 1];
  } else {
    bos = (int64_t)s * T;
    eos = bos + T;
  }
  bos = uniform64(bos);
  eos = uniform64(eos);
}

// Pool row of token `tok` of batch row b in a decode cache: contiguous
// [B, T] rows, or pages of page_size rows (a multiple of CHUNK) found through
// block_table [B, max_blocks] (entries clamped into [0, num_pages) so that no
// address leaves the pool).
__device__ __forceinline__ int64_t cache_row(const int32_t *block_table, int64_t max_blocks,
                                             int page_size, int num_pages, int64_t T, int b,
                                             int tok) {
  if (block_table == nullptr) return (int64_t)b * T + tok;
  const int lp = tok / page_size;
  int pg = block_table[(int64_t)b * max_blocks + lp];
  pg = min(max(pg, 0), num_pages - 1);
  return (int64_t)pg * page_size + (tok - lp * page_size);
}

__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) x = fmaxf(x, __shfl_xor(x, o));
  return x;
}
__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) x += __shfl_xor(x, o);
  return x;
}

}  // namespace wa

// Decode kernels for caches of bf16_t keys (see decode_kernels.h).
#include "decode_kernels.h"

namespace wa {
template hipError_t launch_decode_cache<bf16_t>(const DecodeParams &, int, int64_t, int64_t,
                                             const float *, void *, float *, int64_t, hipStream_t);
}  // namespace wa

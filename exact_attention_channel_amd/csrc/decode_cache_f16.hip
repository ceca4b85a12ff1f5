// Decode kernels for caches of _Float16 keys (see decode_kernels.h).
#include "decode_kernels.h"

namespace wa {
template hipError_t launch_decode_cache<_Float16>(const DecodeParams &, int, int64_t, int64_t,
                                             const float *, void *, float *, int64_t, hipStream_t);
}  // namespace wa

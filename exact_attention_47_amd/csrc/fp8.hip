// FP8 path (placeholder until the kernels land).
#include "common.h"
#include "kernels.h"

namespace attn {
hipError_t launch_hadamard_quant(const void*, void*, float*, const signed char*, int, int, int, int, int,
                                 int, int, hipStream_t) { return hipErrorNotSupported; }
hipError_t launch_quant_per_tensor(const void*, void*, float*, int, int, int, int, int, int,
                                   hipStream_t) { return hipErrorNotSupported; }
hipError_t launch_fwd_fp8(const void*, const void*, const void*, const float*, const float*,
                          const float*, void*, float*, int, int, int, int, int, int, float, int,
                          hipStream_t) { return hipErrorNotSupported; }
}  // namespace attn

// Matrix-core throughput the chip sustains: a measurement aid for the
// roofline report, not part of the attention path.
//
// The data-sheet peaks assume the top engine clock. Under a long stream of
// matrix instructions on every CU the socket reaches its power limit and the
// clock settles lower, so a kernel's rate is also worth stating against what
// the matrix cores deliver there. This kernel runs, on two waves per SIMD of
// every CU, back-to-back MFMAs of one kind on register operands (no memory
// traffic except one store per lane at the end), with eight operand
// fragments in rotation so that consecutive instructions see different
// inputs (fixed operands toggle fewer bits and draw less power).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "common.h"
#include "kernels.h"

namespace attn {
namespace {

__device__ __forceinline__ uint32_t mix32(uint32_t x) {
  x ^= x >> 16;
  x *= 0x7feb352du;
  x ^= x >> 15;
  x *= 0x846ca68bu;
  x ^= x >> 16;
  return x;
}

// bf16 values in [-0.5, 0.5) from a hash of the lane and fragment index
__device__ __forceinline__ v8bf16 frag_bf16(uint32_t seed) {
  v8bf16 f;
#pragma unroll
  for (int e = 0; e < 8; e++) f[e] = (__bf16)((float)(mix32(seed * 8 + e) & 0xffff) / 65536.0f - 0.5f);
  return f;
}

// E4M3 codes with exponent field below 15 (finite, never NaN)
__device__ __forceinline__ v8i frag_e4m3(uint32_t seed) {
  v8i f;
#pragma unroll
  for (int e = 0; e < 8; e++) f[e] = (int)(mix32(seed * 8 + e) & 0x77777777u);
  return f;
}

// KIND 0: v_mfma_f32_32x32x16_bf16; 1: v_mfma_scale_f32_32x32x64_f8f6f4 (E4M3, unit scales);
// 2: v_mfma_f32_16x16x32_bf16. Per iteration and wave: 32 instructions (four
// accumulators, eight fragments).
template <int KIND>
__global__ void __launch_bounds__(256) mfma_stream_kernel(float* __restrict__ sink, int iters) {
  const uint32_t tid = blockIdx.x * blockDim.x + threadIdx.x;
  if constexpr (KIND == 2) {
    v4f acc[4];
#pragma unroll
    for (int a = 0; a < 4; a++)
#pragma unroll
      for (int e = 0; e < 4; e++) acc[a][e] = 0.0f;
    v8bf16 x[8], y[8];
#pragma unroll
    for (int u = 0; u < 8; u++) {
      x[u] = frag_bf16(tid * 16 + u);
      y[u] = frag_bf16(tid * 16 + 8 + u + 0x9e3779b9u);
    }
    for (int it = 0; it < iters; it++) {
#pragma unroll
      for (int u = 0; u < 8; u++)
#pragma unroll
        for (int a = 0; a < 4; a++)
          acc[a] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(x[u], y[(u + a) & 7], acc[a], 0, 0, 0);
    }
    float s = 0.0f;
#pragma unroll
    for (int a = 0; a < 4; a++)
#pragma unroll
      for (int e = 0; e < 4; e++) s += acc[a][e];
    sink[tid] = s;
    return;
  }
  v16f acc[4];
#pragma unroll
  for (int a = 0; a < 4; a++)
#pragma unroll
    for (int e = 0; e < 16; e++) acc[a][e] = 0.0f;
  if constexpr (KIND == 0) {
    v8bf16 x[8], y[8];
#pragma unroll
    for (int u = 0; u < 8; u++) {
      x[u] = frag_bf16(tid * 16 + u);
      y[u] = frag_bf16(tid * 16 + 8 + u + 0x9e3779b9u);
    }
    for (int it = 0; it < iters; it++) {
#pragma unroll
      for (int u = 0; u < 8; u++)
#pragma unroll
        for (int a = 0; a < 4; a++)
          acc[a] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(x[u], y[(u + a) & 7], acc[a], 0, 0, 0);
    }
  } else {
    v8i x[8], y[8];
#pragma unroll
    for (int u = 0; u < 8; u++) {
      x[u] = frag_e4m3(tid * 16 + u);
      y[u] = frag_e4m3(tid * 16 + 8 + u + 0x9e3779b9u);
    }
    for (int it = 0; it < iters; it++) {
#pragma unroll
      for (int u = 0; u < 8; u++)
#pragma unroll
        for (int a = 0; a < 4; a++)
          acc[a] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(x[u], y[(u + a) & 7], acc[a], 0, 0, 0, 127,
                                                                   0, 127);
    }
  }
  float s = 0.0f;
#pragma unroll
  for (int a = 0; a < 4; a++)
#pragma unroll
    for (int e = 0; e < 16; e++) s += acc[a][e];
  sink[tid] = s;
}

}  // namespace

hipError_t launch_mfma_stream(int kind, int iters, float* sink, int blocks, hipStream_t st) {
  if (kind == 0)
    hipLaunchKernelGGL(mfma_stream_kernel<0>, dim3((unsigned)blocks), dim3(256), 0, st, sink, iters);
  else if (kind == 1)
    hipLaunchKernelGGL(mfma_stream_kernel<1>, dim3((unsigned)blocks), dim3(256), 0, st, sink, iters);
  else
    hipLaunchKernelGGL(mfma_stream_kernel<2>, dim3((unsigned)blocks), dim3(256), 0, st, sink, iters);
  return hipGetLastError();
}

}  // namespace attn

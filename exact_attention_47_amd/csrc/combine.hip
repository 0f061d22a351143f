// Merge of key-range partials: for each query row, the partial outputs O_s
// (each normalised over its own key range) and their logsumexps LSE_s give
//   LSE = ln sum_s exp(LSE_s),   O = sum_s exp(LSE_s - LSE) O_s.
// This is the logsumexp combination that makes block-wise softmax exact
// ([GN] "Rueckblick auf den FlashAttention-Ansatz"), applied across
// workgroups that processed disjoint key ranges of the same rows.
// One wave per query row; lanes stride over D.
#include "common.h"
#include "kernels.h"

namespace attn {

template <typename T>
__global__ void __launch_bounds__(256)
combine_kernel(const float* __restrict__ Opart, const float* __restrict__ Lpart, T* __restrict__ O,
               float* __restrict__ LSE, int rows, int n_split, int D)
{
  const int lane = threadIdx.x & 63;
  const int r = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (r >= rows) return;
  float mx = kNegInf;
  for (int s = 0; s < n_split; s++) mx = fmaxf(mx, Lpart[(size_t)s * rows + r]);
  const float ref = mx == kNegInf ? 0.0f : mx;
  float tot = 0.0f;
  for (int s = 0; s < n_split; s++) tot += __expf(Lpart[(size_t)s * rows + r] - ref);
  const float inv = 1.0f / tot;
  for (int d = lane; d < D; d += 64) {
    float acc = 0.0f;
    for (int s = 0; s < n_split; s++) {
      const float w = __expf(Lpart[(size_t)s * rows + r] - ref);
      acc += w * Opart[((size_t)s * rows + r) * D + d];
    }
    O[(size_t)r * D + d] = (T)(acc * inv);
  }
  if (lane == 0) LSE[r] = ref + __logf(tot);
}

hipError_t launch_combine(const FwdArgs& a, hipStream_t st) {
  const int rows = a.B * a.H * a.S_q;
  const dim3 grid((rows + 3) / 4);
  switch (a.dtype) {
    case 0:
      hipLaunchKernelGGL(combine_kernel<float>, grid, dim3(256), 0, st, a.opart, a.lpart, (float*)a.o,
                         a.lse, rows, a.n_split, a.D);
      break;
    case 1:
      hipLaunchKernelGGL(combine_kernel<_Float16>, grid, dim3(256), 0, st, a.opart, a.lpart,
                         (_Float16*)a.o, a.lse, rows, a.n_split, a.D);
      break;
    default:
      hipLaunchKernelGGL(combine_kernel<__bf16>, grid, dim3(256), 0, st, a.opart, a.lpart,
                         (__bf16*)a.o, a.lse, rows, a.n_split, a.D);
      break;
  }
  return hipGetLastError();
}

}  // namespace attn

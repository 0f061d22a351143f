// Fused exact attention forward pass in float32 (vector ALU, no matrix cores).
//
// Same method as the matrix-core kernel (tiles of keys staged in LDS, online
// softmax rescaling, no score matrix in HBM; [NL] "FlashAttention en
// FlashAttention-2"), kept simple because float32 inputs are only used for
// small exact checks. A workgroup of 256 threads owns 32 query rows of one
// (b, h); each row is split over 8 consecutive lanes, each holding D/8
// columns of q and of the output. A score is the sum of the 8 partial dot
// products, reduced with three xor-shuffles inside the 8-lane group, so every
// lane of the group sees every score of its row.
#include "common.h"
#include "kernels.h"

namespace attn {

namespace {
constexpr int F32_ROWS = 32;
constexpr int F32_BN = 32;
}

template <int D, bool CAUSAL, bool SPLIT>
__global__ void __launch_bounds__(256)
fwd_f32_kernel(const float* __restrict__ Q, const float* __restrict__ K, const float* __restrict__ V,
               float* __restrict__ O, float* __restrict__ LSE, float* __restrict__ Opart,
               float* __restrict__ Lpart, int BH, int S_q, int S_k, int n_qt, int n_split,
               int keys_per_split, float c)
{
  constexpr int W = D / 8;                       // columns per lane
  __shared__ float ks[F32_BN][D];
  __shared__ float vs[F32_BN][D];

  const int tid = threadIdx.x;
  const int part = tid & 7;
  const int row = tid >> 3;
  int work = blockIdx.x;
  const int split = work % n_split;
  work /= n_split;
  const int qt = work % n_qt;
  const int bh = work / n_qt;
  const int q = qt * F32_ROWS + row;
  const int diag = S_k - S_q;
  int k_lo = 0, k_hi = S_k;
  if (SPLIT) {
    k_lo = split * keys_per_split;
    k_hi = min(S_k, k_lo + keys_per_split);
  }
  int k_end = k_hi;
  if (CAUSAL) k_end = min(k_end, qt * F32_ROWS + F32_ROWS - 1 + diag + 1);

  const float* Qh = Q + (size_t)bh * S_q * D;
  const float* Kh = K + (size_t)bh * S_k * D;
  const float* Vh = V + (size_t)bh * S_k * D;

  float qr[W], acc[W];
#pragma unroll
  for (int w = 0; w < W; w++) {
    qr[w] = q < S_q ? Qh[(size_t)q * D + part * W + w] : 0.0f;
    acc[w] = 0.0f;
  }
  float m = kNegInf, l = 0.0f;

  for (int key0 = k_lo; key0 < k_end; key0 += F32_BN) {
    __syncthreads();
    for (int i = tid; i < F32_BN * D; i += 256) {
      const int r = i / D, d = i % D;
      const int key = key0 + r;
      ks[r][d] = key < k_hi ? Kh[(size_t)key * D + d] : 0.0f;
      vs[r][d] = key < k_hi ? Vh[(size_t)key * D + d] : 0.0f;
    }
    __syncthreads();
    float s[F32_BN];
    float mx = kNegInf;
#pragma unroll
    for (int j = 0; j < F32_BN; j++) {
      float part_dot = 0.0f;
#pragma unroll
      for (int w = 0; w < W; w++) part_dot = __builtin_fmaf(qr[w], ks[j][part * W + w], part_dot);
      part_dot += __shfl_xor(part_dot, 1);
      part_dot += __shfl_xor(part_dot, 2);
      part_dot += __shfl_xor(part_dot, 4);
      const int key = key0 + j;
      const bool ok = key < k_hi && (!CAUSAL || key <= q + diag);
      s[j] = ok ? part_dot * c : kNegInf;
      mx = fmaxf(mx, s[j]);
    }
    const float mnew = fmaxf(m, mx);
    const float ref = mnew == kNegInf ? 0.0f : mnew;
    const float alpha = fast_exp2(m - ref);
    m = mnew;
    l *= alpha;
#pragma unroll
    for (int w = 0; w < W; w++) acc[w] *= alpha;
#pragma unroll
    for (int j = 0; j < F32_BN; j++) {
      const float p = fast_exp2(s[j] - ref);
      l += p;
#pragma unroll
      for (int w = 0; w < W; w++) acc[w] = __builtin_fmaf(p, vs[j][part * W + w], acc[w]);
    }
  }

  if (q >= S_q) return;
  const bool has = m != kNegInf && l > 0.0f;
  const float inv = has ? 1.0f / l : 0.0f;
  const float lse = has ? (m + __builtin_log2f(l)) * kLn2 : kNegInf;
  if (!SPLIT) {
    float* orow = O + ((size_t)bh * S_q + q) * D + part * W;
#pragma unroll
    for (int w = 0; w < W; w++) orow[w] = acc[w] * inv;
    if (part == 0) LSE[(size_t)bh * S_q + q] = lse;
  } else {
    const size_t prow = ((size_t)split * BH + bh) * S_q + q;
    float* orow = Opart + prow * D + part * W;
#pragma unroll
    for (int w = 0; w < W; w++) orow[w] = acc[w] * inv;
    if (part == 0) Lpart[prow] = lse;
  }
}

template <int D, bool CAUSAL, bool SPLIT>
static hipError_t launch_f32_one(const FwdArgs& a, hipStream_t st) {
  const int n_qt = (a.S_q + F32_ROWS - 1) / F32_ROWS;
  const int n_work = a.B * a.H * n_qt * a.n_split;
  hipLaunchKernelGGL((fwd_f32_kernel<D, CAUSAL, SPLIT>), dim3(n_work), dim3(256), 0, st,
                     (const float*)a.q, (const float*)a.k, (const float*)a.v, (float*)a.o, a.lse,
                     a.opart, a.lpart, a.B * a.H, a.S_q, a.S_k, n_qt, a.n_split, a.keys_per_split, a.c);
  return hipGetLastError();
}

template <int D>
static hipError_t launch_f32_d(const FwdArgs& a, hipStream_t st) {
  const bool split = a.n_split > 1;
  if (a.causal) return split ? launch_f32_one<D, true, true>(a, st) : launch_f32_one<D, true, false>(a, st);
  return split ? launch_f32_one<D, false, true>(a, st) : launch_f32_one<D, false, false>(a, st);
}

int f32_rows_per_block() { return F32_ROWS; }
int f32_keys_per_tile() { return F32_BN; }

hipError_t launch_fwd_f32(const FwdArgs& a, hipStream_t st) {
  switch (a.D) {
    case 64: return launch_f32_d<64>(a, st);
    case 128: return launch_f32_d<128>(a, st);
  }
  return hipErrorInvalidValue;
}

}  // namespace attn

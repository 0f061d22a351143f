// Single-query-row attention over a long key range (decode): the key-range
// split of the forward pass, as a streaming kernel.
//
// With one query row the matrix cores have nothing to reuse: every K and V
// byte is used for exactly two multiply-adds, so the work is bound by HBM
// bandwidth and the kernel is written to stream K and V at full width. The
// method is unchanged: online softmax over the keys of this split, then the
// logsumexp merge of splits (combine.hip) gives the exact result ([NL]
// "FlashAttention en FlashAttention-2"; [GN] "Rueckblick auf den
// FlashAttention-Ansatz").
//
// Work split: one workgroup of 256 threads per (b*h, split). A group of D/8
// consecutive lanes holds one key row (8 elements, one 16-byte load per lane),
// so a wave reads 64*16 bytes of consecutive keys per load instruction. Each
// lane group walks its keys in batches of 8 (16 loads in flight per lane),
// reduces the 8 dot products across its lanes, and updates its own running
// (max, sum, output slice). At the end the 256/(D/8) groups are merged by
// logsumexp through LDS and the split's normalised partial output and LSE
// are written to the workspace.
#include "common.h"
#include "kernels.h"

namespace attn {

namespace {

constexpr int DEC_KEYS = 8;       // keys per batch per lane group

template <typename T>
__device__ __forceinline__ void ld8(const T* p, float* out) {
  const uint4 raw = *(const uint4*)p;
  const T* e = (const T*)&raw;
#pragma unroll
  for (int i = 0; i < 8; i++) out[i] = (float)e[i];
}

template <typename T, int D>
__global__ void __launch_bounds__(256)
decode_kernel(const T* __restrict__ Q, const T* __restrict__ K, const T* __restrict__ V,
              float* __restrict__ Opart, float* __restrict__ Lpart, int BH, int S_k, int n_split,
              int keys_per_split, float c)
{
  constexpr int LG = D / 8;                 // lanes per key row
  constexpr int NG = 256 / LG;              // lane groups per workgroup
  __shared__ float sm_m[NG], sm_l[NG];
  __shared__ float sm_o[NG][D + 4];

  const int tid = threadIdx.x;
  const int sub = tid % LG;                 // which 8 columns
  const int grp = tid / LG;
  const int split = blockIdx.x % n_split;
  const int bh = blockIdx.x / n_split;
  const int k_lo = split * keys_per_split;
  const int k_hi = min(S_k, k_lo + keys_per_split);

  const T* Kh = K + (size_t)bh * S_k * D + sub * 8;
  const T* Vh = V + (size_t)bh * S_k * D + sub * 8;
  float q[8];
  ld8(Q + (size_t)bh * D + sub * 8, q);
#pragma unroll
  for (int i = 0; i < 8; i++) q[i] *= c;      // scores directly in the log2 domain

  float m = kNegInf, l = 0.0f, o[8];
#pragma unroll
  for (int i = 0; i < 8; i++) o[i] = 0.0f;

  // batches of NG*DEC_KEYS consecutive keys; group g takes keys g, g+NG, ...
  for (int base = k_lo; base < k_hi; base += NG * DEC_KEYS) {
    float kk[DEC_KEYS][8], vv[DEC_KEYS][8];
#pragma unroll
    for (int u = 0; u < DEC_KEYS; u++) {
      const int key = min(base + u * NG + grp, k_hi - 1);
      ld8(Kh + (size_t)key * D, kk[u]);
      ld8(Vh + (size_t)key * D, vv[u]);
    }
    float s[DEC_KEYS];
#pragma unroll
    for (int u = 0; u < DEC_KEYS; u++) {
      float a = 0.0f;
#pragma unroll
      for (int i = 0; i < 8; i++) a = __builtin_fmaf(q[i], kk[u][i], a);
#pragma unroll
      for (int off = 1; off < LG; off <<= 1) a += __shfl_xor(a, off);
      s[u] = (base + u * NG + grp < k_hi) ? a : kNegInf;
    }
    float mx = m;
#pragma unroll
    for (int u = 0; u < DEC_KEYS; u++) mx = fmaxf(mx, s[u]);
    const float ref = mx == kNegInf ? 0.0f : mx;
    const float alpha = fast_exp2(m - ref);
    l *= alpha;
#pragma unroll
    for (int i = 0; i < 8; i++) o[i] *= alpha;
#pragma unroll
    for (int u = 0; u < DEC_KEYS; u++) {
      const float p = fast_exp2(s[u] - ref);
      l += p;
#pragma unroll
      for (int i = 0; i < 8; i++) o[i] = __builtin_fmaf(p, vv[u][i], o[i]);
    }
    m = mx;
  }

  // merge the lane groups: M = max m_g, L = sum l_g 2^(m_g - M), O = sum o_g 2^(m_g - M) / L
  if (sub == 0) { sm_m[grp] = m; sm_l[grp] = l; }
#pragma unroll
  for (int i = 0; i < 8; i++) sm_o[grp][sub * 8 + i] = o[i];
  __syncthreads();
  float M = kNegInf;
#pragma unroll
  for (int g = 0; g < NG; g++) M = fmaxf(M, sm_m[g]);
  const float refM = M == kNegInf ? 0.0f : M;
  float L = 0.0f;
#pragma unroll
  for (int g = 0; g < NG; g++) L += sm_l[g] * fast_exp2(sm_m[g] - refM);
  const size_t prow = (size_t)split * BH + bh;
  for (int d = tid; d < D; d += 256) {
    float acc = 0.0f;
#pragma unroll
    for (int g = 0; g < NG; g++) acc += sm_o[g][d] * fast_exp2(sm_m[g] - refM);
    Opart[prow * D + d] = L > 0.0f ? acc / L : 0.0f;
  }
  if (tid == 0) Lpart[prow] = (M != kNegInf && L > 0.0f) ? (M + __builtin_log2f(L)) * kLn2 : kNegInf;
}

template <typename T>
hipError_t launch_t(const FwdArgs& a, hipStream_t st) {
  const dim3 grid((unsigned)(a.B * a.H * a.n_split));
  switch (a.D) {
    case 64:
      hipLaunchKernelGGL((decode_kernel<T, 64>), grid, dim3(256), 0, st, (const T*)a.q, (const T*)a.k,
                         (const T*)a.v, a.opart, a.lpart, a.B * a.H, a.S_k, a.n_split, a.keys_per_split, a.c);
      break;
    case 128:
      hipLaunchKernelGGL((decode_kernel<T, 128>), grid, dim3(256), 0, st, (const T*)a.q, (const T*)a.k,
                         (const T*)a.v, a.opart, a.lpart, a.B * a.H, a.S_k, a.n_split, a.keys_per_split, a.c);
      break;
    case 256:
      hipLaunchKernelGGL((decode_kernel<T, 256>), grid, dim3(256), 0, st, (const T*)a.q, (const T*)a.k,
                         (const T*)a.v, a.opart, a.lpart, a.B * a.H, a.S_k, a.n_split, a.keys_per_split, a.c);
      break;
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace

int decode_keys_per_tile() { return 64; }
int decode_max_rows() { return 1; }

hipError_t launch_fwd_decode(const FwdArgs& a, hipStream_t st) {
  if (a.S_q != 1) return hipErrorInvalidValue;
  if (a.dtype == 2) return launch_t<__bf16>(a, st);
  return launch_t<_Float16>(a, st);
}

}  // namespace attn

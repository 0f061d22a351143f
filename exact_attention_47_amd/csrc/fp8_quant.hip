// FP8 (OCP E4M3) preparation of attention inputs.
//
// hadamard_quant: incoherent processing for Q and K ([NL] "3. Lage precisie
// (FP8) met reductie van kwantisatiefout": multiply by a random orthogonal
// matrix before quantizing so outliers spread over all coordinates; [GN]
// "Niedrige FP8-Praezision und incoherent processing": a random-sign
// Hadamard transform, O(d log d) per head, bound by memory bandwidth). Per
// row: u = FWHT(signs * x) in float32, unnormalised, butterfly strides 1, 2,
// ..., D/2 in that order (every output is the same float32 expression tree as
// the textbook in-place algorithm, so codes are reproducible bit for bit).
// Per block of block_rows rows of one (b, h): a = max |u|, inv = 448 / a,
// code = E4M3(u * inv) rounded to nearest even (the hardware conversion),
// after clamping to +-448 since the conversion does not saturate; scale =
// a / 448, times 1/sqrt(D) when the transform is applied.
//
// Work split for 64-row blocks (the FP8 attention's block size): one
// workgroup of 256 threads per (b, h, block), four lanes per row. Lane s of a
// row holds elements 32k + 8s + i (k < D/32, i < 8), read as D/32 16-byte
// loads issued together and kept in registers for both passes. Strides 1, 2,
// 4, 32, 64 and 128 of the transform are then inside the lane and strides 8
// and 16 are swaps within the 4-lane group (DPP quad permutes, no LDS), still
// taken in the order 1, 2, ..., D/2. Other block sizes use a general kernel
// that spreads a row over D/8 lanes and re-reads the block for its second pass.
//
// rope_hadamard_quant: the same with rotary position embedding applied to
// each row first, in the registers that already hold it ([GN] "Niedrige
// FP8-Praezision und incoherent processing": the transform is memory-bound
// and costs nothing extra when fused with a preceding memory-bound operation
// such as rotary embedding). The angles come as cos/sin tables [S][D/2]
// float32 shared by every (b, h), so they stay in cache; both coordinates of
// a pair (interleaved 2j, 2j+1, or halves j, j + D/2) are in the same lane.
//
// quant_per_tensor: one scale for the whole tensor. Launch 1 clears the
// running maximum, launch 2 reduces max |x| per workgroup and folds it in with
// an integer atomic max on the float bits (exact for non-negative floats and
// independent of order, hence deterministic), launch 3 writes the codes,
// launch 4 turns the maximum into the scale a / 448 (1 if a == 0).
#include "common.h"
#include "kernels.h"

namespace attn {

namespace {

constexpr float kE4M3Max = 448.0f;

template <typename T>
__device__ __forceinline__ void load8(const T* p, float* out) {
  const uint4 raw = *(const uint4*)p;
  const T* e = (const T*)&raw;
#pragma unroll
  for (int i = 0; i < 8; i++) out[i] = (float)e[i];
}

// four floats -> four E4M3 codes in one dword (byte i = code of x[i])
__device__ __forceinline__ uint32_t cvt4(float a, float b, float c, float d) {
  a = fminf(fmaxf(a, -kE4M3Max), kE4M3Max);
  b = fminf(fmaxf(b, -kE4M3Max), kE4M3Max);
  c = fminf(fmaxf(c, -kE4M3Max), kE4M3Max);
  d = fminf(fmaxf(d, -kE4M3Max), kE4M3Max);
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
  w = __builtin_amdgcn_cvt_pk_fp8_f32(c, d, w, true);
  return (uint32_t)w;
}

template <typename T, int D>
__global__ void __launch_bounds__(256)
hadamard_quant_kernel(const T* __restrict__ X, uint8_t* __restrict__ X8, float* __restrict__ scales,
                      const signed char* __restrict__ signs, int S, int block_rows, int n_blk,
                      int apply, float rsqrt_d)
{
  constexpr int LPR = D / 8;                 // lanes per row
  constexpr int RPP = 256 / LPR;             // rows per pass of the workgroup
  __shared__ float red[4];
  const int tid = threadIdx.x;
  const int sub = tid % LPR;                 // position of this lane within its row
  const int rsub = tid / LPR;
  const int blk = blockIdx.x % n_blk;
  const int bh = blockIdx.x / n_blk;
  const int r0 = blk * block_rows;
  const int r1 = min(S, r0 + block_rows);
  const size_t base = (size_t)bh * S * D;

  float sg[8];
#pragma unroll
  for (int i = 0; i < 8; i++) sg[i] = apply ? (float)signs[sub * 8 + i] : 1.0f;

  // pass 1: transform every row of the block, track max |u|
  float amax = 0.0f;
  for (int r = r0 + rsub; r < r1; r += RPP) {
    float u[8];
    load8(X + base + (size_t)r * D + sub * 8, u);
    if (apply) {
#pragma unroll
      for (int i = 0; i < 8; i++) u[i] *= sg[i];
      // strides 1, 2, 4 inside the lane
#pragma unroll
      for (int h = 1; h < 8; h <<= 1)
#pragma unroll
        for (int i = 0; i < 8; i++)
          if ((i & h) == 0) {
            const float a = u[i], b = u[i + h];
            u[i] = a + b;
            u[i + h] = a - b;
          }
      // strides 8 .. D/2 across lanes of the row
#pragma unroll
      for (int lh = 1; lh < LPR; lh <<= 1) {
        const bool upper = (sub & lh) != 0;
#pragma unroll
        for (int i = 0; i < 8; i++) {
          const float other = __shfl_xor(u[i], lh);
          u[i] = upper ? other - u[i] : u[i] + other;
        }
      }
    }
#pragma unroll
    for (int i = 0; i < 8; i++) amax = fmaxf(amax, fabsf(u[i]));
  }
  // block maximum
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) amax = fmaxf(amax, __shfl_xor(amax, off));
  if ((tid & 63) == 0) red[tid >> 6] = amax;
  __syncthreads();
  const float a = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  const bool nz = a > 0.0f;
  const float inv = nz ? __fdiv_rn(kE4M3Max, a) : 0.0f;

  // pass 2: recompute (cheap, the block is in cache) and quantize
  for (int r = r0 + rsub; r < r1; r += RPP) {
    float u[8];
    load8(X + base + (size_t)r * D + sub * 8, u);
    if (apply) {
#pragma unroll
      for (int i = 0; i < 8; i++) u[i] *= sg[i];
#pragma unroll
      for (int h = 1; h < 8; h <<= 1)
#pragma unroll
        for (int i = 0; i < 8; i++)
          if ((i & h) == 0) {
            const float x0 = u[i], x1 = u[i + h];
            u[i] = x0 + x1;
            u[i + h] = x0 - x1;
          }
#pragma unroll
      for (int lh = 1; lh < LPR; lh <<= 1) {
        const bool upper = (sub & lh) != 0;
#pragma unroll
        for (int i = 0; i < 8; i++) {
          const float other = __shfl_xor(u[i], lh);
          u[i] = upper ? other - u[i] : u[i] + other;
        }
      }
    }
    uint2 w = make_uint2(0u, 0u);              // an all-zero block has all-zero codes
    if (nz) {
      w.x = cvt4(u[0] * inv, u[1] * inv, u[2] * inv, u[3] * inv);
      w.y = cvt4(u[4] * inv, u[5] * inv, u[6] * inv, u[7] * inv);
    }
    *(uint2*)(X8 + base + (size_t)r * D + sub * 8) = w;
  }
  if (tid == 0) {
    float sc = nz ? __fdiv_rn(a, kE4M3Max) : 1.0f;
    if (apply && nz) sc = sc * rsqrt_d;
    scales[(size_t)bh * n_blk + blk] = sc;
  }
}

// x' = x * c - y * s, y' = y * c + x * s with every product and sum rounded
// on its own (no fused multiply-add: the result feeds the quantizer, whose
// codes must not depend on how the compiler contracts)
__device__ __forceinline__ void rotate(float& x, float& y, float c, float s) {
#pragma clang fp contract(off)
  const float xc = x * c, ys = y * s, yc = y * c, xs = x * s;
  x = xc - ys;
  y = yc + xs;
}

// one 64-row block per workgroup, four lanes per row (see the header);
// ROPE: 0 none, 1 rotary embedding on interleaved pairs, 2 on half pairs
template <typename T, int D, int ROPE>
__global__ void __launch_bounds__(256)
hadamard_quant64_kernel(const T* __restrict__ X, uint8_t* __restrict__ X8, float* __restrict__ scales,
                        const signed char* __restrict__ signs, int S, int n_blk, int apply, float rsqrt_d,
                        const float* __restrict__ cos_t, const float* __restrict__ sin_t)
{
  constexpr int NK = D / 32;                 // 8-element chunks per lane
  __shared__ float red[4];
  const int tid = threadIdx.x;
  const int sub = tid & 3;
  const int blk = blockIdx.x % n_blk;
  const int bh = blockIdx.x / n_blk;
  const int r = blk * 64 + (tid >> 2);
  const bool valid = r < S;
  const size_t row = ((size_t)bh * S + r) * D;

  float u[NK][8];
  if (valid) {
#pragma unroll
    for (int k = 0; k < NK; k++) load8(X + row + 32 * k + 8 * sub, u[k]);
  } else {
#pragma unroll
    for (int k = 0; k < NK; k++)
#pragma unroll
      for (int i = 0; i < 8; i++) u[k][i] = 0.0f;
  }
  // rotary embedding of position r (tables [S][D/2] float32) before the
  // transform: both coordinates of every pair sit in this lane
  if (ROPE != 0 && valid) {
    const float* cr = cos_t + (size_t)r * (D / 2);
    const float* sr = sin_t + (size_t)r * (D / 2);
    if (ROPE == 1) {                           // pairs (2j, 2j+1): j = 16k + 4*sub + i/2
#pragma unroll
      for (int k = 0; k < NK; k++) {
        const float4 c4 = *(const float4*)(cr + 16 * k + 4 * sub);
        const float4 s4 = *(const float4*)(sr + 16 * k + 4 * sub);
        rotate(u[k][0], u[k][1], c4.x, s4.x);
        rotate(u[k][2], u[k][3], c4.y, s4.y);
        rotate(u[k][4], u[k][5], c4.z, s4.z);
        rotate(u[k][6], u[k][7], c4.w, s4.w);
      }
    } else {                                   // pairs (j, j + D/2): chunks k and k + NK/2
#pragma unroll
      for (int k = 0; k < NK / 2; k++) {
        const float4 c0 = *(const float4*)(cr + 32 * k + 8 * sub), c1 = *(const float4*)(cr + 32 * k + 8 * sub + 4);
        const float4 s0 = *(const float4*)(sr + 32 * k + 8 * sub), s1 = *(const float4*)(sr + 32 * k + 8 * sub + 4);
        const float cc[8] = {c0.x, c0.y, c0.z, c0.w, c1.x, c1.y, c1.z, c1.w};
        const float ss[8] = {s0.x, s0.y, s0.z, s0.w, s1.x, s1.y, s1.z, s1.w};
#pragma unroll
        for (int i = 0; i < 8; i++) rotate(u[k][i], u[k + NK / 2][i], cc[i], ss[i]);
      }
    }
  }
  if (apply) {
#pragma unroll
    for (int k = 0; k < NK; k++) {
      const uint2 sw = *(const uint2*)(signs + 32 * k + 8 * sub);   // eight int8 signs
#pragma unroll
      for (int i = 0; i < 8; i++) {
        const uint32_t byte = ((i < 4 ? sw.x : sw.y) >> (8 * (i & 3))) & 0xffu;
        const uint32_t neg = (byte >> 7) << 31;                     // -1 -> sign bit set
        u[k][i] = __builtin_bit_cast(float, __builtin_bit_cast(uint32_t, u[k][i]) ^ neg);
      }
    }
    // strides 1, 2, 4: inside each chunk
#pragma unroll
    for (int h = 1; h < 8; h <<= 1)
#pragma unroll
      for (int k = 0; k < NK; k++)
#pragma unroll
        for (int i = 0; i < 8; i++)
          if ((i & h) == 0) {
            const float a = u[k][i], b = u[k][i + h];
            u[k][i] = a + b;
            u[k][i + h] = a - b;
          }
    // strides 8, 16: partner lane sub ^ 1, then sub ^ 2 (quad permutes 1,0,3,2 and 2,3,0,1)
#pragma unroll
    for (int lh = 1; lh < 4; lh <<= 1) {
      const bool upper = (sub & lh) != 0;
#pragma unroll
      for (int k = 0; k < NK; k++)
#pragma unroll
        for (int i = 0; i < 8; i++) {
          const int v = __builtin_bit_cast(int, u[k][i]);
          const int o = lh == 1 ? __builtin_amdgcn_mov_dpp(v, 0xB1, 0xF, 0xF, false)
                                : __builtin_amdgcn_mov_dpp(v, 0x4E, 0xF, 0xF, false);
          const float other = __builtin_bit_cast(float, o);
          u[k][i] = upper ? other - u[k][i] : u[k][i] + other;
        }
    }
    // strides 32, 64, 128: across chunks of the lane
#pragma unroll
    for (int h = 1; h < NK; h <<= 1)
#pragma unroll
      for (int k = 0; k < NK; k++)
        if ((k & h) == 0)
#pragma unroll
          for (int i = 0; i < 8; i++) {
            const float a = u[k][i], b = u[k + h][i];
            u[k][i] = a + b;
            u[k + h][i] = a - b;
          }
  }
  float amax = 0.0f;
#pragma unroll
  for (int k = 0; k < NK; k++)
#pragma unroll
    for (int i = 0; i < 8; i++) amax = fmaxf(amax, fabsf(u[k][i]));
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) amax = fmaxf(amax, __shfl_xor(amax, off));
  if ((tid & 63) == 0) red[tid >> 6] = amax;
  __syncthreads();
  const float a = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  const bool nz = a > 0.0f;
  const float inv = nz ? __fdiv_rn(kE4M3Max, a) : 0.0f;
  if (valid) {
#pragma unroll
    for (int k = 0; k < NK; k++) {
      uint2 w = make_uint2(0u, 0u);            // an all-zero block has all-zero codes
      if (nz) {
        w.x = cvt4(u[k][0] * inv, u[k][1] * inv, u[k][2] * inv, u[k][3] * inv);
        w.y = cvt4(u[k][4] * inv, u[k][5] * inv, u[k][6] * inv, u[k][7] * inv);
      }
      *(uint2*)(X8 + row + 32 * k + 8 * sub) = w;
    }
  }
  if (tid == 0) {
    float sc = nz ? __fdiv_rn(a, kE4M3Max) : 1.0f;
    if (apply && nz) sc = sc * rsqrt_d;
    scales[(size_t)bh * n_blk + blk] = sc;
  }
}

__global__ void clear_u32(uint32_t* p) { *p = 0u; }

template <typename T>
__global__ void __launch_bounds__(256)
amax_kernel(const T* __restrict__ X, size_t n8, uint32_t* __restrict__ amax_bits)
{
  __shared__ float red[4];
  float m = 0.0f;
  const size_t step = (size_t)gridDim.x * 256;
  size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
  for (; i + 7 * step < n8; i += 8 * step) {     // eight 16-byte loads in flight per thread
    float v[8][8];
#pragma unroll
    for (int j = 0; j < 8; j++) load8(X + (i + j * step) * 8, v[j]);
#pragma unroll
    for (int j = 0; j < 8; j++)
#pragma unroll
      for (int k = 0; k < 8; k++) m = fmaxf(m, fabsf(v[j][k]));
  }
  for (; i < n8; i += step) {
    float v[8];
    load8(X + i * 8, v);
#pragma unroll
    for (int k = 0; k < 8; k++) m = fmaxf(m, fabsf(v[k]));
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) m = fmaxf(m, __shfl_xor(m, off));
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
  __syncthreads();
  if (threadIdx.x == 0) {
    const float b = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
    atomicMax(amax_bits, __builtin_bit_cast(uint32_t, b));
  }
}

template <typename T>
__global__ void __launch_bounds__(256)
quant_kernel(const T* __restrict__ X, uint8_t* __restrict__ X8, size_t n8,
             const uint32_t* __restrict__ amax_bits)
{
  const float a = __builtin_bit_cast(float, *amax_bits);
  const float inv = a > 0.0f ? __fdiv_rn(kE4M3Max, a) : 0.0f;
  const size_t step = (size_t)gridDim.x * 256;
  size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
  auto put = [&](size_t c, const float* v) {
    uint2 w = make_uint2(0u, 0u);
    if (a > 0.0f) {
      w.x = cvt4(v[0] * inv, v[1] * inv, v[2] * inv, v[3] * inv);
      w.y = cvt4(v[4] * inv, v[5] * inv, v[6] * inv, v[7] * inv);
    }
    *(uint2*)(X8 + c * 8) = w;
  };
  for (; i + 7 * step < n8; i += 8 * step) {     // eight 16-byte loads in flight per thread
    float v[8][8];
#pragma unroll
    for (int j = 0; j < 8; j++) load8(X + (i + j * step) * 8, v[j]);
#pragma unroll
    for (int j = 0; j < 8; j++) put(i + j * step, v[j]);
  }
  for (; i < n8; i += step) {
    float v[8];
    load8(X + i * 8, v);
    put(i, v);
  }
}

// [B, H, S, D] -> codes [B, H, D, S]; one workgroup per (b*h, 64 x 64 tile)
template <typename T>
__global__ void __launch_bounds__(256)
quant_t_kernel(const T* __restrict__ X, uint8_t* __restrict__ X8, int S, int D,
               const uint32_t* __restrict__ amax_bits)
{
  __shared__ uint8_t tile[64][64 + 4];
  const float a = __builtin_bit_cast(float, *amax_bits);
  const float inv = a > 0.0f ? __fdiv_rn(kE4M3Max, a) : 0.0f;
  const int tS = (S + 63) / 64, tD = (D + 63) / 64;
  const int bh = blockIdx.x / (tS * tD);
  const int rem = blockIdx.x % (tS * tD);
  const int s0 = (rem / tD) * 64, d0 = (rem % tD) * 64;
  const size_t base = (size_t)bh * S * D;
  // read: 64 rows x 64 columns, 8 columns per thread
  for (int e = threadIdx.x; e < 64 * 8; e += 256) {
    const int r = e / 8, c8 = (e % 8) * 8;
    const int s = s0 + r, d = d0 + c8;
    if (s < S && d < D) {
      float v[8];
      load8(X + base + (size_t)s * D + d, v);
      const uint32_t w0 = a > 0.0f ? cvt4(v[0] * inv, v[1] * inv, v[2] * inv, v[3] * inv) : 0u;
      const uint32_t w1 = a > 0.0f ? cvt4(v[4] * inv, v[5] * inv, v[6] * inv, v[7] * inv) : 0u;
#pragma unroll
      for (int k = 0; k < 4; k++) {
        tile[c8 + k][r] = (w0 >> (8 * k)) & 255;
        tile[c8 + 4 + k][r] = (w1 >> (8 * k)) & 255;
      }
    }
  }
  __syncthreads();
  // write: 64 rows (d) x 64 columns (s), 4 bytes per thread
  for (int e = threadIdx.x; e < 64 * 16; e += 256) {
    const int dr = e / 16, sc = (e % 16) * 4;
    const int d = d0 + dr, s = s0 + sc;
    if (d < D && s < S) {
      const uint32_t w = tile[dr][sc] | (tile[dr][sc + 1] << 8) | (tile[dr][sc + 2] << 16) |
                         ((uint32_t)tile[dr][sc + 3] << 24);
      *(uint32_t*)(X8 + base + (size_t)d * S + s) = w;
    }
  }
}

__global__ void finish_scale_kernel(float* scale_and_bits) {
  const float a = __builtin_bit_cast(float, *(const uint32_t*)scale_and_bits);
  *scale_and_bits = a > 0.0f ? __fdiv_rn(a, kE4M3Max) : 1.0f;
}

template <typename T, int ROPE>
hipError_t hq64(const void* x, void* x8, float* scales, const signed char* signs, const float* cos_t,
                const float* sin_t, int B, int H, int S, int D, int apply, hipStream_t st) {
  const int n_blk = (S + 63) / 64;
  const dim3 grid((unsigned)(B * H * n_blk));
  const float r = (float)(1.0 / __builtin_sqrt((double)D));
  switch (D) {
    case 64:
      hipLaunchKernelGGL((hadamard_quant64_kernel<T, 64, ROPE>), grid, dim3(256), 0, st, (const T*)x,
                         (uint8_t*)x8, scales, signs, S, n_blk, apply, r, cos_t, sin_t);
      return hipGetLastError();
    case 128:
      hipLaunchKernelGGL((hadamard_quant64_kernel<T, 128, ROPE>), grid, dim3(256), 0, st, (const T*)x,
                         (uint8_t*)x8, scales, signs, S, n_blk, apply, r, cos_t, sin_t);
      return hipGetLastError();
    case 256:
      hipLaunchKernelGGL((hadamard_quant64_kernel<T, 256, ROPE>), grid, dim3(256), 0, st, (const T*)x,
                         (uint8_t*)x8, scales, signs, S, n_blk, apply, r, cos_t, sin_t);
      return hipGetLastError();
  }
  return hipErrorNotSupported;
}

template <typename T>
hipError_t hq_t(const void* x, void* x8, float* scales, const signed char* signs, int B, int H, int S,
                int D, int block_rows, int apply, hipStream_t st) {
  const int n_blk = (S + block_rows - 1) / block_rows;
  const dim3 grid((unsigned)(B * H * n_blk));
  const float r = (float)(1.0 / __builtin_sqrt((double)D));
  if (block_rows == 64) return hq64<T, 0>(x, x8, scales, signs, nullptr, nullptr, B, H, S, D, apply, st);
  switch (D) {
    case 64:
      hipLaunchKernelGGL((hadamard_quant_kernel<T, 64>), grid, dim3(256), 0, st, (const T*)x, (uint8_t*)x8,
                         scales, signs, S, block_rows, n_blk, apply, r);
      break;
    case 128:
      hipLaunchKernelGGL((hadamard_quant_kernel<T, 128>), grid, dim3(256), 0, st, (const T*)x, (uint8_t*)x8,
                         scales, signs, S, block_rows, n_blk, apply, r);
      break;
    case 256:
      hipLaunchKernelGGL((hadamard_quant_kernel<T, 256>), grid, dim3(256), 0, st, (const T*)x, (uint8_t*)x8,
                         scales, signs, S, block_rows, n_blk, apply, r);
      break;
    default:
      return hipErrorNotSupported;
  }
  return hipGetLastError();
}

template <typename T>
hipError_t qpt_t(const void* x, void* x8, float* scale, int B, int H, int S, int D, int transposed,
                 hipStream_t st) {
  uint32_t* bits = (uint32_t*)scale;            // the scale slot holds the running max until the end
  const size_t n8 = (size_t)B * H * S * D / 8;
  hipLaunchKernelGGL(clear_u32, dim3(1), dim3(1), 0, st, bits);
  const unsigned grid = (unsigned)(n8 < 2048 * 256 ? (n8 + 255) / 256 : 2048);
  // the maximum pass ends with one atomic per workgroup on a single word, so
  // it runs on few workgroups that each stream a long stretch (the whole
  // sequence on 64 MiB of bf16: 50 us with 2048 workgroups and four loads in
  // flight per thread, 32 us with 256 and eight, 30 us with 128 and eight)
  const unsigned grid_max = grid < 128 ? grid : 128;
  hipLaunchKernelGGL(amax_kernel<T>, dim3(grid_max), dim3(256), 0, st, (const T*)x, n8, bits);
  if (!transposed) {
    hipLaunchKernelGGL(quant_kernel<T>, dim3(grid), dim3(256), 0, st, (const T*)x, (uint8_t*)x8, n8,
                       (const uint32_t*)bits);
  } else {
    const int tiles = ((S + 63) / 64) * ((D + 63) / 64);
    hipLaunchKernelGGL(quant_t_kernel<T>, dim3((unsigned)(B * H * tiles)), dim3(256), 0, st, (const T*)x,
                       (uint8_t*)x8, S, D, (const uint32_t*)bits);
  }
  hipLaunchKernelGGL(finish_scale_kernel, dim3(1), dim3(1), 0, st, scale);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_hadamard_quant(const void* x, void* x8, float* scales, const signed char* signs, int B,
                                 int H, int S, int D, int block_rows, int apply_hadamard, int in_dtype,
                                 hipStream_t st) {
  if (in_dtype == 2) return hq_t<__bf16>(x, x8, scales, signs, B, H, S, D, block_rows, apply_hadamard, st);
  return hq_t<_Float16>(x, x8, scales, signs, B, H, S, D, block_rows, apply_hadamard, st);
}

hipError_t launch_rope_hadamard_quant(const void* x, void* x8, float* scales, const signed char* signs,
                                      const float* cos_t, const float* sin_t, int B, int H, int S, int D,
                                      int rope_mode, int in_dtype, hipStream_t st) {
  if (in_dtype == 2)
    return rope_mode == 0 ? hq64<__bf16, 1>(x, x8, scales, signs, cos_t, sin_t, B, H, S, D, 1, st)
                          : hq64<__bf16, 2>(x, x8, scales, signs, cos_t, sin_t, B, H, S, D, 1, st);
  return rope_mode == 0 ? hq64<_Float16, 1>(x, x8, scales, signs, cos_t, sin_t, B, H, S, D, 1, st)
                        : hq64<_Float16, 2>(x, x8, scales, signs, cos_t, sin_t, B, H, S, D, 1, st);
}

hipError_t launch_quant_per_tensor(const void* x, void* x8, float* scale, int B, int H, int S, int D,
                                   int in_dtype, int write_transposed, hipStream_t st) {
  if (in_dtype == 2) return qpt_t<__bf16>(x, x8, scale, B, H, S, D, write_transposed, st);
  return qpt_t<_Float16>(x, x8, scale, B, H, S, D, write_transposed, st);
}

}  // namespace attn

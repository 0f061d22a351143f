// Fused attention forward pass on E4M3 inputs (gfx950 FP8 matrix cores).
//
// The low-precision step of the pages ([NL] "3. Lage precisie (FP8) met
// reductie van kwantisatiefout"; [GN] "Niedrige FP8-Praezision und incoherent
// processing"): Q and K arrive as E4M3 codes with one float32 scale per 64
// rows of each (b, h) (after the random-sign Hadamard transform of
// hadamard_quant), V as E4M3 codes with one per-tensor scale. FP8 doubles the
// matrix rate while the exponential stays as expensive ([GN] "Ueberlappung von
// GEMM und Softmax durch Asynchronitaet"), so the softmax is now the longer
// phase and the ping-pong overlap matters more.
//
// Same schedule as the bf16 kernel (8 waves x 32 query rows, two groups
// alternating matrix and softmax phases at workgroup barriers, stage t =
// {K(t), V(t-1)} fetched straight into LDS by group 0), with:
//
// * v_mfma_scale_f32_32x32x64_f8f6f4 (unit scales): S^T = K Q^T takes A =
//   32 keys x 64 d of K from LDS (two 16-byte reads per lane) and B = Q^T from
//   VGPRs; O^T = V^T P^T takes A = 32 d x 64 keys of V^T, assembled with four
//   ds_read_b64_tr_b8 per fragment from V kept in its [S][D] layout, and B =
//   P^T converted from the S^T accumulator.
//
// * Scores: s = scale * qs * ks * (q8 . k8), with qs the block scale of this
//   wave's 32 rows and ks that of each 64-key half of the 128-key tile; the
//   product of the scales and log2(e) is one multiplier per half, folded into
//   the exp2 argument. P is rounded to E4M3 as p * 2^7 (the factor is added to
//   the exponent for free) so small probabilities stay out of the subnormal
//   range; the row sum l is accumulated from the unrounded p * 2^7, and the
//   2^7 cancels in O = acc * vs / l. The running maximum moves whenever a row
//   exceeds it by more than 1.75 (log2), which keeps p * 2^7 <= 430 < 448.
//   At each move the row's largest p is exactly 2^7, which E4M3 holds without
//   rounding; a larger threshold with a smaller factor would make O rescales
//   rarer but lets more small p fall into the subnormal range (2^7 and 1.75
//   leave the O error of N(0,1) inputs unchanged to within 2 %, with about a
//   third fewer rescales than 2^8 and 0.75).
//
// * The transposed V read picks, for element r of read p, the key row that
//   the P fragment holds in that k slot: P^T slot t of lane half h is key
//   64c + 32(t/16) + 8((t%16)/4) + 4h + t%4 of chunk c (the S^T accumulator
//   order), and ds_read_b64_tr_b8 gives lane i element r from the address of
//   lane 2r + i/8 of its 16-lane group, so lane j addresses the key row of
//   slot 8p + j/2 at column 8*(j%2).
//
// * LDS: K and V tiles [128][128 bytes], 16-byte-chunk XOR swizzles chosen so
//   that the K reads (16 lanes per LDS cycle over 16 rows) and the transposed
//   V reads (32 lanes over 8 rows x 32 bytes) hit all 64 banks once.
#include "common.h"
#include "kernels.h"

namespace attn {

namespace {

constexpr int D8 = 128;                 // head dimension (bytes per FP8 row)
constexpr int BN8 = 128;                // keys per tile
constexpr int KB8 = BN8 / 32;           // 32-key blocks per tile
constexpr int PC8 = BN8 / 64;           // 64-key chunks per tile (one P V k-step each)
constexpr int DB8 = D8 / 32;            // 32-row blocks of O^T
constexpr int TILE8 = BN8 * D8;         // bytes per K or V tile
constexpr int STAGE8 = 2 * TILE8;
constexpr int LDS8 = 2 * STAGE8;
constexpr float kTau8 = 1.75f;          // keeps p * 2^7 <= 2^8.75 < 448
constexpr float kPShift8 = 7.0f;        // P is quantized as p * 2^7
constexpr int kVmcnt0_8 = 0x0070 | 0x0F00;

__device__ __forceinline__ int k8_swz(int r) { return (r >> 1) & 7; }
__device__ __forceinline__ int v8_swz(int r) { return 2 * (((r >> 1) & 1) | ((r >> 2) & 2)); }

__device__ __forceinline__ v16f mma8(v8i a, v8i b, v16f c) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 127, 0, 127);
}

__device__ __forceinline__ uint32_t pack_fp8(float a, float b, float c, float d) {
  // the first conversion writes the low half and keeps the high half of its
  // "old" operand, which the second one overwrites: any register will do
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, __builtin_bit_cast(int, d), false);
  w = __builtin_amdgcn_cvt_pk_fp8_f32(c, d, w, true);
  return (uint32_t)w;
}

template <bool CAUSAL>
__global__ void __launch_bounds__(512)
__attribute__((amdgpu_waves_per_eu(2, 2)))
fwd_fp8_kernel(const uint8_t* __restrict__ Q8, const uint8_t* __restrict__ K8, const uint8_t* __restrict__ V8,
               const float* __restrict__ qs, const float* __restrict__ ks, const float* __restrict__ vs,
               __bf16* __restrict__ O, float* __restrict__ LSE, int BH, int S_q, int S_k, int n_qt, float c)
{
  __shared__ __attribute__((aligned(1024))) char lds[LDS8];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int grp = wave >> 2;
  const int hh = lane >> 5;
  const int nn = lane & 31;

  const int n_work = BH * n_qt;
  const int work = xcd_swizzle(blockIdx.x, n_work);
  int qt = work % n_qt;
  const int bh = work / n_qt;
  if (CAUSAL) qt = n_qt - 1 - qt;
  const int q0 = qt * 256;
  const int wr0 = q0 + wave * 32;
  const int diag = S_k - S_q;
  int k_end = S_k;
  if (CAUSAL) k_end = min(k_end, q0 + 255 + diag + 1);
  const int n_tiles = (k_end + BN8 - 1) / BN8;
  const int nq_blk = (S_q + 63) / 64, nk_blk = (S_k + 63) / 64;

  const size_t qoff = (size_t)bh * S_q * D8;
  const size_t koff = (size_t)bh * S_k * D8;
  const uint8_t* Kh = K8 + koff;
  const uint8_t* Vh = V8 + koff;
  const float c_q = c * qs[(size_t)bh * nq_blk + min(wr0, S_q - 1) / 64];
  const float* ksh = ks + (size_t)bh * nk_blk;
  const float v_scale = *vs;

  // Q^T fragments: lane (h, n) holds bytes 64*ks + 32*h .. +31 of query row n
  v8i qf[2];
  {
    const int q = wr0 + nn;
#pragma unroll
    for (int k2 = 0; k2 < 2; k2++) {
      if (q < S_q) {
        const uint4* src = (const uint4*)(Q8 + qoff + (size_t)q * D8 + 64 * k2 + 32 * hh);
        const uint4 lo = src[0], hi = src[1];
        qf[k2] = v8i{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
      } else {
        qf[k2] = v8i{0, 0, 0, 0, 0, 0, 0, 0};
      }
    }
  }

  // stage s = K(s), V(s-1) into buffer s & 1, issued by the 256 threads of
  // group 0 as buffer loads: 32-bit offsets from per-head resources (rows past
  // the key range read zeros, whose scores are masked), one add per load.
  const __amdgpu_buffer_rsrc_t krs = __builtin_amdgcn_make_buffer_rsrc((void*)Kh, (short)0, S_k * D8, 0x00020000);
  const __amdgpu_buffer_rsrc_t vrs = __builtin_amdgcn_make_buffer_rsrc((void*)Vh, (short)0, S_k * D8, 0x00020000);
  int dma_k[TILE8 / 4096], dma_v[TILE8 / 4096];   // this lane's byte offset within a tile
#pragma unroll
  for (int i = 0; i < TILE8 / 4096; i++) {
    const int r = (i * 4 + wave) * 8 + (lane >> 3);    // 8 rows of 128 bytes per 1 KiB wave load
    dma_k[i] = r * D8 + (((lane & 7) ^ k8_swz(r)) * 16);
    dma_v[i] = r * D8 + (((lane & 7) ^ v8_swz(r)) * 16);
  }
  // (offsets and destinations go through locals: a target builtin with
  // template-dependent argument expressions is dropped from the host pass)
  auto issue_stage = [&](int s) {
    char* base = lds + (s & 1) * STAGE8;
    if (s < n_tiles) {
      const int row0 = s * BN8 * D8;
#pragma unroll
      for (int i = 0; i < TILE8 / 4096; i++) {
        char* dst = base + (i * 4 + wave) * 1024;
        const int off = row0 + dma_k[i];
        __builtin_amdgcn_raw_ptr_buffer_load_lds(krs, (__attribute__((address_space(3))) void*)dst, 16, off, 0, 0, 0);
      }
    }
    if (s >= 1 && s - 1 < n_tiles) {
      const int row0 = (s - 1) * BN8 * D8;
#pragma unroll
      for (int i = 0; i < TILE8 / 4096; i++) {
        char* dst = base + TILE8 + (i * 4 + wave) * 1024;
        const int off = row0 + dma_v[i];
        __builtin_amdgcn_raw_ptr_buffer_load_lds(vrs, (__attribute__((address_space(3))) void*)dst, 16, off, 0, 0, 0);
      }
    }
  };

  // per-lane LDS read offsets
  const int xk = k8_swz(nn);
  int k_rd[4];                                   // chunk pairs (ks, h) of row nn
#pragma unroll
  for (int k2 = 0; k2 < 2; k2++)
#pragma unroll
    for (int e = 0; e < 2; e++) k_rd[2 * k2 + e] = nn * D8 + (((4 * k2 + 2 * hh + e) ^ xk) * 16);
  const int g = lane >> 4, jj = lane & 15;
  const int vrow = 8 * (jj >> 3) + 4 * hh + ((jj >> 1) & 3);
  const int xv = v8_swz(vrow);
  int v_rd[DB8];
#pragma unroll
  for (int db = 0; db < DB8; db++)
    v_rd[db] = vrow * D8 + (((2 * db + (g & 1)) ^ xv) * 16) + 8 * (jj & 1);

  v16f o[DB8];
#pragma unroll
  for (int db = 0; db < DB8; db++)
#pragma unroll
    for (int e = 0; e < 16; e++) o[db][e] = 0.0f;
  v16f s[KB8];
  v8i pf[PC8];
  float m = kNegInf, l = 0.0f;

  auto tile_active = [&](int t) { return !CAUSAL || t * BN8 <= wr0 + 31 + diag; };

  auto gemm_phase = [&](int t) {
    const char* st = lds + (t & 1) * STAGE8;
    if (t >= 1 && tile_active(t - 1)) {
      const char* vl = st + TILE8;
#pragma unroll
      for (int pc = 0; pc < PC8; pc++)
#pragma unroll
        for (int db = 0; db < DB8; db++) {
          v2i part[4];
#pragma unroll
          for (int p = 0; p < 4; p++) {
            const int row0 = 64 * pc + 32 * (p >> 1) + 16 * (p & 1);
            part[p] = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_v2i*)(vl + v_rd[db] + row0 * D8));
          }
          const v8i a = {part[0][0], part[0][1], part[1][0], part[1][1],
                         part[2][0], part[2][1], part[3][0], part[3][1]};
          o[db] = mma8(a, pf[pc], o[db]);
          __builtin_amdgcn_sched_barrier(0);
        }
    }
    if (t < n_tiles && tile_active(t)) {
#pragma unroll
      for (int k2 = 0; k2 < 2; k2++)
#pragma unroll
        for (int kb = 0; kb < KB8; kb++) {
          const char* kp = st + kb * 32 * D8;
          const uint4 lo = *(const uint4*)(kp + k_rd[2 * k2]);
          const uint4 hi = *(const uint4*)(kp + k_rd[2 * k2 + 1]);
          const v8i a = {(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
          if (k2 == 0) {
            const v16f zero = {};
            s[kb] = mma8(a, qf[0], zero);
          } else {
            s[kb] = mma8(a, qf[1], s[kb]);
          }
          __builtin_amdgcn_sched_barrier(0);
        }
    }
  };

  auto softmax_phase = [&](int t) {
    if (t < 0 || t >= n_tiles || !tile_active(t)) return;
    const int key0 = t * BN8;
    const float c0 = c_q * ksh[min(key0, S_k - 1) / 64];
    const float c1 = c_q * ksh[min(key0 + 64, S_k - 1) / 64];
    const bool need_mask = (key0 + BN8 > S_k) || (CAUSAL && key0 + BN8 - 1 > wr0 + diag);
    if (need_mask) {
      const int q = wr0 + nn;
#pragma unroll
      for (int kb = 0; kb < KB8; kb++)
#pragma unroll
        for (int i = 0; i < 4; i++)
#pragma unroll
          for (int j = 0; j < 4; j++) {
            const int key = key0 + kb * 32 + 8 * i + 4 * hh + j;
            const bool ok = key < S_k && (!CAUSAL || key <= q + diag);
            if (!ok) s[kb][4 * i + j] = kNegInf;
          }
    }
    // running maxima as plain chains, which compile to v_max3 (a pairwise
    // max of two matrix results costs an extra canonicalizing max each)
    float x0 = kNegInf, x1 = kNegInf;
#pragma unroll
    for (int e = 0; e < 16; e++) x0 = fmaxf(x0, s[0][e]);
#pragma unroll
    for (int e = 0; e < 16; e++) x0 = fmaxf(x0, s[1][e]);
#pragma unroll
    for (int e = 0; e < 16; e++) x1 = fmaxf(x1, s[2][e]);
#pragma unroll
    for (int e = 0; e < 16; e++) x1 = fmaxf(x1, s[3][e]);
    const float x = pair_max(fmaxf(x0 * c0, x1 * c1));
    if (__any(x > m + kTau8)) {
      const float mnew = fmaxf(m, x);
      const float ref = mnew == kNegInf ? 0.0f : mnew;
      const float alpha = fast_exp2(m - ref);
      m = mnew;
      l *= alpha;
#pragma unroll
      for (int db = 0; db < DB8; db++)
#pragma unroll
        for (int e = 0; e < 16; e++) o[db][e] *= alpha;
    }
    const float ref = (m == kNegInf ? 0.0f : m) - kPShift8;   // p * 2^7 = 2^(s*c - m + 7)
    float ls = 0.0f;
#pragma unroll
    for (int pc = 0; pc < PC8; pc++) {
      const float cc = pc == 0 ? c0 : c1;
      uint32_t w[8];
#pragma unroll
      for (int half = 0; half < 2; half++)
#pragma unroll
        for (int q4 = 0; q4 < 4; q4++) {
          float p[4];
#pragma unroll
          for (int e = 0; e < 4; e++) {
            p[e] = fast_exp2(__builtin_fmaf(s[2 * pc + half][4 * q4 + e], cc, -ref));
            ls += p[e];
          }
          w[4 * half + q4] = pack_fp8(p[0], p[1], p[2], p[3]);
        }
      pf[pc] = v8i{(int)w[0], (int)w[1], (int)w[2], (int)w[3], (int)w[4], (int)w[5], (int)w[6], (int)w[7]};
    }
    l += ls;
  };

  auto barrier = [] {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
    asm volatile("" ::: "memory");
  };
  if (n_tiles > 0) {
    if (grp == 0) issue_stage(0);
    __builtin_amdgcn_s_waitcnt(kVmcnt0_8);
    __syncthreads();
    if (grp == 1) barrier();
    for (int j = 0; j <= n_tiles; j++) {
      __builtin_amdgcn_s_setprio(1);
      gemm_phase(j);
      __builtin_amdgcn_s_setprio(0);
      barrier();
      if (grp == 0) issue_stage(j + 1);
      softmax_phase(j);
      __builtin_amdgcn_s_waitcnt(kVmcnt0_8);
      barrier();
    }
    if (grp == 0) barrier();
  }

  // epilogue: O = acc * vs / l (the 2^7 of p cancels), LSE = ln2 * (m + log2 l - 7)
  const int q = wr0 + nn;
  const float lt = pair_sum(l);
  const bool has = m != kNegInf && lt > 0.0f;
  const float inv = has ? v_scale / lt : 0.0f;
  const float lse = has ? (m + __builtin_log2f(lt) - kPShift8) * kLn2 : kNegInf;
  if (q < S_q) {
    __bf16* orow = O + qoff + (size_t)q * D8;
#pragma unroll
    for (int db = 0; db < DB8; db++)
#pragma unroll
      for (int i = 0; i < 4; i++) {
        typedef __bf16 v4b __attribute__((ext_vector_type(4)));
        v4b w4;
#pragma unroll
        for (int j = 0; j < 4; j++) w4[j] = (__bf16)(o[db][4 * i + j] * inv);
        *(v4b*)(orow + db * 32 + 8 * i + 4 * hh) = w4;
      }
    if (hh == 0) LSE[(size_t)bh * S_q + q] = lse;
  }
}

}  // namespace

hipError_t launch_fwd_fp8(const void* q8, const void* k8, const void* v8, const float* qs, const float* ks,
                          const float* vs, void* o, float* lse, int B, int H, int S_q, int S_k, int D,
                          int causal, float c, int v_transposed, hipStream_t st) {
  if (D != D8 || v_transposed) return hipErrorNotSupported;
  if ((long long)(S_k + BN8) * D8 > 0x7fffffffLL) return hipErrorInvalidValue;   // 32-bit buffer offsets
  const int n_qt = (S_q + 255) / 256;
  const dim3 grid((unsigned)(B * H * n_qt));
  if (causal)
    hipLaunchKernelGGL(fwd_fp8_kernel<true>, grid, dim3(512), 0, st, (const uint8_t*)q8, (const uint8_t*)k8,
                       (const uint8_t*)v8, qs, ks, vs, (__bf16*)o, lse, B * H, S_q, S_k, n_qt, c);
  else
    hipLaunchKernelGGL(fwd_fp8_kernel<false>, grid, dim3(512), 0, st, (const uint8_t*)q8, (const uint8_t*)k8,
                       (const uint8_t*)v8, qs, ks, vs, (__bf16*)o, lse, B * H, S_q, S_k, n_qt, c);
  return hipGetLastError();
}

}  // namespace attn

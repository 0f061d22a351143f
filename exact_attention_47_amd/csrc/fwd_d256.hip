// Fused exact attention forward pass for head dimension 256 (bf16 / fp16).
//
// Same method and operand layout as the ping-pong kernel (transposed GEMMs
// S^T = K Q^T and O^T = V^T P^T on v_mfma_f32_32x32x16, one lane per query
// row, base-2 online softmax with lazy rescaling, [NL] "FlashAttention en
// FlashAttention-2"; [GN] "Rueckblick auf den FlashAttention-Ansatz"), with a
// simpler schedule: at D = 256, Q^T (64 VGPRs) and O^T (128 VGPRs) leave too
// few of the 256 registers of two waves per SIMD for the ping-pong's extra
// live state, and the matrix work per key tile is four times the softmax
// work, so a single barrier per tile with register-staged loads suffices.
//
// Work split: 8 waves x 32 query rows per workgroup, 32-key tiles, two LDS
// buffers; the global loads of tile t+1 go to registers before tile t is
// computed and are written to the other buffer after it. LDS rows are
// padded (K: 2*D + 16 bytes, V: 2*D + 64 bytes) so that the K reads (16 lanes
// per cycle over 16 rows) and the transposed V reads (32 lanes per cycle over
// 4 rows x 64 bytes) fall on distinct banks of the 64-bank LDS.
#include "common.h"
#include "kernels.h"

namespace attn {

template <typename T> struct Mma256;
template <> struct Mma256<__bf16> {
  typedef v8bf16 frag;
  static __device__ __forceinline__ v16f mma(frag a, frag b, v16f c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
  }
  static __device__ __forceinline__ frag cvt(v8f x) { return __builtin_convertvector(x, v8bf16); }
};
template <> struct Mma256<_Float16> {
  typedef v8f16 frag;
  static __device__ __forceinline__ v16f mma(frag a, frag b, v16f c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
  }
  static __device__ __forceinline__ frag cvt(v8f x) { return __builtin_convertvector(x, v8f16); }
};

template <int D, int QB, int NW_, int BN_>
struct Cfg256 {
  static constexpr int NW = NW_;                // waves per workgroup
  static constexpr int NT = NW * 64;            // threads per workgroup
  static constexpr int RPW = 32 * QB;           // query rows per wave
  static constexpr int BM = NW * RPW;           // query rows per workgroup
  static constexpr int BN = BN_;                // keys per tile
  static constexpr int KB = BN / 32;            // 32-key blocks per tile
  static constexpr int DS = D / 16;             // k-steps of the S^T product
  static constexpr int DB = D / 32;             // 32-wide column blocks of O^T
  static constexpr int CH = D / 8;              // 16-byte chunks per row
  static constexpr int KS = 2 * D + 16;         // K row stride in LDS (bytes)
  static constexpr int VS = 2 * D + 64;         // V row stride in LDS (bytes)
  static constexpr int KT = BN * KS;            // K tile bytes
  static constexpr int VT = BN * VS;            // V tile bytes
  static constexpr int STAGE = KT + VT;
  static constexpr int LDS = 2 * STAGE;
  static constexpr int NCH = BN * CH / NT;      // 16-byte chunks per thread per tile
  static_assert(BN * CH % NT == 0, "tile chunks must divide evenly over the threads");
};

constexpr float kTau256 = 8.0f;   // lazy-rescale threshold, log2 domain

template <typename T, int D, int QB, int NW, int BN, bool CAUSAL, bool SPLIT>
__global__ void __launch_bounds__(NW * 64)
__attribute__((amdgpu_waves_per_eu(NW / 4, NW / 4)))
fwd_d256_kernel(const T* __restrict__ Q, const T* __restrict__ K, const T* __restrict__ V,
                T* __restrict__ O, float* __restrict__ LSE,
                float* __restrict__ Opart, float* __restrict__ Lpart,
                int BH, int S_q, int S_k, int n_qt, int n_split, int keys_per_split, float c)
{
  using C = Cfg256<D, QB, NW, BN>;
  using M = Mma256<T>;
  typedef typename M::frag frag;
  __shared__ __attribute__((aligned(16))) char lds[C::LDS];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int hh = lane >> 5;        // lane half
  const int nn = lane & 31;        // query column owned by this lane

  // ---- which (b*h, q tile, split) this workgroup computes
  const int n_work = BH * n_qt * n_split;
  int work = xcd_swizzle(blockIdx.x, n_work);
  const int split = work % n_split;
  work /= n_split;
  int qt = work % n_qt;
  const int bh = work / n_qt;
  if (CAUSAL) qt = n_qt - 1 - qt;  // heaviest query tiles first

  const int q0 = qt * C::BM;
  const int wr0 = q0 + wave * C::RPW;          // first row of this wave
  const int diag = S_k - S_q;                  // causal: key j allowed iff j <= i + diag
  int k_lo = 0, k_hi = S_k;
  if (SPLIT) {
    k_lo = split * keys_per_split;
    k_hi = min(S_k, k_lo + keys_per_split);
  }
  int k_end = k_hi;
  if (CAUSAL) k_end = min(k_end, q0 + C::BM - 1 + diag + 1);
  const int n_tiles = k_end > k_lo ? (k_end - k_lo + C::BN - 1) / C::BN : 0;

  const size_t qoff = (size_t)bh * S_q * D;
  const size_t koff = (size_t)bh * S_k * D;
  const T* Qh = Q + qoff;
  const T* Kh = K + koff;
  const T* Vh = V + koff;

  // ---- Q^T fragments (B operand of S^T), kept in registers
  frag qf[QB][C::DS];
#pragma unroll
  for (int qb = 0; qb < QB; qb++) {
    const int q = wr0 + qb * 32 + nn;
#pragma unroll
    for (int ds = 0; ds < C::DS; ds++) {
      if (q < S_q) {
        qf[qb][ds] = *(const frag*)(Qh + (size_t)q * D + ds * 16 + 8 * hh);
      } else {
#pragma unroll
        for (int e = 0; e < 8; e++) qf[qb][ds][e] = (T)0.0f;
      }
    }
  }

  // ---- global -> register staging of one K/V tile
  uint4 kst[C::NCH], vst[C::NCH];
  auto gload = [&](int key0) {
#pragma unroll
    for (int i = 0; i < C::NCH; i++) {
      const int id = i * C::NT + tid;
      const int r = id / C::CH, cc = id % C::CH;
      const int key = key0 + r;
      if (key < k_hi) {
        kst[i] = *(const uint4*)(Kh + (size_t)key * D + cc * 8);
        vst[i] = *(const uint4*)(Vh + (size_t)key * D + cc * 8);
      } else {
        kst[i] = make_uint4(0, 0, 0, 0);
        vst[i] = make_uint4(0, 0, 0, 0);
      }
    }
  };
  auto swrite = [&](int buf) {
    char* kb = lds + buf * C::STAGE;
    char* vb = kb + C::KT;
#pragma unroll
    for (int i = 0; i < C::NCH; i++) {
      const int id = i * C::NT + tid;
      const int r = id / C::CH, cc = id % C::CH;
      *(uint4*)(kb + r * C::KS + cc * 16) = kst[i];
      *(uint4*)(vb + r * C::VS + cc * 16) = vst[i];
    }
  };

  // per-lane LDS bases
  const int kbase = nn * C::KS + hh * 16;
  const int g = lane >> 4, jj = lane & 15;
  const int vbase = (4 * hh + (jj >> 2)) * C::VS + 32 * (g & 1) + 8 * (jj & 3);

  v16f o[QB][C::DB];
#pragma unroll
  for (int qb = 0; qb < QB; qb++)
#pragma unroll
    for (int db = 0; db < C::DB; db++)
#pragma unroll
      for (int e = 0; e < 16; e++) o[qb][db][e] = 0.0f;
  float m[QB], l[QB];
#pragma unroll
  for (int qb = 0; qb < QB; qb++) { m[qb] = kNegInf; l[qb] = 0.0f; }

  if (n_tiles > 0) {
    gload(k_lo);
    swrite(0);
  }
  __syncthreads();

  for (int t = 0; t < n_tiles; t++) {
    const int key0 = k_lo + t * C::BN;
    if (t + 1 < n_tiles) gload(key0 + C::BN);
    const char* kl = lds + (t & 1) * C::STAGE;
    const char* vl = kl + C::KT;

    // causal: this wave's rows may all precede the tile
    const bool active = !CAUSAL || key0 <= wr0 + C::RPW - 1 + diag;
    if (active) {
      // ---- S^T = K Q^T
      v16f s[C::KB][QB];
#pragma unroll
      for (int kb = 0; kb < C::KB; kb++)
#pragma unroll
        for (int qb = 0; qb < QB; qb++)
#pragma unroll
          for (int e = 0; e < 16; e++) s[kb][qb][e] = 0.0f;
#pragma unroll
      for (int ds = 0; ds < C::DS; ds++) {
#pragma unroll
        for (int kb = 0; kb < C::KB; kb++) {
          const frag a = *(const frag*)(kl + kbase + kb * 32 * C::KS + ds * 32);
#pragma unroll
          for (int qb = 0; qb < QB; qb++) s[kb][qb] = M::mma(a, qf[qb][ds], s[kb][qb]);
        }
      }

      // ---- mask: keys past the range end, and the causal diagonal
      const bool need_mask = (key0 + C::BN > k_hi) || (CAUSAL && key0 + C::BN - 1 > wr0 + diag);
      if (need_mask) {
#pragma unroll
        for (int kb = 0; kb < C::KB; kb++)
#pragma unroll
          for (int qb = 0; qb < QB; qb++) {
            const int q = wr0 + qb * 32 + nn;
#pragma unroll
            for (int i = 0; i < 4; i++)
#pragma unroll
              for (int j = 0; j < 4; j++) {
                const int key = key0 + kb * 32 + 8 * i + 4 * hh + j;
                const bool ok = key < k_hi && (!CAUSAL || key <= q + diag);
                if (!ok) s[kb][qb][4 * i + j] = kNegInf;
              }
          }
      }

      // ---- online softmax (base 2, scale folded into c)
      float mx[QB];
      bool grow = false;
#pragma unroll
      for (int qb = 0; qb < QB; qb++) {
        float x = kNegInf;
#pragma unroll
        for (int kb = 0; kb < C::KB; kb++)
#pragma unroll
          for (int e = 0; e < 16; e++) x = fmaxf(x, s[kb][qb][e]);
        x = pair_max(x) * c;
        mx[qb] = x;
        grow |= x > m[qb] + kTau256;
      }
      if (__any(grow)) {
#pragma unroll
        for (int qb = 0; qb < QB; qb++) {
          const float mnew = fmaxf(m[qb], mx[qb]);
          const float ref = mnew == kNegInf ? 0.0f : mnew;
          const float alpha = fast_exp2(m[qb] - ref);   // 0 when m was -inf
          m[qb] = mnew;
          l[qb] *= alpha;
#pragma unroll
          for (int db = 0; db < C::DB; db++)
#pragma unroll
            for (int e = 0; e < 16; e++) o[qb][db][e] *= alpha;
        }
      }
#pragma unroll
      for (int qb = 0; qb < QB; qb++) {
        const float ref = m[qb] == kNegInf ? 0.0f : m[qb];
        float ls = 0.0f;
#pragma unroll
        for (int kb = 0; kb < C::KB; kb++)
#pragma unroll
          for (int e = 0; e < 16; e++) {
            const float p = fast_exp2(__builtin_fmaf(s[kb][qb][e], c, -ref));
            s[kb][qb][e] = p;
            ls += p;
          }
        l[qb] += ls;
      }

      // ---- O^T += V^T P^T
#pragma unroll
      for (int kb = 0; kb < C::KB; kb++)
#pragma unroll
        for (int ks = 0; ks < 2; ks++) {
          frag pf[QB];
#pragma unroll
          for (int qb = 0; qb < QB; qb++) {
            v8f x;
#pragma unroll
            for (int e = 0; e < 8; e++) x[e] = s[kb][qb][8 * ks + e];
            pf[qb] = M::cvt(x);
          }
#pragma unroll
          for (int db = 0; db < C::DB; db++) {
            const int off = (kb * 32 + 16 * ks) * C::VS + db * 64;
            v4i16 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)(vl + vbase + off));
            v4i16 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)(vl + vbase + off + 8 * C::VS));
            v8i16 a16 = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
            const frag a = __builtin_bit_cast(frag, a16);
#pragma unroll
            for (int qb = 0; qb < QB; qb++) o[qb][db] = M::mma(a, pf[qb], o[qb][db]);
          }
        }
    }

    if (t + 1 < n_tiles) swrite((t + 1) & 1);
    __syncthreads();
  }

  // ---- epilogue: normalise, logsumexp, store
#pragma unroll
  for (int qb = 0; qb < QB; qb++) {
    const int q = wr0 + qb * 32 + nn;
    const float lt = pair_sum(l[qb]);
    const bool has = m[qb] != kNegInf && lt > 0.0f;
    const float inv = has ? 1.0f / lt : 0.0f;
    const float lse = has ? (m[qb] + __builtin_log2f(lt)) * kLn2 : kNegInf;
    if (q < S_q) {
      if (!SPLIT) {
        T* orow = O + qoff + (size_t)q * D;
#pragma unroll
        for (int db = 0; db < C::DB; db++)
#pragma unroll
          for (int i = 0; i < 4; i++) {
            typedef T v4t __attribute__((ext_vector_type(4)));
            v4t w;
#pragma unroll
            for (int j = 0; j < 4; j++) w[j] = (T)(o[qb][db][4 * i + j] * inv);
            *(v4t*)(orow + db * 32 + 8 * i + 4 * hh) = w;
          }
        if (hh == 0) LSE[(size_t)bh * S_q + q] = lse;
      } else {
        const size_t prow = ((size_t)split * BH + bh) * S_q + q;
        float* orow = Opart + prow * D;
#pragma unroll
        for (int db = 0; db < C::DB; db++)
#pragma unroll
          for (int i = 0; i < 4; i++) {
            float4 w;
            w.x = o[qb][db][4 * i + 0] * inv;
            w.y = o[qb][db][4 * i + 1] * inv;
            w.z = o[qb][db][4 * i + 2] * inv;
            w.w = o[qb][db][4 * i + 3] * inv;
            *(float4*)(orow + db * 32 + 8 * i + 4 * hh) = w;
          }
        if (hh == 0) Lpart[prow] = lse;
      }
    }
  }
}

// ---------------------------------------------------------------- launcher

template <typename T, bool CAUSAL, bool SPLIT>
static hipError_t launch_256(const FwdArgs& a, hipStream_t st) {
  using C = Cfg256<256, 1, 8, 32>;
  const int n_qt = (a.S_q + C::BM - 1) / C::BM;
  const int n_work = a.B * a.H * n_qt * a.n_split;
  hipLaunchKernelGGL((fwd_d256_kernel<T, 256, 1, 8, 32, CAUSAL, SPLIT>), dim3(n_work), dim3(C::NT), 0, st,
                     (const T*)a.q, (const T*)a.k, (const T*)a.v, (T*)a.o, a.lse, a.opart, a.lpart,
                     a.B * a.H, a.S_q, a.S_k, n_qt, a.n_split, a.keys_per_split, a.c);
  return hipGetLastError();
}

template <typename T>
static hipError_t launch_256_t(const FwdArgs& a, hipStream_t st) {
  const bool split = a.n_split > 1;
  if (a.causal) return split ? launch_256<T, true, true>(a, st) : launch_256<T, true, false>(a, st);
  return split ? launch_256<T, false, true>(a, st) : launch_256<T, false, false>(a, st);
}

int d256_keys_per_tile() { return 32; }

hipError_t launch_fwd_d256(const FwdArgs& a, hipStream_t st) {
  if (a.dtype == 2) return launch_256_t<__bf16>(a, st);
  return launch_256_t<_Float16>(a, st);
}

}  // namespace attn

// Fused exact attention forward pass for head dimension 256 (bf16 / fp16).
//
// Same method and operand layout as the ping-pong kernel (transposed GEMMs
// S^T = K Q^T and O^T = V^T P^T on v_mfma_f32_32x32x16, one lane per query
// row, base-2 online softmax with lazy rescaling, [NL] "FlashAttention en
// FlashAttention-2"; [GN] "Rueckblick auf den FlashAttention-Ansatz"), with a
// simpler schedule: at D = 256, Q^T (64 VGPRs) and O^T (128 VGPRs) leave too
// few of the 256 registers of two waves per SIMD for the ping-pong's extra
// live state, and the matrix work per key tile is four times the softmax
// work, so all eight waves run the same phases with one barrier per tile
// (both waves of a SIMD then issue matrix instructions together).
//
// Work split: 8 waves x 32 query rows per workgroup, BN-key tiles, two LDS
// stages held in two separate arrays (so the compiler can tell a direct load
// into one from a read of the other; the loop is unrolled by two). Tile t+1
// is fetched with buffer loads straight into LDS (no registers) while tile t
// is computed, and waited for before the tile's closing barrier. Rows are
// stored unpadded with a 16-byte-chunk XOR swizzle (K: chunk ^ (row & 15),
// V: chunk ^ 4 (row & 3)) so that the K reads (16 lanes per cycle over 16
// rows) and the transposed V reads (32 lanes per cycle over 4 rows x 64
// bytes) touch every bank of the 64-bank LDS once. Rows past the end of K/V
// read zeros (their scores are masked): the tile that reaches past the end
// is loaded with range-checked offsets.
//
// Packed batches (VARLEN): [total, H, D] rows H*D elements apart, each
// workgroup looking up its sequence's offsets; the load offsets step by that
// row pitch and the buffer range ends after the sequence's last row.
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
  static constexpr int RB = 2 * D;              // bytes per K/V row
  static constexpr int TILE = BN * RB;          // bytes per K or V tile
  static constexpr int STAGE = 2 * TILE;        // K(t) then V(t)
  static constexpr int NI = TILE / (NT * 16);   // direct-load instructions per thread per tile
  static constexpr int RPI = 1024 / RB;         // rows written by one wave instruction
  static_assert(TILE % (NT * 16) == 0, "tile must split evenly into 1 KiB wave loads");
  static_assert(RPI * NW % 8 == 0, "a lane's rows must step by a multiple of 8 between its loads");
};

constexpr float kTau256 = 8.0f;   // lazy-rescale threshold, log2 domain

template <typename T, int D, int QB, int NW, int BN, bool CAUSAL, bool SPLIT, bool VARLEN>
__global__ void __launch_bounds__(NW * 64)
__attribute__((amdgpu_waves_per_eu(2, 2)))   // two waves per SIMD: one 8-wave or two 4-wave workgroups per CU
fwd_d256_kernel(const T* __restrict__ Q, const T* __restrict__ K, const T* __restrict__ V,
                T* __restrict__ O, float* __restrict__ LSE,
                float* __restrict__ Opart, float* __restrict__ Lpart,
                int BH, int S_q_, int S_k_, int n_qt, int n_split, int keys_per_split, float c,
                const int* __restrict__ cu_q, const int* __restrict__ cu_k, int H, int total_q)
{
  static_assert(!(VARLEN && SPLIT), "packed batches run unsplit");
  using C = Cfg256<D, QB, NW, BN>;
  using M = Mma256<T>;
  typedef typename M::frag frag;
  __shared__ __attribute__((aligned(1024))) char st0[C::STAGE];
  __shared__ __attribute__((aligned(1024))) char st1[C::STAGE];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform (scalar offsets)
  const int hh = lane >> 5;        // lane half
  const int nn = lane & 31;        // query column owned by this lane

  // ---- which (b*h, q tile, split) this workgroup computes
  int split = 0, qt, bh;
  if (VARLEN) {
    // packed batches: XCD x takes heads x, x+8, ... one at a time with all
    // their query tiles (highest first) when B*H is a multiple of 8, so a
    // head's K and V stay in one L2; otherwise query tiles heaviest first
    // over all heads
    if (BH % 8 == 0) {
      const int x = blockIdx.x % 8, j = blockIdx.x / 8;
      bh = x + 8 * (j / n_qt);
      qt = n_qt - 1 - j % n_qt;
    } else {
      qt = n_qt - 1 - (int)(blockIdx.x / BH);
      bh = blockIdx.x % BH;
    }
  } else if (CAUSAL && !SPLIT && n_qt >= 16) {
    // query tiles heaviest first over all (b, h) at a time; consecutive
    // workgroups go to the 8 XCDs in turn, so (b, h) stays on XCD bh % 8
    // when B*H is a multiple of 8
    qt = n_qt - 1 - (int)(blockIdx.x / BH);
    bh = blockIdx.x % BH;
  } else {
    const int n_work = BH * n_qt * n_split;
    int work = xcd_swizzle(blockIdx.x, n_work);
    split = work % n_split;
    work /= n_split;
    qt = work % n_qt;
    bh = work / n_qt;
    if (CAUSAL) qt = n_qt - 1 - qt;  // heaviest query tiles first
  }

  const int q0 = qt * C::BM;
  const int wr0 = q0 + wave * C::RPW;          // first row of this wave

  // ---- where this (b, h) lives. Dense: [B, H, S, D], rows D elements apart.
  // Packed ([GN] "Weitere Optimierungen und kuenftige Integration" names
  // variable-length sequences): [total, H, D], sequence b at rows
  // cu[b] .. cu[b+1]-1, rows H*D elements apart; LSE is [H, total_q].
  int S_q = S_q_, S_k = S_k_;
  const int pitch = VARLEN ? H * D : D;        // elements between consecutive rows
  const T *Qh, *Kh, *Vh;
  T* Oh;
  float* lseh;
  if (VARLEN) {
    const int b = bh / H, h = bh % H;
    const int q_beg = cu_q[b], k_beg = cu_k[b];
    S_q = cu_q[b + 1] - q_beg;
    S_k = cu_k[b + 1] - k_beg;
    if (q0 >= S_q) return;                     // whole workgroup: past this sequence's rows
    Qh = Q + ((size_t)q_beg * H + h) * D;
    Kh = K + ((size_t)k_beg * H + h) * D;
    Vh = V + ((size_t)k_beg * H + h) * D;
    Oh = O + ((size_t)q_beg * H + h) * D;
    lseh = LSE + (size_t)h * total_q + q_beg;
  } else {
    Qh = Q + (size_t)bh * S_q * D;
    Kh = K + (size_t)bh * S_k * D;
    Vh = V + (size_t)bh * S_k * D;
    Oh = O + (size_t)bh * S_q * D;
    lseh = LSE + (size_t)bh * S_q;
  }
  const int RBg = pitch * (int)sizeof(T);      // bytes between consecutive rows in memory
  const int diag = S_k - S_q;                  // causal: key j allowed iff j <= i + diag
  int k_lo = 0, k_hi = S_k;
  if (SPLIT) {
    k_lo = split * keys_per_split;
    k_hi = min(S_k, k_lo + keys_per_split);
  }
  int k_end = k_hi;
  if (CAUSAL) k_end = min(k_end, q0 + C::BM - 1 + diag + 1);
  const int n_tiles = k_end > k_lo ? (k_end - k_lo + C::BN - 1) / C::BN : 0;

  // ---- Q^T fragments (B operand of S^T), kept in registers
  frag qf[QB][C::DS];
#pragma unroll
  for (int qb = 0; qb < QB; qb++) {
    const int q = wr0 + qb * 32 + nn;
#pragma unroll
    for (int ds = 0; ds < C::DS; ds++) {
      if (q < S_q) {
        qf[qb][ds] = *(const frag*)(Qh + (size_t)q * pitch + ds * 16 + 8 * hh);
      } else {
#pragma unroll
        for (int e = 0; e < 8; e++) qf[qb][ds][e] = (T)0.0f;
      }
    }
  }

  // ---- direct loads of one K/V tile: per-head buffer resources, one
  // lane-constant offset (a lane's rows step by a multiple of 16 between its
  // loads, which leaves both swizzles unchanged) plus wave-uniform scalars.
  // The range ends after the last row (packed rows are RBg bytes apart), so
  // rows past it read zeros.
  const int kv_bytes = VARLEN ? (S_k > 0 ? (S_k - 1) * RBg + C::RB : 0) : S_k * C::RB;
  const __amdgpu_buffer_rsrc_t krs = __builtin_amdgcn_make_buffer_rsrc((void*)Kh, (short)0, kv_bytes, 0x00020000);
  const __amdgpu_buffer_rsrc_t vrs = __builtin_amdgcn_make_buffer_rsrc((void*)Vh, (short)0, kv_bytes, 0x00020000);
  // with 4 waves a lane's rows step by 8 between its loads (ALT)
  constexpr bool ALT = (C::RPI * C::NW) % 16 != 0;
  static_assert(!(ALT && !SPLIT), "four-wave workgroups serve key-range splits only");
  int lane_k, lane_k1, lane_v;
  {
    const int rsub = (lane * 16) / C::RB;
    const int u = ((lane * 16) % C::RB) / 16;
    const int r = wave * C::RPI + rsub;
    lane_k = rsub * RBg + ((u ^ (r & 15)) * 16);
    // ALT: odd loads take the K swizzle of row r + 8 (the V swizzle repeats
    // every 4 rows)
    lane_k1 = ALT ? rsub * RBg + ((u ^ ((r + 8) & 15)) * 16) : lane_k;
    lane_v = rsub * RBg + ((u ^ (4 * (r & 3))) * 16);
  }
  // (offsets and destinations go through locals: a target builtin with
  // template-dependent argument expressions is dropped from the host pass)
  // The buffer range check covers the per-lane offset and not the scalar
  // one: a tile that reaches past the last row puts its whole offset in the
  // per-lane part (dense), or gets one resource per instruction based at the
  // instruction's first row with the bytes left after it as its range
  // (packed, where the per-lane offsets spilled), so that its rows past the
  // end read zeros.
  auto issue_tile = [&](int key0, char* base) {
    if (key0 + C::BN <= S_k) {
#pragma unroll
      for (int i = 0; i < C::NI; i++) {
        const int blk = i * C::NW + wave;
        char* kdst = base + blk * 1024;
        char* vdst = base + C::TILE + blk * 1024;
        const int soff = (key0 + blk * C::RPI) * RBg;
        if constexpr (ALT) {
          const int lk = (i & 1) ? lane_k1 : lane_k;
          __builtin_amdgcn_raw_ptr_buffer_load_lds(krs, (__attribute__((address_space(3))) void*)kdst, 16, lk,
                                                   soff, 0, 0);
        } else {
          __builtin_amdgcn_raw_ptr_buffer_load_lds(krs, (__attribute__((address_space(3))) void*)kdst, 16, lane_k,
                                                   soff, 0, 0);
        }
        __builtin_amdgcn_raw_ptr_buffer_load_lds(vrs, (__attribute__((address_space(3))) void*)vdst, 16, lane_v,
                                                 soff, 0, 0);
      }
    } else {
#pragma unroll
      for (int i = 0; i < C::NI; i++) {
        const int blk = i * C::NW + wave;
        char* kdst = base + blk * 1024;
        char* vdst = base + C::TILE + blk * 1024;
        if constexpr (VARLEN) {
          const int off = (key0 + blk * C::RPI) * RBg;
          const int left = kv_bytes > off ? kv_bytes - off : 0;
          const __amdgpu_buffer_rsrc_t k1 =
              __builtin_amdgcn_make_buffer_rsrc((void*)((const char*)Kh + off), (short)0, left, 0x00020000);
          const __amdgpu_buffer_rsrc_t v1 =
              __builtin_amdgcn_make_buffer_rsrc((void*)((const char*)Vh + off), (short)0, left, 0x00020000);
          const int lk = ALT && (i & 1) ? lane_k1 : lane_k;
          __builtin_amdgcn_raw_ptr_buffer_load_lds(k1, (__attribute__((address_space(3))) void*)kdst, 16, lk,
                                                   0, 0, 0);
          __builtin_amdgcn_raw_ptr_buffer_load_lds(v1, (__attribute__((address_space(3))) void*)vdst, 16, lane_v,
                                                   0, 0, 0);
        } else {
          const int koff = lane_k + (key0 + blk * C::RPI) * RBg;
          const int voff = lane_v + (key0 + blk * C::RPI) * RBg;
          __builtin_amdgcn_raw_ptr_buffer_load_lds(krs, (__attribute__((address_space(3))) void*)kdst, 16, koff,
                                                   0, 0, 0);
          __builtin_amdgcn_raw_ptr_buffer_load_lds(vrs, (__attribute__((address_space(3))) void*)vdst, 16, voff,
                                                   0, 0, 0);
        }
      }
    }
  };

  // per-lane LDS read offsets (swizzle folded in; it only reaches the low 4 /
  // 2 bits of the chunk index, so the offsets repeat every 8 k-steps / 4
  // column blocks up to a constant)
  int k_rd[8];
#pragma unroll
  for (int ds = 0; ds < 8; ds++) k_rd[ds] = nn * C::RB + (((2 * ds + hh) ^ (nn & 15)) * 16);
  const int g = lane >> 4, jj = lane & 15;
  const int vrow = 4 * hh + (jj >> 2);
  int v_rd[4];
#pragma unroll
  for (int db = 0; db < 4; db++)
    v_rd[db] = vrow * C::RB + (((4 * db + 2 * (g & 1) + ((jj & 3) >> 1)) ^ (4 * (vrow & 3))) * 16) + 8 * (jj & 1);

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

  // one tile: fetch tile t+1 into the other stage, compute tile t, wait for
  // this wave's loads, barrier
  auto step = [&](int t, const char* kl, char* nxt) {
    const int key0 = k_lo + t * C::BN;
    if (t + 1 < n_tiles) issue_tile(key0 + C::BN, nxt);
    const char* vl = kl + C::TILE;
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
            const frag a = *(const frag*)(kl + k_rd[ds % 8] + (ds / 8) * 256 + kb * 32 * C::RB);
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
        // a row's keys are split over the two halves of the wave: when
        // neither half's maximum passes the bound, the row's does not either,
        // so the exchange between the halves waits for a move
        float xh[QB];
        bool grow = false;
  #pragma unroll
        for (int qb = 0; qb < QB; qb++) {
          float x = kNegInf;
  #pragma unroll
          for (int kb = 0; kb < C::KB; kb++)
  #pragma unroll
            for (int e = 0; e < 16; e++) x = fmaxf(x, s[kb][qb][e]);
          xh[qb] = x;
          grow |= x * c > m[qb] + kTau256;
        }
        if (__any(grow)) {
  #pragma unroll
          for (int qb = 0; qb < QB; qb++) {
            const float mnew = fmaxf(m[qb], pair_max(xh[qb]) * c);
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
              const char* va = vl + v_rd[db % 4] + (db / 4) * 256 + (kb * 32 + 16 * ks) * C::RB;
              v4i16 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)va);
              v4i16 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)(va + 8 * C::RB));
              v8i16 a16 = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
              const frag a = __builtin_bit_cast(frag, a16);
  #pragma unroll
              for (int qb = 0; qb < QB; qb++) o[qb][db] = M::mma(a, pf[qb], o[qb][db]);
            }
          }
      }

    __builtin_amdgcn_s_waitcnt(0x0070 | 0x0F00);   // vmcnt(0): this wave's share of tile t+1
    __syncthreads();
  };
  if (n_tiles > 0) {
    issue_tile(k_lo, st0);
    __builtin_amdgcn_s_waitcnt(0x0070 | 0x0F00);
    __syncthreads();
    int t = 0;
    for (; t + 1 < n_tiles; t += 2) {
      step(t, st0, st1);
      step(t + 1, st1, st0);
    }
    if (t < n_tiles) step(t, st0, st1);
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
        T* orow = Oh + (size_t)q * pitch;
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
        if (hh == 0) lseh[q] = lse;
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

#ifndef D256_BN
#define D256_BN 32
#endif

template <typename T, bool CAUSAL, bool SPLIT, int NW>
static hipError_t launch_256_nw(const FwdArgs& a, hipStream_t st) {
  using C = Cfg256<256, 1, NW, D256_BN>;
  if ((long long)(a.S_k + C::BN) * C::RB > 0x7fffffffLL) return hipErrorInvalidValue;   // 32-bit buffer offsets
  const int n_qt = (a.S_q + C::BM - 1) / C::BM;
  const int n_work = a.B * a.H * n_qt * a.n_split;
  hipLaunchKernelGGL((fwd_d256_kernel<T, 256, 1, NW, D256_BN, CAUSAL, SPLIT, false>), dim3(n_work), dim3(C::NT), 0,
                     st, (const T*)a.q, (const T*)a.k, (const T*)a.v, (T*)a.o, a.lse, a.opart, a.lpart,
                     a.B * a.H, a.S_q, a.S_k, n_qt, a.n_split, a.keys_per_split, a.c, nullptr, nullptr, a.H, 0);
  return hipGetLastError();
}

// Eight-wave workgroups (256 rows); a key-range split of at most 128 query
// rows runs on four-wave workgroups (128 rows, two per CU), which carry half
// the idle rows (on full grids the eight-wave form is faster).
template <typename T, bool CAUSAL, bool SPLIT>
static hipError_t launch_256(const FwdArgs& a, hipStream_t st) {
  if constexpr (SPLIT) {
    if (a.S_q <= Cfg256<256, 1, 4, D256_BN>::BM) return launch_256_nw<T, CAUSAL, SPLIT, 4>(a, st);
  }
  return launch_256_nw<T, CAUSAL, SPLIT, 8>(a, st);
}

// packed batches: S_q / S_k are the longest sequences; the grid covers
// B*H*ceil(S_q / 256) workgroups, and those past their sequence exit at once
template <typename T, bool CAUSAL>
static hipError_t launch_256_varlen(const FwdArgs& a, hipStream_t st) {
  using C = Cfg256<256, 1, 8, D256_BN>;
  // 32-bit buffer offsets over H*D-element row steps
  if ((long long)(a.S_k + C::BN) * a.H * C::RB > 0x7fffffffLL) return hipErrorInvalidValue;
  const int n_qt = (a.S_q + C::BM - 1) / C::BM;
  const int n_work = a.B * a.H * n_qt;
  hipLaunchKernelGGL((fwd_d256_kernel<T, 256, 1, 8, D256_BN, CAUSAL, false, true>), dim3(n_work), dim3(C::NT), 0,
                     st, (const T*)a.q, (const T*)a.k, (const T*)a.v, (T*)a.o, a.lse, nullptr, nullptr,
                     a.B * a.H, a.S_q, a.S_k, n_qt, 1, 0, a.c, a.cu_q, a.cu_k, a.H, a.total_q);
  return hipGetLastError();
}

template <typename T>
static hipError_t launch_256_t(const FwdArgs& a, hipStream_t st) {
  const bool split = a.n_split > 1;
  if (a.causal) return split ? launch_256<T, true, true>(a, st) : launch_256<T, true, false>(a, st);
  return split ? launch_256<T, false, true>(a, st) : launch_256<T, false, false>(a, st);
}

int d256_keys_per_tile() { return D256_BN; }

hipError_t launch_fwd_d256(const FwdArgs& a, hipStream_t st) {
  if (a.dtype == 2) return launch_256_t<__bf16>(a, st);
  return launch_256_t<_Float16>(a, st);
}

hipError_t launch_fwd_d256_varlen(const FwdArgs& a, hipStream_t st) {
  if (a.dtype == 2)
    return a.causal ? launch_256_varlen<__bf16, true>(a, st) : launch_256_varlen<__bf16, false>(a, st);
  return a.causal ? launch_256_varlen<_Float16, true>(a, st) : launch_256_varlen<_Float16, false>(a, st);
}

}  // namespace attn

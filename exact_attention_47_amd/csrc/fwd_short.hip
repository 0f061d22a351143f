// Fused exact attention forward pass for short key ranges (bf16 / fp16,
// D = 64 / 128): three or four small workgroups per CU, each wave running its
// tiles in order.
//
// Same method as the main kernel (O = softmax(scale Q K^T [+ causal]) V and
// the row logsumexp by tiles with online softmax rescaling, [NL]
// "FlashAttention en FlashAttention-2"; [GN] "Rueckblick auf den
// FlashAttention-Ansatz") and the same transposed operand layout (S^T = K Q^T,
// O^T = V^T P^T, one lane per query row, base-2 softmax, lazy rescaling).
// What changes is the schedule, for key ranges of a few tiles, where the main
// kernel's one workgroup per CU leaves its start-up latency and memory waits
// exposed:
//
// * 4 waves x 32 query rows per workgroup and 32-key tiles, so three LDS
//   stages take 48 KiB (D = 128) or 24 KiB (D = 64). Each wave keeps only one
//   tile's scores and probabilities live (at most 168 VGPRs at D = 128, 112 at
//   D = 64), so three (D = 128) or four (D = 64) workgroups share a CU: one
//   wave of each per SIMD.
//
// * Each wave runs its tiles in order: S(t) = K(t) Q^T, mask (tiles that
//   need one, the key-range tail and the causal diagonal, are a suffix of a
//   wave's tiles and run in a second unrolled loop), online softmax, P(t) to
//   matrix fragments, O += V(t)^T P(t)^T. The overlap of matrix and vector
//   work ([GN] "Overlap innerhalb einer Warpgroup") comes from the other
//   waves of the SIMD, which are at other points of their steps. A software
//   pipeline inside each wave (exponentials of tile t between the MFMAs of
//   tile t+1) needs two tiles' scores live and so allowed only two waves per
//   SIMD; the plain order with three or four waves measured 7-33 % faster on
//   these ranges.
//
// * Stage j = {K(j), V(j)} lives in one of three separate __shared__ arrays
//   (so the compiler can tell the direct load into one from the reads of
//   another; the loop is unrolled by three). Stage t+2 is fetched with buffer
//   loads into the array that step t-1 finished with, and waited for at the
//   end of step t+1.
#include "common.h"
#include "kernels.h"


namespace attn {

namespace {

template <typename T> struct Mma;
template <> struct Mma<__bf16> {
  typedef v8bf16 frag;
  static __device__ __forceinline__ v16f mma(frag a, frag b, v16f c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
  }
  static __device__ __forceinline__ frag cvt(v8f x) { return __builtin_convertvector(x, v8bf16); }
};
template <> struct Mma<_Float16> {
  typedef v8f16 frag;
  static __device__ __forceinline__ v16f mma(frag a, frag b, v16f c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
  }
  static __device__ __forceinline__ frag cvt(v8f x) { return __builtin_convertvector(x, v8f16); }
};

template <int D>
struct ShortCfg {
  static constexpr int NW = 4;                  // waves per workgroup (one per SIMD)
  static constexpr int NT = NW * 64;
  static constexpr int BM = NW * 32;            // query rows per workgroup
  static constexpr int BN = 32;                 // keys per tile
  static constexpr int KB = BN / 32;            // 32-key blocks per tile
  static constexpr int DS = D / 16;             // k-steps of the S^T product
  static constexpr int DB = D / 32;             // 32-wide column blocks of O^T
  static constexpr int RB = 2 * D;              // bytes per K/V row
  static constexpr int TILE = BN * RB;          // bytes per K or V tile
  static constexpr int STAGE = 2 * TILE;        // K(j) then V(j)
  static constexpr int NI = TILE / (NT * 16);   // direct-load instructions per thread per tile
  static constexpr int RPI = 1024 / RB;         // rows written by one wave instruction
  static_assert(TILE % (NT * 16) == 0, "tile must split evenly into 1 KiB wave loads");
};

// Row-dependent 16-byte-chunk XOR swizzles of the K and V tiles.
template <int D> __device__ __forceinline__ int k_swz(int r) { return D == 64 ? (r >> 1) & 7 : r & 15; }
template <int D> __device__ __forceinline__ int v_swz(int r) { return D == 64 ? 4 * ((r >> 1) & 1) : 4 * (r & 3); }

constexpr float kSumMax = 256.0f;   // lazy rescale: a lane's tile sum of P may reach 2^8

template <int N> struct IC { static constexpr int value = N; };

template <typename T, int D, bool CAUSAL, bool SPLIT, bool VARLEN>
__global__ void __launch_bounds__(256)
__attribute__((amdgpu_waves_per_eu(D == 64 ? 4 : 3, D == 64 ? 4 : 3)))
fwd_short_kernel(const T* __restrict__ Q, const T* __restrict__ K, const T* __restrict__ V,
                T* __restrict__ O, float* __restrict__ LSE,
                float* __restrict__ Opart, float* __restrict__ Lpart,
                int BH, int S_q_, int S_k_, int n_qt, int n_split, int keys_per_split, float c,
                const int* __restrict__ cu_q, const int* __restrict__ cu_k, int H, int total_q)
{
  static_assert(!(VARLEN && SPLIT), "packed batches run unsplit");
  using C = ShortCfg<D>;
  using M = Mma<T>;
  typedef typename M::frag frag;
  // three stage buffers as separate objects, so that the compiler can tell a
  // direct load into one from a read of another
  __shared__ __attribute__((aligned(1024))) char st0[C::STAGE];
  __shared__ __attribute__((aligned(1024))) char st1[C::STAGE];
  __shared__ __attribute__((aligned(1024))) char st2[C::STAGE];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int hh = lane >> 5;        // lane half
  const int nn = lane & 31;        // query column owned by this lane

  // ---- which (b*h, q tile, split) this workgroup computes
  int split = 0, qt, bh;
  if (VARLEN) {
    // packed batches: XCD x takes heads x, x+8, ... one at a time with all
    // their query tiles (highest first) when B*H is a multiple of 8
    if (BH % 8 == 0) {
      const int x = blockIdx.x % 8, j = blockIdx.x / 8;
      bh = x + 8 * (j / n_qt);
      qt = n_qt - 1 - j % n_qt;
    } else {
      qt = n_qt - 1 - (int)(blockIdx.x / BH);
      bh = blockIdx.x % BH;
    }
  } else if (CAUSAL && !SPLIT && (D == 64 || n_qt >= 16)) {
    // query tiles heaviest first over all (b, h) at a time; consecutive
    // workgroups go to the 8 XCDs in turn, so (b, h) stays on XCD bh % 8
    // when B*H is a multiple of 8. Measured against the contiguous share of
    // heads per XCD below: D = 128 causal 2048 keys +10 %, 1024 -3 %, 512 -8 %
    // (few tiles per head: there a head's tiles running together share its
    // K and V in L2); D = 64 causal 512 +5.5 %, 4096 +10 %.
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
  const int wr0 = q0 + wave * 32;              // first row of this wave

  // ---- where this (b, h) lives. Dense: [B, H, S, D]. Packed: [total, H, D],
  // sequence b at rows cu[b] .. cu[b+1]-1, rows H*D elements apart; LSE is
  // [H, total_q].
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
  frag qf[C::DS];
  {
    const int q = wr0 + nn;
#pragma unroll
    for (int ds = 0; ds < C::DS; ds++) {
      if (q < S_q) {
        qf[ds] = *(const frag*)(Qh + (size_t)q * pitch + ds * 16 + 8 * hh);
      } else {
#pragma unroll
        for (int e = 0; e < 8; e++) qf[ds][e] = (T)0.0f;
      }
    }
  }

  // ---- direct global -> LDS loads: stage j = K(j) and V(j). Every wave
  // issues its share (NI instructions per tile, 1 KiB each, lane i landing at
  // byte 16*i and fetching the logical chunk the swizzle stores there), as
  // buffer loads on per-head resources: rows outside K/V read zeros (their
  // scores are masked, or the tile is never read), and every stage issues the
  // same number of instructions, which keeps the wait counts exact.
  // (packed rows are RBg bytes apart; the range ends after the last row)
  const int kv_bytes = VARLEN ? (S_k > 0 ? (S_k - 1) * RBg + C::RB : 0) : S_k * C::RB;
  const __amdgpu_buffer_rsrc_t krs = __builtin_amdgcn_make_buffer_rsrc((void*)Kh, (short)0, kv_bytes, 0x00020000);
  const __amdgpu_buffer_rsrc_t vrs = __builtin_amdgcn_make_buffer_rsrc((void*)Vh, (short)0, kv_bytes, 0x00020000);
  const int dma_rsub = (lane * 16) / C::RB;
  const int dma_u = ((lane * 16) % C::RB) / 16;
  // (offsets and destinations go through locals: a target builtin with
  // template-dependent argument expressions is dropped from the host pass)
  auto issue_stage = [&](int j, char* base) {
    const int krow0 = k_lo + j * C::BN;               // past the end: reads 0
#pragma unroll
    for (int i = 0; i < C::NI; i++) {
      const int blk = i * C::NW + wave;
      const int r = blk * C::RPI + dma_rsub;
      const int koff = (krow0 + r) * RBg + ((dma_u ^ k_swz<D>(r)) * 16);
      const int voff = (krow0 + r) * RBg + ((dma_u ^ v_swz<D>(r)) * 16);
      char* kdst = base + blk * 1024;
      char* vdst = base + C::TILE + blk * 1024;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(krs, (__attribute__((address_space(3))) void*)kdst, 16, koff, 0, 0, 0);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(vrs, (__attribute__((address_space(3))) void*)vdst, 16, voff, 0, 0, 0);
    }
  };

  // ---- per-lane LDS read offsets (swizzle folded in)
  constexpr int NKR = C::DS < 8 ? C::DS : 8;
  constexpr int NVR = C::DB < 4 ? C::DB : 4;
  const int xk = k_swz<D>(nn);
  int k_rd[NKR];
#pragma unroll
  for (int ds = 0; ds < NKR; ds++) k_rd[ds] = nn * C::RB + (((2 * ds + hh) ^ xk) * 16);
  const int g = lane >> 4, jj = lane & 15;
  const int vrow = 4 * hh + (jj >> 2);
  const int xv = v_swz<D>(vrow);
  int v_rd[NVR];
#pragma unroll
  for (int db = 0; db < NVR; db++)
    v_rd[db] = vrow * C::RB + (((4 * db + 2 * (g & 1) + ((jj & 3) >> 1)) ^ xv) * 16) + 8 * (jj & 1);

  v16f o[C::DB];
#pragma unroll
  for (int db = 0; db < C::DB; db++)
#pragma unroll
    for (int e = 0; e < 16; e++) o[db][e] = 0.0f;
  float m = kNegInf, l = 0.0f;

  auto barrier = [] {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
    asm volatile("" ::: "memory");
  };

  // One step per tile t, in order: S(t) = K(t) Q^T, mask, online softmax,
  // P(t) -> fragments, O += V(t)^T P(t). Stage t (K(t), V(t)) is read from
  // buffer t % 3 while stage t+2 is fetched into buffer (t+2) % 3.
  auto step = [&](auto bi, auto masked, int t) {
    constexpr int B = decltype(bi)::value;
    constexpr bool MASKED = decltype(masked)::value;
    const char* rbuf = B == 0 ? st0 : B == 1 ? st1 : st2;
    char* dbuf = B == 0 ? st2 : B == 1 ? st0 : st1;
    barrier();
    issue_stage(t + 2, dbuf);
    v16f s[C::KB];
    {
      constexpr int NS = C::DS * C::KB;
      auto load = [&](int j) {
        const int kb = j / C::DS, ds = j % C::DS;
        return *(const frag*)(rbuf + k_rd[ds % NKR] + (ds / NKR) * 256 + kb * 32 * C::RB);
      };
      frag ring[2];
      ring[0] = load(0);
#pragma unroll
      for (int j = 0; j < NS; j++) {
        if (j + 1 < NS) ring[(j + 1) & 1] = load(j + 1);
        const int kb = j / C::DS, ds = j % C::DS;
        if (ds == 0) {
          const v16f zero = {};
          s[kb] = M::mma(ring[j & 1], qf[ds], zero);
        } else {
          s[kb] = M::mma(ring[j & 1], qf[ds], s[kb]);
        }
      }
    }
    if (MASKED) {
      const int key0 = k_lo + t * C::BN;
      const int q = wr0 + nn;
#pragma unroll
      for (int kb = 0; kb < C::KB; kb++)
#pragma unroll
        for (int i = 0; i < 4; i++)
#pragma unroll
          for (int jx = 0; jx < 4; jx++) {
            const int key = key0 + kb * 32 + 8 * i + 4 * hh + jx;
            const bool ok = key < k_hi && (!CAUSAL || key <= q + diag);
            if (!ok) s[kb][4 * i + jx] = kNegInf;
          }
    }
    // P = 2^(s*c - m) with the row's current reference m. The reference only
    // has to keep every P <= 2^8.
    frag pf[C::KB][2];
    auto exps = [&](float& acc) {
      const float ref = m == kNegInf ? 0.0f : m;
#pragma unroll
      for (int kb = 0; kb < C::KB; kb++)
#pragma unroll
        for (int ks = 0; ks < 2; ks++) {
          v8f pv;
#pragma unroll
          for (int e = 0; e < 8; e++) {
            pv[e] = fast_exp2(__builtin_fmaf(s[kb][8 * ks + e], c, -ref));
            acc += pv[e];
          }
          pf[kb][ks] = M::cvt(pv);
        }
    };
    auto move_reference = [&](float x) {     // m -> max(m, x), O and l rescaled
      const float mnew = fmaxf(m, x);
      const float r = mnew == kNegInf ? 0.0f : mnew;
      const float alpha = fast_exp2(m - r);      // 0 when m was -inf, 1 when m stays
      m = mnew;
      l *= alpha;
#pragma unroll
      for (int db = 0; db < C::DB; db++)
#pragma unroll
        for (int e = 0; e < 16; e++) o[db][e] *= alpha;
    };
    auto half_max = [&]() {                  // this lane's half of the row
      float x = kNegInf;
#pragma unroll
      for (int kb = 0; kb < C::KB; kb++)
#pragma unroll
        for (int e = 0; e < 16; e++) x = fmaxf(x, s[kb][e]);
      return x;
    };
    auto row_max = [&]() { return pair_max(half_max()) * c; };
    if constexpr (D == 64) {
      // A lane's tile sum bounds each of its P, so the row maximum is
      // computed only when some sum exceeds 2^8 (or a row has no reference
      // yet): then m moves to the maximum and P is recomputed. The final
      // O / l and LSE use the same m, so any reference reached this way
      // gives the exact result. (At D = 128 the extra code costs the
      // three-wave register budget more than the skipped maximum saves.)
      float ls = __builtin_inff();               // forces the slow path below
      if (!__any(m == kNegInf)) {
        ls = 0.0f;
        exps(ls);
      }
      if (__any(!(ls <= kSumMax))) {
        move_reference(row_max());
        ls = 0.0f;
        exps(ls);
      }
      l += ls;
    } else {
      // the reference moves when a row's maximum exceeds it by more than 8;
      // the row's keys are split over the two halves of the wave, and when
      // neither half's maximum passes the bound the row's does not either, so
      // the exchange between the halves is needed only when it moves
      const float xh = half_max();
      if (__any(xh * c > m + 8.0f)) move_reference(pair_max(xh) * c);
      exps(l);
    }
    {
      constexpr int NP = C::KB * 2 * C::DB;
      const char* vl = rbuf + C::TILE;
      auto load = [&](int j) {
        const int kb = j / (2 * C::DB), ks = (j / C::DB) % 2, db = j % C::DB;
        const int off = (kb * 32 + 16 * ks) * C::RB;
        const char* va = vl + v_rd[db % NVR] + (db / NVR) * 256 + off;
        v4i16 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)va);
        v4i16 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)(va + 8 * C::RB));
        return __builtin_bit_cast(frag, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
      };
      frag ring[2];
      ring[0] = load(0);
#pragma unroll
      for (int j = 0; j < NP; j++) {
        if (j + 1 < NP) ring[(j + 1) & 1] = load(j + 1);
        const int kb = j / (2 * C::DB), ks = (j / C::DB) % 2, db = j % C::DB;
        o[db] = M::mma(ring[j & 1], pf[kb][ks], o[db]);
      }
    }
    __builtin_amdgcn_s_waitcnt(0x0070 | 0x0F00 | (2 * C::NI));   // stage t+1 complete
  };

  // Steps run over the wave's tiles with an allowed key (causal: a prefix);
  // tiles that need no mask for any row of the wave come first, the masked
  // ones (key-range tail, causal diagonal) are a suffix. After its last tile
  // a wave only keeps the barriers and its share of the loads going.
  if (n_tiles > 0) {
    int t_last = n_tiles - 1;
    if (CAUSAL) {
      const int lim = wr0 + 31 + diag - k_lo;
      t_last = lim < 0 ? -1 : min(t_last, lim / C::BN);
    }
    issue_stage(0, st0);
    issue_stage(1, st1);
    __builtin_amdgcn_s_waitcnt(0x0070 | 0x0F00 | (2 * C::NI));   // stage 0 complete
    int u_mask = (k_hi - k_lo) / C::BN;
    if (CAUSAL) {
      const int lim2 = wr0 + diag - k_lo + 1;
      u_mask = min(u_mask, lim2 < 0 ? 0 : lim2 / C::BN);
    }
    const IC<0> P;
    const IC<1> Mk;
    int t = 0;
    const int t_plain = min(t_last + 1, u_mask);
    for (; t + 2 < t_plain; t += 3) {
      step(IC<0>(), P, t);
      step(IC<1>(), P, t + 1);
      step(IC<2>(), P, t + 2);
    }
    for (; t + 2 <= t_last; t += 3) {
      step(IC<0>(), Mk, t);
      step(IC<1>(), Mk, t + 1);
      step(IC<2>(), Mk, t + 2);
    }
    if (t <= t_last) { step(IC<0>(), Mk, t); t++; }
    if (t <= t_last) { step(IC<1>(), Mk, t); t++; }
    for (; t < n_tiles; t++) {
      const int bsel = (t + 2) % 3;
      barrier();
      issue_stage(t + 2, bsel == 0 ? st0 : bsel == 1 ? st1 : st2);
      __builtin_amdgcn_s_waitcnt(0x0070 | 0x0F00 | (2 * C::NI));
    }
    __builtin_amdgcn_s_waitcnt(0x0070 | 0x0F00);
  }

  // ---- epilogue: normalise, logsumexp, store
  const int q = wr0 + nn;
  const float lt = pair_sum(l);
  const bool has = m != kNegInf && lt > 0.0f;
  const float inv = has ? 1.0f / lt : 0.0f;
  const float lse = has ? (m + __builtin_log2f(lt)) * kLn2 : kNegInf;
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
          for (int j = 0; j < 4; j++) w[j] = (T)(o[db][4 * i + j] * inv);
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
          w.x = o[db][4 * i + 0] * inv;
          w.y = o[db][4 * i + 1] * inv;
          w.z = o[db][4 * i + 2] * inv;
          w.w = o[db][4 * i + 3] * inv;
          *(float4*)(orow + db * 32 + 8 * i + 4 * hh) = w;
        }
      if (hh == 0) Lpart[prow] = lse;
    }
  }
}

// ---------------------------------------------------------------- launchers

template <typename T, int D, bool CAUSAL, bool SPLIT, bool VARLEN = false>
hipError_t launch_one(const FwdArgs& a, hipStream_t st) {
  using C = ShortCfg<D>;
  // K and V are addressed per head through 32-bit buffer offsets (packed:
  // over H*D-element row steps; S_k is then the longest key sequence)
  const long long row_bytes = VARLEN ? (long long)a.H * C::RB : C::RB;
  if ((long long)(a.S_k + 4 * C::BN) * row_bytes > 0x7fffffffLL) return hipErrorInvalidValue;
  const int n_qt = (a.S_q + C::BM - 1) / C::BM;
  const int n_work = a.B * a.H * n_qt * a.n_split;
  hipLaunchKernelGGL((fwd_short_kernel<T, D, CAUSAL, SPLIT, VARLEN>), dim3(n_work), dim3(C::NT), 0, st,
                     (const T*)a.q, (const T*)a.k, (const T*)a.v, (T*)a.o, a.lse, a.opart, a.lpart,
                     a.B * a.H, a.S_q, a.S_k, n_qt, a.n_split, a.keys_per_split, a.c, a.cu_q, a.cu_k, a.H,
                     a.total_q);
  return hipGetLastError();
}

template <typename T, int D>
hipError_t launch_varlen_d(const FwdArgs& a, hipStream_t st) {
  return a.causal ? launch_one<T, D, true, false, true>(a, st) : launch_one<T, D, false, false, true>(a, st);
}

template <typename T>
hipError_t launch_varlen_t(const FwdArgs& a, hipStream_t st) {
  switch (a.D) {
    case 64: return launch_varlen_d<T, 64>(a, st);
    case 128: return launch_varlen_d<T, 128>(a, st);
  }
  return hipErrorInvalidValue;
}

template <typename T, int D>
hipError_t launch_d(const FwdArgs& a, hipStream_t st) {
  const bool split = a.n_split > 1;
  if (a.causal) return split ? launch_one<T, D, true, true>(a, st) : launch_one<T, D, true, false>(a, st);
  return split ? launch_one<T, D, false, true>(a, st) : launch_one<T, D, false, false>(a, st);
}

template <typename T>
hipError_t launch_t(const FwdArgs& a, hipStream_t st) {
  switch (a.D) {
    case 64: return launch_d<T, 64>(a, st);
    case 128: return launch_d<T, 128>(a, st);
  }
  return hipErrorInvalidValue;
}

}  // namespace

int short_keys_per_tile() { return ShortCfg<128>::BN; }
int short_rows_per_block() { return ShortCfg<128>::BM; }

hipError_t launch_fwd_short(const FwdArgs& a, hipStream_t st) {
  if (a.dtype == 2) return launch_t<__bf16>(a, st);
  return launch_t<_Float16>(a, st);
}

hipError_t launch_fwd_short_varlen(const FwdArgs& a, hipStream_t st) {
  if (a.n_split != 1) return hipErrorInvalidValue;
  if (a.dtype == 2) return launch_varlen_t<__bf16>(a, st);
  return launch_varlen_t<_Float16>(a, st);
}

}  // namespace attn

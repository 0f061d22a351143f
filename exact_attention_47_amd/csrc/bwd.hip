// Backward pass of the fused attention on gfx950 matrix cores (bf16 / fp16,
// D = 64 / 128).
//
// The forward pass keeps the row logsumexp so that the backward pass can
// recompute the probabilities block by block instead of storing them ([GN]
// "Rueckblick auf den FlashAttention-Ansatz"). With S = scale Q K^T,
// P = exp(S - LSE), the gradients of O = P V are
//
//   dV = P^T dO,  dP = dO V^T,  dS = P * (dP - Dd),  Dd_i = sum_d dO_id O_id,
//   dQ = scale dS K,  dK = scale dS^T Q.
//
// Two launches of one kernel template share the forward kernel's operand
// layout (a 32-row "outer" block per wave held as the B operand, 32-row
// "inner" tiles streamed through LDS, every product on the 16x16x32 MFMA with
// accumulators transposed so that lane (g, n) owns outer rows n and 16 + n
// and holds inner rows 4g .. 4g+3 of each 16-row inner block):
//
//   mode dQ:  outer = query rows, inner = keys:  S^T = K Q^T, dP^T = V dO^T,
//             dQ^T += K^T dS^T
//   mode dKV: outer = keys, inner = query rows:  S = Q K^T,  dP = dO V^T,
//             dK^T += Q^T dS,  dV^T += dO^T P
//
// dQ and dKV each compute S and P (seven products per tile pair instead of
// five), and every gradient is a plain sum in a fixed order: results are
// deterministic (no atomics). At D = 128 the dKV mode's two accumulators and
// the outer K rows fill the 256 registers of two waves per SIMD, so its outer
// V rows (the B operand of dP) are read from LDS. The A operands of the
// accumulations (K^T,
// Q^T, dO^T) are read from the staged tiles with ds_read_b64_tr_b16, choosing
// for each k slot the inner row that the probability fragment holds there
// (a lane's four rows of inner block 0, then its four of block 1), exactly as
// the forward pass reads V^T. Staged tiles use an XOR swizzle that suits both
// read patterns (see bswz).
//
// A small first kernel (one row per D/8 lanes, float32 sum) writes -Dd and
// -log2(e) LSE per query row, the forms the tiles consume: P = exp2(S c +
// (-log2(e) LSE)) is one multiply-add and an exp2, and dKV's dP product
// starts its accumulator at -Dd, so that dS = P * dP is one multiply.
#include "common.h"
#include "kernels.h"

namespace attn {

namespace {

template <typename T> struct BMma;
template <> struct BMma<__bf16> {
  typedef v8bf16 frag;
  static __device__ __forceinline__ v4f mma(frag a, frag b, v4f c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
  }
  static __device__ __forceinline__ frag cvt(v8f x) { return __builtin_convertvector(x, v8bf16); }
};
template <> struct BMma<_Float16> {
  typedef v8f16 frag;
  static __device__ __forceinline__ v4f mma(frag a, frag b, v4f c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
  }
  static __device__ __forceinline__ frag cvt(v8f x) { return __builtin_convertvector(x, v8f16); }
};

constexpr int kDQ = 0, kDKV = 1;   // dQ; dK and dV in one pass

template <int D>
struct BwdCfg {
  static constexpr int NW = 4;                  // waves per workgroup
  static constexpr int NT = NW * 64;
  static constexpr int BO = NW * 32;            // outer rows per workgroup
  static constexpr int BI = 32;                 // inner rows per tile
  static constexpr int DS = D / 32;             // k-steps over D
  static constexpr int DB = D / 16;             // 16-wide blocks of D
  static constexpr int RB = 2 * D;              // bytes per row
  static constexpr int TILE = BI * RB;
  static constexpr int STAGE = 2 * TILE + 512;  // X, Y, then 64 -log2(e) LSE and 64 -Dd values (inner = queries)
  static constexpr int NI = TILE / (NT * 16);   // direct loads per thread per tile
  static constexpr int RPI = 1024 / RB;         // rows per 1 KiB wave load
  static_assert(TILE % (NT * 16) == 0, "tile must split into 1 KiB wave loads");
};

// Row-dependent 16-byte-chunk XOR swizzle of the staged tiles, which are read
// both by rows (16-byte reads: one chunk of each of 16 consecutive rows) and
// transposed (8-byte transposing reads, 32 lanes per LDS cycle: one 32-byte
// segment of each of 8 consecutive rows). chunk ^ 2 (r & 7) at D = 128
// (chunk ^ 2 ((r >> 1) & 3) at D = 64, whose odd rows start on bank 32)
// gives 8 aligned rows 8 distinct segments, and the 16-byte reads, which the
// LDS serves eight lanes at a time, 8 distinct chunks per eight rows: both
// patterns touch every bank once (measured with a probe of both patterns:
// 0 conflicts; a swizzle that also spread 16 rows over 16 chunks cost 2.7
// conflict cycles per 16-byte read).
template <int D> __device__ __forceinline__ int bswz(int r) {
  return D == 64 ? 2 * ((r >> 1) & 3) : 2 * (r & 7);
}

template <typename T>
__device__ __forceinline__ void load8f(const T* p, float* out) {
  const uint4 raw = *(const uint4*)p;
  const T* e = (const T*)&raw;
#pragma unroll
  for (int i = 0; i < 8; i++) out[i] = (float)e[i];
}

// nDd[row] = -sum_d dO[row][d] * O[row][d] (float32, D/8 lanes per row) and
// nl2[row] = -log2(e) * LSE[row]
template <typename T, int D>
__global__ void __launch_bounds__(256) bwd_dot_kernel(const T* __restrict__ O, const T* __restrict__ dO,
                                                       const float* __restrict__ LSE, float* __restrict__ nDd,
                                                       float* __restrict__ nl2, long rows)
{
  constexpr int LPR = D / 8;
  const long g = (long)blockIdx.x * 256 + threadIdx.x;
  const long row = g / LPR;
  const int part = (int)(g % LPR);
  float acc = 0.0f;
  if (row < rows) {
    float a[8], b[8];
    load8f(O + row * D + part * 8, a);
    load8f(dO + row * D + part * 8, b);
#pragma unroll
    for (int i = 0; i < 8; i++) acc += a[i] * b[i];
  }
#pragma unroll
  for (int off = LPR / 2; off >= 1; off >>= 1) acc += __shfl_xor(acc, off);
  if (row < rows && part == 0) {
    nDd[row] = -acc;
    nl2[row] = -(LSE[row] * kLog2e);
  }
}

template <bool B> struct BIC { static constexpr bool value = B; };

template <typename T, int D, int MODE, bool CAUSAL>
__global__ void __launch_bounds__(256)
__attribute__((amdgpu_waves_per_eu(2, 2)))
bwd_kernel(const T* __restrict__ Q, const T* __restrict__ K, const T* __restrict__ V,
           const T* __restrict__ dO, const float* __restrict__ NL2, const float* __restrict__ NDd,
           T* __restrict__ Gout, T* __restrict__ Gout2, int BH, int S_q, int S_k, int n_ot, float c,
           float gscale)
{
  using C = BwdCfg<D>;
  using M = BMma<T>;
  typedef typename M::frag frag;
  constexpr bool DQ = MODE == kDQ;
  // dKV at D = 128: the outer V rows (B operand of dP) are read from LDS
  // instead of registers, which keeps both accumulators within the 256
  // registers of two waves per SIMD
  constexpr bool OF2_LDS = !DQ && D == 128;
  __shared__ __attribute__((aligned(1024))) char st0[C::STAGE];
  __shared__ __attribute__((aligned(1024))) char st1[C::STAGE];
  __shared__ __attribute__((aligned(1024))) char ovs[OF2_LDS ? C::BO * C::RB : 16];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 4;                      // 16-lane group: inner rows 4g..4g+3 of each 16-row block
  const int n = lane & 15;                      // outer rows n and 16 + n of the wave

  int ot, bh;
  if (!CAUSAL) {
    const int work = xcd_swizzle(blockIdx.x, BH * n_ot);
    ot = work % n_ot;
    bh = work / n_ot;
  } else {
    // causal: outer blocks go out heaviest first over all (b, h) at a time
    // (late query tiles for dQ, early key blocks for dK and dV), so that no
    // XCD is left with a head's heavy blocks at the end; the hardware deals
    // consecutive workgroups to the 8 XCDs in turn, so (b, h) stays on XCD
    // bh % 8 when B*H is a multiple of 8
    const int level = blockIdx.x / BH;
    bh = blockIdx.x % BH;
    ot = DQ ? n_ot - 1 - level : level;
  }
  const int S_o = DQ ? S_q : S_k;
  const int S_i = DQ ? S_k : S_q;
  const int o0 = ot * C::BO;
  const int wr0 = o0 + wave * 32;               // this wave's outer rows
  const int diag = S_k - S_q;                   // key j allowed for query i iff j <= i + diag

  // inner rows that any outer row of the workgroup can see
  int i_lo = 0, i_hi = S_i;
  if (CAUSAL) {
    if (DQ) i_hi = min(S_k, o0 + C::BO - 1 + diag + 1);
    else i_lo = max(0, o0 - diag);
  }
  const int t_begin = i_lo / C::BI;
  const int t_end = i_hi > i_lo ? (i_hi + C::BI - 1) / C::BI : t_begin;

  const size_t qo = (size_t)bh * S_q * D, ko = (size_t)bh * S_k * D;
  const T* O1 = DQ ? Q + qo : K + ko;           // outer, first product
  const T* O2 = DQ ? dO + qo : V + ko;          // outer, second product
  const T* Xg = DQ ? K + ko : Q + qo;           // inner, first product (and dQ / dK accumulation)
  const T* Yg = DQ ? V + ko : dO + qo;          // inner, second product (and dV accumulation)
  const float* nl2h = NL2 + (size_t)bh * S_q;   // -log2(e) LSE
  const float* nddh = NDd + (size_t)bh * S_q;   // -Dd

  // outer rows as B operands: lane (g, n) holds row wr0 + 16 ob + n, d = 32 ds + 8 g .. +7
  constexpr bool OF2_REG = !OF2_LDS;
  frag of1[C::DS][2], of2[OF2_REG ? C::DS : 1][2];
#pragma unroll
  for (int ob = 0; ob < 2; ob++) {
    const int r = wr0 + 16 * ob + n;
#pragma unroll
    for (int ds = 0; ds < C::DS; ds++) {
      if (r < S_o) {
        of1[ds][ob] = *(const frag*)(O1 + (size_t)r * D + ds * 32 + 8 * g);
        if constexpr (OF2_REG) of2[ds][ob] = *(const frag*)(O2 + (size_t)r * D + ds * 32 + 8 * g);
      } else {
#pragma unroll
        for (int e = 0; e < 8; e++) {
          of1[ds][ob][e] = (T)0.0f;
          if constexpr (OF2_REG) of2[ds][ob][e] = (T)0.0f;
        }
      }
    }
  }
  // OF2_LDS: each wave writes its 32 outer V rows to its 32-row slice of ovs
  // (rows past S_o as zeros), with the staged tiles' swizzle, and reads them
  // back with the row-read offsets below
  if constexpr (OF2_LDS) {
    char* ow = ovs + wave * 32 * C::RB;
#pragma unroll
    for (int i = 0; i < 32 * C::RB / (64 * 16); i++) {
      const int cidx = i * 64 + lane;               // 16-byte chunk of the wave's slice
      const int row = cidx / (C::RB / 16), u = cidx % (C::RB / 16);
      uint4 val = make_uint4(0u, 0u, 0u, 0u);
      if (wr0 + row < S_o) val = *(const uint4*)(O2 + (size_t)(wr0 + row) * D + u * 8);
      *(uint4*)(ow + row * C::RB + ((u ^ bswz<D>(row)) * 16)) = val;
    }
    __syncthreads();
  }
  // per-lane scalars of the outer query rows (mode dQ)
  float nl2_o[2] = {0.0f, 0.0f}, ndd_o[2] = {0.0f, 0.0f};
  if (DQ) {
#pragma unroll
    for (int ob = 0; ob < 2; ob++) {
      const int r = wr0 + 16 * ob + n;
      if (r < S_q) {
        nl2_o[ob] = nl2h[r];
        ndd_o[ob] = nddh[r];
      }
    }
  }

  // stage t: X rows 32t.., Y rows 32t.. (buffer loads; rows past the end read 0)
  const __amdgpu_buffer_rsrc_t xrs = __builtin_amdgcn_make_buffer_rsrc((void*)Xg, (short)0, S_i * C::RB, 0x00020000);
  const __amdgpu_buffer_rsrc_t yrs = __builtin_amdgcn_make_buffer_rsrc((void*)Yg, (short)0, S_i * C::RB, 0x00020000);
  const int dma_rsub = (lane * 16) / C::RB;
  const int dma_u = ((lane * 16) % C::RB) / 16;
  // (offsets and destinations go through locals: a target builtin with
  // template-dependent argument expressions is dropped from the host pass)
  // (inner = queries: wave 0 also stages the tile's -log2(e) LSE and -Dd
  // values, 64 rows per instruction, rows past S_q read 0)
  const __amdgpu_buffer_rsrc_t lrs = __builtin_amdgcn_make_buffer_rsrc((void*)nl2h, (short)0, S_q * 4, 0x00020000);
  const __amdgpu_buffer_rsrc_t drs = __builtin_amdgcn_make_buffer_rsrc((void*)nddh, (short)0, S_q * 4, 0x00020000);
  auto issue_stage = [&](int t, char* base) {
    if (!DQ && wave == 0) {
      char* ld = base + 2 * C::TILE;
      char* dd = base + 2 * C::TILE + 256;
      const int off = (t * C::BI + lane) * 4;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(lrs, (__attribute__((address_space(3))) void*)ld, 4, off, 0, 0, 0);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(drs, (__attribute__((address_space(3))) void*)dd, 4, off, 0, 0, 0);
    }
#pragma unroll
    for (int i = 0; i < C::NI; i++) {
      const int blk = i * C::NW + wave;
      const int r = blk * C::RPI + dma_rsub;
      const int off = (t * C::BI + r) * C::RB + ((dma_u ^ bswz<D>(r)) * 16);
      char* xd = base + blk * 1024;
      char* yd = base + C::TILE + blk * 1024;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(xrs, (__attribute__((address_space(3))) void*)xd, 16, off, 0, 0, 0);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(yrs, (__attribute__((address_space(3))) void*)yd, 16, off, 0, 0, 0);
    }
  };

  // LDS read offsets (the swizzle depends on the low four row bits only, so
  // the offsets of inner block 1 are those of block 0 plus 16 rows).
  // Row reads (A of the two products): inner row n, chunk 4 ds + g.
  int k_rd[C::DS];
#pragma unroll
  for (int ds = 0; ds < C::DS; ds++) k_rd[ds] = n * C::RB + (((4 * ds + g) ^ bswz<D>(n)) * 16);
  // Transposed reads (A of the accumulations): lane n of group g addresses
  // inner row 4g + n/4 (and 16 rows further), columns 16 db + 4 (n % 4) .. +3.
  const int vrow = 4 * g + (n >> 2);
  int tr_rd[C::DB];
#pragma unroll
  for (int db = 0; db < C::DB; db++)
    tr_rd[db] = vrow * C::RB + (((2 * db + ((n & 3) >> 1)) ^ bswz<D>(vrow)) * 16) + 8 * (n & 1);

  v4f acc[C::DB][2];
#pragma unroll
  for (int db = 0; db < C::DB; db++)
#pragma unroll
    for (int ob = 0; ob < 2; ob++)
#pragma unroll
      for (int e = 0; e < 4; e++) acc[db][ob][e] = 0.0f;
  // second accumulator (mode dKV: dV^T next to dK^T)
  constexpr int DB2 = DQ ? 1 : C::DB;
  v4f acc2[DB2][2];
#pragma unroll
  for (int db = 0; db < DB2; db++)
#pragma unroll
    for (int ob = 0; ob < 2; ob++)
#pragma unroll
      for (int e = 0; e < 4; e++) acc2[db][ob][e] = 0.0f;

  auto barrier = [] {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
    asm volatile("" ::: "memory");
  };

  // acc^T[d x outer] += Z^T[d x inner] F[inner x outer] for one staged tile Z
  auto accumulate = [&](v4f (*dst)[2], const char* zs, const frag* f) {
#pragma unroll
    for (int db = 0; db < C::DB; db++) {
      v4i16 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)(zs + tr_rd[db]));
      v4i16 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)(zs + tr_rd[db] + 16 * C::RB));
      const frag a = __builtin_bit_cast(frag, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
      dst[db][0] = M::mma(a, f[0], dst[db][0]);
      dst[db][1] = M::mma(a, f[1], dst[db][1]);
    }
  };

  auto step = [&](int t, const char* st) {
    const char* xs = st;
    const char* ys = st + C::TILE;
    // C[inner 32 x outer 32] = X_tile O1^T: block (ib, ob) of lane (g, n) holds
    // inner rows 16 ib + 4g + i of outer row 16 ob + n
    v4f s[2][2];
#pragma unroll
    for (int ds = 0; ds < C::DS; ds++)
#pragma unroll
      for (int ib = 0; ib < 2; ib++) {
        const frag a = *(const frag*)(xs + k_rd[ds] + ib * 16 * C::RB);
        if (ds == 0) {
          const v4f zero = {};
          s[ib][0] = M::mma(a, of1[ds][0], zero);
          s[ib][1] = M::mma(a, of1[ds][1], zero);
        } else {
          s[ib][0] = M::mma(a, of1[ds][0], s[ib][0]);
          s[ib][1] = M::mma(a, of1[ds][1], s[ib][1]);
        }
      }
    v4f dp[2][2];
#pragma unroll
    for (int ib = 0; ib < 2; ib++) {
      if constexpr (DQ) {
        // every element of a block belongs to its outer (query) row: the
        // product starts from that row's -Dd
#pragma unroll
        for (int ob = 0; ob < 2; ob++)
#pragma unroll
          for (int e = 0; e < 4; e++) dp[ib][ob][e] = ndd_o[ob];
      } else {
        // dP - Dd in one product: the accumulator starts at the staged -Dd
        // of the inner (query) row that each element belongs to
        const float4 d4 = *(const float4*)(st + 2 * C::TILE + 256 + (16 * ib + 4 * g) * 4);
#pragma unroll
        for (int ob = 0; ob < 2; ob++) {
          dp[ib][ob][0] = d4.x; dp[ib][ob][1] = d4.y; dp[ib][ob][2] = d4.z; dp[ib][ob][3] = d4.w;
        }
      }
    }
#pragma unroll
    for (int ds = 0; ds < C::DS; ds++) {
      frag b0, b1;
      if constexpr (OF2_LDS) {
        const char* ow = ovs + wave * 32 * C::RB;
        b0 = *(const frag*)(ow + k_rd[ds]);
        b1 = *(const frag*)(ow + k_rd[ds] + 16 * C::RB);
      } else {
        b0 = of2[ds][0];
        b1 = of2[ds][1];
      }
#pragma unroll
      for (int ib = 0; ib < 2; ib++) {
        const frag a = *(const frag*)(ys + k_rd[ds] + ib * 16 * C::RB);
        dp[ib][0] = M::mma(a, b0, dp[ib][0]);
        dp[ib][1] = M::mma(a, b1, dp[ib][1]);
      }
    }
    // probabilities (and dS), masked where the key is outside the range or
    // after the causal limit. The mask is evaluated only on tiles that hold
    // such a pair for this wave's 32 outer rows (range tails, the causal
    // diagonal); elsewhere every pair is allowed.
    const int t0 = t * C::BI;
    const bool full = DQ ? (wr0 + 32 <= S_q && t0 + C::BI <= S_k && (!CAUSAL || t0 + C::BI - 1 <= wr0 + diag))
                         : (t0 + C::BI <= S_q && wr0 + 32 <= S_k && (!CAUSAL || wr0 + 31 <= t0 + diag));
    float gv[2][2][4], gp[2][2][4];
    auto probs = [&](auto masked) {
      constexpr bool MASKED = decltype(masked)::value;
#pragma unroll
      for (int ib = 0; ib < 2; ib++) {
        const int ir0 = t0 + 16 * ib + 4 * g;          // inner rows ir0 .. ir0+3
        float l4[4] = {0.0f, 0.0f, 0.0f, 0.0f};
        if (!DQ) {
          const float4 lv = *(const float4*)(st + 2 * C::TILE + (16 * ib + 4 * g) * 4);
          l4[0] = lv.x; l4[1] = lv.y; l4[2] = lv.z; l4[3] = lv.w;
        }
#pragma unroll
        for (int ob = 0; ob < 2; ob++) {
          const int orow = wr0 + 16 * ob + n;
#pragma unroll
          for (int i = 0; i < 4; i++) {
            const int ir = ir0 + i;
            const int query = DQ ? orow : ir;
            const int key = DQ ? ir : orow;
            const bool ok = !MASKED || (query < S_q && key < S_k && (!CAUSAL || key <= query + diag));
            const float nl2 = DQ ? nl2_o[ob] : l4[i];
            const float p = ok ? fast_exp2(__builtin_fmaf(s[ib][ob][i], c, nl2)) : 0.0f;
            gv[ib][ob][i] = p * dp[ib][ob][i];          // dp already holds dP - Dd
            if (!DQ) gp[ib][ob][i] = p;
          }
        }
      }
    };
    if (full) probs(BIC<false>());
    else probs(BIC<true>());
    // B operand of the accumulation, k order: the lane's four rows of inner
    // block 0, then its four of block 1
    frag gf[2];
#pragma unroll
    for (int ob = 0; ob < 2; ob++) {
      v8f w;
#pragma unroll
      for (int e = 0; e < 8; e++) w[e] = gv[e >> 2][ob][e & 3];
      gf[ob] = M::cvt(w);
    }
    // acc^T += X^T dS (dQ^T += K^T dS^T, dK^T += Q^T dS)
    accumulate(acc, xs, gf);
    if constexpr (!DQ) {
      // dV^T[d x outer] += dO^T[d x inner] P[inner x outer], from the same stage
      frag pf2[2];
#pragma unroll
      for (int ob = 0; ob < 2; ob++) {
        v8f w;
#pragma unroll
        for (int e = 0; e < 8; e++) w[e] = gp[e >> 2][ob][e & 3];
        pf2[ob] = M::cvt(w);
      }
      accumulate(acc2, ys, pf2);
    }
  };

  // Causal dK and dV: each workgroup's inner range starts at its own diagonal
  // and ends at the last query tile. Walked backwards from the end, the
  // workgroups of one head read the same query tiles at about the same time
  // (one moving window in L2 instead of one per starting point).
  auto tile = [&](int u) { return (CAUSAL && !DQ) ? t_begin + t_end - 1 - u : u; };
  if (t_end > t_begin) {
    issue_stage(tile(t_begin), st0);
    __builtin_amdgcn_s_waitcnt(0x0070 | 0x0F00);
    int t = t_begin;
    for (; t + 1 < t_end; t += 2) {
      barrier();
      issue_stage(tile(t + 1), st1);
      step(tile(t), st0);
      __builtin_amdgcn_s_waitcnt(0x0070 | 0x0F00);
      barrier();
      if (t + 2 < t_end) issue_stage(tile(t + 2), st0);
      step(tile(t + 1), st1);
      __builtin_amdgcn_s_waitcnt(0x0070 | 0x0F00);
    }
    if (t < t_end) {
      barrier();
      step(tile(t), st0);
    }
  }

  // store the gradient rows of this wave: lane (g, n) holds rows wr0 + 16 ob
  // + n, columns 16 db + 4g .. +3. The lane index passes through an empty asm
  // statement, so that the compiler does not keep the outer rows' addresses
  // live across the tile loop for these stores.
  int lane_e = lane;
  asm volatile("" : "+v"(lane_e));
  const int n_e = lane_e & 15, g_e = lane_e >> 4;
#pragma unroll
  for (int ob = 0; ob < 2; ob++) {
    const int r = wr0 + 16 * ob + n_e;
    if (r < S_o) {
      typedef T v4t __attribute__((ext_vector_type(4)));
      T* grow = Gout + (size_t)bh * S_o * D + (size_t)r * D;
#pragma unroll
      for (int db = 0; db < C::DB; db++) {
        v4t w;
#pragma unroll
        for (int e = 0; e < 4; e++) w[e] = (T)(acc[db][ob][e] * gscale);
        *(v4t*)(grow + db * 16 + 4 * g_e) = w;
      }
      if constexpr (!DQ) {
        T* grow2 = Gout2 + (size_t)bh * S_o * D + (size_t)r * D;
#pragma unroll
        for (int db = 0; db < DB2; db++) {
          v4t w;
#pragma unroll
          for (int e = 0; e < 4; e++) w[e] = (T)acc2[db][ob][e];
          *(v4t*)(grow2 + db * 16 + 4 * g_e) = w;
        }
      }
    }
  }
}

template <typename T, int D, int MODE>
hipError_t launch_mode(const BwdArgs& a, hipStream_t st) {
  using C = BwdCfg<D>;
  const int S_o = MODE == kDQ ? a.S_q : a.S_k;
  const int n_ot = (S_o + C::BO - 1) / C::BO;
  const dim3 grid((unsigned)(a.B * a.H * n_ot));
  T* out = (T*)(MODE == kDQ ? a.dq : a.dk);
  T* out2 = (T*)(MODE == kDKV ? a.dv : nullptr);
  const float gscale = a.scale;
  if (a.causal)
    hipLaunchKernelGGL((bwd_kernel<T, D, MODE, true>), grid, dim3(C::NT), 0, st, (const T*)a.q, (const T*)a.k,
                       (const T*)a.v, (const T*)a.dout, a.nl2, a.dd, out, out2, a.B * a.H, a.S_q, a.S_k, n_ot,
                       a.scale * kLog2e, gscale);
  else
    hipLaunchKernelGGL((bwd_kernel<T, D, MODE, false>), grid, dim3(C::NT), 0, st, (const T*)a.q, (const T*)a.k,
                       (const T*)a.v, (const T*)a.dout, a.nl2, a.dd, out, out2, a.B * a.H, a.S_q, a.S_k, n_ot,
                       a.scale * kLog2e, gscale);
  return hipGetLastError();
}

template <typename T, int D>
hipError_t launch_d(const BwdArgs& a, hipStream_t st) {
  // K and V (and Q, dO) are addressed through 32-bit buffer offsets
  if ((long long)(a.S_k > a.S_q ? a.S_k : a.S_q) * 2 * D + 2LL * 32 * 2 * D > 0x7fffffffLL) return hipErrorInvalidValue;
  const long rows = (long)a.B * a.H * a.S_q;
  const long threads = rows * (D / 8);
  hipLaunchKernelGGL((bwd_dot_kernel<T, D>), dim3((unsigned)((threads + 255) / 256)), dim3(256), 0, st,
                     (const T*)a.o, (const T*)a.dout, a.lse, a.dd, a.nl2, rows);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if ((e = launch_mode<T, D, kDQ>(a, st)) != hipSuccess) return e;
  // dK and dV in one pass: S and P computed once for both (measured against
  // separate dK and dV passes: +18 % on the whole backward at D = 64 4K,
  // +11 to +13 % at D = 128 4K-16K, with the outer V rows in LDS there)
  return launch_mode<T, D, kDKV>(a, st);
}

template <typename T>
hipError_t launch_t(const BwdArgs& a, hipStream_t st) {
  switch (a.D) {
    case 64: return launch_d<T, 64>(a, st);
    case 128: return launch_d<T, 128>(a, st);
  }
  return hipErrorNotSupported;
}

}  // namespace

hipError_t launch_bwd(const BwdArgs& a, hipStream_t st) {
  if (a.dtype == 2) return launch_t<__bf16>(a, st);
  return launch_t<_Float16>(a, st);
}

}  // namespace attn

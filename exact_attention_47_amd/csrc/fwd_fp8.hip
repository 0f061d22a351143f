// Fused attention forward pass on E4M3 inputs (gfx950 FP8 matrix cores).
//
// The low-precision step of the pages ([NL] "3. Lage precisie (FP8) met
// reductie van kwantisatiefout"; [GN] "Niedrige FP8-Praezision und incoherent
// processing"): Q and K arrive as E4M3 codes with one float32 scale per 64
// rows of each (b, h) (after the random-sign Hadamard transform of
// hadamard_quant), V as E4M3 codes with one per-tensor scale. FP8 doubles the
// matrix rate while the exponential stays as expensive ([GN] "Ueberlappung von
// GEMM und Softmax durch Asynchronitaet"): the vector unit, not the matrix
// core, bounds this kernel (about five vector instructions per score against
// a quarter of a matrix instruction; on gfx950 an exponential holds the
// vector unit about twice as long as an FMA, and the two do not overlap).
// The schedule therefore aims at keeping the vector unit busy from as many
// waves as the register file allows.
//
// * Work split: 4 waves x 32 query rows per workgroup, 64-key tiles (one K
//   scale block and one k-step of the P V product each). Three LDS stages of
//   16 KiB and at most 168 VGPRs per lane: three workgroups share a CU, one
//   wave of each per SIMD.
//
// * Each wave runs its tiles in order: S(t) = K(t) Q^T
//   (v_mfma_scale_f32_32x32x64_f8f6f4, unit scales), mask (a suffix of the
//   wave's tiles: key-range tail, causal diagonal), softmax, E4M3 packing,
//   then O += V(t)^T P(t)^T. The overlap of matrix and vector work that the
//   pages build inside a warpgroup ([GN] "Overlap innerhalb einer
//   Warpgroup") comes here from the three waves of a SIMD, which are at
//   different points of their steps; with the software pipeline inside each
//   wave the registers allowed only two waves per SIMD, and three plain waves
//   measured 4-6 % faster.
//
// * Scores: s = scale * qs * ks * (q8 . k8), with qs the block scale of this
//   wave's 32 rows and ks that of the tile's 64 keys; their product with
//   log2(e) is one multiplier per tile, folded into the exp2 argument (the
//   next tile's scale is fetched a step ahead with a vector load: a scalar
//   load in flight would turn every LDS wait into a full one). P is rounded
//   to E4M3 as p * 2^7 (the factor is added to the exponent for free) so
//   small probabilities stay out of the subnormal range. The row sum l is
//   the sum of the rounded values, so O = acc * vs / l is the average of the
//   V rows under the weights the product used (the 2^7 cancels) and the LSE
//   is the log of their sum. l comes from the matrix core: one
//   v_mfma_scale_f32_16x16x128_f8f6f4 per tile multiplies the P fragment by
//   a selector of E4M3 ones (lane group G of A holds ones in rows r with
//   r/4 of G's parity), which leaves in every element of output lane L the
//   tile's sum for query L % 32 over both key halves, and takes the 32
//   vector adds per lane and tile off the vector unit. The running maximum
//   moves whenever a row exceeds it by more than 1.75 (log2), which keeps
//   p * 2^7 <= 430 < 448; at each move the row's largest p is exactly 2^7,
//   which E4M3 holds without rounding.
//
// * V comes as [S_k, D] codes (read transposed in flight, below) or, with
//   v_transposed, as [D, S_k] codes: those tiles are stored [128 d][64 keys]
//   and read with eight 4-byte loads per fragment, dword q holding keys
//   8q + 4h .. 8q + 4h + 3 (the P fragment's k order, below).
//
// * The transposed V read picks, for element r of read p, the key row that
//   the P fragment holds in that k slot: P^T slot t of lane half h is key
//   32(t/16) + 8((t%16)/4) + 4h + t%4 (the S^T accumulator order), and
//   ds_read_b64_tr_b8 gives lane i element r from the address of lane
//   2r + i/8 of its 16-lane group, so lane j addresses the key row of slot
//   8p + j/2 at column 8*(j%2).
//
// * LDS: K and V tiles [64][128 bytes], 16-byte-chunk XOR swizzles chosen so
//   that the K reads (16 lanes per LDS cycle over 16 rows) and the transposed
//   V reads (32 lanes over 8 rows x 32 bytes) hit all 64 banks once. Stage
//   j = {K(j), V(j)} lives in one of three separate __shared__ arrays (the
//   compiler can then tell a direct load into one from a read of another;
//   the loop is unrolled by three); stage t+2 is fetched with buffer loads at
//   the start of step t and waited for at the end of step t+1.
#include "common.h"
#include "kernels.h"

namespace attn {

namespace {

constexpr int D8 = 128;                 // head dimension (bytes per FP8 row)
constexpr int BN8 = 64;                 // keys per tile
constexpr int KB8 = BN8 / 32;           // 32-key blocks per tile
constexpr int DB8 = D8 / 32;            // 32-row blocks of O^T
constexpr int NW8 = 4;                  // waves per workgroup
constexpr int NT8 = NW8 * 64;
constexpr int BM8 = NW8 * 32;           // query rows per workgroup
constexpr int TILE8 = BN8 * D8;         // bytes per K or V tile
constexpr int STAGE8 = 2 * TILE8;
constexpr int NI8 = TILE8 / (NT8 * 16); // direct-load instructions per thread per tile
constexpr float kTau8 = 1.75f;          // keeps p * 2^7 <= 2^8.75 < 448
constexpr float kPShift8 = 7.0f;        // P is quantized as p * 2^7
static_assert(TILE8 % (NT8 * 16) == 0, "tile must split evenly into 1 KiB wave loads");

__device__ __forceinline__ int k8_swz(int r) { return (r >> 1) & 7; }
__device__ __forceinline__ int v8_swz(int r) { return 2 * (((r >> 1) & 1) | ((r >> 2) & 2)); }

__device__ __forceinline__ v16f mma8(v8i a, v8i b, v16f c) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 127, 0, 127);
}

// the same product with a 16x16 output: the P tile's row sums (above)
__device__ __forceinline__ v4f mma8_rows(v8i a, v8i b, v4f c) {
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, 0, 127, 0, 127);
}

__device__ __forceinline__ uint32_t pack_fp8(float a, float b, float c, float d) {
  // the first conversion writes the low half and keeps the high half of its
  // "old" operand, which the second one overwrites: any register will do, and
  // one whose value dies here saves a copy
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, __builtin_bit_cast(int, a), false);
  w = __builtin_amdgcn_cvt_pk_fp8_f32(c, d, w, true);
  return (uint32_t)w;
}

template <int N> struct IC8 { static constexpr int value = N; };

// V^T tiles ([128 d][64 keys], VT = true): 16-byte chunk c of row d sits
// at chunk position c ^ vt8_swz(d)
__device__ __forceinline__ int vt8_swz(int d) { return (d >> 2) & 3; }

template <bool CAUSAL, bool VT, bool SPLIT>
__global__ void __launch_bounds__(NT8)
__attribute__((amdgpu_waves_per_eu(3, 3)))
fwd_fp8_kernel(const uint8_t* __restrict__ Q8, const uint8_t* __restrict__ K8, const uint8_t* __restrict__ V8,
               const float* __restrict__ qs, const float* __restrict__ ks, const float* __restrict__ vs,
               __bf16* __restrict__ O, float* __restrict__ LSE, float* __restrict__ Opart, float* __restrict__ Lpart,
               int BH, int S_q, int S_k, int n_qt, int n_split, int keys_per_split, float c)
{
  __shared__ __attribute__((aligned(1024))) char st0[STAGE8];
  __shared__ __attribute__((aligned(1024))) char st1[STAGE8];
  __shared__ __attribute__((aligned(1024))) char st2[STAGE8];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int hh = lane >> 5;
  const int nn = lane & 31;

  const int n_work = BH * n_qt;
  int qt, bh, split = 0;
  if (SPLIT) {
    // key-range split: equal work per item, contiguous shares per XCD
    int work = xcd_swizzle(blockIdx.x, n_work * n_split);
    split = work % n_split;
    work /= n_split;
    qt = work % n_qt;
    bh = work / n_qt;
  } else if (CAUSAL && n_qt >= 16) {
    // query tiles heaviest first over all (b, h) at a time; consecutive
    // workgroups go to the 8 XCDs in turn, so (b, h) stays on XCD bh % 8
    // when B*H is a multiple of 8
    qt = n_qt - 1 - (int)(blockIdx.x / BH);
    bh = blockIdx.x % BH;
  } else {
    const int work = xcd_swizzle(blockIdx.x, n_work);
    qt = work % n_qt;
    bh = work / n_qt;
    if (CAUSAL) qt = n_qt - 1 - qt;     // heaviest query tiles first
  }
  const int q0 = qt * BM8;
  const int wr0 = q0 + wave * 32;
  const int diag = S_k - S_q;
  // this workgroup's keys: k_lo .. k_hi - 1 (a 64-key multiple apart), as
  // tiles t0 .. t_end - 1 counted from key 0
  const int k_lo = SPLIT ? split * keys_per_split : 0;
  const int k_hi = SPLIT ? min(S_k, k_lo + keys_per_split) : S_k;
  int k_end = k_hi;
  if (CAUSAL) k_end = min(k_end, q0 + BM8 - 1 + diag + 1);
  const int t0 = k_lo / BN8;
  const int t_end = k_end > k_lo ? (k_end + BN8 - 1) / BN8 : t0;
  const int nq_blk = (S_q + 63) / 64, nk_blk = (S_k + 63) / 64;

  const size_t qoff = (size_t)bh * S_q * D8;
  const size_t koff = (size_t)bh * S_k * D8;
  const uint8_t* Kh = K8 + koff;
  const uint8_t* Vh = V8 + koff;
  const float c_q = c * qs[(size_t)bh * nq_blk + min(wr0, S_q - 1) / 64];
  const float* ksh = ks + (size_t)bh * nk_blk;
  const float v_scale = *vs;

  // Q^T fragments: lane (h, n) holds bytes 64*k2 + 32*h .. +31 of query row n
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

  // stage j = K(j), V(j): every wave issues NI8 K and NI8 V loads (1 KiB =
  // 8 rows each). Each stage has its own buffer resources, built in scalar
  // registers: base at the tile's first row, range the bytes of K / V left
  // from there (at most one tile). The per-lane offsets stay below one tile
  // and are all the range check sees, so rows past the end (the last tile's
  // tail, and the two stages fetched past the end so that every step issues
  // the same loads and the wait counts stay exact) read zeros and touch no
  // memory outside the tensors.
  int lane_k[NI8], lane_v[NI8];
#pragma unroll
  for (int i = 0; i < NI8; i++) {
    const int r = (i * NW8 + wave) * 8 + (lane >> 3);
    lane_k[i] = r * D8 + (((lane & 7) ^ k8_swz(r)) * 16);
    if (VT) {
      // V^T [D][S_k] per head: a 1 KiB wave load fills 16 rows d of 64 key
      // bytes; the tile's key offset (64 j) is added per stage
      const int d = (i * NW8 + wave) * 16 + (lane >> 2);
      lane_v[i] = d * S_k + (((lane & 3) ^ vt8_swz(d)) * 16);
    } else {
      lane_v[i] = r * D8 + (((lane & 7) ^ v8_swz(r)) * 16);
    }
  }
  // V^T: one resource over the head's D rows of S_k bytes. Key bytes past
  // S_k in a tile belong to the next row (finite codes whose P is 0); past
  // the last row the range check returns zeros.
  const __amdgpu_buffer_rsrc_t vtrs = __builtin_amdgcn_make_buffer_rsrc((void*)Vh, (short)0, D8 * S_k, 0x00020000);
  // (offsets and destinations go through locals: a target builtin with
  // template-dependent argument expressions is dropped from the host pass)
  auto issue_stage = [&](int j, char* base) {
    const int off = j * TILE8;
    const int left = S_k * D8 > off ? min(S_k * D8 - off, TILE8) : 0;
    const __amdgpu_buffer_rsrc_t krs =
        __builtin_amdgcn_make_buffer_rsrc((void*)(Kh + off), (short)0, left, 0x00020000);
    const __amdgpu_buffer_rsrc_t vrs =
        __builtin_amdgcn_make_buffer_rsrc((void*)(Vh + off), (short)0, left, 0x00020000);
#pragma unroll
    for (int i = 0; i < NI8; i++) {
      char* kdst = base + (i * NW8 + wave) * 1024;
      char* vdst = base + TILE8 + (i * NW8 + wave) * 1024;
      const int lk = lane_k[i], lv = lane_v[i];
      __builtin_amdgcn_raw_ptr_buffer_load_lds(krs, (__attribute__((address_space(3))) void*)kdst, 16, lk, 0, 0, 0);
      if (VT) {
        const int lvt = lv + j * BN8;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(vtrs, (__attribute__((address_space(3))) void*)vdst, 16, lvt, 0, 0,
                                                 0);
      } else {
        __builtin_amdgcn_raw_ptr_buffer_load_lds(vrs, (__attribute__((address_space(3))) void*)vdst, 16, lv, 0, 0, 0);
      }
    }
  };

  // per-lane LDS read offsets
  const int xk = k8_swz(nn);
  int k_rd[4];                                   // chunk pairs (k2, h) of row nn
#pragma unroll
  for (int k2 = 0; k2 < 2; k2++)
#pragma unroll
    for (int e = 0; e < 2; e++) k_rd[2 * k2 + e] = nn * D8 + (((4 * k2 + 2 * hh + e) ^ xk) * 16);
  const int g = lane >> 4, jj = lane & 15;
  const int vrow = 8 * (jj >> 3) + 4 * hh + ((jj >> 1) & 3);
  const int xv = v8_swz(vrow);
  int v_rd[DB8];
#pragma unroll
  for (int db = 0; db < DB8; db++) {
    if (VT) {
      // V^T row d = 32 db + nn, chunk db: dword q of the fragment holds keys
      // 8 q + 4 h .. +3, byte 8 (q & 1) + 4 h of chunk q / 2
      v_rd[db] = nn * BN8 + ((db ^ vt8_swz(nn)) * 16) + 4 * hh;
    } else {
      v_rd[db] = vrow * D8 + (((2 * db + (g & 1)) ^ xv) * 16) + 8 * (jj & 1);
    }
  }

  v16f o[DB8];
#pragma unroll
  for (int db = 0; db < DB8; db++)
#pragma unroll
    for (int e = 0; e < 16; e++) o[db][e] = 0.0f;
  float m = kNegInf, l = 0.0f, rf = 0.0f;
  // A operand of the row-sum product: lane (G = lane / 16, r = lane % 16)
  // holds E4M3 ones (0x38) when G and r / 4 have the same parity. B lane
  // 16 G + n holds query n + 16 (G % 2), key half G / 2, so output row r
  // (lanes G' = r / 4) sums the two B lane groups of its query
  v8i ones_sel;
  {
    const int sel = ((lane >> 4) & 1) == ((lane >> 2) & 1) ? 0x38383838 : 0;
#pragma unroll
    for (int i = 0; i < 8; i++) ones_sel[i] = sel;
  }

  const __amdgpu_buffer_rsrc_t ksrs = __builtin_amdgcn_make_buffer_rsrc((void*)ksh, (short)0, nk_blk * 4, 0x00020000);
  auto tile_scale_v = [&](int t) {
    const int off = (min(t * BN8, S_k - 1) / 64) * 4;
    return c_q * __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(ksrs, off, 0, 0));
  };
  float cs_cur = c_q * ksh[t0];

  auto barrier = [] {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
    asm volatile("" ::: "memory");
  };

  // One step per tile t: S(t) = K(t) Q^T, softmax of tile t, O += V(t)^T P(t).
  // The wave runs them in order; the three waves per SIMD (one of each of the
  // CU's three workgroups) overlap one another's matrix and vector work.
  auto step = [&](auto bi, auto masked, int t) {
    constexpr int B = decltype(bi)::value;
    constexpr bool MASKED = decltype(masked)::value;
    const char* rbuf = B == 0 ? st0 : B == 1 ? st1 : st2;
    char* dbuf = B == 0 ? st2 : B == 1 ? st0 : st1;    // buffer (t + 2) % 3
    const float cc = cs_cur;
    barrier();
    const float c_nx = tile_scale_v(t + 1);
    issue_stage(t + 2, dbuf);
    // S^T = K Q^T: four 32x32x64 steps (k2-major within each 32-key block)
    v16f s[KB8];
    {
      auto load = [&](int j) {
        const int kb = j / 2, k2 = j % 2;
        const char* kp = rbuf + kb * 32 * D8;
        const uint4 lo = *(const uint4*)(kp + k_rd[2 * k2]);
        const uint4 hi = *(const uint4*)(kp + k_rd[2 * k2 + 1]);
        return v8i{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
      };
      v8i ring[2];
      ring[0] = load(0);
#pragma unroll
      for (int j = 0; j < 4; j++) {
        if (j + 1 < 4) ring[(j + 1) & 1] = load(j + 1);
        const int kb = j / 2, k2 = j % 2;
        if (k2 == 0) {
          const v16f zero = {};
          s[kb] = mma8(ring[j & 1], qf[0], zero);
        } else {
          s[kb] = mma8(ring[j & 1], qf[1], s[kb]);
        }
      }
    }
    if (MASKED) {
      const int key0 = t * BN8;
      const int q = wr0 + nn;
#pragma unroll
      for (int kb = 0; kb < KB8; kb++)
#pragma unroll
        for (int i = 0; i < 4; i++)
#pragma unroll
          for (int jx = 0; jx < 4; jx++) {
            const int key = key0 + kb * 32 + 8 * i + 4 * hh + jx;
            const bool ok = key < k_hi && (!CAUSAL || key <= q + diag);
            if (!ok) s[kb][4 * i + jx] = kNegInf;
          }
    }
    // the row's keys are split over the two halves of the wave: when neither
    // half's maximum passes the bound, the row's does not either, so the
    // exchange between the halves is needed only when the reference moves
    float xh = kNegInf;
#pragma unroll
    for (int kb = 0; kb < KB8; kb++)
#pragma unroll
      for (int e = 0; e < 16; e++) xh = fmaxf(xh, s[kb][e]);
    if (__any(xh * cc > m + kTau8)) {
      const float x = pair_max(xh) * cc;
      const float mnew = fmaxf(m, x);
      const float r = mnew == kNegInf ? 0.0f : mnew;
      const float alpha = fast_exp2(m - r);      // 0 when m was -inf
      m = mnew;
      rf = r;
      l *= alpha;
#pragma unroll
      for (int db = 0; db < DB8; db++)
#pragma unroll
        for (int e = 0; e < 16; e++) o[db][e] *= alpha;
    }
    const float nref = kPShift8 - rf;            // p * 2^7 = 2^(s*cc - rf + 7)
    v8i pf;
#pragma unroll
    for (int quad = 0; quad < 8; quad++) {
      const int b = quad / 4, q4 = quad % 4;
      float p[4];
#pragma unroll
      for (int e = 0; e < 4; e++) {
        p[e] = fast_exp2(__builtin_fmaf(s[b][4 * q4 + e], cc, nref));
      }
      pf[quad] = (int)pack_fp8(p[0], p[1], p[2], p[3]);
    }
    // O^T += V^T P^T: four 32x32x64 steps, one per 32-row block of O^T, and
    // the tile's row sums (issued first: they need no LDS read)
    {
      const char* vl = rbuf + TILE8;
      auto load = [&](int db) {
        if (VT) {
          // rows 32 db + nn of the V^T tile; v_rd holds the chunk of q / 2 = c
          const char* row = vl + db * 32 * BN8;
          v8i r;
#pragma unroll
          for (int q = 0; q < 8; q++) r[q] = *(const int*)(row + v_rd[q >> 1] + 8 * (q & 1));
          return r;
        }
        v2i part[4];
#pragma unroll
        for (int p = 0; p < 4; p++) {
          const int row0 = 32 * (p >> 1) + 16 * (p & 1);
          part[p] = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_v2i*)(vl + v_rd[db] + row0 * D8));
        }
        return v8i{part[0][0], part[0][1], part[1][0], part[1][1], part[2][0], part[2][1], part[3][0], part[3][1]};
      };
      v8i ring[2];
      ring[0] = load(0);
      const v4f zero4 = {};
      const v4f lt = mma8_rows(ones_sel, pf, zero4);
#pragma unroll
      for (int db = 0; db < DB8; db++) {
        if (db + 1 < DB8) ring[(db + 1) & 1] = load(db + 1);
        o[db] = mma8(ring[db & 1], pf, o[db]);
      }
      l += lt[0];
    }
    cs_cur = c_nx;
    __builtin_amdgcn_s_waitcnt(0x0070 | 0x0F00 | (2 * NI8 + 1));   // stage t+1 complete
  };

  if (t_end > t0) {
    int t_last = t_end - 1;
    if (CAUSAL) {
      const int lim = wr0 + 31 + diag;
      t_last = lim < 0 ? -1 : min(t_last, lim / BN8);
    }
    issue_stage(t0, st0);
    issue_stage(t0 + 1, st1);
    __builtin_amdgcn_s_waitcnt(0x0070 | 0x0F00 | (2 * NI8));      // stage 0 complete
    int u_mask = k_hi / BN8;                     // tiles that need no mask for any row of the wave
    if (CAUSAL) {
      const int lim2 = wr0 + diag + 1;
      u_mask = min(u_mask, lim2 < 0 ? 0 : lim2 / BN8);
    }
    const IC8<0> P;
    const IC8<1> Mk;
    int t = t0;                                  // tile t sits in buffer (t - t0) % 3
    const int t_plain = min(t_last + 1, u_mask);  // tiles before this one need no mask
    for (; t + 2 < t_plain; t += 3) {
      step(IC8<0>(), P, t);
      step(IC8<1>(), P, t + 1);
      step(IC8<2>(), P, t + 2);
    }
    for (; t + 2 <= t_last; t += 3) {
      step(IC8<0>(), Mk, t);
      step(IC8<1>(), Mk, t + 1);
      step(IC8<2>(), Mk, t + 2);
    }
    if (t <= t_last) { step(IC8<0>(), Mk, t); t++; }
    if (t <= t_last) { step(IC8<1>(), Mk, t); t++; }
    for (; t < t_end; t++) {                     // the wave is done: keep the barriers and loads going
      const int bsel = (t - t0 + 2) % 3;
      barrier();
      issue_stage(t + 2, bsel == 0 ? st0 : bsel == 1 ? st1 : st2);
      __builtin_amdgcn_s_waitcnt(0x0070 | 0x0F00 | (2 * NI8));
    }
    __builtin_amdgcn_s_waitcnt(0x0070 | 0x0F00);
  }

  // epilogue: O = acc * vs / l (the 2^7 of p cancels), LSE = ln2 * (m + log2 l - 7)
  const int q = wr0 + nn;
  const float lt = l;                           // the whole row's sum in both halves
  const bool has = m != kNegInf && lt > 0.0f;
  const float inv = has ? v_scale / lt : 0.0f;
  const float lse = has ? (m + __builtin_log2f(lt) - kPShift8) * kLn2 : kNegInf;
  if (q < S_q) {
    if (!SPLIT) {
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
    } else {
      // this split's normalised partial output and LSE (merged by logsumexp)
      const size_t prow = ((size_t)split * BH + bh) * S_q + q;
      float* orow = Opart + prow * D8;
#pragma unroll
      for (int db = 0; db < DB8; db++)
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

}  // namespace

struct Fp8Launch {
  const void *q8, *k8, *v8;
  const float *qs, *ks, *vs;
  void* o;
  float* lse;
  float *opart, *lpart;
  int BH, S_q, S_k, n_qt, n_split, keys_per_split;
  float c;
};

template <bool CAUSAL, bool VT, bool SPLIT>
static void launch_fp8(const Fp8Launch& a, hipStream_t st) {
  const dim3 grid((unsigned)(a.BH * a.n_qt * (SPLIT ? a.n_split : 1)));
  hipLaunchKernelGGL((fwd_fp8_kernel<CAUSAL, VT, SPLIT>), grid, dim3(NT8), 0, st, (const uint8_t*)a.q8,
                     (const uint8_t*)a.k8, (const uint8_t*)a.v8, a.qs, a.ks, a.vs, (__bf16*)a.o, a.lse, a.opart,
                     a.lpart, a.BH, a.S_q, a.S_k, a.n_qt, a.n_split, a.keys_per_split, a.c);
}

template <bool SPLIT>
static void launch_fp8_s(const Fp8Launch& a, int causal, int v_transposed, hipStream_t st) {
  if (causal) {
    if (v_transposed) launch_fp8<true, true, SPLIT>(a, st);
    else launch_fp8<true, false, SPLIT>(a, st);
  } else {
    if (v_transposed) launch_fp8<false, true, SPLIT>(a, st);
    else launch_fp8<false, false, SPLIT>(a, st);
  }
}

int fp8_keys_per_tile() { return BN8; }
int fp8_rows_per_block() { return BM8; }

hipError_t launch_fwd_fp8(const void* q8, const void* k8, const void* v8, const float* qs, const float* ks,
                          const float* vs, void* o, float* lse, int B, int H, int S_q, int S_k, int D,
                          int causal, float c, int v_transposed, int n_split, int keys_per_split, float* opart,
                          float* lpart, hipStream_t st) {
  if (D != D8) return hipErrorNotSupported;
  if (v_transposed && S_k % 16 != 0) return hipErrorNotSupported;            // 16-byte aligned V^T rows
  if ((long long)(S_k + 4 * BN8) * D8 > 0x7fffffffLL) return hipErrorInvalidValue;   // 32-bit buffer offsets
  if (n_split > 1 && (keys_per_split % BN8 != 0 || !opart || !lpart)) return hipErrorInvalidValue;
  Fp8Launch a{q8, k8, v8, qs, ks, vs, o, lse, opart, lpart, B * H, S_q, S_k, (S_q + BM8 - 1) / BM8,
              n_split, keys_per_split, c};
  if (n_split > 1) launch_fp8_s<true>(a, causal, v_transposed, st);
  else launch_fp8_s<false>(a, causal, v_transposed, st);
  return hipGetLastError();
}

}  // namespace attn

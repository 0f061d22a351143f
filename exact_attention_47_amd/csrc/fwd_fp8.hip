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
// vector unit about twice as long as an FMA, and the two do not overlap), so
// its schedule keeps the vector unit fed from two waves per SIMD at all times.
//
// * Work split: 4 waves x 32 query rows per workgroup, 64-key tiles (one K
//   scale block and one k-step of the P V product each). Three LDS stages of
//   16 KiB: two workgroups share a CU, one wave of each per SIMD.
//
// * Overlap inside each wave ([GN] "Overlap innerhalb einer Warpgroup"): step
//   t computes S(t+1) = K(t+1) Q^T (v_mfma_scale_f32_32x32x64_f8f6f4, unit
//   scales) with the exponentials and E4M3 packing of tile t spread between
//   its matrix instructions, then O += V(t)^T P(t)^T with the row maximum of
//   tile t+1 in between. Each step is straight-line code with a scheduling
//   barrier after every matrix instruction; masked tiles (key-range tail,
//   causal diagonal) are a suffix of a wave's tiles and run in a second
//   unrolled loop; scores past the range are -inf instead of skipped; a move
//   of the row maximum is applied to O at the next step, after that tile's
//   P V (still exact).
//
// * Scores: s = scale * qs * ks * (q8 . k8), with qs the block scale of this
//   wave's 32 rows and ks that of the tile's 64 keys; their product with
//   log2(e) is one multiplier per tile, folded into the exp2 argument. P is
//   rounded to E4M3 as p * 2^7 (the factor is added to the exponent for free)
//   so small probabilities stay out of the subnormal range; the row sum l is
//   accumulated from the unrounded p * 2^7, and the 2^7 cancels in
//   O = acc * vs / l. The running maximum moves whenever a row exceeds it by
//   more than 1.75 (log2), which keeps p * 2^7 <= 430 < 448; at each move the
//   row's largest p is exactly 2^7, which E4M3 holds without rounding.
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
//   j = {K(j), V(j-1)} lives in one of three separate __shared__ arrays (the
//   compiler can then tell a direct load into one from a read of another;
//   the loop is unrolled by three); stage t+3 is fetched with buffer loads at
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

__device__ __forceinline__ uint32_t pack_fp8(float a, float b, float c, float d) {
  // the first conversion writes the low half and keeps the high half of its
  // "old" operand, which the second one overwrites: any register will do, and
  // one whose value dies here saves a copy
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, __builtin_bit_cast(int, a), false);
  w = __builtin_amdgcn_cvt_pk_fp8_f32(c, d, w, true);
  return (uint32_t)w;
}

template <int N> struct IC8 { static constexpr int value = N; };

template <bool CAUSAL>
__global__ void __launch_bounds__(NT8)
__attribute__((amdgpu_waves_per_eu(2, 2)))
fwd_fp8_kernel(const uint8_t* __restrict__ Q8, const uint8_t* __restrict__ K8, const uint8_t* __restrict__ V8,
               const float* __restrict__ qs, const float* __restrict__ ks, const float* __restrict__ vs,
               __bf16* __restrict__ O, float* __restrict__ LSE, int BH, int S_q, int S_k, int n_qt, float c)
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
  const int work = xcd_swizzle(blockIdx.x, n_work);
  int qt = work % n_qt;
  const int bh = work / n_qt;
  if (CAUSAL) qt = n_qt - 1 - qt;       // heaviest query tiles first
  const int q0 = qt * BM8;
  const int wr0 = q0 + wave * 32;
  const int diag = S_k - S_q;
  int k_end = S_k;
  if (CAUSAL) k_end = min(k_end, q0 + BM8 - 1 + diag + 1);
  const int n_tiles = k_end > 0 ? (k_end + BN8 - 1) / BN8 : 0;
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

  // stage j = K(j), V(j-1): every wave issues NI8 K and NI8 V instructions
  // (1 KiB = 8 rows each), buffer loads on per-head resources; rows outside
  // K/V read zeros, so every stage issues the same number of instructions
  const __amdgpu_buffer_rsrc_t krs = __builtin_amdgcn_make_buffer_rsrc((void*)Kh, (short)0, S_k * D8, 0x00020000);
  const __amdgpu_buffer_rsrc_t vrs = __builtin_amdgcn_make_buffer_rsrc((void*)Vh, (short)0, S_k * D8, 0x00020000);
  // lane part of each load's offset (lane-constant: the swizzle repeats every
  // 16 rows and every load covers 8 rows at a multiple of 8) plus a
  // wave-uniform stage offset; stage 0 has no V tile (its V loads would
  // start before the buffer) and is waited for in full before the loop
  int lane_k[NI8], lane_v[NI8];
#pragma unroll
  for (int i = 0; i < NI8; i++) {
    const int r = (i * NW8 + wave) * 8 + (lane >> 3);
    lane_k[i] = r * D8 + (((lane & 7) ^ k8_swz(r)) * 16);
    lane_v[i] = r * D8 + (((lane & 7) ^ v8_swz(r)) * 16);
  }
  // (offsets and destinations go through locals: a target builtin with
  // template-dependent argument expressions is dropped from the host pass)
  auto issue_stage = [&](int j, char* base) {
    const int soff_k = j * TILE8;
    const int soff_v = (j - 1) * TILE8;
#pragma unroll
    for (int i = 0; i < NI8; i++) {
      char* kdst = base + (i * NW8 + wave) * 1024;
      const int lk = lane_k[i];
      __builtin_amdgcn_raw_ptr_buffer_load_lds(krs, (__attribute__((address_space(3))) void*)kdst, 16, lk, soff_k, 0, 0);
    }
    if (j >= 1) {
#pragma unroll
      for (int i = 0; i < NI8; i++) {
        char* vdst = base + TILE8 + (i * NW8 + wave) * 1024;
        const int lv = lane_v[i];
        __builtin_amdgcn_raw_ptr_buffer_load_lds(vrs, (__attribute__((address_space(3))) void*)vdst, 16, lv, soff_v, 0, 0);
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
  for (int db = 0; db < DB8; db++)
    v_rd[db] = vrow * D8 + (((2 * db + (g & 1)) ^ xv) * 16) + 8 * (jj & 1);

  v16f o[DB8];
#pragma unroll
  for (int db = 0; db < DB8; db++)
#pragma unroll
    for (int e = 0; e < 16; e++) o[db][e] = 0.0f;
  v16f sacc[3][KB8];               // scores of tiles j, j+1 (index j % 3)
#pragma unroll
  for (int kb = 0; kb < KB8; kb++)
#pragma unroll
    for (int e = 0; e < 16; e++) sacc[2][kb][e] = kNegInf;   // "tile -1"
  v8i pf;
  float m = kNegInf, l = 0.0f, rf = 0.0f, alpha = 1.0f, xmax = kNegInf;
  bool resc = false;

  auto tile_active = [&](int t) { return !CAUSAL || t * BN8 <= wr0 + 31 + diag; };
  auto tile_scale = [&](int t) { return c_q * ksh[min(t * BN8, S_k - 1) / 64]; };
  float cs_cur = 1.0f, cs_nxt = 1.0f;        // scales of the current and next tile
  const __amdgpu_buffer_rsrc_t ksrs = __builtin_amdgcn_make_buffer_rsrc((void*)ksh, (short)0, nk_blk * 4, 0x00020000);
  auto tile_scale_v = [&](int t) {
    const int off = (min(t * BN8, S_k - 1) / 64) * 4;
    return c_q * __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(ksrs, off, 0, 0));
  };

  auto mask = [&](v16f* sn, int t) {
    const int key0 = t * BN8;
    const int q = wr0 + nn;
#pragma unroll
    for (int kb = 0; kb < KB8; kb++)
#pragma unroll
      for (int i = 0; i < 4; i++)
#pragma unroll
        for (int jx = 0; jx < 4; jx++) {
          const int key = key0 + kb * 32 + 8 * i + 4 * hh + jx;
          const bool ok = key < S_k && (!CAUSAL || key <= q + diag);
          if (!ok) sn[kb][4 * i + jx] = kNegInf;
        }
  };
  // row maximum of a new tile: decide whether the reference moves (applied to
  // O and l once the previous tile's P V is in)
  auto maxdec = [&] {
    const float x = xmax;
    resc = __any(x > m + kTau8);
    if (resc) {
      const float mnew = fmaxf(m, x);
      const float r = mnew == kNegInf ? 0.0f : mnew;
      alpha = fast_exp2(m - r);            // 0 when m was -inf
      m = mnew;
      rf = r;
    }
  };

  // S(t+1)^T = K Q^T (four 32x32x64 steps: k2-major within each 32-key block)
  // with the exponentials and E4M3 packing of tile t spread over the steps
  constexpr int LA = 2;
  auto sblock = [&](const char* st, v16f* sd, const v16f* sc, float cc) {
    constexpr int NS = KB8 * 2;
    constexpr int EPS = 16 * KB8 / NS;           // exponentials per step (8)
    auto load = [&](int j) {
      const int kb = j / 2, k2 = j % 2;
      const char* kp = st + kb * 32 * D8;
      const uint4 lo = *(const uint4*)(kp + k_rd[2 * k2]);
      const uint4 hi = *(const uint4*)(kp + k_rd[2 * k2 + 1]);
      return v8i{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
    };
    v8i ring[LA + 1];
#pragma unroll
    for (int j = 0; j < LA; j++) ring[j] = load(j);
    const float nref = -(rf - kPShift8);         // p * 2^7 = 2^(s*cc - rf + 7)
#pragma unroll
    for (int j = 0; j < NS; j++) {
      if (j + LA < NS) ring[(j + LA) % (LA + 1)] = load(j + LA);
      const int kb = j / 2, k2 = j % 2;
      if (k2 == 0) {
        const v16f zero = {};
        sd[kb] = mma8(ring[j % (LA + 1)], qf[0], zero);
      } else {
        sd[kb] = mma8(ring[j % (LA + 1)], qf[1], sd[kb]);
      }
      // slots 4*q4 .. 4*q4+3 of block b go to word 4*b + q4 of P^T; the
      // packed words and the row sum are written in place each step, which
      // keeps this step's exponentials in this step (values only used at the
      // end would be sunk past the scheduling barriers)
#pragma unroll
      for (int u = 0; u < EPS / 4; u++) {
        const int quad = j * (EPS / 4) + u, b = quad / 4, q4 = quad % 4;
        float p[4];
#pragma unroll
        for (int e = 0; e < 4; e++) {
          p[e] = fast_exp2(__builtin_fmaf(sc[b][4 * q4 + e], cc, nref));
          l += p[e];
        }
        pf[4 * b + q4] = (int)pack_fp8(p[0], p[1], p[2], p[3]);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  // O^T += V(t)^T P(t)^T (four 32x32x64 steps, one per 32-row block of O^T)
  // with the row maximum of tile t+1 spread over the steps
  auto pblock = [&](auto do_m, const char* st, const v16f* sn, float cn) {
    constexpr bool DM = decltype(do_m)::value;
    constexpr int MPS = 16 * KB8 / DB8;          // score elements per step (8)
    const char* vl = st + TILE8;
    auto load = [&](int db) {
      v2i part[4];
#pragma unroll
      for (int p = 0; p < 4; p++) {
        const int row0 = 32 * (p >> 1) + 16 * (p & 1);
        part[p] = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_v2i*)(vl + v_rd[db] + row0 * D8));
      }
      return v8i{part[0][0], part[0][1], part[1][0], part[1][1], part[2][0], part[2][1], part[3][0], part[3][1]};
    };
    v8i ring[LA + 1];
#pragma unroll
    for (int j = 0; j < LA; j++) ring[j] = load(j);
    if (DM) xmax = kNegInf;
#pragma unroll
    for (int db = 0; db < DB8; db++) {
      if (db + LA < DB8) ring[(db + LA) % (LA + 1)] = load(db + LA);
      o[db] = mma8(ring[db % (LA + 1)], pf, o[db]);
      if (DM) {                                  // (in place, like the row sum)
#pragma unroll
        for (int u = 0; u < MPS; u++) {
          const int idx = db * MPS + u;
          xmax = fmaxf(xmax, sn[idx / 16][idx % 16]);
        }
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    if (DM) xmax = pair_max(xmax) * cn;
  };
  auto barrier = [] {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
    asm volatile("" ::: "memory");
  };

  // One step t (-1 <= t < n_tiles): stage t+1 (K(t+1), V(t)) is read from
  // buffer (t+1) % 3 while stage t+3 is fetched into buffer t % 3.
  auto step = [&](auto bi, auto masked, int t) {
    constexpr int B = decltype(bi)::value;
    constexpr bool MASKED = decltype(masked)::value;
    char* dbuf = B == 0 ? st0 : B == 1 ? st1 : st2;
    const char* rbuf = B == 0 ? st1 : B == 1 ? st2 : st0;
    v16f* scur = sacc[B];
    v16f* snx = sacc[(B + 1) % 3];
    // tile scales: loaded one step ahead as vector loads before the stage's
    // loads (complete at this step's final wait), so that no scalar load is
    // in flight while the step waits for its LDS reads: scalar and LDS loads
    // share one counter, and a pending scalar load makes every wait a full one
    const float c_cur = cs_cur, c_nxt = cs_nxt;
    barrier();
    const float c_pre = tile_scale_v(t + 2);
    issue_stage(t + 3, dbuf);
    if (resc) {
      l *= alpha;
#pragma unroll
      for (int db = 0; db < DB8; db++)
#pragma unroll
        for (int e = 0; e < 16; e++) o[db][e] *= alpha;
    }
    sblock(rbuf, snx, scur, c_cur);
    if (MASKED) {
      mask(snx, t + 1);
      pblock(IC8<0>(), rbuf, snx, c_nxt);
      float x = kNegInf;
#pragma unroll
      for (int kb = 0; kb < KB8; kb++)
#pragma unroll
        for (int e = 0; e < 16; e++) x = fmaxf(x, snx[kb][e]);
      xmax = pair_max(x) * c_nxt;
    } else {
      pblock(IC8<1>(), rbuf, snx, c_nxt);
    }
    maxdec();
    cs_cur = c_nxt;
    cs_nxt = c_pre;
    __builtin_amdgcn_s_waitcnt(0x0070 | 0x0F00 | (2 * NI8));   // stage t+2 complete
  };

  // steps from t = -1 to the wave's last tile with an allowed key (see the
  // main kernel's schedule notes); then only barriers and loads
  if (n_tiles > 0) {
    int t_last = n_tiles - 1;
    if (CAUSAL) {
      const int lim = wr0 + 31 + diag;
      t_last = lim < 0 ? -1 : min(t_last, lim / BN8);
    }
    cs_cur = tile_scale(0);
    cs_nxt = tile_scale(0);
    {
      // stage 0 holds no V tile; the first step multiplies its zero
      // probabilities with that part of the buffer, which must not be NaN
      uint4* vz = (uint4*)(st0 + TILE8);
#pragma unroll
      for (int i = 0; i < TILE8 / (NT8 * 16); i++) vz[i * NT8 + tid] = uint4{0, 0, 0, 0};
    }
    issue_stage(0, st0);
    issue_stage(1, st1);
    __builtin_amdgcn_s_waitcnt(0x0070 | 0x0F00);
    __syncthreads();
    int u_mask = S_k / BN8;                      // tiles that need no mask for any row of the wave
    if (CAUSAL) {
      const int lim2 = wr0 + diag + 1;
      u_mask = min(u_mask, lim2 < 0 ? 0 : lim2 / BN8);
    }
    const IC8<0> P;
    const IC8<1> Mk;
    int t = -1;
    const int t_plain = min(t_last, u_mask - 2);
    for (; t + 2 <= t_plain; t += 3) {
      step(IC8<2>(), P, t);
      step(IC8<0>(), P, t + 1);
      step(IC8<1>(), P, t + 2);
    }
    for (; t + 2 <= t_last; t += 3) {
      step(IC8<2>(), Mk, t);
      step(IC8<0>(), Mk, t + 1);
      step(IC8<1>(), Mk, t + 2);
    }
    if (t <= t_last) { step(IC8<2>(), Mk, t); t++; }
    if (t <= t_last) { step(IC8<0>(), Mk, t); t++; }
    for (; t < n_tiles; t++) {
      const int bsel = (t + 3) % 3;
      barrier();
      issue_stage(t + 3, bsel == 0 ? st0 : bsel == 1 ? st1 : st2);
      __builtin_amdgcn_s_waitcnt(0x0070 | 0x0F00 | (2 * NI8));
    }
    __builtin_amdgcn_s_waitcnt(0x0070 | 0x0F00);
    if (resc) {                    // a reference change not yet applied (cannot happen: the
      l *= alpha;                  // last scores a wave looks at are fully masked)
#pragma unroll
      for (int db = 0; db < DB8; db++)
#pragma unroll
        for (int e = 0; e < 16; e++) o[db][e] *= alpha;
    }
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
  if ((long long)(S_k + 4 * BN8) * D8 > 0x7fffffffLL) return hipErrorInvalidValue;   // 32-bit buffer offsets
  const int n_qt = (S_q + BM8 - 1) / BM8;
  const dim3 grid((unsigned)(B * H * n_qt));
  if (causal)
    hipLaunchKernelGGL(fwd_fp8_kernel<true>, grid, dim3(NT8), 0, st, (const uint8_t*)q8, (const uint8_t*)k8,
                       (const uint8_t*)v8, qs, ks, vs, (__bf16*)o, lse, B * H, S_q, S_k, n_qt, c);
  else
    hipLaunchKernelGGL(fwd_fp8_kernel<false>, grid, dim3(NT8), 0, st, (const uint8_t*)q8, (const uint8_t*)k8,
                       (const uint8_t*)v8, qs, ks, vs, (__bf16*)o, lse, B * H, S_q, S_k, n_qt, c);
  return hipGetLastError();
}

}  // namespace attn

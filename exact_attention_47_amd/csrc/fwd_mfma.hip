// Fused exact attention forward pass on gfx950 matrix cores (bf16 / fp16,
// D = 64 / 128).
//
// What is computed: O = softmax(scale * Q K^T [+ causal mask]) V and the row
// logsumexp, block by block with online softmax rescaling, so the score matrix
// never reaches HBM ([NL] "FlashAttention en FlashAttention-2"; [GN]
// "Rueckblick auf den FlashAttention-Ansatz").
//
// CDNA4 mapping of the pages' Hopper schedule:
//
// * Work split. One workgroup of 8 waves per (b, h, 256 query rows); each wave
//   owns 32 query rows for the whole key loop and holds Q^T in registers. Keys
//   are processed in tiles of 128.
//
// * Ping-pong ([GN] "Pingpong-Scheduling zwischen Warpgroups"). Waves w and
//   w+4 share a SIMD. Waves 0-3 (group 0) and 4-7 (group 1) run the same
//   loop half a step apart: while one group issues its matrix instructions
//   (P V of the previous tile, then Q K^T of the current one) the other group
//   runs the softmax of its latest tile on the vector ALU, and at each
//   workgroup barrier they swap. The group issuing matrix instructions raises
//   its wave priority so the MFMA pipe is fed first.
//
// * Loads in the shadow of compute ([NL] "2. Minimalisatie van
//   geheugenoperaties"). Stage t of a two-buffer LDS ring holds K(t) and
//   V(t-1): exactly the operands of the matrix phase that reads it. Stage t+1
//   is fetched with buffer_load_dwordx4 ... lds (global memory straight into
//   LDS, no registers) at the start of the step that reads stage t, and
//   waited for just before the step's closing barrier.
//
// * Both products run on v_mfma_f32_16x16x32 (16 cycles for a 16 x 16 x 32
//   block; under the chip's power limit the matrix cores sustain it at a
//   higher rate than the 32x32x16 form, which this kernel used before:
//   +3 to +7 % on the same schedule). Both are transposed so that a lane
//   owns query rows:
//   - S^T = K Q^T per 16-key block kb and 16-query block qb (A = 16 keys x 32
//     d from LDS, B = Q^T from registers). Lane (g = lane / 16, n = lane %
//     16) holds keys kb*16 + 4g + i (i < 4) of query qb*16 + n: a lane owns
//     two query rows (qb = 0, 1) with 32 scores each per tile. Each K
//     fragment serves both query blocks, so the LDS bytes per product are
//     those of a 32-row block.
//   - O^T += V^T P^T per 32-key pair p of S blocks (2p, 2p+1) and 16-wide d
//     block: the B operand's eight k rows of lane (g, n) are the lane's four
//     keys of block 2p then its four of block 2p+1, i.e. the lane's S values
//     of that pair after exp2 and conversion. The A operand takes the same
//     key order: two ds_read_b64_tr_b16 per fragment (rows 32p + 4g + r and
//     32p + 16 + 4g + r), which transpose 4 x 16 blocks in flight.
//   - Row maxima (rare) and the final row sums reduce over the four lanes of
//     a query: one exchange 16 lanes away, one 32 lanes away.
//
// * Softmax in base 2 with the scale folded in: p = 2^(s * c - m), c =
//   scale * log2(e). The reference m moves only when a lane's sum of P over
//   a tile exceeds 2^8 (which bounds every P by 2^8): the row maximum is
//   then computed and P recomputed, so most tiles need neither the maximum
//   nor a rescale of O, and the result is still exact because the final
//   O / l and LSE use the same m.
//
// * LDS layout. Tiles are stored unpadded ([128][D]) with a 16-byte-chunk
//   XOR swizzle that depends on the row, so that a K fragment read (16 rows,
//   one chunk each per LDS cycle) and a transposed V read (8 rows, one
//   32-byte segment each per LDS cycle) each touch all 64 banks once. The
//   direct loads write 1 KiB per wave instruction, lane i at byte 16*i; each
//   lane fetches the global chunk that the swizzle places there.
#include "common.h"
#include "kernels.h"

namespace attn {
namespace {

template <typename T> struct Mma;
template <> struct Mma<__bf16> {
  typedef v8bf16 frag;
  static __device__ __forceinline__ v4f mma(frag a, frag b, v4f c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
  }
  static __device__ __forceinline__ frag cvt(v8f x) { return __builtin_convertvector(x, v8bf16); }
};
template <> struct Mma<_Float16> {
  typedef v8f16 frag;
  static __device__ __forceinline__ v4f mma(frag a, frag b, v4f c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
  }
  static __device__ __forceinline__ frag cvt(v8f x) { return __builtin_convertvector(x, v8f16); }
};

template <int D_>
struct FwdCfg {
  static constexpr int D = D_;
  static constexpr int NW = 8;                  // waves per workgroup (two groups of 4)
  static constexpr int NT = NW * 64;
  static constexpr int BM = NW * 32;            // query rows per workgroup
  static constexpr int BN = 128;                // keys per tile
  static constexpr int KB = BN / 16;            // 16-key blocks of S^T
  static constexpr int KP = BN / 32;            // 32-key steps of O^T
  static constexpr int DS = D / 32;             // k-steps of S^T
  static constexpr int DB = D / 16;             // 16-wide column blocks of O^T
  static constexpr int RB = 2 * D;              // bytes per K/V row in LDS
  static constexpr int TILE = BN * RB;          // bytes per K or V tile
  static constexpr int STAGE = 2 * TILE;        // K(t) then V(t-1)
  static constexpr int LDS = 2 * STAGE;
  static constexpr int NI = TILE / (NT * 16);   // direct-load instructions per thread per tile
  static constexpr int RPI = 1024 / RB;         // rows written by one wave instruction
  static_assert(TILE % (NT * 16) == 0, "tile must split evenly into 1 KiB wave loads");
};

// Row-dependent 16-byte-chunk XOR swizzles. A K fragment read serves 16 rows
// with one chunk each per LDS cycle; a transposed V read 8 rows with one
// 32-byte segment each. With 256-byte rows (D = 128) every row starts on bank
// 0; with 128-byte rows (D = 64) odd rows start on bank 32, so the swizzle
// takes the row bits above the lowest.
template <int D> __device__ __forceinline__ int k_swz(int r) { return D == 64 ? (r >> 1) & 7 : r & 15; }
template <int D> __device__ __forceinline__ int v_swz(int r) { return D == 64 ? 2 * ((r >> 1) & 3) : 2 * (r & 7); }

constexpr float kSumMax = 256.0f;        // lazy rescale: a lane's tile sum of P may reach 2^8
constexpr int kVmcnt0 = 0x0070 | 0x0F00;  // s_waitcnt vmcnt(0), other counters unconstrained

// maximum / sum over the four lanes n, n+16, n+32, n+48 of a query
__device__ __forceinline__ float quad_max(float x) { return pair_max(fmaxf(x, __shfl_xor(x, 16))); }
__device__ __forceinline__ float quad_sum(float x) { return pair_sum(x + __shfl_xor(x, 16)); }

template <typename T, int D, bool CAUSAL, bool SPLIT, bool VARLEN, bool PERSIST>
__global__ void __launch_bounds__(512)
__attribute__((amdgpu_waves_per_eu(2, 2)))
fwd_mfma_kernel(const T* __restrict__ Q, const T* __restrict__ K, const T* __restrict__ V,
                  T* __restrict__ O, float* __restrict__ LSE,
                  float* __restrict__ Opart, float* __restrict__ Lpart,
                  int BH, int S_q_, int S_k_, int n_qt, int n_split, int keys_per_split, float c,
                  const int* __restrict__ cu_q, const int* __restrict__ cu_k, int H, int total_q)
{
  static_assert(!(VARLEN && SPLIT), "packed batches run unsplit");
  static_assert(!(PERSIST && (VARLEN || SPLIT)), "the persistent grid runs dense, unsplit work");
  using C = FwdCfg<D>;
  using M = Mma<T>;
  typedef typename M::frag frag;
  __shared__ __attribute__((aligned(1024))) char lds[C::LDS];

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int grp = wave >> 2;       // ping-pong group

  // A persistent grid (PERSIST) runs this body once per work item it is
  // dealt; otherwise there is one workgroup per item and one pass.
  for (int it = 0;; it++) {
  // (per item, the lane index is read afresh and passes through an empty asm
  // statement, so that no lane-dependent value is hoisted out of the item
  // loop, where it would hold a register across every item)
  int lane = PERSIST ? (int)__builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u)) : tid & 63;
  if (PERSIST) asm volatile("" : "+v"(lane));
  const int g = lane >> 4;         // 16-lane group: rows 4g..4g+3 of each 16 x 16 output block
  const int n = lane & 15;         // query column within a 16-query block
  // ---- which (b*h, q tile, split) this workgroup computes
  int split, qt, bh;
  if (PERSIST) {
    // Fixed grid of G workgroups (at most one per CU, all resident). The
    // items, heaviest query tiles first, are dealt in a snake: on even
    // rounds workgroup j takes the j-th item of the round, on odd rounds the
    // (G-1-j)-th, so heavy and light causal tiles pair up. When B*H and G
    // are multiples of 8 the deal runs per XCD (workgroup g sits on XCD
    // g % 8) over that XCD's heads, and within an XCD by head, heaviest
    // query tile first: the workgroups of a round share one or two heads'
    // K and V in L2.
    const int G = gridDim.x;
    const bool per_xcd = (BH & 7) == 0 && (G & 7) == 0;
    const int x = per_xcd ? blockIdx.x & 7 : 0;
    const int j = per_xcd ? blockIdx.x >> 3 : blockIdx.x;
    const int gx = per_xcd ? G >> 3 : G;
    const int nbh = per_xcd ? BH >> 3 : BH;
    const long long i = (long long)it * gx + ((it & 1) ? gx - 1 - j : j);
    if (i >= (long long)nbh * n_qt) break;
    const int level = (int)(i % n_qt);
    const int hsel = (int)(i / n_qt);
    bh = per_xcd ? x + 8 * hsel : hsel;
    qt = n_qt - 1 - level;
    split = 0;
  } else if (!VARLEN && (SPLIT || !CAUSAL)) {
    // equal work per item: contiguous shares of the items per XCD
    const int n_work = BH * n_qt * n_split;
    int work = xcd_swizzle(blockIdx.x, n_work);
    split = work % n_split;
    work /= n_split;
    qt = work % n_qt;
    bh = work / n_qt;
    if (CAUSAL) qt = n_qt - 1 - qt;  // heaviest query tiles first
  } else {
    // Packed batches and unsplit causal work: query tiles in descending
    // order (the heaviest work first), and (b, h) on XCD bh % 8 for every
    // tile when B*H is a multiple of 8 (the hardware deals consecutive
    // workgroups to the 8 XCDs in turn), so its K and V stay in one L2.
    split = 0;
    if (VARLEN && BH % 8 == 0) {
      // packed: XCD x takes heads x, x+8, ..., one at a time with all
      // their query tiles (highest first)
      const int x = blockIdx.x % 8, j = blockIdx.x / 8;
      bh = x + 8 * (j / n_qt);
      qt = n_qt - 1 - j % n_qt;
    } else {
      qt = n_qt - 1 - (int)(blockIdx.x / BH);
      bh = blockIdx.x % BH;
    }
  }

  const int q0 = qt * C::BM;
  const int wr0 = q0 + wave * 32;              // first row of this wave

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

  // ---- Q^T fragments (B operand of S^T): 8 d of query qb*16 + n, kept in registers
  frag qf[C::DS][2];
#pragma unroll
  for (int qb = 0; qb < 2; qb++) {
    const int q = wr0 + qb * 16 + n;
#pragma unroll
    for (int ds = 0; ds < C::DS; ds++) {
      if (q < S_q) {
        qf[ds][qb] = *(const frag*)(Qh + (size_t)q * pitch + ds * 32 + 8 * g);
      } else {
#pragma unroll
        for (int e = 0; e < 8; e++) qf[ds][qb][e] = (T)0.0f;
      }
    }
  }

  // ---- direct global -> LDS loads by the 256 threads of group 0: stage s =
  // K(s) (if s < n_tiles) and V(s-1) (if s >= 1) into buffer s & 1. Each wave
  // instruction fills 1 KiB (RPI rows); lane i lands at byte 16*i and fetches
  // the logical chunk the swizzle stores there. A lane's rows step by 16
  // (D = 128) or 32 (D = 64) between its instructions, which leaves both
  // swizzles unchanged, so its part of the offset is one constant and the
  // rest is wave-uniform. Tiles wholly inside K and V use the per-head buffer
  // resources (whose range check covers the per-lane offset only); a tile
  // reaching past the last row gets one resource per instruction, based at
  // the instruction's first row with the bytes left after it as its range,
  // so the rows past the end read zeros (their scores are masked, and zero V
  // rows keep 0 * V finite whatever memory follows).
  const int kv_bytes = VARLEN ? (S_k > 0 ? (S_k - 1) * RBg + C::RB : 0) : S_k * C::RB;
  const __amdgpu_buffer_rsrc_t krs = __builtin_amdgcn_make_buffer_rsrc((void*)Kh, (short)0, kv_bytes, 0x00020000);
  const __amdgpu_buffer_rsrc_t vrs = __builtin_amdgcn_make_buffer_rsrc((void*)Vh, (short)0, kv_bytes, 0x00020000);
  int lane_k, lane_v;
  {
    const int rsub = (lane * 16) / C::RB;           // row within the wave instruction
    const int u = ((lane * 16) % C::RB) / 16;       // physical chunk within the row
    const int r = wave * C::RPI + rsub;
    lane_k = rsub * RBg + ((u ^ k_swz<D>(r)) * 16);
    lane_v = rsub * RBg + ((u ^ v_swz<D>(r)) * 16);
  }
  auto load_tile = [&](__amdgpu_buffer_rsrc_t rs, const T* head, int lane_off, int row0, char* tb) {
    if (row0 + C::BN <= S_k) {
#pragma unroll
      for (int i = 0; i < 2 * C::NI; i++) {
        const int blk = i * 4 + wave;                // 1 KiB block of the tile
        char* dst = tb + blk * 1024;
        const int soff = (row0 + blk * C::RPI) * RBg;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (__attribute__((address_space(3))) void*)dst, 16, lane_off,
                                                 soff, 0, 0);
      }
    } else {
#pragma unroll
      for (int i = 0; i < 2 * C::NI; i++) {
        const int blk = i * 4 + wave;
        char* dst = tb + blk * 1024;
        const int off = (row0 + blk * C::RPI) * RBg;
        const int left = kv_bytes > off ? kv_bytes - off : 0;
        const __amdgpu_buffer_rsrc_t r1 =
            __builtin_amdgcn_make_buffer_rsrc((void*)((const char*)head + off), (short)0, left, 0x00020000);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(r1, (__attribute__((address_space(3))) void*)dst, 16, lane_off,
                                                 0, 0, 0);
      }
    }
  };
  auto issue_stage = [&](int s) {
    char* base = lds + (s & 1) * C::STAGE;
    if (s < n_tiles) load_tile(krs, Kh, lane_k, k_lo + s * C::BN, base);
    if (s >= 1 && s - 1 < n_tiles) load_tile(vrs, Vh, lane_v, k_lo + (s - 1) * C::BN, base + C::TILE);
  };

  // ---- per-lane LDS read offsets (swizzle folded in)
  // K fragment (kb, ds): row kb*16 + n, logical chunk 4*ds + g.
  int k_rd[C::DS];
#pragma unroll
  for (int ds = 0; ds < C::DS; ds++) k_rd[ds] = n * C::RB + (((4 * ds + g) ^ k_swz<D>(n)) * 16);
  // V fragment (p, db): lane n of group g addresses row 32p + 4g + n/4 (and
  // 16 rows further for the second half), columns 16*db + 4*(n % 4) .. +3.
  const int vrow = 4 * g + (n >> 2);
  int v_rd[C::DB];
#pragma unroll
  for (int db = 0; db < C::DB; db++)
    v_rd[db] = vrow * C::RB + (((2 * db + ((n & 3) >> 1)) ^ v_swz<D>(vrow)) * 16) + 8 * (n & 1);

  v4f o[C::DB][2];
#pragma unroll
  for (int db = 0; db < C::DB; db++)
#pragma unroll
    for (int qb = 0; qb < 2; qb++)
#pragma unroll
      for (int e = 0; e < 4; e++) o[db][qb][e] = 0.0f;
  v4f s[C::KB][2];
  frag pf[C::KP][2];
  float m[2] = {kNegInf, kNegInf}, l[2] = {0.0f, 0.0f};

  // causal: tiles that lie wholly after this wave's last row are skipped
  auto tile_active = [&](int t) { return !CAUSAL || k_lo + t * C::BN <= wr0 + 31 + diag; };

  // matrix phase: O^T += V(t-1)^T P(t-1)^T, then S(t)^T = K(t) Q^T. Each step
  // loads one A fragment from LDS (LA steps ahead) and multiplies it into both
  // query blocks; a scheduling barrier after every step keeps the compiler
  // from hoisting further loads (registers the two waves per SIMD lack).
  constexpr int LA = 3;
  constexpr int NPV = C::KP * C::DB;
  constexpr int NSK = C::DS * C::KB;
  auto gemm_phase = [&](int t) {
    const char* st = lds + (t & 1) * C::STAGE;
    if (t >= 1 && tile_active(t - 1)) {
      const char* vl = st + C::TILE;
      auto load = [&](int j) {
        const int p = j / C::DB, db = j % C::DB;
        const char* va = vl + v_rd[db] + p * 32 * C::RB;
        v4i16 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)va);
        v4i16 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)(va + 16 * C::RB));
        return __builtin_bit_cast(frag, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
      };
      frag ring[LA + 1];
#pragma unroll
      for (int j = 0; j < LA; j++) ring[j] = load(j);
#pragma unroll
      for (int j = 0; j < NPV; j++) {
        if (j + LA < NPV) ring[(j + LA) % (LA + 1)] = load(j + LA);
        const int p = j / C::DB, db = j % C::DB;
        o[db][0] = M::mma(ring[j % (LA + 1)], pf[p][0], o[db][0]);
        o[db][1] = M::mma(ring[j % (LA + 1)], pf[p][1], o[db][1]);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    if (t < n_tiles && tile_active(t)) {
      auto load = [&](int j) {
        const int ds = j / C::KB, kb = j % C::KB;
        return *(const frag*)(st + k_rd[ds] + kb * 16 * C::RB);
      };
      frag ring[LA + 1];
#pragma unroll
      for (int j = 0; j < LA; j++) ring[j] = load(j);
#pragma unroll
      for (int j = 0; j < NSK; j++) {
        if (j + LA < NSK) ring[(j + LA) % (LA + 1)] = load(j + LA);
        const int ds = j / C::KB, kb = j % C::KB;
        if (ds == 0) {
          const v4f zero = {};
          s[kb][0] = M::mma(ring[j % (LA + 1)], qf[ds][0], zero);
          s[kb][1] = M::mma(ring[j % (LA + 1)], qf[ds][1], zero);
        } else {
          s[kb][0] = M::mma(ring[j % (LA + 1)], qf[ds][0], s[kb][0]);
          s[kb][1] = M::mma(ring[j % (LA + 1)], qf[ds][1], s[kb][1]);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  };

  // vector phase: mask, online softmax of S(t), P(t) -> matrix-operand fragments
  auto softmax_phase = [&](int t) {
    if (t < 0 || t >= n_tiles || !tile_active(t)) return;
    const int key0 = k_lo + t * C::BN;
    const bool need_mask = (key0 + C::BN > k_hi) || (CAUSAL && key0 + C::BN - 1 > wr0 + diag);
    if (need_mask) {
      // Key key0 + kb*16 + 4g + i is allowed iff kb*16 + i <= lim. The sign
      // of the difference picks -inf or +inf as the bound of a minimum: two
      // vector instructions per score and no lane masks (64 compares per
      // tile would hold their 64-bit results in scalar registers).
#pragma unroll
      for (int qb = 0; qb < 2; qb++) {
        const int last = CAUSAL ? min(k_hi - 1, wr0 + qb * 16 + n + diag) : k_hi - 1;
        const int lim = last - key0 - 4 * g;
#pragma unroll
        for (int kb = 0; kb < C::KB; kb++)
#pragma unroll
          for (int i = 0; i < 4; i++) {
            const uint32_t sgn = (uint32_t)(lim - (kb * 16 + i)) & 0x80000000u;
            s[kb][qb][i] = fminf(s[kb][qb][i], __builtin_bit_cast(float, sgn | 0x7f800000u));
          }
      }
    }
    // P = 2^(s*c - m) per query row with its current reference, summed in
    // float32 and converted to the matrix operand type (keys of block 2p,
    // then of block 2p+1).
    auto exps = [&](float* ls) {
#pragma unroll
      for (int qb = 0; qb < 2; qb++) {
        const float ref = m[qb] == kNegInf ? 0.0f : m[qb];
        float acc = 0.0f;
#pragma unroll
        for (int p = 0; p < C::KP; p++) {
          v8f pv;
#pragma unroll
          for (int e = 0; e < 8; e++) {
            pv[e] = fast_exp2(__builtin_fmaf(s[2 * p + (e >> 2)][qb][e & 3], c, -ref));
            acc += pv[e];
          }
          pf[p][qb] = M::cvt(pv);
        }
        ls[qb] = acc;
      }
    };
    // Only the sums are needed while every lane's tile sum of P stays within
    // 2^8 (which bounds each P): the maximum is taken, O and l rescaled and P
    // recomputed only when some sum exceeds it or a row has no reference
    // yet. Any reference reached this way gives the exact result, as the
    // final O / l and LSE use the same m.
    float ls[2] = {__builtin_inff(), __builtin_inff()};
    if (!__any(m[0] == kNegInf || m[1] == kNegInf)) exps(ls);
    if (__any(!(ls[0] <= kSumMax) || !(ls[1] <= kSumMax))) {
#pragma unroll
      for (int qb = 0; qb < 2; qb++) {
        float x = kNegInf;
#pragma unroll
        for (int kb = 0; kb < C::KB; kb++)
#pragma unroll
          for (int i = 0; i < 4; i++) x = fmaxf(x, s[kb][qb][i]);
        x = quad_max(x) * c;
        const float mnew = fmaxf(m[qb], x);
        const float ref = mnew == kNegInf ? 0.0f : mnew;
        const float alpha = fast_exp2(m[qb] - ref);   // 0 when m was -inf, 1 when m stays
        m[qb] = mnew;
        l[qb] *= alpha;
#pragma unroll
        for (int db = 0; db < C::DB; db++)
#pragma unroll
          for (int e = 0; e < 4; e++) o[db][qb][e] *= alpha;
      }
      exps(ls);
    }
    l[0] += ls[0];
    l[1] += ls[1];
  };

  // gemm(j) | barrier | softmax(j) | barrier, group 1 one barrier behind
  // group 0, so each group's matrix phase overlaps the other's softmax.
  // Group 0 fetches stage j+1 at the start of its softmax phase j and waits
  // for it before that phase's closing barrier: both groups have finished
  // reading stage j-1 (the buffer it overwrites) by then, stage j+1 is
  // complete before either group reads it, and no LDS read is issued while
  // a direct load is in flight. Inside the loop the barriers are bare
  // s_barrier: the staged tile is the only memory to settle, waited for
  // explicitly.
  auto barrier = [] {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
    asm volatile("" ::: "memory");
  };
  if (n_tiles > 0) {
    if (grp == 0) issue_stage(0);
    __builtin_amdgcn_s_waitcnt(kVmcnt0);
    __syncthreads();
    if (grp == 1) barrier();
    for (int j = 0; j <= n_tiles; j++) {
      __builtin_amdgcn_s_setprio(1);
      gemm_phase(j);
      __builtin_amdgcn_s_setprio(0);
      barrier();
      if (grp == 0) issue_stage(j + 1);
      softmax_phase(j);
      __builtin_amdgcn_s_waitcnt(kVmcnt0);
      barrier();
    }
    if (grp == 0) barrier();
  }

  // ---- epilogue: normalise, logsumexp, store. The lane index passes
  // through an empty asm statement here too: otherwise the compiler shares
  // the row addresses of the Q loads with the O stores and keeps them live
  // across the tile loop (8-10 registers, which spilled on some variants).
  int lane_e = lane;
  asm volatile("" : "+v"(lane_e));
  const int n_e = lane_e & 15, g_e = lane_e >> 4;
#pragma unroll
  for (int qb = 0; qb < 2; qb++) {
    const int q = wr0 + qb * 16 + n_e;
    const float lt = quad_sum(l[qb]);
    const bool has = m[qb] != kNegInf && lt > 0.0f;
    const float inv = has ? 1.0f / lt : 0.0f;
    const float lse = has ? (m[qb] + __builtin_log2f(lt)) * kLn2 : kNegInf;
    if (q < S_q) {
      if (!SPLIT) {
        T* orow = Oh + (size_t)q * pitch;
#pragma unroll
        for (int db = 0; db < C::DB; db++) {
          typedef T v4t __attribute__((ext_vector_type(4)));
          v4t w;
#pragma unroll
          for (int e = 0; e < 4; e++) w[e] = (T)(o[db][qb][e] * inv);
          *(v4t*)(orow + db * 16 + 4 * g_e) = w;
        }
        if (g_e == 0) lseh[q] = lse;
      } else {
        const size_t prow = ((size_t)split * BH + bh) * S_q + q;
        float* orow = Opart + prow * D;
#pragma unroll
        for (int db = 0; db < C::DB; db++) {
          float4 w;
          w.x = o[db][qb][0] * inv;
          w.y = o[db][qb][1] * inv;
          w.z = o[db][qb][2] * inv;
          w.w = o[db][qb][3] * inv;
          *(float4*)(orow + db * 16 + 4 * g_e) = w;
        }
        if (g_e == 0) Lpart[prow] = lse;
      }
    }
  }
  // Persistent: every wave has passed the loop's last barrier after its last
  // LDS read, so the next item's first stage may overwrite the buffers.
  if (!PERSIST) break;
  }
}

template <typename T, int D, bool CAUSAL, bool SPLIT, bool VARLEN = false, bool PERSIST = false>
hipError_t launch_one(const FwdArgs& a, hipStream_t st, int n_wg = 0) {
  using C = FwdCfg<D>;
  // 32-bit buffer offsets (packed rows: S_k is the longest sequence's length)
  const long long row_bytes = VARLEN ? (long long)a.H * C::RB : C::RB;
  if ((long long)(a.S_k + C::BN) * row_bytes > 0x7fffffffLL) return hipErrorInvalidValue;
  const int n_qt = (a.S_q + C::BM - 1) / C::BM;
  const int n_work = a.B * a.H * n_qt * a.n_split;
  const int grid = PERSIST ? (n_wg < n_work ? n_wg : n_work) : n_work;
  hipLaunchKernelGGL((fwd_mfma_kernel<T, D, CAUSAL, SPLIT, VARLEN, PERSIST>), dim3(grid), dim3(C::NT), 0, st,
                     (const T*)a.q, (const T*)a.k, (const T*)a.v, (T*)a.o, a.lse, a.opart, a.lpart, a.B * a.H,
                     a.S_q, a.S_k, n_qt, a.n_split, a.keys_per_split, a.c, a.cu_q, a.cu_k, a.H, a.total_q);
  return hipGetLastError();
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

template <typename T>
hipError_t launch_varlen_t(const FwdArgs& a, hipStream_t st) {
  switch (a.D) {
    case 64: return a.causal ? launch_one<T, 64, true, false, true>(a, st) : launch_one<T, 64, false, false, true>(a, st);
    case 128: return a.causal ? launch_one<T, 128, true, false, true>(a, st) : launch_one<T, 128, false, false, true>(a, st);
  }
  return hipErrorInvalidValue;
}

template <typename T>
hipError_t launch_persistent_t(const FwdArgs& a, int n_wg, hipStream_t st) {
  switch (a.D) {
    case 64: return a.causal ? launch_one<T, 64, true, false, false, true>(a, st, n_wg)
                             : launch_one<T, 64, false, false, false, true>(a, st, n_wg);
    case 128: return a.causal ? launch_one<T, 128, true, false, false, true>(a, st, n_wg)
                              : launch_one<T, 128, false, false, false, true>(a, st, n_wg);
  }
  return hipErrorInvalidValue;
}

}  // namespace

int mfma_keys_per_tile(int D) { return D == 64 || D == 128 ? FwdCfg<128>::BN : d256_keys_per_tile(); }
int mfma_rows_per_block(int D) { (void)D; return FwdCfg<128>::BM; }

hipError_t launch_fwd_mfma(const FwdArgs& a, hipStream_t st) {
  if (a.D == 256) return launch_fwd_d256(a, st);
  if (a.dtype == 2) return launch_t<__bf16>(a, st);
  return launch_t<_Float16>(a, st);
}

hipError_t launch_fwd_varlen(const FwdArgs& a, hipStream_t st) {
  if (a.dtype == 2) return launch_varlen_t<__bf16>(a, st);
  return launch_varlen_t<_Float16>(a, st);
}

hipError_t launch_fwd_persistent(const FwdArgs& a, int n_wg, hipStream_t st) {
  if (a.n_split != 1 || n_wg < 1) return hipErrorInvalidValue;
  if (a.dtype == 2) return launch_persistent_t<__bf16>(a, n_wg, st);
  return launch_persistent_t<_Float16>(a, n_wg, st);
}

}  // namespace attn

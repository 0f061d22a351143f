// Fused exact attention forward pass on gfx950 matrix cores (bf16 / fp16).
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
//   are processed in tiles of BN.
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
// * Both GEMMs are transposed so that one lane owns one query row:
//   S^T = K Q^T with v_mfma_f32_32x32x16 (A = K rows from LDS, B = Q^T from
//   VGPRs): lane (h, n) holds 16 keys of query n, so row max and row sum need
//   one exchange with lane n+32 only. O^T = V^T P^T (A = V^T read with
//   ds_read_b64_tr_b16, which transposes in flight; B = P^T, which is the S^T
//   accumulator after exp2 and conversion, already in the B operand's k order
//   given the matching choice of keys for V^T).
//
// * Softmax in base 2 with the scale folded in: p = 2^(s * c - m), c =
//   scale * log2(e). The reference m moves only when a lane's sum of P over
//   a tile exceeds 2^8 (which bounds every P by 2^8): the row maximum is
//   then computed and P recomputed, so most tiles need neither the maximum
//   nor a rescale of O, and the result is still exact because the final
//   O / l and LSE use the same m.
//
// * LDS layout. Tiles are stored unpadded ([BN][D]) with a 16-byte-chunk XOR
//   swizzle that depends on the row, so that the K reads (16 lanes per LDS
//   cycle: 16 rows, one chunk each) and the transposed V reads (32 lanes per
//   cycle: 4 rows x 64 bytes) each touch all 64 banks once. The direct loads
//   write 1 KiB per wave instruction, lane i at byte 16*i; each lane fetches
//   the global chunk that the swizzle places there.
#include "common.h"
#include "kernels.h"

namespace attn {

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

template <int D, int BN_>
struct FwdCfg {
  static constexpr int NW = 8;                  // waves per workgroup (two groups of 4)
  static constexpr int NT = NW * 64;
  static constexpr int BM = NW * 32;            // query rows per workgroup
  static constexpr int BN = BN_;                // keys per tile
  static constexpr int KB = BN / 32;            // 32-key blocks per tile
  static constexpr int DS = D / 16;             // k-steps of the S^T product
  static constexpr int DB = D / 32;             // 32-wide column blocks of O^T
  static constexpr int RB = 2 * D;              // bytes per K/V row
  static constexpr int TILE = BN * RB;          // bytes per K or V tile
  static constexpr int STAGE = 2 * TILE;        // K(t) then V(t-1)
  static constexpr int LDS = 2 * STAGE;
  static constexpr int NI = TILE / (NT * 16);   // direct-load instructions per thread per tile
  static constexpr int RPI = 1024 / RB;         // rows written by one wave instruction
  static_assert(TILE % (NT * 16) == 0, "tile must split evenly into 1 KiB wave loads");
};

// Row-dependent 16-byte-chunk XOR swizzles of the K and V tiles.
template <int D> __device__ __forceinline__ int k_swz(int r) { return D == 64 ? (r >> 1) & 7 : r & 15; }
template <int D> __device__ __forceinline__ int v_swz(int r) { return D == 64 ? 4 * ((r >> 1) & 1) : 4 * (r & 3); }

constexpr float kSumMax = 256.0f;   // lazy rescale: a lane's tile sum of P may reach 2^8
constexpr int kVmcnt0 = 0x0070 | 0x0F00;   // s_waitcnt vmcnt(0), other counters unconstrained

template <typename T, int D, int BN, bool CAUSAL, bool SPLIT, bool VARLEN, bool PERSIST>
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
  using C = FwdCfg<D, BN>;
  using M = Mma<T>;
  typedef typename M::frag frag;
  __shared__ __attribute__((aligned(1024))) char lds[C::LDS];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int grp = wave >> 2;       // ping-pong group
  const int hh = lane >> 5;        // lane half
  const int nn = lane & 31;        // query column owned by this lane

  // A persistent grid (PERSIST) runs this body once per work item it is
  // dealt; otherwise there is one workgroup per item and one pass.
  for (int it = 0;; it++) {
  // ---- which (b*h, q tile, split) this workgroup computes
  int split, qt, bh;
  if (PERSIST) {
    // Fixed grid of G workgroups (at most one per CU, all resident). The
    // items, heaviest query tiles first, are dealt in a snake: on even
    // rounds workgroup j takes the j-th item of the round, on odd rounds the
    // (G-1-j)-th, so the heavy and light causal tiles pair up and every
    // workgroup gets about the same number of keys. When B*H and G are
    // multiples of 8 the deal runs per XCD (workgroup g sits on XCD g % 8)
    // over the heads of that XCD only, so a head's tiles share one L2.
    const int G = gridDim.x;
    const bool per_xcd = (BH & 7) == 0 && (G & 7) == 0;
    const int x = per_xcd ? blockIdx.x & 7 : 0;
    const int j = per_xcd ? blockIdx.x >> 3 : blockIdx.x;
    const int gx = per_xcd ? G >> 3 : G;
    const int nbh = per_xcd ? BH >> 3 : BH;
    const long long i = (long long)it * gx + ((it & 1) ? gx - 1 - j : j);
    if (i >= (long long)nbh * n_qt) break;
    // items by head, heaviest query tile first within a head: the workgroups
    // of a round share one or two heads' K and V in L2, and when the tile
    // count and the workgroups per XCD divide one another the snake pairs
    // every tile with its mirror (level l with n_qt - 1 - l)
    const int level = (int)(i % n_qt);
    const int hsel = (int)(i / n_qt);
    bh = per_xcd ? x + 8 * hsel : hsel;
    qt = n_qt - 1 - level;
    split = 0;
  } else if (!VARLEN && (SPLIT || !CAUSAL)) {
    const int n_work = BH * n_qt * n_split;
    int work = xcd_swizzle(blockIdx.x, n_work);
    split = work % n_split;
    work /= n_split;
    qt = work % n_qt;
    bh = work / n_qt;
    if (CAUSAL) qt = n_qt - 1 - qt;  // heaviest query tiles first
  } else {
    // Packed batches and unsplit causal work: the workgroups' loads differ,
    // so a contiguous share of the work per XCD (as above) would leave some
    // XCDs with all the long sequences (packed) or all the late query tiles.
    // Query tiles go out in descending order instead, all (b, h) at a time:
    // high tiles exist only in long sequences, and causal tiles grow with the
    // index, so the heaviest work starts first; the hardware deals
    // consecutive workgroups to the 8 XCDs in turn, so (b, h) lands on XCD
    // bh % 8 for every tile when B*H is a multiple of 8 (its K and V stay in
    // one L2). Measured on causal D=128 8K: +2.5 % over the contiguous shares.
    split = 0;
    if (VARLEN && BH % 8 == 0) {
      // packed: XCD x (workgroups x, x+8, ...) takes heads bh = x, x+8, ...,
      // one at a time with all their query tiles (highest first): every XCD
      // gets the same share of each sequence, and the tiles of one head run
      // together, so its K and V are read from L2 rather than once per tile
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

  // ---- direct global -> LDS loads, issued by the 256 threads of group 0:
  // stage s = K(s) (if s < n_tiles) and V(s-1) (if s >= 1) into buffer s & 1.
  // Each wave instruction fills 1 KiB (RPI rows); lane i lands at byte 16*i
  // and fetches the logical chunk the swizzle stores there. The loads are
  // buffer loads on per-head resources. The rows a lane loads step by 16
  // (D=128) or 32 (D=64) between its instructions, which leaves both swizzles
  // unchanged, so its part of the offset is one constant and the rest (tile
  // row and 1 KiB block) is wave-uniform: no vector arithmetic per load.
  // The buffer range check covers the per-lane offset and not the scalar
  // one, so that split serves only tiles that lie wholly inside K and V. A
  // tile that reaches past the last row gets one resource per load
  // instruction instead, built in scalar registers: its base is the
  // instruction's first row and its range the bytes left after it, so the
  // per-lane offset alone is checked and the rows past the end read zeros
  // (their scores are masked, and zero V rows keep 0 * V finite whatever
  // memory follows).
  // (packed rows are strided: the range ends after the last row's D elements)
  const int kv_bytes = VARLEN ? (S_k > 0 ? (S_k - 1) * RBg + C::RB : 0) : S_k * C::RB;
  const __amdgpu_buffer_rsrc_t krs = __builtin_amdgcn_make_buffer_rsrc((void*)Kh, (short)0, kv_bytes, 0x00020000);
  const __amdgpu_buffer_rsrc_t vrs = __builtin_amdgcn_make_buffer_rsrc((void*)Vh, (short)0, kv_bytes, 0x00020000);
  int lane_k, lane_v;
  {
    const int rsub = (lane * 16) / C::RB;           // row within the wave instruction
    const int u = ((lane * 16) % C::RB) / 16;       // physical chunk within the row
    const int r = wave * C::RPI + rsub;             // first row; later rows differ by a multiple of 16
    lane_k = rsub * RBg + ((u ^ k_swz<D>(r)) * 16);
    lane_v = rsub * RBg + ((u ^ v_swz<D>(r)) * 16);
  }
  // (offsets and destinations go through locals: a target builtin with
  // template-dependent argument expressions is dropped from the host pass)
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
  // The XOR only reaches the low 3 (K) / 2 (V) bits of the chunk index, so
  // the offsets repeat every 8 k-steps / 4 column blocks up to a constant.
  constexpr int NKR = C::DS < 8 ? C::DS : 8;
  constexpr int NVR = C::DB < 4 ? C::DB : 4;
  const int xk = k_swz<D>(nn);                 // K row = kb*32 + nn: swizzle depends on nn only
  int k_rd[NKR];
#pragma unroll
  for (int ds = 0; ds < NKR; ds++) k_rd[ds] = nn * C::RB + (((2 * ds + hh) ^ xk) * 16);
  const int g = lane >> 4, jj = lane & 15;
  const int vrow = 4 * hh + (jj >> 2);         // V row = vrow + kb*32 + 16*ks + 8*part
  const int xv = v_swz<D>(vrow);               // depends on vrow's low bits only
  int v_rd[NVR];
#pragma unroll
  for (int db = 0; db < NVR; db++)
    v_rd[db] = vrow * C::RB + (((4 * db + 2 * (g & 1) + ((jj & 3) >> 1)) ^ xv) * 16) + 8 * (jj & 1);

  v16f o[C::DB];
#pragma unroll
  for (int db = 0; db < C::DB; db++)
#pragma unroll
    for (int e = 0; e < 16; e++) o[db][e] = 0.0f;
  v16f s[C::KB];
  frag pf[C::KB][2];
  float m = kNegInf, l = 0.0f;

  // causal: tiles that lie wholly after this wave's last row are skipped
  auto tile_active = [&](int t) { return !CAUSAL || k_lo + t * C::BN <= wr0 + 31 + diag; };

  // matrix phase: O^T += V(t-1)^T P(t-1)^T, then S(t)^T = K(t) Q^T.
  // Each product is a list of steps (one A fragment from LDS, one MFMA); the
  // fragment of step j+LA is loaded while step j multiplies, and a scheduling
  // barrier after every step keeps the compiler from hoisting further loads
  // (which would cost registers the two waves per SIMD do not have).
  constexpr int LA = 3;
  constexpr int NPV = C::KB * 2 * C::DB;      // steps of O^T += V^T P^T
  constexpr int NSK = C::DS * C::KB;          // steps of S^T = K Q^T
  auto gemm_phase = [&](int t) {
    const char* st = lds + (t & 1) * C::STAGE;
    if (t >= 1 && tile_active(t - 1)) {
      const char* vl = st + C::TILE;
      auto load = [&](int j) {
        const int kb = j / (2 * C::DB), ks = (j / C::DB) % 2, db = j % C::DB;
        const int off = (kb * 32 + 16 * ks) * C::RB;
        const char* va = vl + v_rd[db % NVR] + (db / NVR) * 256 + off;
        v4i16 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)va);
        v4i16 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)(va + 8 * C::RB));
        return __builtin_bit_cast(frag, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
      };
      frag ring[LA + 1];
#pragma unroll
      for (int j = 0; j < LA; j++) ring[j] = load(j);
#pragma unroll
      for (int j = 0; j < NPV; j++) {
        if (j + LA < NPV) ring[(j + LA) % (LA + 1)] = load(j + LA);
        const int kb = j / (2 * C::DB), ks = (j / C::DB) % 2, db = j % C::DB;
        o[db] = M::mma(ring[j % (LA + 1)], pf[kb][ks], o[db]);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    if (t < n_tiles && tile_active(t)) {
      auto load = [&](int j) {
        const int ds = j / C::KB, kb = j % C::KB;
        return *(const frag*)(st + k_rd[ds % NKR] + (ds / NKR) * 256 + kb * 32 * C::RB);
      };
      frag ring[LA + 1];
#pragma unroll
      for (int j = 0; j < LA; j++) ring[j] = load(j);
#pragma unroll
      for (int j = 0; j < NSK; j++) {
        if (j + LA < NSK) ring[(j + LA) % (LA + 1)] = load(j + LA);
        const int ds = j / C::KB, kb = j % C::KB;
        if (ds == 0) {
          const v16f zero = {};
          s[kb] = M::mma(ring[j % (LA + 1)], qf[ds], zero);
        } else {
          s[kb] = M::mma(ring[j % (LA + 1)], qf[ds], s[kb]);
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
      const int q = wr0 + nn;
#pragma unroll
      for (int kb = 0; kb < C::KB; kb++)
#pragma unroll
        for (int i = 0; i < 4; i++)
#pragma unroll
          for (int j = 0; j < 4; j++) {
            const int key = key0 + kb * 32 + 8 * i + 4 * hh + j;
            const bool ok = key < k_hi && (!CAUSAL || key <= q + diag);
            if (!ok) s[kb][4 * i + j] = kNegInf;
          }
    }
    // P = 2^(s*c - m) with the row's current reference m, summed in float32
    // and converted to the matrix operand type.
    auto exps = [&]() {
      const float ref = m == kNegInf ? 0.0f : m;
      float ls = 0.0f;
#pragma unroll
      for (int kb = 0; kb < C::KB; kb++)
#pragma unroll
        for (int ks = 0; ks < 2; ks++) {
          v8f pv;
#pragma unroll
          for (int e = 0; e < 8; e++) {
            pv[e] = fast_exp2(__builtin_fmaf(s[kb][8 * ks + e], c, -ref));
            ls += pv[e];
          }
          pf[kb][ks] = M::cvt(pv);
        }
      return ls;
    };
    // The reference only has to keep every P <= 2^8. A lane's tile sum
    // bounds each of its P, so the row maximum is computed only when some
    // sum exceeds 2^8 (or a row has no reference yet): then m moves to
    // the maximum, O and l are rescaled, and P is recomputed. Any reference
    // reached this way gives the exact result, as the final O / l and LSE
    // use the same m.
    float ls = __builtin_inff();                 // forces the slow path below
    if (!__any(m == kNegInf)) ls = exps();
    if (__any(!(ls <= kSumMax))) {
      float x = kNegInf;
#pragma unroll
      for (int kb = 0; kb < C::KB; kb++)
#pragma unroll
        for (int e = 0; e < 16; e++) x = fmaxf(x, s[kb][e]);
      x = pair_max(x) * c;
      const float mnew = fmaxf(m, x);
      const float ref = mnew == kNegInf ? 0.0f : mnew;
      const float alpha = fast_exp2(m - ref);   // 0 when m was -inf, 1 when m stays
      m = mnew;
      l *= alpha;
#pragma unroll
      for (int db = 0; db < C::DB; db++)
#pragma unroll
        for (int e = 0; e < 16; e++) o[db][e] *= alpha;
      ls = exps();
    }
    l += ls;
  };

  // Both groups run the same body, gemm(j) | barrier | softmax(j) | barrier;
  // group 1 starts one barrier later and group 0 ends one barrier later, so
  // group 1's matrix phase overlaps group 0's softmax and vice versa. Group 0
  // fetches stage j+1 at the start of its softmax phase j and waits for it
  // before that phase's closing barrier: both groups have finished reading
  // stage j-1 (the buffer it overwrites) by then, stage j+1 is complete
  // before either group reads it, and no LDS read is ever issued while a
  // direct load is in flight (so the compiler adds no waits of its own).
  // Inside the loop the barriers are bare s_barrier: the only memory that
  // must be settled at a barrier is the staged tile, waited for explicitly.
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
  // Persistent: every wave has passed the loop's last barrier after its last
  // LDS read, so the next item's first stage may overwrite the buffers.
  if (!PERSIST) break;
  }
}

// ---------------------------------------------------------------- launchers

// Keys per tile for each head dimension (LDS: 2 stages x (K + V) tiles).
#ifndef FWD_D64_BN
#define FWD_D64_BN 128
#endif
#ifndef FWD_D128_BN
#define FWD_D128_BN 128
#endif

template <int D> struct Shape;
template <> struct Shape<64> { static constexpr int BN = FWD_D64_BN; };
template <> struct Shape<128> { static constexpr int BN = FWD_D128_BN; };

template <typename T, int D, bool CAUSAL, bool SPLIT, bool VARLEN = false, bool PERSIST = false>
static hipError_t launch_one(const FwdArgs& a, hipStream_t st, int n_wg = 0) {
  using C = FwdCfg<D, Shape<D>::BN>;
  // 32-bit buffer offsets (packed rows: S_k is the longest sequence's length)
  const long long row_bytes = VARLEN ? (long long)a.H * C::RB : C::RB;
  if ((long long)(a.S_k + C::BN) * row_bytes > 0x7fffffffLL) return hipErrorInvalidValue;
  const int n_qt = (a.S_q + C::BM - 1) / C::BM;
  const int n_work = a.B * a.H * n_qt * a.n_split;
  const int grid = PERSIST ? (n_wg < n_work ? n_wg : n_work) : n_work;
  hipLaunchKernelGGL((fwd_mfma_kernel<T, D, Shape<D>::BN, CAUSAL, SPLIT, VARLEN, PERSIST>), dim3(grid), dim3(C::NT), 0,
                     st, (const T*)a.q, (const T*)a.k, (const T*)a.v, (T*)a.o, a.lse, a.opart, a.lpart,
                     a.B * a.H, a.S_q, a.S_k, n_qt, a.n_split, a.keys_per_split, a.c, a.cu_q, a.cu_k, a.H,
                     a.total_q);
  return hipGetLastError();
}

template <typename T, int D>
static hipError_t launch_d(const FwdArgs& a, hipStream_t st) {
  const bool split = a.n_split > 1;
  if (a.causal) return split ? launch_one<T, D, true, true>(a, st) : launch_one<T, D, true, false>(a, st);
  return split ? launch_one<T, D, false, true>(a, st) : launch_one<T, D, false, false>(a, st);
}

template <typename T>
static hipError_t launch_t(const FwdArgs& a, hipStream_t st) {
  switch (a.D) {
    case 64: return launch_d<T, 64>(a, st);
    case 128: return launch_d<T, 128>(a, st);
  }
  return hipErrorInvalidValue;
}

int mfma_keys_per_tile(int D) {
  return D == 64 ? Shape<64>::BN : D == 128 ? Shape<128>::BN : d256_keys_per_tile();
}
int mfma_rows_per_block(int D) { (void)D; return 256; }

template <typename T>
static hipError_t launch_varlen_t(const FwdArgs& a, hipStream_t st) {
  switch (a.D) {
    case 64: return a.causal ? launch_one<T, 64, true, false, true>(a, st) : launch_one<T, 64, false, false, true>(a, st);
    case 128: return a.causal ? launch_one<T, 128, true, false, true>(a, st) : launch_one<T, 128, false, false, true>(a, st);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_fwd_varlen(const FwdArgs& a, hipStream_t st) {
  if (a.dtype == 2) return launch_varlen_t<__bf16>(a, st);
  return launch_varlen_t<_Float16>(a, st);
}

template <typename T>
static hipError_t launch_persistent_t(const FwdArgs& a, int n_wg, hipStream_t st) {
  switch (a.D) {
    case 64: return a.causal ? launch_one<T, 64, true, false, false, true>(a, st, n_wg)
                             : launch_one<T, 64, false, false, false, true>(a, st, n_wg);
    case 128: return a.causal ? launch_one<T, 128, true, false, false, true>(a, st, n_wg)
                              : launch_one<T, 128, false, false, false, true>(a, st, n_wg);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_fwd_persistent(const FwdArgs& a, int n_wg, hipStream_t st) {
  if (a.n_split != 1 || n_wg < 1) return hipErrorInvalidValue;
  if (a.dtype == 2) return launch_persistent_t<__bf16>(a, n_wg, st);
  return launch_persistent_t<_Float16>(a, n_wg, st);
}

hipError_t launch_fwd_mfma(const FwdArgs& a, hipStream_t st) {
  if (a.D == 256) return launch_fwd_d256(a, st);
  if (a.dtype == 2) return launch_t<__bf16>(a, st);
  return launch_t<_Float16>(a, st);
}

}  // namespace attn

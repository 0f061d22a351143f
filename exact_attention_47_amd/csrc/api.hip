// C ABI of libattn (declared in include/attn.h): argument validation, choice
// of kernel and key-range split, workspace handling and launches.
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

#include <mutex>

#include "../../include/attn.h"
#include "common.h"
#include "kernels.h"

namespace {

bool verbose() {
  static int v = -1;
  if (v < 0) v = getenv("ATTN_VERBOSE") != nullptr;
  return v != 0;
}

void say(const char* what, int status) {
  if (verbose()) fprintf(stderr, "[attn] %s: %s\n", what, attn_status_string(status));
}

bool aligned(const void* p, uintptr_t a) { return ((uintptr_t)p & (a - 1)) == 0; }

int key_tile(int dtype, int D) {
  return dtype == ATTN_F32 ? attn::f32_keys_per_tile() : attn::mfma_keys_per_tile(D);
}

// Split plan: effective split count and keys per split (a multiple of the key tile).
struct Plan {
  int n_split;
  int keys_per_split;
};

constexpr int kChipCUs = 256;   // compute units of the MI355X

// tile: the kernel's keys per tile; rows: query rows per workgroup
Plan plan_core(int tile, int rows, int B, int H, int S_q, int S_k, int D, int req) {
  const int n_tiles = (S_k + tile - 1) / tile;
  int n = 1;
  if (req > 1) {
    n = req;
  } else if (req == 0) {
    if (S_q <= 64 && S_k >= 8192) {
      // short query block against a long key range: split the keys so that
      // many workgroups stream the key range in parallel
      n = (S_k + 4095) / 4096;
    } else if (S_k >= 8192) {
      // too few query tiles to fill half the chip against a long key range:
      // split the keys so that about one workgroup per compute unit runs,
      // into at most ceil(S_k / 2048) splits, with partial results that fit
      // ATTN_NOALLOC_SCRATCH_BYTES (for attn_fwd: so that attn_fwd_noalloc
      // plans alike; for attn_fwd_fp8: a modest merge buffer)
      const long long n_work = (long long)B * H * ((S_q + rows - 1) / rows);
      if (n_work < kChipCUs / 2) {
        const long long per_split = (long long)B * H * S_q * (D + 1) * (long long)sizeof(float);
        long long m = (kChipCUs + n_work - 1) / n_work;
        m = std::min(m, (long long)(S_k + 2047) / 2048);
        m = std::min(m, ((long long)ATTN_NOALLOC_SCRATCH_BYTES - 512) / per_split);
        if (m > 1) n = (int)m;
      }
    }
  }
  if (n > n_tiles) n = n_tiles;
  if (n > 256) n = 256;
  if (n < 1) n = 1;
  const int tiles_per = (n_tiles + n - 1) / n;
  const int kps = tiles_per * tile;
  n = (S_k + kps - 1) / kps;          // drop splits that would be empty
  return Plan{n, kps};
}

// attn_fwd / attn_fwd_ex: 256-row workgroups at the key tile of the dtype
// and D (the main kernel's 128 keys at D = 64 / 128, which the short-range
// kernel's 32-key tile divides; the D = 256 and float32 kernels' own tiles)
Plan plan_splits(int dtype, int B, int H, int S_q, int S_k, int D, int req) {
  return plan_core(key_tile(dtype, D), 256, B, H, S_q, S_k, D, req);
}

size_t round_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

// Short key ranges run on the short-range kernel (three or four small
// workgroups per CU hide one another's start-up and memory waits), long ones
// on the main kernel. Crossovers measured on the sweeps (short-range over
// main kernel; run-to-run spread about 1.5 %): D = 64 up to 4096 keys (+17 %
// at 1024, +4.5 % at 2048, -1.4 % at 4096), causal D = 64 up to 8192 (+9 % at
// 2048, +14 % at 4096, +5.6 % at 8192, equal at 16384), D = 128 causal up to
// 2048 (+20 % at 512, +2.6 % at 1024, +1.4 % at 2048, equal at 4096), D = 128
// non-causal up to 1024 (+13 % at 512, +2.4 % at 1024). Key-range splits go
// to the main kernel, whose key tile the split plan uses, except those of
// short query blocks (use_short_split).
bool use_short_kernel(int D, int causal, int S_k, int n_split) {
  if (n_split != 1) return false;
  if (D == 64) return S_k <= (causal ? 8192 : 4096);
  if (D == 128) return S_k <= (causal ? 2048 : 1024);
  return false;
}

// A key-range split of a short query block (more than the decode kernel's one
// row, at most one short-range workgroup's rows) runs on the short-range
// kernel: its 128-row workgroups carry half the main kernel's idle rows, and
// the main kernel's 256 rows of matrix work per key tile then no longer stand
// beside the K/V stream. (The split plan's key granularity, the main kernel's
// 128-key tile, is a multiple of the short-range kernel's 32-key tile.)
bool use_short_split(int D, int S_q, int n_split) {
  return n_split > 1 && (D == 64 || D == 128) && S_q <= attn::short_rows_per_block();
}

// Causal D = 128 on the main kernel runs on the persistent grid: its snake
// deal measured +0.8 to +2 % over the hardware-dealt grid from 4K to 16K
// keys on the 32x32x16 form of the kernel; on the 16x16x32 form the two
// grids are within 0.7 % of each other there, and D = 64 and non-causal work
// gain 0.1 to 1.4 % on the persistent grid (all within the run-to-run
// spread), so the choice stands.
bool use_persistent(int D, int causal, int n_split) { return causal && D == 128 && n_split == 1; }

// Compute units of the current device, asked once per device.
int cu_count() {
  static int cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return 0;
  int n = dev < 64 ? cache[dev] : 0;
  if (n > 0) return n;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) return 0;
  if (dev < 64) cache[dev] = n;
  return n;
}

size_t ws_bytes(const Plan& p, int B, int H, int S_q, int D) {
  if (p.n_split <= 1) return 0;
  const size_t rows = (size_t)p.n_split * B * H * S_q;
  return round_up(rows * D * sizeof(float), 256) + round_up(rows * sizeof(float), 256);
}

int check_args(const void* q, const void* k, const void* v, const void* o, const float* lse, int B,
               int H, int S_q, int S_k, int D, int causal, float scale, int dtype) {
  if (!q || !k || !v || !o || !lse) return ATTN_ERR_INVALID_ARG;
  if (B <= 0 || H <= 0 || S_q <= 0 || S_k <= 0 || D <= 0) return ATTN_ERR_INVALID_ARG;
  if (dtype != ATTN_F32 && dtype != ATTN_F16 && dtype != ATTN_BF16) return ATTN_ERR_INVALID_ARG;
  if (causal != 0 && causal != 1) return ATTN_ERR_INVALID_ARG;
  if (!(scale > 0.0f) || !isfinite(scale)) return ATTN_ERR_INVALID_ARG;
  if (D != 64 && D != 128 && D != 256) return ATTN_ERR_UNSUPPORTED;
  if (dtype == ATTN_F32 && D == 256) return ATTN_ERR_UNSUPPORTED;
  if (causal && S_q > S_k) return ATTN_ERR_UNSUPPORTED;
  // launch grid must fit in 31 bits
  const long long blocks = (long long)B * H * ((S_q + 31) / 32) * 256;
  if (blocks > 0x7fffffffLL) return ATTN_ERR_UNSUPPORTED;
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(o, 16) || !aligned(lse, 4))
    return ATTN_ERR_MISALIGNED;
  return ATTN_OK;
}

int run_fwd(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int S_q,
            int S_k, int D, int causal, float scale, int dtype, int req_split, void* ws,
            size_t ws_size, bool own_ws, hipStream_t st) {
  int rc = check_args(q, k, v, o, lse, B, H, S_q, S_k, D, causal, scale, dtype);
  if (rc != ATTN_OK) return rc;
  if (req_split < 0) return ATTN_ERR_INVALID_ARG;
  const Plan p = plan_splits(dtype, B, H, S_q, S_k, D, req_split);
  const size_t need = ws_bytes(p, B, H, S_q, D);
  if (!own_ws && need > 0 && (ws == nullptr || ws_size < need || !aligned(ws, 256)))
    return ATTN_ERR_WORKSPACE;

  attn::FwdArgs a;
  a.q = q; a.k = k; a.v = v; a.o = o; a.lse = lse;
  a.B = B; a.H = H; a.S_q = S_q; a.S_k = S_k; a.D = D;
  a.causal = causal; a.dtype = dtype;
  a.n_split = p.n_split; a.keys_per_split = p.keys_per_split;
  a.c = scale * attn::kLog2e;
  a.opart = nullptr; a.lpart = nullptr;

  void* buf = ws;
  if (need > 0) {
    if (own_ws) {
      if (hipMallocAsync(&buf, need, st) != hipSuccess) return ATTN_ERR_LAUNCH;
    }
    const size_t rows = (size_t)p.n_split * B * H * S_q;
    a.opart = (float*)buf;
    a.lpart = (float*)((char*)buf + round_up(rows * D * sizeof(float), 256));
  }
  hipError_t e;
  int n_cu = 0;
  if (dtype == ATTN_F32) e = attn::launch_fwd_f32(a, st);
  else if (p.n_split > 1 && S_q <= attn::decode_max_rows()) e = attn::launch_fwd_decode(a, st);
  else if (use_short_kernel(D, causal, S_k, p.n_split) || use_short_split(D, S_q, p.n_split))
    e = attn::launch_fwd_short(a, st);
  else if (use_persistent(D, causal, p.n_split) && (n_cu = cu_count()) > 0) e = attn::launch_fwd_persistent(a, n_cu, st);
  else e = attn::launch_fwd_mfma(a, st);
  if (e == hipSuccess && p.n_split > 1) e = attn::launch_combine(a, st);
  if (need > 0 && own_ws) {
    if (hipFreeAsync(buf, st) != hipSuccess && e == hipSuccess) e = hipErrorUnknown;
  }
  if (e != hipSuccess) {
    if (verbose()) fprintf(stderr, "[attn] launch failed: %s\n", hipGetErrorString(e));
    return ATTN_ERR_LAUNCH;
  }
  return ATTN_OK;
}

// Scratch memory of attn_fwd_noalloc: a fixed device array in place of the
// stream-ordered allocation attn_fwd makes for a key-range split. Each device
// the library runs on holds its own copy until the process ends. Host code
// never uses the array's name as an address (on the host it only stands for
// the symbol): the device address comes from hipGetSymbolAddress, asked once
// per device with that device current, and is kept per device.
__device__ __align__(256) char scratch[ATTN_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex scratch_mu;
void* scratch_ptr[kMaxDevices];

// Device address of the current device's scratch array, or nullptr if the
// runtime cannot give it.
void* device_scratch() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> g(scratch_mu);
  if (scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) return nullptr;
    scratch_ptr[dev] = p;
  }
  return scratch_ptr[dev];
}

}  // namespace

extern "C" {

int attn_abi_version(void) { return ATTN_ABI_VERSION; }

int attn_mfma_stream(int kind, int iters, float* sink, size_t sink_bytes, double* flop, void* stream) {
  if (kind < 0 || kind > 2 || iters <= 0 || sink == nullptr || flop == nullptr) return ATTN_ERR_INVALID_ARG;
  if (!aligned(sink, 16)) return ATTN_ERR_MISALIGNED;
  const int n_cu = cu_count();
  if (n_cu <= 0) return ATTN_ERR_LAUNCH;
  const long long blocks = 2LL * n_cu;   // four waves each: two waves per SIMD on every CU
  if ((long long)sink_bytes < blocks * 256 * (long long)sizeof(float)) return ATTN_ERR_INVALID_ARG;
  const double per_instr = kind == 0 ? 2.0 * 32 * 32 * 16 : kind == 1 ? 2.0 * 32 * 32 * 64 : 2.0 * 16 * 16 * 32;
  *flop = per_instr * 32.0 * (double)iters * (double)(blocks * 4);
  if (attn::launch_mfma_stream(kind, iters, sink, (int)blocks, (hipStream_t)stream) != hipSuccess) {
    say("attn_mfma_stream", ATTN_ERR_LAUNCH);
    return ATTN_ERR_LAUNCH;
  }
  return ATTN_OK;
}

const char* attn_status_string(int status) {
  switch (status) {
    case ATTN_OK: return "ok";
    case ATTN_ERR_INVALID_ARG: return "invalid argument";
    case ATTN_ERR_UNSUPPORTED: return "unsupported configuration";
    case ATTN_ERR_MISALIGNED: return "misaligned pointer";
    case ATTN_ERR_LAUNCH: return "HIP launch failure";
    case ATTN_ERR_WORKSPACE: return "workspace missing or too small";
  }
  return "unknown status";
}

int attn_check_args(const void* q, const void* k, const void* v, const void* o, const float* lse,
                    int B, int H, int S_q, int S_k, int D, int causal, float scale, int dtype) {
  return check_args(q, k, v, o, lse, B, H, S_q, S_k, D, causal, scale, dtype);
}

int attn_fwd_num_splits(int B, int H, int S_q, int S_k, int D, int dtype, int num_splits) {
  if (B <= 0 || H <= 0 || S_q <= 0 || S_k <= 0 || num_splits < 0) return 1;
  if (dtype != ATTN_F32 && dtype != ATTN_F16 && dtype != ATTN_BF16) return 1;
  return plan_splits(dtype, B, H, S_q, S_k, D, num_splits).n_split;
}

size_t attn_fwd_workspace_size(int B, int H, int S_q, int S_k, int D, int num_splits) {
  if (B <= 0 || H <= 0 || S_q <= 0 || S_k <= 0 || D <= 0 || num_splits < 0) return 0;
  // the float32 kernel uses a smaller key tile and can need more splits
  const Plan a = plan_splits(ATTN_BF16, B, H, S_q, S_k, D, num_splits);
  const Plan b = plan_splits(ATTN_F32, B, H, S_q, S_k, D, num_splits);
  const size_t x = ws_bytes(a, B, H, S_q, D), y = ws_bytes(b, B, H, S_q, D);
  return x > y ? x : y;
}

int attn_fwd(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H,
             int S_q, int S_k, int D, int causal, float scale, int dtype, void* stream) {
  const int rc = run_fwd(q, k, v, o, lse, B, H, S_q, S_k, D, causal, scale, dtype, 0, nullptr, 0,
                         true, (hipStream_t)stream);
  if (rc != ATTN_OK) say("attn_fwd", rc);
  return rc;
}

int attn_fwd_ex(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H,
                int S_q, int S_k, int D, int causal, float scale, int dtype, int num_splits,
                void* workspace, size_t workspace_bytes, void* stream) {
  const int rc = run_fwd(q, k, v, o, lse, B, H, S_q, S_k, D, causal, scale, dtype, num_splits,
                         workspace, workspace_bytes, false, (hipStream_t)stream);
  if (rc != ATTN_OK) say("attn_fwd_ex", rc);
  return rc;
}

int attn_fwd_noalloc(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H,
                     int S_q, int S_k, int D, int causal, float scale, int dtype, void* stream) {
  int rc = check_args(q, k, v, o, lse, B, H, S_q, S_k, D, causal, scale, dtype);
  // the split attn_fwd would choose must fit the fixed scratch array; this is
  // decided on the host before anything touches the device
  if (rc == ATTN_OK) {
    const Plan p = plan_splits(dtype, B, H, S_q, S_k, D, 0);
    if (ws_bytes(p, B, H, S_q, D) > (size_t)ATTN_NOALLOC_SCRATCH_BYTES) rc = ATTN_ERR_WORKSPACE;
  }
  void* ws = nullptr;
  if (rc == ATTN_OK && (ws = device_scratch()) == nullptr) rc = ATTN_ERR_LAUNCH;
  if (rc == ATTN_OK)
    rc = run_fwd(q, k, v, o, lse, B, H, S_q, S_k, D, causal, scale, dtype, 0, ws, ATTN_NOALLOC_SCRATCH_BYTES,
                 false, (hipStream_t)stream);
  if (rc != ATTN_OK) say("attn_fwd_noalloc", rc);
  return rc;
}

int attn_fwd_persistent(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H,
                        int S_q, int S_k, int D, int causal, float scale, int dtype, int num_workgroups,
                        void* stream) {
  int rc = check_args(q, k, v, o, lse, B, H, S_q, S_k, D, causal, scale, dtype);
  if (rc == ATTN_OK && num_workgroups < 0) rc = ATTN_ERR_INVALID_ARG;
  if (rc == ATTN_OK && (dtype == ATTN_F32 || (D != 64 && D != 128))) rc = ATTN_ERR_UNSUPPORTED;
  int n_cu = 0;
  if (rc == ATTN_OK && (n_cu = cu_count()) <= 0) rc = ATTN_ERR_LAUNCH;
  // one workgroup per CU at most: the kernel's workgroup fills a CU, so a
  // larger grid would no longer be resident at once
  if (rc == ATTN_OK && num_workgroups > n_cu) rc = ATTN_ERR_INVALID_ARG;
  if (rc != ATTN_OK) {
    say("attn_fwd_persistent", rc);
    return rc;
  }
  attn::FwdArgs a;
  a.q = q; a.k = k; a.v = v; a.o = o; a.lse = lse;
  a.B = B; a.H = H; a.S_q = S_q; a.S_k = S_k; a.D = D;
  a.causal = causal; a.dtype = dtype;
  a.n_split = 1; a.keys_per_split = 0;
  a.c = scale * attn::kLog2e;
  a.opart = nullptr; a.lpart = nullptr;
  const hipError_t e = attn::launch_fwd_persistent(a, num_workgroups > 0 ? num_workgroups : n_cu,
                                                   (hipStream_t)stream);
  if (e != hipSuccess) {
    if (verbose()) fprintf(stderr, "[attn] launch failed: %s\n", hipGetErrorString(e));
    say("attn_fwd_persistent", ATTN_ERR_LAUNCH);
    return ATTN_ERR_LAUNCH;
  }
  return ATTN_OK;
}

int attn_fwd_varlen(const void* q, const void* k, const void* v, void* o, float* lse,
                    const int* cu_seqlens_q, const int* cu_seqlens_k, int B, int H, int total_q,
                    int total_k, int max_seqlen_q, int max_seqlen_k, int D, int causal, float scale,
                    int dtype, void* stream) {
  int rc = ATTN_OK;
  // (tensors of zero rows may be NULL)
  if (((!q || !o || !lse) && total_q > 0) || ((!k || !v) && total_k > 0) || !cu_seqlens_q || !cu_seqlens_k)
    rc = ATTN_ERR_INVALID_ARG;
  else if (B <= 0 || H <= 0 || D <= 0 || total_q < 0 || total_k < 0 || max_seqlen_q < 0 ||
           max_seqlen_k < 0 || max_seqlen_q > total_q || max_seqlen_k > total_k)
    rc = ATTN_ERR_INVALID_ARG;
  else if (dtype != ATTN_F32 && dtype != ATTN_F16 && dtype != ATTN_BF16) rc = ATTN_ERR_INVALID_ARG;
  else if (causal != 0 && causal != 1) rc = ATTN_ERR_INVALID_ARG;
  else if (!(scale > 0.0f) || !isfinite(scale)) rc = ATTN_ERR_INVALID_ARG;
  else if (dtype == ATTN_F32 || (D != 64 && D != 128 && D != 256)) rc = ATTN_ERR_UNSUPPORTED;
  else if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(o, 16) || !aligned(lse, 4) ||
           !aligned(cu_seqlens_q, 4) || !aligned(cu_seqlens_k, 4))
    rc = ATTN_ERR_MISALIGNED;
  if (rc == ATTN_OK && total_q > 0 && max_seqlen_q > 0) {
    const int bm = attn::mfma_rows_per_block(D);
    const long long blocks = (long long)B * H * ((max_seqlen_q + bm - 1) / bm);
    if (blocks > 0x7fffffffLL) rc = ATTN_ERR_UNSUPPORTED;
  }
  if (rc != ATTN_OK) {
    say("attn_fwd_varlen", rc);
    return rc;
  }
  if (total_q == 0 || max_seqlen_q == 0) return ATTN_OK;
  attn::FwdArgs a;
  a.q = q; a.k = k; a.v = v; a.o = o; a.lse = lse;
  a.B = B; a.H = H; a.S_q = max_seqlen_q; a.S_k = max_seqlen_k; a.D = D;
  a.causal = causal; a.dtype = dtype;
  a.n_split = 1; a.keys_per_split = 0;
  a.c = scale * attn::kLog2e;
  a.opart = nullptr; a.lpart = nullptr;
  a.cu_q = cu_seqlens_q; a.cu_k = cu_seqlens_k; a.total_q = total_q;
  // D = 256 runs on its own kernel; D = 64 / 128 on the short-range kernel
  // when the longest key sequence is within its range (as for attn_fwd),
  // else on the main one
  const hipError_t e = D == 256 ? attn::launch_fwd_d256_varlen(a, (hipStream_t)stream)
                       : use_short_kernel(D, causal, max_seqlen_k, 1) ? attn::launch_fwd_short_varlen(a, (hipStream_t)stream)
                                                                       : attn::launch_fwd_varlen(a, (hipStream_t)stream);
  if (e != hipSuccess) {
    rc = e == hipErrorInvalidValue ? ATTN_ERR_UNSUPPORTED : ATTN_ERR_LAUNCH;
    if (verbose()) fprintf(stderr, "[attn] varlen launch failed: %s\n", hipGetErrorString(e));
    say("attn_fwd_varlen", rc);
  }
  return rc;
}

int attn_bwd(const void* q, const void* k, const void* v, const void* o, const float* lse, const void* dout,
             void* dq, void* dk, void* dv, int B, int H, int S_q, int S_k, int D, int causal, float scale,
             int dtype, void* stream) {
  int rc = ATTN_OK;
  if (!q || !k || !v || !o || !lse || !dout || !dq || !dk || !dv) rc = ATTN_ERR_INVALID_ARG;
  else if (B <= 0 || H <= 0 || S_q <= 0 || S_k <= 0 || D <= 0) rc = ATTN_ERR_INVALID_ARG;
  else if (dtype != ATTN_F32 && dtype != ATTN_F16 && dtype != ATTN_BF16) rc = ATTN_ERR_INVALID_ARG;
  else if (causal != 0 && causal != 1) rc = ATTN_ERR_INVALID_ARG;
  else if (!(scale > 0.0f) || !isfinite(scale)) rc = ATTN_ERR_INVALID_ARG;
  else if (dtype == ATTN_F32 || (D != 64 && D != 128)) rc = ATTN_ERR_UNSUPPORTED;
  else if (causal && S_q > S_k) rc = ATTN_ERR_UNSUPPORTED;
  else if ((long long)B * H * ((S_q > S_k ? S_q : S_k) + 127) / 128 > 0x7fffffffLL) rc = ATTN_ERR_UNSUPPORTED;
  else if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(o, 16) || !aligned(dout, 16) ||
           !aligned(dq, 16) || !aligned(dk, 16) || !aligned(dv, 16) || !aligned(lse, 4))
    rc = ATTN_ERR_MISALIGNED;
  if (rc != ATTN_OK) {
    say("attn_bwd", rc);
    return rc;
  }
  hipStream_t st = (hipStream_t)stream;
  void* dd = nullptr;
  const size_t rows = (size_t)B * H * S_q;
  if (hipMallocAsync(&dd, 2 * rows * sizeof(float), st) != hipSuccess) return ATTN_ERR_LAUNCH;
  attn::BwdArgs a;
  a.q = q; a.k = k; a.v = v; a.o = o; a.dout = dout; a.lse = lse; a.dd = (float*)dd; a.nl2 = (float*)dd + rows;
  a.dq = dq; a.dk = dk; a.dv = dv;
  a.B = B; a.H = H; a.S_q = S_q; a.S_k = S_k; a.D = D; a.causal = causal; a.dtype = dtype; a.scale = scale;
  hipError_t e = attn::launch_bwd(a, st);
  if (hipFreeAsync(dd, st) != hipSuccess && e == hipSuccess) e = hipErrorUnknown;
  if (e != hipSuccess) {
    rc = e == hipErrorInvalidValue ? ATTN_ERR_UNSUPPORTED : ATTN_ERR_LAUNCH;
    say("attn_bwd", rc);
  }
  return rc;
}

int hadamard_quant(const void* x, void* x8, float* scales, const signed char* signs, int B, int H,
                   int S, int D, int block_rows, int apply_hadamard, int in_dtype, void* stream) {
  if (!x || !x8 || !scales || !signs) return ATTN_ERR_INVALID_ARG;
  if (B <= 0 || H <= 0 || S <= 0 || D <= 0 || block_rows <= 0 || block_rows > 1024)
    return ATTN_ERR_INVALID_ARG;
  if (apply_hadamard != 0 && apply_hadamard != 1) return ATTN_ERR_INVALID_ARG;
  if (in_dtype != ATTN_BF16 && in_dtype != ATTN_F16) return ATTN_ERR_INVALID_ARG;
  if (D != 64 && D != 128 && D != 256) return ATTN_ERR_UNSUPPORTED;
  if (!aligned(x, 16) || !aligned(x8, 16) || !aligned(scales, 4) || !aligned(signs, 8))
    return ATTN_ERR_MISALIGNED;
  const hipError_t e = attn::launch_hadamard_quant(x, x8, scales, signs, B, H, S, D, block_rows,
                                                   apply_hadamard, in_dtype, (hipStream_t)stream);
  return e == hipSuccess ? ATTN_OK : (e == hipErrorNotSupported ? ATTN_ERR_UNSUPPORTED : ATTN_ERR_LAUNCH);
}

int rope_hadamard_quant(const void* x, void* x8, float* scales, const signed char* signs, const float* cos_t,
                        const float* sin_t, int B, int H, int S, int D, int block_rows, int rope_mode,
                        int in_dtype, void* stream) {
  if (!x || !x8 || !scales || !signs || !cos_t || !sin_t) return ATTN_ERR_INVALID_ARG;
  if (B <= 0 || H <= 0 || S <= 0 || D <= 0 || block_rows <= 0) return ATTN_ERR_INVALID_ARG;
  if (rope_mode != 0 && rope_mode != 1) return ATTN_ERR_INVALID_ARG;
  if (in_dtype != ATTN_BF16 && in_dtype != ATTN_F16) return ATTN_ERR_INVALID_ARG;
  if ((D != 64 && D != 128 && D != 256) || block_rows != 64) return ATTN_ERR_UNSUPPORTED;
  if (!aligned(x, 16) || !aligned(x8, 16) || !aligned(scales, 4) || !aligned(signs, 8) || !aligned(cos_t, 16) ||
      !aligned(sin_t, 16))
    return ATTN_ERR_MISALIGNED;
  const hipError_t e = attn::launch_rope_hadamard_quant(x, x8, scales, signs, cos_t, sin_t, B, H, S, D, rope_mode,
                                                        in_dtype, (hipStream_t)stream);
  return e == hipSuccess ? ATTN_OK : (e == hipErrorNotSupported ? ATTN_ERR_UNSUPPORTED : ATTN_ERR_LAUNCH);
}

int quant_per_tensor(const void* x, void* x8, float* scale, int B, int H, int S, int D, int in_dtype,
                     int write_transposed, void* stream) {
  if (!x || !x8 || !scale) return ATTN_ERR_INVALID_ARG;
  if (B <= 0 || H <= 0 || S <= 0 || D <= 0) return ATTN_ERR_INVALID_ARG;
  if (in_dtype != ATTN_BF16 && in_dtype != ATTN_F16) return ATTN_ERR_INVALID_ARG;
  if (write_transposed != 0 && write_transposed != 1) return ATTN_ERR_INVALID_ARG;
  if (D % 8 != 0) return ATTN_ERR_UNSUPPORTED;
  if (write_transposed && S % 16 != 0) return ATTN_ERR_UNSUPPORTED;
  if (!aligned(x, 16) || !aligned(x8, 16) || !aligned(scale, 4)) return ATTN_ERR_MISALIGNED;
  const hipError_t e = attn::launch_quant_per_tensor(x, x8, scale, B, H, S, D, in_dtype,
                                                     write_transposed, (hipStream_t)stream);
  return e == hipSuccess ? ATTN_OK : (e == hipErrorNotSupported ? ATTN_ERR_UNSUPPORTED : ATTN_ERR_LAUNCH);
}

int attn_fwd_fp8(const void* q8, const void* k8, const void* v8, const float* q_scales,
                 const float* k_scales, const float* v_scale, void* o, float* lse, int B, int H,
                 int S_q, int S_k, int D, int causal, float scale, int block_rows, int v_transposed,
                 void* stream) {
  if (!q8 || !k8 || !v8 || !q_scales || !k_scales || !v_scale || !o || !lse) return ATTN_ERR_INVALID_ARG;
  if (B <= 0 || H <= 0 || S_q <= 0 || S_k <= 0 || D <= 0) return ATTN_ERR_INVALID_ARG;
  if (causal != 0 && causal != 1) return ATTN_ERR_INVALID_ARG;
  if (v_transposed != 0 && v_transposed != 1) return ATTN_ERR_INVALID_ARG;
  if (!(scale > 0.0f) || !isfinite(scale)) return ATTN_ERR_INVALID_ARG;
  if (D != 128 || block_rows != 64) return ATTN_ERR_UNSUPPORTED;
  if (causal && S_q > S_k) return ATTN_ERR_UNSUPPORTED;
  if (v_transposed && S_k % 16 != 0) return ATTN_ERR_UNSUPPORTED;
  if (!aligned(q8, 16) || !aligned(k8, 16) || !aligned(v8, 16) || !aligned(o, 16) || !aligned(lse, 4) ||
      !aligned(q_scales, 4) || !aligned(k_scales, 4) || !aligned(v_scale, 4))
    return ATTN_ERR_MISALIGNED;
  // key-range split by the rules of attn_fwd, at the FP8 kernel's 64-key
  // tile and 128-row workgroups; the partials come from the stream-ordered
  // allocator and are merged into o / lse by logsumexp
  const Plan p = plan_core(attn::fp8_keys_per_tile(), attn::fp8_rows_per_block(), B, H, S_q, S_k, D, 0);
  const hipStream_t st = (hipStream_t)stream;
  const size_t need = ws_bytes(p, B, H, S_q, D);
  void* buf = nullptr;
  float *opart = nullptr, *lpart = nullptr;
  if (need > 0) {
    if (hipMallocAsync(&buf, need, st) != hipSuccess) return ATTN_ERR_LAUNCH;
    const size_t rows = (size_t)p.n_split * B * H * S_q;
    opart = (float*)buf;
    lpart = (float*)((char*)buf + round_up(rows * D * sizeof(float), 256));
  }
  hipError_t e = attn::launch_fwd_fp8(q8, k8, v8, q_scales, k_scales, v_scale, o, lse, B, H, S_q, S_k, D, causal,
                                      scale * attn::kLog2e, v_transposed, p.n_split, p.keys_per_split, opart, lpart,
                                      st);
  if (e == hipSuccess && p.n_split > 1) {
    attn::FwdArgs a;
    a.o = o; a.lse = lse; a.B = B; a.H = H; a.S_q = S_q; a.S_k = S_k; a.D = D;
    a.dtype = ATTN_BF16; a.n_split = p.n_split; a.opart = opart; a.lpart = lpart;
    e = attn::launch_combine(a, st);
  }
  if (need > 0 && hipFreeAsync(buf, st) != hipSuccess && e == hipSuccess) e = hipErrorUnknown;
  return e == hipSuccess ? ATTN_OK : (e == hipErrorNotSupported ? ATTN_ERR_UNSUPPORTED : ATTN_ERR_LAUNCH);
}

}  // extern "C"

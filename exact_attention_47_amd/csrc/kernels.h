// Host-side view of the kernels: argument bundles and launch functions.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>

namespace attn {

struct FwdArgs {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;
  float* opart;        // [n_split][B*H][S_q][D] float32, when n_split > 1
  float* lpart;        // [n_split][B*H][S_q] float32, when n_split > 1
  int B, H, S_q, S_k, D;
  int causal;
  int dtype;           // ATTN_F32 / ATTN_F16 / ATTN_BF16
  int n_split;         // >= 1
  int keys_per_split;  // multiple of the kernel's key tile
  float c;             // scale * log2(e)
  // packed batches ([total, H, D] with cumulative sequence starts): S_q and
  // S_k above are then the longest query / key sequence
  const int* cu_q = nullptr;
  const int* cu_k = nullptr;
  int total_q = 0;
};

// bf16 / fp16 matrix-core kernel
hipError_t launch_fwd_mfma(const FwdArgs& a, hipStream_t st);
int mfma_rows_per_block(int D);
int mfma_keys_per_tile(int D);

// backward pass (bf16 / fp16, D = 64 / 128): Dd, then dQ, dK, dV
struct BwdArgs {
  const void* q;
  const void* k;
  const void* v;
  const void* o;
  const void* dout;
  const float* lse;    // [B*H][S_q], natural log, from the forward pass
  float* dd;           // workspace [B*H][S_q]: -rowsum(dO * O)
  float* nl2;          // workspace [B*H][S_q]: -log2(e) * LSE
  void* dq;
  void* dk;
  void* dv;
  int B, H, S_q, S_k, D;
  int causal;
  int dtype;
  float scale;
};
hipError_t launch_bwd(const BwdArgs& a, hipStream_t st);

// packed (variable-length) batches on the bf16 / fp16 kernel, D = 64 / 128
hipError_t launch_fwd_varlen(const FwdArgs& a, hipStream_t st);

// the bf16 / fp16 kernel on a persistent grid of n_wg workgroups (unsplit,
// D = 64 / 128); n_wg at most the CU count keeps every workgroup resident
hipError_t launch_fwd_persistent(const FwdArgs& a, int n_wg, hipStream_t st);

// short causal key ranges, D = 64 / 128 (two co-resident 4-wave workgroups per CU)
hipError_t launch_fwd_short(const FwdArgs& a, hipStream_t st);
int short_rows_per_block();
// packed batches ([total, H, D] through cu_q / cu_k, unsplit)
hipError_t launch_fwd_short_varlen(const FwdArgs& a, hipStream_t st);
int short_keys_per_tile();

// head dimension 256 (dense: called through launch_fwd_mfma; packed: from attn_fwd_varlen)
hipError_t launch_fwd_d256(const FwdArgs& a, hipStream_t st);
hipError_t launch_fwd_d256_varlen(const FwdArgs& a, hipStream_t st);
int d256_keys_per_tile();

// float32 kernel
hipError_t launch_fwd_f32(const FwdArgs& a, hipStream_t st);
int f32_rows_per_block();
int f32_keys_per_tile();

// single-query-row decode kernel (S_q small, long key range)
hipError_t launch_fwd_decode(const FwdArgs& a, hipStream_t st);
int decode_keys_per_tile();
int decode_max_rows();

// merge of split partials into O (dtype) and LSE
hipError_t launch_combine(const FwdArgs& a, hipStream_t st);

// FP8 path
hipError_t launch_hadamard_quant(const void* x, void* x8, float* scales, const signed char* signs,
                                 int B, int H, int S, int D, int block_rows, int apply_hadamard,
                                 int in_dtype, hipStream_t st);
hipError_t launch_rope_hadamard_quant(const void* x, void* x8, float* scales, const signed char* signs,
                                      const float* cos_t, const float* sin_t, int B, int H, int S, int D,
                                      int rope_mode, int in_dtype, hipStream_t st);
hipError_t launch_quant_per_tensor(const void* x, void* x8, float* scale, int B, int H, int S, int D,
                                   int in_dtype, int write_transposed, hipStream_t st);
// n_split > 1: keys_per_split a multiple of fp8_keys_per_tile(); normalised
// partial outputs / LSEs go to opart / lpart (merged by launch_combine)
hipError_t launch_fwd_fp8(const void* q8, const void* k8, const void* v8, const float* qs,
                          const float* ks, const float* vs, void* o, float* lse, int B, int H,
                          int S_q, int S_k, int D, int causal, float c, int v_transposed,
                          int n_split, int keys_per_split, float* opart, float* lpart, hipStream_t st);
int fp8_keys_per_tile();
int fp8_rows_per_block();

// matrix-core stream for the roofline report (kind 0: bf16 32x32x16, 1: fp8
// 32x32x64, 2: bf16 16x16x32), `blocks` workgroups of four waves, one float
// per thread to sink
hipError_t launch_mfma_stream(int kind, int iters, float* sink, int blocks, hipStream_t st);

}  // namespace attn

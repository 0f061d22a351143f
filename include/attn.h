/*
 * attn.h -- C ABI of libattn, the exact fused attention forward pass for
 * AMD MI355X (gfx950).
 *
 * Sources (cited by page title and section):
 *   [NL] "FlashAttention-3 (NL)", systems-analysis.info
 *   [GN] "FlashAttention-3: Schnellere und praezisere Attention durch
 *        Asynchronitaet und geringe Praezision", GeekNews (de.news.hada.io)
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - Tensors are contiguous [B, H, S, D] with D innermost (element (b,h,s,d)
 *    at ((b*H + h)*S + s)*D + d). LSE is contiguous [B, H, S_q] float32.
 *  - Every pointer is a device pointer allocated by the caller, who owns it.
 *    The library never frees caller memory and keeps no state between calls.
 *  - `stream` is a hipStream_t passed as an opaque pointer (NULL = the null
 *    stream). Every call only enqueues work on it and returns; nothing is
 *    synchronised inside the library.
 *  - Return value: ATTN_OK or a negative status. On any error status nothing
 *    has been enqueued and no output has been touched, except ATTN_ERR_LAUNCH,
 *    which reports a failure of the HIP runtime at launch time.
 *  - Device pointers must be 16-byte aligned; sizes must be positive.
 *  - Results are bitwise deterministic for fixed inputs and arguments (no
 *    atomics whose order can change a floating-point result).
 */
#ifndef ATTN_H
#define ATTN_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

#define ATTN_ABI_VERSION 4

/* element types */
#define ATTN_F32  0
#define ATTN_F16  1
#define ATTN_BF16 2

/* status codes */
#define ATTN_OK                0
#define ATTN_ERR_INVALID_ARG  (-1) /* null pointer, non-positive size, unknown dtype */
#define ATTN_ERR_UNSUPPORTED  (-2) /* valid but not implemented: D not in {64,128,256}, causal with S_q > S_k, ... */
#define ATTN_ERR_MISALIGNED   (-3) /* a device pointer is not 16-byte aligned */
#define ATTN_ERR_LAUNCH       (-4) /* the HIP runtime reported an error when enqueuing */
#define ATTN_ERR_WORKSPACE    (-5) /* workspace missing or smaller than attn_fwd_workspace_size() */

/* Version of this interface (ATTN_ABI_VERSION). */
int attn_abi_version(void);

/* Static, human-readable text for a status code. */
const char* attn_status_string(int status);

/*
 * attn_fwd -- O = softmax(scale * Q K^T [+ causal mask]) V and its row-wise
 * logsumexp, computed tile by tile with online softmax rescaling so that the
 * S_q x S_k score matrix never reaches device memory.
 *
 * Defined by: the attention computation of [NL] "Het probleem van het
 * aandachtsmechanisme"; the tiled, fused, exact method of [NL] "FlashAttention
 * en FlashAttention-2" and [GN] "Rueckblick auf den FlashAttention-Ansatz".
 *
 *   q      [B, H, S_q, D]   dtype
 *   k, v   [B, H, S_k, D]   dtype
 *   o      [B, H, S_q, D]   dtype (written)
 *   lse    [B, H, S_q]      float32 (written): natural-log logsumexp of the
 *                           scaled, masked scores of each query row
 *   causal 0 or 1: key j is allowed for query i iff j <= i + (S_k - S_q)
 *          (bottom-right aligned); causal with S_q > S_k is ATTN_ERR_UNSUPPORTED
 *   scale  multiplier of Q K^T (commonly 1/sqrt(D)); must be finite and > 0
 *   dtype  ATTN_F32, ATTN_F16 or ATTN_BF16; accumulation is float32 in all cases
 *   D      64, 128 or 256 (ATTN_F32: 64 or 128)
 *
 * Against long key ranges (8192 keys or more) the library splits the key
 * range and merges the partial results by logsumexp when the query block is
 * short (at most 64 rows) or the grid too small for the chip (fewer 256-row
 * query tiles over all (b, h) than half its 256 compute units; then only as
 * far as the partial results fit ATTN_NOALLOC_SCRATCH_BYTES). The temporary
 * buffer it needs is taken from the stream-ordered allocator on `stream` and
 * released on the same stream.
 */
int attn_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
             int B, int H, int S_q, int S_k, int D, int causal, float scale,
             int dtype, void* stream);

/*
 * attn_fwd_ex -- attn_fwd with explicit control of the key-range split.
 *
 *   num_splits  0 = choose automatically (as attn_fwd), 1 = never split,
 *               n > 1 = split the key range into n near-equal chunks
 *               (clamped to the number of key tiles)
 *   workspace   device buffer of at least
 *               attn_fwd_workspace_size(B, H, S_q, S_k, D, num_splits) bytes,
 *               used when the effective split count is > 1; may be NULL when
 *               no split happens. Partial outputs (float32) and partial LSEs
 *               are staged there; it holds no state after the call.
 */
int attn_fwd_ex(const void* q, const void* k, const void* v, void* o, float* lse,
                int B, int H, int S_q, int S_k, int D, int causal, float scale,
                int dtype, int num_splits, void* workspace, size_t workspace_bytes,
                void* stream);

/*
 * attn_fwd_noalloc -- attn_fwd that allocates nothing, for callers that cannot
 * allocate device memory during the call (code under HIP graph capture, tight
 * serving loops, harnesses that forbid hipMalloc).
 *
 * Same arguments, kernels, split choice, outputs and errors as attn_fwd, and
 * the same bits. Where attn_fwd would take its key-range split workspace from
 * the stream-ordered allocator, this entry point uses a fixed device array of
 * ATTN_NOALLOC_SCRATCH_BYTES inside the library instead (one per GPU, held
 * until the process ends; its address is looked up once per device on the
 * first call, with the stream's device current). Shapes whose split needs
 * more than that (attn_fwd_workspace_size(B, H, S_q, S_k, D, 0) above the
 * limit) return ATTN_ERR_WORKSPACE before anything is enqueued; shapes that
 * need no split never touch the array. Nothing in the array has to start at
 * zero: every split writes its whole partial result before the merge reads
 * it. All calls on one GPU share its array, so two calls that overlap in
 * time on one GPU (on different streams, or from different host threads
 * without ordering) race on it; calls ordered on one stream do not.
 */
#define ATTN_NOALLOC_SCRATCH_BYTES (16u << 20)
int attn_fwd_noalloc(const void* q, const void* k, const void* v, void* o, float* lse,
                     int B, int H, int S_q, int S_k, int D, int causal, float scale,
                     int dtype, void* stream);

/*
 * attn_fwd_persistent -- attn_fwd on a persistent grid: a fixed number of
 * workgroups, each resident on its own CU for the whole call, loops over the
 * (b, h, query tile) items dealt to it ([GN] "Weitere Optimierungen und
 * kuenftige Integration" lists the persistent kernel among the full paper's
 * optimizations). Same operands, layout, masking, outputs and errors as
 * attn_fwd, and the same bits as attn_fwd where attn_fwd runs the unsplit
 * main kernel (long key ranges); the key range is never split.
 *
 *   dtype           ATTN_F16 or ATTN_BF16 (others: ATTN_ERR_UNSUPPORTED)
 *   D               64 or 128 (others: ATTN_ERR_UNSUPPORTED)
 *   num_workgroups  0 = one per CU of the current device; 1 .. CU count =
 *                   that many (uses only that many CUs, leaving the others to
 *                   concurrent work); more than the CU count or negative:
 *                   ATTN_ERR_INVALID_ARG
 *
 * Items are dealt heaviest query tile first in a snake order (even rounds
 * forward, odd rounds backward), which pairs heavy and light causal tiles so
 * the workgroups finish together; the deal is fixed, so the results do not
 * depend on timing. No workspace.
 */
int attn_fwd_persistent(const void* q, const void* k, const void* v, void* o, float* lse,
                        int B, int H, int S_q, int S_k, int D, int causal, float scale,
                        int dtype, int num_workgroups, void* stream);

/*
 * attn_fwd_varlen -- attn_fwd over a packed batch of sequences of different
 * lengths ([GN] "Weitere Optimierungen und kuenftige Integration" lists
 * variable-length sequences among the full paper's optimizations; each
 * sequence is attended exactly as attn_fwd would attend it alone).
 *
 *   q, o          [total_q, H, D], sequence b at rows cu_seqlens_q[b] ..
 *                 cu_seqlens_q[b+1]-1 (element (t,h,d) at (t*H + h)*D + d)
 *   k, v          [total_k, H, D], indexed by cu_seqlens_k the same way
 *   lse           [H, total_q] float32 (natural-log logsumexp of the scaled
 *                 scores of each row)
 *   cu_seqlens_q, cu_seqlens_k
 *                 device int32 arrays of B+1 entries: 0, then the running
 *                 totals; nondecreasing, last entry total_q / total_k. They are
 *                 read on the device only, so the library cannot check them:
 *                 the caller guarantees this shape (and that no sequence is
 *                 longer than max_seqlen_q / max_seqlen_k); otherwise the
 *                 kernel reads and writes outside the tensors.
 *   max_seqlen_q, max_seqlen_k
 *                 upper bounds of the sequence lengths (they size the grid)
 *   causal        per sequence, bottom-right aligned: key j of a sequence with
 *                 S_q query and S_k key rows is allowed for its query i iff
 *                 j <= i + S_k - S_q
 *
 * A query row with no allowed key (an empty key sequence, or causal rows
 * above the diagonal when S_q > S_k) gets O = 0 and LSE = -inf. Empty query
 * sequences write nothing. dtype is ATTN_BF16 or ATTN_F16 (ATTN_F32 returns
 * ATTN_ERR_UNSUPPORTED); D is 64, 128 or 256 (others ATTN_ERR_UNSUPPORTED;
 * so is a longest key sequence whose rows span 2^31 bytes or more of K,
 * (max_seqlen_k + 128) * H * D * 2 at D = 64 / 128 and (max_seqlen_k + 32) *
 * H * 512 at D = 256). q, k, v, o must be
 * 16-byte aligned, lse and the cu arrays 4-byte aligned; q, o, lse may be
 * NULL when total_q = 0 and k, v when total_k = 0. total_q = 0 returns
 * ATTN_OK without launching.
 */
int attn_fwd_varlen(const void* q, const void* k, const void* v, void* o, float* lse,
                    const int* cu_seqlens_q, const int* cu_seqlens_k, int B, int H,
                    int total_q, int total_k, int max_seqlen_q, int max_seqlen_k, int D,
                    int causal, float scale, int dtype, void* stream);

/*
 * attn_bwd -- gradients of attn_fwd's output: dQ, dK, dV from Q, K, V, the
 * forward output O and its LSE, and dO. The forward pass keeps the LSE so
 * that the backward pass recomputes the probabilities instead of storing them
 * ([GN] "Rueckblick auf den FlashAttention-Ansatz").
 *
 *   q, o, dout, dq  [B, H, S_q, D];  k, v, dk, dv  [B, H, S_k, D]  (dtype)
 *   lse             [B, H, S_q] float32, as written by attn_fwd
 *   scale, causal   as given to attn_fwd
 *
 * dQ = scale dS K, dK = scale dS^T Q, dV = P^T dO with P = exp(scale Q K^T - LSE)
 * (masked like the forward pass), dS = P * (dO V^T - rowsum(dO * O)). dtype is
 * ATTN_BF16 or ATTN_F16 and D is 64 or 128 (otherwise ATTN_ERR_UNSUPPORTED);
 * causal with S_q > S_k is ATTN_ERR_UNSUPPORTED as in attn_fwd. Accumulation
 * is float32 in a fixed order (deterministic); the gradients are rounded to
 * dtype. A float32 scratch of 2*B*H*S_q values (per query row: -rowsum(dO * O)
 * and -log2(e) LSE) comes from the stream-ordered allocator on `stream` and is
 * released on it.
 */
int attn_bwd(const void* q, const void* k, const void* v, const void* o, const float* lse,
             const void* dout, void* dq, void* dk, void* dv, int B, int H, int S_q, int S_k,
             int D, int causal, float scale, int dtype, void* stream);

/* Bytes of workspace attn_fwd_ex needs for these sizes and split request
 * (0 when the effective split count is 1). num_splits = 0 means "automatic". */
size_t attn_fwd_workspace_size(int B, int H, int S_q, int S_k, int D, int num_splits);

/* The split count attn_fwd would use for these sizes and element type (or
 * attn_fwd_ex with num_splits), after clamping; 1 means no split. The key
 * tile, and so the clamping, depends on dtype (ATTN_F32: 32 keys;
 * ATTN_F16 / ATTN_BF16: 128 keys at D = 64 / 128, 32 at D = 256); an unknown
 * dtype or a non-positive size returns 1. Host-only, never touches the
 * device. */
int attn_fwd_num_splits(int B, int H, int S_q, int S_k, int D, int dtype, int num_splits);

/*
 * attn_check_args -- the argument validation attn_fwd performs, without
 * enqueuing anything. Returns the status attn_fwd would return for these
 * arguments if the launch itself succeeded. Host-only.
 */
int attn_check_args(const void* q, const void* k, const void* v, const void* o, const float* lse,
                    int B, int H, int S_q, int S_k, int D, int causal, float scale, int dtype);

/*
 * hadamard_quant -- incoherent processing for FP8: x' = H_D diag(signs) x /
 * sqrt(D) along D for every row, then E4M3 quantization with one scale per
 * block of `block_rows` consecutive rows of each (b, h).
 *
 * Defined by: [NL] "3. Lage precisie (FP8) met reductie van kwantisatiefout"
 * (multiply Q and K by a random orthogonal matrix before quantizing) and
 * [GN] "Niedrige FP8-Praezision und incoherent processing" (random-sign
 * Hadamard, O(d log d) per head, memory-bound).
 *
 *   x        [B, H, S, D] in_dtype (ATTN_BF16 or ATTN_F16)
 *   x8       [B, H, S, D] uint8 E4M3 codes (written)
 *   scales   [B, H, ceil(S / block_rows)] float32 (written): dequantized
 *            value = E4M3(code) * scale of the code's block
 *   signs    device int8[D], every entry +1 or -1 (values are not checked)
 *   block_rows  1..1024
 *   x and x8 must be 16-byte aligned, scales 4-byte and signs 8-byte aligned
 *   (ATTN_ERR_MISALIGNED otherwise)
 *   apply_hadamard  1: transform then quantize; 0: quantize x itself
 *
 * Arithmetic (all float32, so the codes are unique): u = FWHT(signs * x) with
 * butterfly strides 1, 2, ..., D/2 (unnormalised); per block a = max |u|;
 * inv = 448 / a; code = E4M3_RNE(u * inv) (saturating); scale = a / 448,
 * then scale *= 1/sqrt(D) when the transform is applied. A block with a == 0
 * gets scale 1 and codes 0. D in {64, 128, 256}.
 */
int hadamard_quant(const void* x, void* x8, float* scales, const signed char* signs,
                   int B, int H, int S, int D, int block_rows, int apply_hadamard,
                   int in_dtype, void* stream);

/*
 * rope_hadamard_quant -- hadamard_quant with rotary position embedding applied
 * to every row first, fused into the same pass over x ([GN] "Niedrige
 * FP8-Praezision und incoherent processing": the Hadamard transform is bound
 * by memory bandwidth and costs nothing extra when fused with a preceding
 * memory-bound operation such as rotary embedding).
 *
 *   x, x8, scales, signs, B, H, S, D, in_dtype  as for hadamard_quant
 *   cos_t, sin_t  device float32 tables [S][D/2] (16-byte aligned): row p, pair
 *                 j holds cos / sin of that position's angle for pair j; shared
 *                 by every (b, h)
 *   rope_mode     0: pairs (2j, 2j+1); 1: pairs (j, j + D/2)
 *   block_rows    must be 64
 *
 * Row p of each (b, h) becomes x'_a = x_a cos - x_b sin, x'_b = x_b cos + x_a
 * sin for each pair (a, b), every product and sum rounded to float32 on its
 * own (no fused multiply-add), and then goes through hadamard_quant's
 * transform and block quantization unchanged (codes are reproducible bit for
 * bit). Returns ATTN_ERR_UNSUPPORTED for block_rows != 64 or D not in
 * {64, 128, 256}; other errors as for hadamard_quant.
 */
int rope_hadamard_quant(const void* x, void* x8, float* scales, const signed char* signs,
                        const float* cos_t, const float* sin_t, int B, int H, int S, int D,
                        int block_rows, int rope_mode, int in_dtype, void* stream);

/*
 * quant_per_tensor -- E4M3 quantization with one scale for the whole tensor
 * (four small launches on `stream`: clear, max |x|, quantize, final scale).
 * Used for V on the FP8 path and for the plain per-tensor FP8 baseline
 * without a transform: the pages compare incoherent processing against FP8
 * with no transform applied and report the error ratio ([NL] "3. Lage
 * precisie (FP8) met reductie van kwantisatiefout"; [GN] "Niedrige
 * FP8-Praezision und incoherent processing").
 *
 *   x       [B, H, S, D] in_dtype (ATTN_BF16 or ATTN_F16)
 *   x8      uint8 E4M3 codes (written), [B, H, S, D], or [B, H, D, S] when
 *           write_transposed = 1
 *   scale   one device float32 (written): a / 448 with a = max |x|, 1 if a == 0;
 *           it also serves as the reduction target and is cleared on-stream first
 *   code = E4M3_RNE(x * (448 / a)), saturating.
 */
int quant_per_tensor(const void* x, void* x8, float* scale, int B, int H, int S, int D,
                     int in_dtype, int write_transposed, void* stream);

/*
 * attn_fwd_fp8 -- attention on E4M3 inputs with float32 accumulation,
 * bfloat16 output and float32 LSE ([NL] "3. Lage precisie (FP8) met reductie
 * van kwantisatiefout"; [GN] "Niedrige FP8-Praezision und incoherent
 * processing").
 *
 *   q8, k8      [B, H, S_q|S_k, D] E4M3 codes
 *   q_scales    [B, H, ceil(S_q / block_rows)] float32 block scales of q8
 *   k_scales    [B, H, ceil(S_k / block_rows)] float32 block scales of k8
 *   v8          E4M3 codes of V: [B, H, S_k, D] with v_transposed = 0 (the
 *               kernel transposes V in flight), or [B, H, D, S_k] with
 *               v_transposed = 1 (the layout quant_per_tensor writes with
 *               write_transposed = 1; S_k must then be a multiple of 16,
 *               else ATTN_ERR_UNSUPPORTED). Both give the same bits.
 *   v_scale     one device float32: the per-tensor scale of v8
 *   o           [B, H, S_q, D] bfloat16 (written); lse [B, H, S_q] float32
 *   block_rows  must be 64 (the key tile of the kernel)
 * Scores are scale * (q8 . k8) * q_scale(row block) * k_scale(key block).
 * The probabilities entering P V are rounded to E4M3 after multiplication by
 * 2^7 (relative to the row's running reference, which moves when the row
 * grows by more than 1.75 in log2); the row sums are those of the rounded
 * values, so O is normalised by the weights that multiply V and the LSE is the
 * log of their sum. D = 128. The key range is split and the partial results
 * merged by logsumexp as attn_fwd does (at least 8192 keys, and a query block
 * of at most 64 rows or fewer than 128 query tiles of 128 rows over all
 * (b, h)); the merge buffer is taken from the stream-ordered allocator on
 * `stream` and released on the same stream.
 */
int attn_fwd_fp8(const void* q8, const void* k8, const void* v8,
                 const float* q_scales, const float* k_scales, const float* v_scale,
                 void* o, float* lse, int B, int H, int S_q, int S_k, int D,
                 int causal, float scale, int block_rows, int v_transposed, void* stream);

/*
 * attn_mfma_stream -- a measurement aid for the roofline report, outside the
 * attention path. The data-sheet peaks assume the top engine clock; under a
 * long stream of matrix instructions the socket reaches its power limit and
 * the clock settles lower. This call enqueues one kernel that runs
 * back-to-back matrix instructions of one kind on register operands on every
 * compute unit (two waves per SIMD, 32 * iters instructions per wave, eight
 * operand fragments in rotation, no memory traffic but one float per thread
 * to `sink`), so that the rate the matrix cores sustain can be stated beside
 * the peak. Time it with events around the call, after a warm-up launch.
 *   kind        0: v_mfma_f32_32x32x16_bf16 (that of the D = 256 forward,
 *               short-range and backward kernels); 1:
 *               v_mfma_scale_f32_32x32x64_f8f6f4 on E4M3 codes with unit
 *               scales (that of attn_fwd_fp8); 2: v_mfma_f32_16x16x32_bf16
 *               (that of the main D = 64 / 128 forward kernel)
 *   iters       iterations per wave, > 0 (50000 runs for about 60 ms at kind 0,
 *               about 30 ms at kind 2)
 *   sink        device buffer of float, 16-byte aligned, that receives one
 *               value per thread: 2 * (compute units) * 256 floats
 *   sink_bytes  its size in bytes
 *   flop        host pointer; receives the floating-point operations the
 *               launch performs (2 * M * N * K per instruction)
 * Errors: ATTN_ERR_INVALID_ARG (unknown kind, iters <= 0, null pointer, sink
 * smaller than needed), ATTN_ERR_MISALIGNED, ATTN_ERR_LAUNCH.
 */
int attn_mfma_stream(int kind, int iters, float* sink, size_t sink_bytes, double* flop, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* ATTN_H */

/*
 * fa.h -- C ABI of libfa.so: exact tiled scaled-dot-product attention on MI355X (gfx950).
 *
 * The operation (ainews.cool, "flash-attention transformer optimization", technical deep
 * dive): O = Softmax(S) V with S = scale * Q K^T, computed without materialising the
 * N x N matrix S in device memory.  The softmax runs block by block with a running row
 * maximum and running normaliser (same page, same section, last paragraph; bmjup.com,
 * "FlashAttention-2 ... 实战解析", section 2.2: numerator and denominator kept apart and
 * combined only at the end).  The backward pass recomputes the probability matrix from
 * Q, K and the stored per-row logsumexp instead of storing it (ainews.cool page, technical
 * deep dive, item 2 "recomputation").
 *
 * Layout (bmjup.com page, section 4, usage example: (batch, seqlen, nheads, headdim)):
 *   q, o, dO, dq : [B, N, Hq,  d]  contiguous, row-major ("BSHD")
 *   k, v, dk, dv : [B, N, Hkv, d]  contiguous, row-major
 *   lse          : [B, Hq, N]      float32, natural log: lse[i] = ln sum_j exp(s_ij)
 * Query head hq reads KV head hq / (Hq / Hkv): consecutive groups of Hq/Hkv query heads
 * share one KV head (MQA/GQA, hysenlabs.com "dao-ailab flash-attention", hardware-boundary
 * section).
 *
 * Masks (bmjup.com page, sections 2.3 and 3.3):
 *   causal != 0 : query row i attends keys j <= i
 *   window  > 0 : query row i attends keys j >= i - window + 1 (a left bound; together
 *                 with causal these are the `window` keys i-window+1 .. i)
 *   window == 0 : no window
 * A masked entry has probability zero: it never enters the normaliser.
 *
 * Position bias (bmjup.com page, FAQ on inference: an optional alibi_slopes argument, no
 * bias when it is absent; hysenlabs.com page, hardware-boundary section: ALiBi): the
 * *_alibi entry points take a device array `alibi_slopes` of Hq float32 slopes m_h
 * (caller-owned, read by the kernels only, used as given, any finite value; NULL is
 * rejected: the plain entry points are the no-bias case).  Query head h then scores
 * s_ij = scale * q_i . k_j - m_h * |i - j| before the mask and the softmax, with positions
 * counted from the start of each sequence; lse is the logsumexp of those biased scores, and
 * the backward treats the slopes as constants.
 *
 * Conventions for every entry point:
 *   - The caller owns every buffer (device memory, e.g. from hipMalloc or a framework
 *     allocator).  The library never allocates, frees or synchronises.
 *   - Calls enqueue work on `stream` (a hipStream_t; NULL = the null stream) and return.
 *     Results are valid once the stream has reached that point.
 *   - Arguments are validated before anything is launched.  On a non-FA_OK status
 *     nothing was enqueued and fa_last_error() describes the problem.
 *   - Re-entrant.  The library keeps no state between calls except two thread-local items:
 *     the message of the last error and a pending timing request (fa_bwd_time_main_kernel,
 *     a benchmark hook that only the next backward or decode call on the same thread reads
 *     and clears).
 *   - Output buffers must not alias input buffers.
 *   - Tensor pointers (q, k, v, o, dO, dq, dk, dv, the caches) must be 16-byte aligned
 *     and the float32 / int32 arrays (lse, cu_seqlens, seqlens_k, alibi_slopes) 4-byte
 *     aligned, as any framework allocation is; FA_ERR_INVALID_ARG otherwise.
 */
#ifndef FA_H_
#define FA_H_

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  FA_OK = 0,
  FA_ERR_INVALID_ARG = 1, /* null or misaligned pointer, non-positive size, Hq % Hkv != 0,
                             window < 0, non-finite scale, size product overflowing 2^31
                             elements                                                   */
  FA_ERR_UNSUPPORTED = 2, /* head dim outside {64, 128, 256}; a probe variant not built   */
  FA_ERR_WORKSPACE = 3,   /* workspace missing, too small or not 256-byte aligned        */
  FA_ERR_HIP = 4          /* the HIP runtime reported an error at launch                  */
} fa_status;

/*
 * Forward, bfloat16 in and out, float32 accumulation.
 *   q [B,N,Hq,d], k/v [B,N,Hkv,d] : inputs, device pointers to bfloat16
 *   o [B,N,Hq,d]                  : output, bfloat16 (rounded to nearest even once)
 *   lse [B,Hq,N]                  : output, float32 natural-log logsumexp of each row of S
 *   scale                         : any finite float (1/sqrt(d) for standard attention)
 * d must be 64, 128 or 256.  A row that attends no key (impossible with causal or
 * window >= 1 masks) gets o = 0 and lse = -inf.
 */
fa_status fa_fwd(const void* q, const void* k, const void* v, void* o, float* lse, int B,
                 int Hq, int Hkv, int N, int d, int causal, int window, float scale,
                 void* stream);

/*
 * fa_fwd with the ALiBi position bias (see the header comment): `alibi_slopes` is a device
 * array of Hq float32 slopes; NULL returns FA_ERR_INVALID_ARG.  Other rules as fa_fwd.
 */
fa_status fa_fwd_alibi(const void* q, const void* k, const void* v, void* o, float* lse, int B,
                       int Hq, int Hkv, int N, int d, int causal, int window, float scale,
                       const float* alibi_slopes, void* stream);

/*
 * Forward with 8-bit inputs.  The pages name an FP8 forward pass of a later version of the
 * method (ainews.cool, "flash-attention transformer optimization", opening overview;
 * hysenlabs.com, "dao-ailab flash-attention", hardware-boundary section) and fix no format;
 * this entry point takes OCP FP8 E4M3 codes ("fn": bias 7, 3 mantissa bits, max 448,
 * NaN = 0x7F / 0xFF, no infinities) with one float32 dequantisation factor per tensor.
 *   q [B,N,Hq,d], k/v [B,N,Hkv,d] : device pointers to E4M3 codes (one byte each), BSHD
 *   descale_q/k/v                 : the real inputs are descale_x * decoded code; each
 *                                   must be finite and > 0
 *   o [B,N,Hq,d]                  : output, bfloat16; lse [B,Hq,N] float32 natural log
 *   scale                         : softmax scale applied to the dequantised Q K^T
 * Computed: the attention of the dequantised inputs, with both products on the 8-bit
 * matrix cores.  Those sum their 64 code products with less than float32 precision
 * (measured: error within 2^-11 of the largest single product), so each score is off by up
 * to about (d/64) 2^-11 |scale| max_c |q_c k_c|, and lse by as much.  The probability
 * weights are rounded to E4M3 for the second product (each off by at most 2^-4 of itself,
 * or 2^-10 of the row's largest weight) and O is normalised by the unrounded weight sum.
 * Returns
 * FA_ERR_INVALID_ARG also for a factor that is not finite and positive, or
 * |scale| * descale_q * descale_k above 3e38.  Other rules as fa_fwd.
 */
fa_status fa_fwd_fp8(const void* q, const void* k, const void* v, void* o, float* lse,
                     float descale_q, float descale_k, float descale_v, int B, int Hq, int Hkv,
                     int N, int d, int causal, int window, float scale, void* stream);

/*
 * Forward, float32 in and out (same contract and layouts as fa_fwd, every tensor float32).
 * Dot products, softmax and accumulation are all float32.  The pages name float32 inputs
 * as a data type of the ROCm Triton backend only (hysenlabs.com, "dao-ailab
 * flash-attention", hardware-boundary section; the CUDA build takes fp16 / bf16 only,
 * bmjup.com page, section 4); this entry point is that float32 forward.
 */
fa_status fa_fwd_fp32(const float* q, const float* k, const float* v, float* o, float* lse,
                      int B, int Hq, int Hkv, int N, int d, int causal, int window,
                      float scale, void* stream);

/*
 * Bytes of device workspace fa_bwd needs for these sizes: D = rowsum(dO * O) as float32
 * [B, Hq, N], rounded up to a multiple of 256 bytes.  Linear in N: the backward keeps one
 * float per query row besides its inputs and outputs, never an N x N matrix (ainews.cool,
 * "flash-attention transformer optimization", technical deep dive: item 2, recomputation
 * instead of storing the attention matrix, and the memory table, linear growth with the
 * sequence length).  Returns 0 for arguments fa_bwd would reject.
 */
size_t fa_bwd_workspace_size(int B, int Hq, int Hkv, int N, int d, int causal, int window);

/*
 * Backward of L = sum(O * dO) for bfloat16 tensors (analytic gradient of fa_fwd).
 *   q, k, v        : the forward inputs
 *   o, lse         : the forward outputs (o bfloat16, lse float32) for the same q, k, v,
 *                    masks and scale
 *   dO [B,N,Hq,d]  : upstream gradient, bfloat16
 *   dq [B,N,Hq,d], dk/dv [B,N,Hkv,d] : outputs, bfloat16; dk and dv of a KV head are
 *                    summed over the query heads of its group
 *   workspace      : device buffer of at least fa_bwd_workspace_size(...) bytes, 256-byte
 *                    aligned; its contents on entry are ignored and on return hold D
 * The pass computes D = rowsum(dO * O) from the stored O, then recomputes P = exp(S - lse)
 * block by block twice: once per key block, accumulating dV = P^T dO and
 * dK = scale * dS^T Q with dS = P * (dO V^T - D), and once per query block, accumulating
 * dQ = scale * dS K.  No atomics are used: all outputs are deterministic.
 */
fa_status fa_bwd(const void* q, const void* k, const void* v, const void* o, const void* dO,
                 const float* lse, void* dq, void* dk, void* dv, int B, int Hq, int Hkv,
                 int N, int d, int causal, int window, float scale, void* workspace,
                 size_t workspace_bytes, void* stream);

/*
 * fa_bwd without a workspace argument, for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid allocation).
 * D = rowsum(dO * O) goes to a static device array of the library instead: 16 MiB per GPU
 * (B * Hq * N <= 4194304 rows of float32), held by every GPU the library runs on until the
 * process ends.  The call allocates nothing.  Larger sizes return FA_ERR_WORKSPACE.  All
 * calls on one GPU share that array and each overwrites it completely before reading it:
 * calls that overlap on one GPU (different streams or threads without ordering between
 * them) race and give wrong gradients.  Results are bitwise those of fa_bwd.  Other rules
 * as fa_bwd.
 */
fa_status fa_bwd_noalloc(const void* q, const void* k, const void* v, const void* o,
                         const void* dO, const float* lse, void* dq, void* dk, void* dv, int B,
                         int Hq, int Hkv, int N, int d, int causal, int window, float scale,
                         void* stream);

/* fa_bwd for the forward of fa_fwd_alibi (the same slopes); NULL slopes are rejected. */
fa_status fa_bwd_alibi(const void* q, const void* k, const void* v, const void* o,
                       const void* dO, const float* lse, void* dq, void* dk, void* dv, int B,
                       int Hq, int Hkv, int N, int d, int causal, int window, float scale,
                       void* workspace, size_t workspace_bytes, const float* alibi_slopes,
                       void* stream);

/*
 * Packed variable-length sequences.  bmjup.com, "FlashAttention-2 ... 实战解析", FAQ Q4,
 * names a variable-length interface beside the fixed-length one; what it computes is the
 * attention above applied to each sequence on its own (self-attention inside a sequence,
 * masks counted from the sequence's first row).
 *   q, o, dO, dq [total, Hq, d] and k, v, dk, dv [total, Hkv, d], bfloat16, contiguous:
 *                    sequence s occupies rows cu_seqlens[s] .. cu_seqlens[s + 1] - 1 of
 *                    every tensor (the same rows for queries and keys)
 *   cu_seqlens       device array of num_seqs + 1 int32 offsets, non-decreasing, first 0,
 *                    last total (an empty sequence is allowed); caller-owned, read by the
 *                    kernels only
 *   max_seqlen       an upper bound on every sequence length, <= total.  The offsets are not
 *                    read on the host: a sequence longer than max_seqlen is computed on its
 *                    first max_seqlen rows only, and offsets outside [0, total] are clamped
 *                    into it, so bad offsets give wrong values but no out-of-bounds access.
 *   lse (and the workspace's D) float32 [Hq, total]
 * Other arguments, the error codes and the stream rules are those of fa_fwd / fa_bwd
 * (B = num_seqs and N = max_seqlen for the size checks); FA_ERR_INVALID_ARG also for a
 * null cu_seqlens, non-positive counts or max_seqlen > total.
 */
fa_status fa_fwd_varlen(const void* q, const void* k, const void* v, void* o, float* lse,
                        const int* cu_seqlens, int num_seqs, int total, int max_seqlen, int Hq,
                        int Hkv, int d, int causal, int window, float scale, void* stream);

/* Packed sequences with the ALiBi position bias (positions counted from each sequence's
 * first row); NULL slopes are rejected. */
fa_status fa_fwd_varlen_alibi(const void* q, const void* k, const void* v, void* o, float* lse,
                              const int* cu_seqlens, int num_seqs, int total, int max_seqlen,
                              int Hq, int Hkv, int d, int causal, int window, float scale,
                              const float* alibi_slopes, void* stream);

/* Workspace bytes for fa_bwd_varlen: D as float32 [Hq, total] rounded up to 256; 0 for
 * invalid sizes. */
size_t fa_bwd_varlen_workspace_size(int total, int Hq, int Hkv, int d);

fa_status fa_bwd_varlen(const void* q, const void* k, const void* v, const void* o,
                        const void* dO, const float* lse, void* dq, void* dk, void* dv,
                        const int* cu_seqlens, int num_seqs, int total, int max_seqlen, int Hq,
                        int Hkv, int d, int causal, int window, float scale, void* workspace,
                        size_t workspace_bytes, void* stream);

fa_status fa_bwd_varlen_alibi(const void* q, const void* k, const void* v, const void* o,
                              const void* dO, const float* lse, void* dq, void* dk, void* dv,
                              const int* cu_seqlens, int num_seqs, int total, int max_seqlen,
                              int Hq, int Hkv, int d, int causal, int window, float scale,
                              void* workspace, size_t workspace_bytes,
                              const float* alibi_slopes, void* stream);

/*
 * Decoding: the newest queries of each sequence over its KV cache, the method at inference
 * over large context caches (bmjup.com, "FlashAttention-2 ... 实战解析", FAQ on inference).
 *   q [B, Nq, Hq, d]        : bf16, the Nq newest tokens of each sequence
 *   k_cache, v_cache        : bf16 [B, Nk, Hkv, d]; sequence b uses its first seqlens_k[b]
 *                             rows
 *   seqlens_k               : device int32 [B], or NULL for Nk everywhere; values are
 *                             clamped into [0, Nk] by the kernels (not read on the host)
 *   o [B, Nq, Hq, d] bf16, lse [B, Hq, Nq] float32 natural log
 * Query i of sequence b sits at position seqlens_k[b] - Nq + i; causal and window masks
 * count from there (without causal every query sees the whole cached sequence; a window
 * still bounds from the left).  A query with no allowed key gets o = 0 and lse = -inf.
 * The keys any query of a sequence may attend are split into num_splits chunks (0: the
 * library chooses, see fa_decode_num_splits); each chunk's workgroups write a partial
 * output and logsumexp to the workspace and a second kernel merges them exactly
 * (LSE = ln sum e^LSE_s, O = sum e^(LSE_s - LSE) O_s).  With one chunk no workspace is
 * used (it may be NULL).  d must be 64 or 128 (FA_ERR_UNSUPPORTED otherwise); Nq >= 1;
 * num_splits in [0, 256].  Other rules as fa_fwd.
 */
int fa_decode_num_splits(int B, int Hq, int Hkv, int Nq, int Nk, int d, int num_splits);

/* Workspace bytes fa_decode needs for these sizes and num_splits (0 when one chunk or
 * invalid sizes). */
size_t fa_decode_workspace_size(int B, int Hq, int Hkv, int Nq, int Nk, int d, int num_splits);

fa_status fa_decode(const void* q, const void* k_cache, const void* v_cache,
                    const int* seqlens_k, void* o, float* lse, int B, int Hq, int Hkv, int Nq,
                    int Nk, int d, int causal, int window, float scale, int num_splits,
                    void* workspace, size_t workspace_bytes, void* stream);

/*
 * Benchmark hook (no counterpart on the pages): the next backward (fa_bwd, fa_bwd_alibi,
 * fa_bwd_varlen, fa_bwd_varlen_alibi) or fa_decode call made on this thread records `start_event` on its stream right before its main kernel
 * (the key-block kernel for dK, dV; the chunk kernel of fa_decode) and `stop_event` right
 * after it (the dQ kernel, or the chunk merge, follows), so a caller can time the kernels
 * separately with hipEventElapsedTime.  Arguments are hipEvent_t handles owned by the caller; passing NULL
 * for both clears a pending request.  Returns FA_ERR_INVALID_ARG if exactly one is NULL.
 */
fa_status fa_bwd_time_main_kernel(void* start_event, void* stop_event);

/*
 * Measurement aid (no counterpart on the pages): enqueue `blocks` workgroups of 256
 * threads, each wave running four independent chains of `iters` bf16 32x32x16 matrix-core
 * products (32768 flop each; 4 waves per workgroup), so the sustained matrix throughput is
 * blocks * 4 * 4 * iters * 32768 flop / elapsed time.  `out` is a caller-owned device buffer
 * of blocks * 256 floats that receives per-lane sums (values are meaningless).  Returns
 * FA_ERR_INVALID_ARG for a null `out` or non-positive sizes, FA_ERR_HIP on launch failure.
 */
fa_status fa_mfma_probe(float* out, int blocks, int iters, void* stream);

/*
 * Measurement aid (no counterpart on the pages): price the atomic alternative to the
 * separate dQ pass.  Enqueues `blocks` workgroups of 256 threads; each adds, `iters` times,
 * a 32 x 128 tile of float32 values (1/1024 each) with global float atomics into the
 * caller-owned accumulator `acc` of row_blocks * 32 rows whose rows are `stride` floats
 * apart, visiting row blocks in a pseudo-random order.  The adds follow the layout of a
 * 32 x 32 MFMA accumulator: each wave-wide atomic covers two rows of 32 consecutive floats.  So blocks * iters * 4096 atomic
 * adds are issued; their rate is that count over the elapsed time.  `acc` must hold
 * row_blocks * 32 * stride floats; its contents change.  FA_ERR_INVALID_ARG for a null
 * pointer, non-positive counts, stride < 128 or row_blocks * 32 * stride >= 2^31.
 */
fa_status fa_atomic_probe(float* acc, int row_blocks, int stride, int blocks, int iters,
                          void* stream);

/*
 * Measurement aid (no counterpart on the pages): how much other work the matrix core's
 * issue pattern leaves room for.  Enqueues `blocks` workgroups of 256 * waves_per_simd
 * threads (waves_per_simd 1 or 2; with `blocks` = 256 that is one workgroup per CU); every
 * wave runs `iters` rounds of four v_mfma_f32_32x32x16_bf16 products (4 * 32768 flop per
 * wave and round) and writes one float per lane to `out`, which must hold
 * blocks * 256 * waves_per_simd floats.  `kind` selects what sits beside the products:
 *   0  param in {0,2,4,6,8,12}: param independent float32 FMAs after each product;
 *   1  param in {1,2,3,4,6,8}:  param independent v_exp_f32 after each product;
 *   2  param in {1,2,4,8}:      the round's products spread over param accumulation
 *                               chains (eight products per round for this kind);
 *   3  param in {0,1,2}:        param operands of each product read from LDS (16 bytes per
 *                               lane, one round ahead; 64 KiB of LDS per workgroup; iters
 *                               is rounded up to an even count); param in {10,11,12}: the
 *                               same with param - 10 LDS operands and the accumulators
 *                               held in AGPRs instead of VGPRs; param in {20,21,22}:
 *                               param - 20 LDS operands, every operand value drawn
 *                               uniformly from [-2, 2) (element-to-element variation).
 *   6  param in {1,2,3}:        the A operand of each product read from global memory
 *                               (16-byte loads three rounds ahead, inside a 32 KiB window of
 *                               `out` per workgroup; `out` is overwritten, its values are
 *                               the operands): 1 a contiguous 1 KiB run per wave, 2 the
 *                               K-operand pattern of the forward (32 rows of 256 bytes, 32
 *                               bytes per row per load), 3 half the products as 2 and half
 *                               with the A operand from LDS; needs blocks * waves_per_simd
 *                               >= 32 (FA_ERR_INVALID_ARG otherwise); iters is rounded up
 *                               to a multiple of 4.
 *   4, 5  param = width * 10000 + stride, width in {4,8,16} bytes, stride in [1, 4096]:
 *                               no products; every wave stores (4) or loads (5) `width`
 *                               bytes per lane at LDS byte lane * stride (masked to 64 KiB
 *                               and aligned down to the width), `iters` times, so the LDS
 *                               bank-conflict counters of the launch measure the banks and
 *                               the lanes served per cycle at that width.
 * The caller times the launch.  FA_ERR_UNSUPPORTED for another (kind, param),
 * FA_ERR_INVALID_ARG for a null pointer, waves_per_simd not 1 or 2, or non-positive counts.
 */
fa_status fa_issue_probe(float* out, int kind, int param, int waves_per_simd, int blocks,
                         int iters, void* stream);

/*
 * Measurement aid for the 8-bit forward's error bound (no counterpart on the pages): one
 * v_mfma_f32_32x32x64_f8f6f4 per operand set from a zero accumulator, C = A B with
 * A[m][k] = a[s][m][k] and B[k][n] = bt[s][n][k] for s < sets (E4M3 codes, 32 x 64 bytes per
 * set and operand, row-major), written as float32 to c[s][m][n] (32 x 32 per set).  The
 * caller owns the device buffers: a and bt hold sets * 2048 bytes and are 16-byte aligned, c
 * holds sets * 1024 floats.  FA_ERR_INVALID_ARG for a null or misaligned pointer,
 * sets <= 0 or sets * 2048 >= 2^31.
 */
fa_status fa_fp8_product_probe(const void* a, const void* bt, float* c, int sets,
                               void* stream);

/* Message for the last non-FA_OK status returned on this thread ("" if none). */
const char* fa_last_error(void);

/* Library version string. */
const char* fa_version(void);

#ifdef __cplusplus
}
#endif

#endif /* FA_H_ */

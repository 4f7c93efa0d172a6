/*
 * libfa: exact attention O = softmax(scale * Q K^T) V for AMD MI355X (gfx950),
 * computed tile by tile with an online softmax so that the N x N score matrix
 * never reaches device memory.
 *
 * The operation is the attention formula of the page "FlashAttention v2相比于v1
 * 有哪些更新" (blogweb.cn), section 1; the tiling and the running max/sum
 * recurrence are those of "FlashAttention技术解析：优化Transformer注意力机制"
 * (mhpq.cn), sections 2.1-2.2, with the normalisation deferred to the end of
 * the key loop as in the blogweb.cn page, section 3 ("Rescale操作"). The
 * backward pass recomputes the probabilities from the stored row logsumexp,
 * which is the "store only the softmax normalisation factor" strategy of the
 * page "4.3 FlashAttention-2与FlashAttention-3演进", FlashAttention-3
 * section 3 ("反向传播优化").
 *
 * Conventions shared by every entry point
 * ----------------------------------------
 *  Layout    q, o, dout, dq : contiguous [B, Hq, N, d]   (row-major, d fastest)
 *            k, v, dk, dv   : contiguous [B, Hkv, N, d]
 *            lse            : contiguous [B, Hq, N] float32
 *  Heads     query head h reads key/value head h / (Hq / Hkv) (grouped heads;
 *            Hkv == Hq is ordinary multi-head attention).
 *  Mask      causal != 0: key j is visible to query i iff j <= i.
 *  Scale     applied to q.k before the softmax (usually 1/sqrt(d)).
 *  lse       natural-log logsumexp of the scaled, masked scores of each query
 *            row: lse_i = log(sum_j exp(scale * q_i.k_j)).
 *  Memory    every pointer is a device pointer owned by the caller; the
 *            library never allocates, frees or keeps a pointer past the call.
 *            Base pointers must be 16-byte aligned. (fa_bwd_noalloc keeps its
 *            scratch in a fixed array of the library's own, one per GPU.)
 *  Streams   work is enqueued on `stream` (NULL = the default stream) and the
 *            call returns without synchronising; a device-side fault shows at
 *            the caller's next synchronisation.
 *  Empty     B == 0 or N == 0 is a valid empty problem: FA_OK, nothing is
 *            touched (pointers may then be NULL).
 *  Errors    a status code is returned; nothing is printed and nothing aborts.
 *            Argument checks run before any HIP call, so FA_ERR_INVALID_ARG and
 *            FA_ERR_UNSUPPORTED (shape) never depend on a device being present.
 *  Threads   the library keeps no state besides a per-device architecture
 *            check cached on first use (and the per-device address of
 *            fa_bwd_noalloc's scratch); calls from several host threads are
 *            safe, except overlapping fa_bwd_noalloc calls on one GPU.
 */
#ifndef FA_H
#define FA_H

#include <stddef.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  FA_OK = 0,
  FA_ERR_INVALID_ARG = -1, /* null/misaligned pointer, negative or inconsistent sizes, bad flag */
  FA_ERR_UNSUPPORTED = -2, /* head dim not supported, or device is not gfx950 */
  FA_ERR_DEVICE = -3,      /* no usable HIP device / device query failed */
  FA_ERR_LAUNCH = -4,      /* a kernel launch reported an error */
  FA_ERR_INTERNAL = -5,
  FA_ERR_TOO_LARGE = -6    /* the problem needs more scratch than fa_bwd_noalloc holds */
} fa_status;

/* Forward, bf16 storage (q, k, v, o as bf16 bit patterns), float32 arithmetic
 * for the softmax and the accumulators, float32 lse. o is rounded to bf16
 * round-to-nearest-even. Supported d: 64, 128, 256. Sizes: B >= 0, N >= 0,
 * Hq >= 1, Hkv >= 1, Hq % Hkv == 0, B*Hq*N*d < 2^31 elements per tensor. */
int fa_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
           int B, int Hq, int Hkv, int N, int d, int causal, float scale,
           hipStream_t stream);

/* Forward, float32 storage and float32 arithmetic throughout (no bf16
 * rounding anywhere). Same arguments, layouts and limits as fa_fwd, except
 * that d is 64 or 128. */
int fa_fwd_f32(const float* q, const float* k, const float* v, float* o, float* lse,
               int B, int Hq, int Hkv, int N, int d, int causal, float scale,
               hipStream_t stream);

/* Bytes of device workspace fa_fwd_splitkv needs for these sizes and
 * n_splits (0 on invalid sizes or n_splits outside 0..64; 0 = the automatic
 * choice of fa_fwd_splitkv). */
size_t fa_fwd_splitkv_workspace_bytes(int B, int Hq, int Hkv, int N, int d, int n_splits);

/* Forward attention, bf16, with the keys of every query tile split into
 * n_splits contiguous ranges processed by separate workgroups: more
 * parallelism when B * Hq * ceil(N / 256) workgroups cannot fill the GPU
 * (few heads, long sequences). Each range produces its partial output
 * O_s (fp32, normalised by its own row sum) and lse_s; a second kernel
 * combines them with the online-softmax rule one level up, lse = log sum_s
 * exp(lse_s), O = sum_s exp(lse_s - lse) O_s (the merge of per-device
 * partial results in "FlashAttention技术解析" (mhpq.cn), section 4.2).
 * Same arguments, layouts and results as fa_fwd (up to rounding), plus
 * workspace: device memory of at least fa_fwd_splitkv_workspace_bytes(...)
 * bytes, 16-byte aligned, contents ignored on entry.
 * n_splits: 1..64, or 0 to let the library choose (enough parts for the
 * plain forward's B * Hq * ceil(N / 256) workgroups to cover the GPU's 256
 * compute units, 1 when they already do, at most one part per 4 key tiles);
 * FA_ERR_INVALID_ARG otherwise. Ranges are balanced over the key tiles each
 * query tile actually visits (causal included). One part runs exactly
 * fa_fwd (the workspace is then not touched). */
int fa_fwd_splitkv(const void* q, const void* k, const void* v, void* o, float* lse,
                   void* workspace, size_t workspace_bytes,
                   int B, int Hq, int Hkv, int N, int d, int causal, float scale,
                   int n_splits, hipStream_t stream);

/* Block size (queries and keys) of the block mask of fa_fwd_blocksparse, and
 * the largest N it accepts (1024 blocks). */
#define FA_SPARSE_BLOCK 128
#define FA_SPARSE_MAX_N 131072

/* Forward attention, bf16, restricted by a block mask: the query rows and
 * the keys are cut into blocks of FA_SPARSE_BLOCK (the last one ragged),
 * n_blk = ceil(N / FA_SPARSE_BLOCK), and key j is visible to query i iff
 * the mask entry of (i / FA_SPARSE_BLOCK, j / FA_SPARSE_BLOCK) is non-zero
 * (and j <= i when causal). Key blocks that no query of a workgroup sees are
 * never loaded (the block-sparse integration of "FlashAttention技术解析"
 * (mhpq.cn), section 6.2; each query row takes one softmax over all the keys
 * it sees). A row that sees no key gets o = 0 and lse = -inf.
 * block_mask: device uint8, caller-owned; the entry (b, h, qb, kb) for query
 * head h is block_mask[b * mask_stride_b + h * mask_stride_h + qb * n_blk + kb]
 * (strides in bytes, >= 0; 0 shares one mask across batches or heads), so
 * each [n_blk, n_blk] mask is row-major and contiguous.
 * Other arguments, layouts and limits as fa_fwd, plus N <= FA_SPARSE_MAX_N
 * (FA_ERR_UNSUPPORTED beyond) and negative strides FA_ERR_INVALID_ARG. */
int fa_fwd_blocksparse(const void* q, const void* k, const void* v, void* o, float* lse,
                       const unsigned char* block_mask, long long mask_stride_b, long long mask_stride_h,
                       int B, int Hq, int Hkv, int N, int d, int causal, float scale,
                       hipStream_t stream);

/* FP8 inputs: e4m3 codes (OCP 8-bit float: 1 sign, 4 exponent bits with bias 7,
 * 3 mantissa bits; largest value 448) with one float32 scale per
 * FA_FP8_BLOCK consecutive rows of a head, x ~= value(code) * scale. */
#define FA_FP8_BLOCK 64

/* Block-wise quantisation of a bf16 tensor x [B, H, N, d] (d = 64, 128 or
 * 256) for fa_fwd_fp8: per block of FA_FP8_BLOCK rows of one (b, h),
 * scale = max|block| / 448 (1 for a block of zeros) and code = e4m3(x / scale),
 * both float32 divisions correctly rounded, codes rounded to nearest even
 * (the block scale factors of "Flash Attention V3技术解析" (mlqm.cn), section
 * 3.2, with the largest e4m3 value as the divisor). codes: device uint8
 * [B, H, N, d]; scale: device float32 [B, H, ceil(N / FA_FP8_BLOCK)]. Same
 * pointer, alignment and error rules as fa_fwd. */
int fa_quantize_fp8(const void* x, unsigned char* codes, float* scale, int B, int H, int N, int d,
                    hipStream_t stream);

/* Forward attention with FP8 queries and keys (mixed precision: the Q K^T
 * product runs on the FP8 matrix unit, as the FP8 variant of "Flash Attention
 * V3技术解析" (mlqm.cn), sections 1.3 and 3.2, does with block-wise scales; the
 * softmax, P and V stay float32 / bf16, where "4.3 FlashAttention-2与
 * FlashAttention-3演进" (aiknowledge.cn), FlashAttention-3 section 2, keeps
 * BF16). q_codes [B, Hq, N, d] and k_codes [B, Hkv, N, d] are e4m3 codes with
 * scales q_scale [B, Hq, ceil(N / 64)] and k_scale [B, Hkv, ceil(N / 64)]
 * (as written by fa_quantize_fp8); v is bf16 [B, Hkv, N, d]; o bf16, lse
 * float32 as in fa_fwd. The result is attention on the dequantised Q and K.
 * d = 128 or 256 (FA_ERR_UNSUPPORTED otherwise); other rules as fa_fwd. */
int fa_fwd_fp8(const unsigned char* q_codes, const unsigned char* k_codes, const void* v,
               const float* q_scale, const float* k_scale, void* o, float* lse,
               int B, int Hq, int Hkv, int N, int d, int causal, float scale,
               hipStream_t stream);

/* Bytes of device workspace fa_bwd needs for these sizes (0 on invalid sizes). */
size_t fa_bwd_workspace_bytes(int B, int Hq, int Hkv, int N, int d);

/* Backward, bf16 storage. q, k, v are the forward inputs; o and lse are the
 * forward outputs (fa_fwd); dout = dL/dO. Writes dq, dk, dv (bf16, RNE) =
 * dL/dq, dL/dk, dL/dv. The probabilities are recomputed from lse. For grouped
 * heads dk and dv sum over the query heads that read each key/value head.
 * workspace: device memory of at least fa_bwd_workspace_bytes(...) bytes,
 * 16-byte aligned, contents ignored on entry (float32 scratch for the row
 * term, stored negated as -D_i = -sum_c dout_ic o_ic, and for lse_i * log2 e,
 * both written by the first kernel for the second; and, for grouped heads on
 * grids too small to reach every compute unit, float32 partial dK, dV sums
 * over parts of each K/V head's query heads, added up by a third kernel). All three outputs are bitwise repeatable
 * (no atomics). Supported d: 64, 128, 256. */
int fa_bwd(const void* q, const void* k, const void* v, const void* o,
           const void* dout, const float* lse, void* dq, void* dk, void* dv,
           void* workspace, size_t workspace_bytes,
           int B, int Hq, int Hkv, int N, int d, int causal, float scale,
           hipStream_t stream);

/* Instrumentation variant of fa_bwd for measurement: identical arguments and
 * results, plus `events`, an array of 3 hipEvent_t created by the caller (or
 * NULL, then this is exactly fa_bwd). The events are recorded on `stream`
 * before the dQ kernel (which also computes the row term D), between it and
 * the dK/dV kernel, and after the dK/dV kernel (and the reduction of split
 * head groups, when there is one), so that each of the two stages can be
 * timed on its own. */
int fa_bwd_timed(const void* q, const void* k, const void* v, const void* o,
                 const void* dout, const float* lse, void* dq, void* dk, void* dv,
                 void* workspace, size_t workspace_bytes,
                 int B, int Hq, int Hkv, int N, int d, int causal, float scale,
                 hipStream_t stream, hipEvent_t* events);

/* Scratch held per GPU by fa_bwd_noalloc: 32 MiB. */
#define FA_BWD_NOALLOC_SCRATCH_BYTES (32u << 20)

/* For callers that cannot allocate device memory: code under HIP graph
 * capture, tight serving loops, and harnesses that forbid hipMalloc.
 * fa_bwd with the same arguments, layouts, kernels and results (bit for bit),
 * minus the workspace: it uses a scratch array of FA_BWD_NOALLOC_SCRATCH_BYTES
 * that the library holds in each GPU's memory from that GPU's first call
 * until the process ends, and it calls no hipMalloc, hipFree or allocating
 * library routine. Problems whose fa_bwd_workspace_bytes(...) exceed it get
 * FA_ERR_TOO_LARGE before any HIP call (about 2^22 query rows B * Hq * N
 * without split head groups). Every call on one GPU shares that GPU's
 * array: calls that overlap in time on one GPU (several streams or host
 * threads) race and must be serialised by the caller. */
int fa_bwd_noalloc(const void* q, const void* k, const void* v, const void* o,
                   const void* dout, const float* lse, void* dq, void* dk, void* dv,
                   int B, int Hq, int Hkv, int N, int d, int causal, float scale,
                   hipStream_t stream);

/* Static description of a status code; never NULL. */
const char* fa_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* FA_H */

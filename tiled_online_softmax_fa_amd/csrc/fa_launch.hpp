// Kernel parameter blocks and host-side launchers (C++ linkage, internal to libfa).
#pragma once

#include <hip/hip_runtime_api.h>
#include <stddef.h>

namespace fa {

struct FwdParams {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;
  int B, Hq, Hkv, N;
  float scale_log2;  // scale * log2(e): scores are exponentiated with exp2
  int n_tiles;       // query tiles per head (filled in by the launcher)
  // split-KV only: key-range parts per query tile, and the per-part outputs
  // o_part [n_splits][B*Hq][N][d] fp32 (normalised by the part's own row sum)
  // and lse_part [n_splits][B*Hq][N] fp32 (natural log; -inf for no key)
  int n_splits;
  float* o_part;
  float* lse_part;
  // block-sparse only: uint8 mask, element (b, h, qb, kb) at
  // block_mask[b * mask_stride_b + h * mask_stride_h + qb * n_blk + kb]
  const unsigned char* block_mask;
  long long mask_stride_b, mask_stride_h;
  // FP8 only: q and k hold e4m3 codes; one fp32 scale per 64 rows of a head,
  // q_descale [B][Hq][n_qblk], k_descale [B][Hkv][n_qblk], n_qblk = ceil(N / 64)
  const float* q_descale;
  const float* k_descale;
};

struct BwdParams {
  const void* q;
  const void* k;
  const void* v;
  const void* o;
  const void* dout;
  const float* lse;
  void* dq;
  void* dk;
  void* dv;
  float* delta;   // [B, Hq, N] workspace: -D_i = -sum_c dout_ic o_ic (the dP accumulators start there)
  float* lse2;    // [B, Hq, N] workspace: lse_i * log2(e), written with D by the dQ kernel
  int n_gsplit;     // parts of each dK/dV workgroup's (query head, query tile) sequence (1: none)
  float* dkv_part;  // n_gsplit > 1: [2][n_gsplit][B * Hkv][N][d] fp32 partial dV^T, dK^T sums (dK unscaled)
  int B, Hq, Hkv, N;
  float scale;
  float scale_log2;
  int n_tiles;
};

hipError_t launch_fwd_bf16(const FwdParams& p, int d, bool causal, hipStream_t stream);
hipError_t launch_fwd_f32(const FwdParams& p, int d, bool causal, hipStream_t stream);
// split-KV forward: the partial kernel then the merge (p.n_splits >= 1, workspace in p.o_part / p.lse_part)
hipError_t launch_fwd_bf16_splitkv(const FwdParams& p, int d, bool causal, hipStream_t stream);
// block-sparse forward (p.block_mask set; N <= kSparseMaxN)
constexpr int kSparseBlock = 128;
constexpr int kSparseMaxBlocks = 1024;
constexpr int kSparseMaxN = kSparseBlock * kSparseMaxBlocks;
hipError_t launch_fwd_bf16_blocksparse(const FwdParams& p, int d, bool causal, hipStream_t stream);
// FP8 forward (p.q, p.k e4m3 codes with p.q_descale / p.k_descale; d = 128 or 256)
constexpr int kFp8Block = 64;
hipError_t launch_fwd_fp8(const FwdParams& p, int d, bool causal, hipStream_t stream);
// block-wise e4m3 quantisation of a bf16 [heads][N][d] tensor (d = 64, 128 or 256)
hipError_t launch_quantize_fp8(const void* x, unsigned char* codes, float* scale, int heads, int N, int d,
                               hipStream_t stream);
// events: NULL or 3 events recorded before/between/after the two backward kernels
hipError_t launch_bwd_bf16(const BwdParams& p, int d, bool causal, hipStream_t stream, hipEvent_t* events);
// device address of this GPU's scratch array for fa_bwd_noalloc (FA_BWD_NOALLOC_SCRATCH_BYTES bytes),
// looked up on the current device's first call and cached per device
hipError_t bwd_noalloc_scratch(void** ptr);

}  // namespace fa

// Block-wise FP8 (e4m3) quantisation of a bf16 tensor [heads][N][d] (gfx950).
//
// One scale per 64 rows of a head across the whole head dim: scale =
// max|block| / 448 and code = e4m3(x / scale), rounded to nearest even (the
// block scale factors of "Flash Attention V3技术解析" (mlqm.cn) section 3.2,
// with 448, the largest e4m3 value, as the divisor). A block of zeros gets
// scale 1. Both divisions are correctly rounded float32 divisions, and
// v_cvt_pk_fp8_f32 rounds to nearest even, so codes and scales are exact
// functions of the input bits.
//
// HBM-bound: one workgroup of 256 threads per (64-row block, head) reads the
// block twice (the second read hits L2) and writes one byte per element.
#include "fa_common.hpp"
#include "fa_launch.hpp"

namespace fa {

template <int D>
__global__ __launch_bounds__(256) void fa_quantize_fp8_kernel(const __bf16* __restrict__ x,
                                                              unsigned char* __restrict__ codes,
                                                              float* __restrict__ scale, int N, int n_blk) {
  constexpr int BR = kFp8Block;
  const int blk = workgroup_index() % n_blk;
  const size_t head = (size_t)workgroup_index() / n_blk;
  const int r0 = blk * BR;
  const int rows = min(BR, N - r0);
  const size_t base = (head * N + r0) * D;  // first element of the block
  const int n8 = rows * D / 8;              // groups of 8 elements (16 bytes of input)
  const u32x4* src = (const u32x4*)(x + base);

  float amax = 0.f;
  for (int i = (int)threadIdx.x; i < n8; i += 256) {
    const bf16x8 v = __builtin_bit_cast(bf16x8, src[i]);
#pragma unroll
    for (int e = 0; e < 8; ++e) amax = fmaxf(amax, fabsf((float)v[e]));
  }
  // block maximum: within the wave, then across the 4 waves
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) amax = fmaxf(amax, __shfl_xor(amax, off, 64));
  __shared__ float wmax[4];
  if ((threadIdx.x & 63) == 0) wmax[threadIdx.x >> 6] = amax;
  __syncthreads();
  amax = fmaxf(fmaxf(wmax[0], wmax[1]), fmaxf(wmax[2], wmax[3]));
  const float s = amax > 0.f ? amax / 448.0f : 1.0f;

  u32x2* dst = (u32x2*)(codes + base);
  for (int i = (int)threadIdx.x; i < n8; i += 256) {
    const bf16x8 v = __builtin_bit_cast(bf16x8, src[i]);
    float y[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) y[e] = (float)v[e] / s;
    uint32_t lo = 0, hi = 0;
    lo = __builtin_amdgcn_cvt_pk_fp8_f32(y[0], y[1], lo, false);
    lo = __builtin_amdgcn_cvt_pk_fp8_f32(y[2], y[3], lo, true);
    hi = __builtin_amdgcn_cvt_pk_fp8_f32(y[4], y[5], hi, false);
    hi = __builtin_amdgcn_cvt_pk_fp8_f32(y[6], y[7], hi, true);
    dst[i] = u32x2{lo, hi};
  }
  if (threadIdx.x == 0) scale[head * n_blk + blk] = s;
}

hipError_t launch_quantize_fp8(const void* x, unsigned char* codes, float* scale, int heads, int N, int d,
                               hipStream_t stream) {
  const int n_blk = (N + kFp8Block - 1) / kFp8Block;
  const dim3 grid((unsigned)((size_t)heads * n_blk));
  if (d == 64) hipLaunchKernelGGL((fa_quantize_fp8_kernel<64>), grid, dim3(256), 0, stream, (const __bf16*)x, codes, scale, N, n_blk);
  else if (d == 128) hipLaunchKernelGGL((fa_quantize_fp8_kernel<128>), grid, dim3(256), 0, stream, (const __bf16*)x, codes, scale, N, n_blk);
  else if (d == 256) hipLaunchKernelGGL((fa_quantize_fp8_kernel<256>), grid, dim3(256), 0, stream, (const __bf16*)x, codes, scale, N, n_blk);
  else return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace fa

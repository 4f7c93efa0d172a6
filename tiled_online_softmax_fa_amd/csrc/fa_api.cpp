// C ABI of libfa: argument validation, device check, dispatch to the kernels.
// Every check that depends only on the arguments runs before any HIP call.
#include <hip/hip_runtime_api.h>

#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstdint>
#include <cstring>

#include "fa.h"
#include "fa_launch.hpp"

namespace {

constexpr int kMaxDevices = 64;
// 0 = unknown, 1 = gfx950, 2 = other architecture
std::atomic<int> g_arch_state[kMaxDevices];

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Shapes common to forward and backward. Returns FA_OK, or the error code.
// Head dims: 64 and 128 everywhere, 256 where `d256` (every bf16 entry point).
int check_shapes(int B, int Hq, int Hkv, int N, int d, int causal, float scale, bool d256 = false) {
  if (B < 0 || N < 0 || Hq < 1 || Hkv < 1) return FA_ERR_INVALID_ARG;
  if (Hq % Hkv != 0) return FA_ERR_INVALID_ARG;
  if (causal != 0 && causal != 1) return FA_ERR_INVALID_ARG;
  if (!std::isfinite(scale) || !(scale > 0.0f)) return FA_ERR_INVALID_ARG;
  if (d != 64 && d != 128 && !(d256 && d == 256)) return FA_ERR_UNSUPPORTED;
  // every tensor must index with 32-bit element offsets inside one head and
  // with size_t across heads; keep the whole tensor below 2^31 elements
  const long long elems = (long long)B * Hq * N * d;
  if (elems >= (1LL << 31)) return FA_ERR_INVALID_ARG;
  return FA_OK;
}

int check_ptrs(std::initializer_list<const void*> ptrs) {
  for (const void* p : ptrs) {
    if (p == nullptr) return FA_ERR_INVALID_ARG;
    if (!aligned16(p)) return FA_ERR_INVALID_ARG;
  }
  return FA_OK;
}

// gfx950 check for the current device, cached per device id.
int check_device() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return FA_ERR_DEVICE;
  if (dev < kMaxDevices) {
    const int st = g_arch_state[dev].load(std::memory_order_relaxed);
    if (st == 1) return FA_OK;
    if (st == 2) return FA_ERR_UNSUPPORTED;
  }
  hipDeviceProp_t prop;
  if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return FA_ERR_DEVICE;
  const bool ok = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0;
  if (dev < kMaxDevices) g_arch_state[dev].store(ok ? 1 : 2, std::memory_order_relaxed);
  return ok ? FA_OK : FA_ERR_UNSUPPORTED;
}

int launch_status(hipError_t e) { return e == hipSuccess ? FA_OK : FA_ERR_LAUNCH; }

constexpr float kLog2e = 1.4426950408889634f;

template <typename T>
int fwd_common(const T* q, const T* k, const T* v, T* o, float* lse, int B, int Hq, int Hkv, int N, int d,
               int causal, float scale, hipStream_t stream, bool bf16) {
  int st = check_shapes(B, Hq, Hkv, N, d, causal, scale, bf16);
  if (st != FA_OK) return st;
  if (B == 0 || N == 0) return FA_OK;
  st = check_ptrs({q, k, v, o, lse});
  if (st != FA_OK) return st;
  st = check_device();
  if (st != FA_OK) return st;
  fa::FwdParams p{};
  p.q = q;
  p.k = k;
  p.v = v;
  p.o = o;
  p.lse = lse;
  p.B = B;
  p.Hq = Hq;
  p.Hkv = Hkv;
  p.N = N;
  p.scale_log2 = scale * kLog2e;
  return launch_status(bf16 ? fa::launch_fwd_bf16(p, d, causal != 0, stream)
                            : fa::launch_fwd_f32(p, d, causal != 0, stream));
}

constexpr int kMaxSplits = 64;
constexpr int kComputeUnits = 256;  // MI355X

// n_splits = 0: as many key-range parts as it takes for the workgroups of the
// plain forward (one per query tile and head) to cover the compute units once,
// at most one part per 4 key tiles of the longest query tile.
int auto_splits(int B, int Hq, int N, int d) {
  const int bm = d == 256 ? 128 : 256, bn = d == 256 ? 32 : 64;  // the forward's tiles
  const long long n_wg = (long long)B * Hq * ((N + bm - 1) / bm);
  if (n_wg <= 0) return 1;  // empty problem
  int s = n_wg >= kComputeUnits ? 1 : (int)(kComputeUnits / n_wg);
  s = std::min(s, std::max(1, ((N + bn - 1) / bn) / 4));
  return std::max(1, std::min(s, kMaxSplits));
}

// split-KV workspace: o_part [S][rows][d] fp32, then (256-byte aligned) lse_part [S][rows] fp32
size_t splitkv_o_bytes(int B, int Hq, int N, int d, int n_splits) {
  const size_t rows = (size_t)B * Hq * N;
  return (rows * (size_t)d * sizeof(float) * (size_t)n_splits + 255) & ~(size_t)255;
}
size_t splitkv_workspace(int B, int Hq, int N, int d, int n_splits) {
  const size_t rows = (size_t)B * Hq * N;
  return splitkv_o_bytes(B, Hq, N, d, n_splits) + ((rows * sizeof(float) * (size_t)n_splits + 255) & ~(size_t)255);
}

// per query row: D_i, then (256-byte aligned) lse_i * log2(e)
size_t bwd_row_bytes(int B, int Hq, int N) { return ((size_t)B * Hq * N * sizeof(float) + 255) & ~(size_t)255; }

// Parts the (query head, query tile) steps of each dK/dV workgroup are split
// into: enough for its grid of (key tile, batch * K/V head) workgroups to
// reach every compute unit (1: no split), with about 4 steps per part or more
// on the longest sequence, and at most kMaxDkdvParts. Each part writes fp32
// partial dK, dV sums, added up by a reduction kernel.
constexpr int kMaxDkdvParts = 16;
int bwd_group_splits(int B, int Hq, int Hkv, int N, int d) {
  const int bnk = d == 256 ? 64 : 128, bmq = d == 256 ? 32 : 64;  // keys per workgroup, query rows per step
  const long long n_wg = (long long)((N + bnk - 1) / bnk) * B * Hkv;
  if (n_wg == 0 || n_wg >= kComputeUnits) return 1;  // (empty problems launch nothing)
  const long long steps = (long long)((N + bmq - 1) / bmq) * (Hq / Hkv);  // key tile 0: every query tile
  long long s = (kComputeUnits + n_wg - 1) / n_wg;
  s = std::min<long long>(s, std::max<long long>(1, steps / 4));
  return (int)std::min<long long>(s, kMaxDkdvParts);
}
// split dK/dV partial sums: dV^T parts then dK^T parts, [2][S][B * Hkv][N][d] fp32
size_t bwd_part_bytes(int B, int Hq, int Hkv, int N, int d) {
  const int S = bwd_group_splits(B, Hq, Hkv, N, d);
  if (S <= 1) return 0;
  return ((size_t)2 * S * B * Hkv * N * (size_t)d * sizeof(float) + 255) & ~(size_t)255;
}
size_t bwd_workspace(int B, int Hq, int Hkv, int N, int d) {
  return 2 * bwd_row_bytes(B, Hq, N) + bwd_part_bytes(B, Hq, Hkv, N, d);
}

}  // namespace

extern "C" {

int fa_fwd(const void* q, const void* k, const void* v, void* o, float* lse, int B, int Hq, int Hkv, int N, int d,
           int causal, float scale, hipStream_t stream) {
  return fwd_common<void>(q, k, v, o, lse, B, Hq, Hkv, N, d, causal, scale, stream, true);
}

int fa_fwd_f32(const float* q, const float* k, const float* v, float* o, float* lse, int B, int Hq, int Hkv, int N,
               int d, int causal, float scale, hipStream_t stream) {
  return fwd_common<float>(q, k, v, o, lse, B, Hq, Hkv, N, d, causal, scale, stream, false);
}

size_t fa_fwd_splitkv_workspace_bytes(int B, int Hq, int Hkv, int N, int d, int n_splits) {
  if (check_shapes(B, Hq, Hkv, N, d, 0, 1.0f, true) != FA_OK) return 0;
  if (n_splits == 0) n_splits = auto_splits(B, Hq, N, d);
  if (n_splits < 1 || n_splits > kMaxSplits) return 0;
  return splitkv_workspace(B, Hq, N, d, n_splits);
}

int fa_fwd_splitkv(const void* q, const void* k, const void* v, void* o, float* lse, void* workspace,
                   size_t workspace_bytes, int B, int Hq, int Hkv, int N, int d, int causal, float scale, int n_splits,
                   hipStream_t stream) {
  int st = check_shapes(B, Hq, Hkv, N, d, causal, scale, true);
  if (st != FA_OK) return st;
  if (n_splits == 0) n_splits = auto_splits(B, Hq, N, d);
  if (n_splits < 1 || n_splits > kMaxSplits) return FA_ERR_INVALID_ARG;
  if (B == 0 || N == 0) return FA_OK;
  st = check_ptrs({q, k, v, o, lse, workspace});
  if (st != FA_OK) return st;
  if (workspace_bytes < splitkv_workspace(B, Hq, N, d, n_splits)) return FA_ERR_INVALID_ARG;
  st = check_device();
  if (st != FA_OK) return st;
  fa::FwdParams p{};
  p.q = q;
  p.k = k;
  p.v = v;
  p.o = o;
  p.lse = lse;
  p.B = B;
  p.Hq = Hq;
  p.Hkv = Hkv;
  p.N = N;
  p.scale_log2 = scale * kLog2e;
  // one part is the plain forward: no partial results, no merge
  if (n_splits == 1) return launch_status(fa::launch_fwd_bf16(p, d, causal != 0, stream));
  p.n_splits = n_splits;
  p.o_part = (float*)workspace;
  p.lse_part = (float*)((char*)workspace + splitkv_o_bytes(B, Hq, N, d, n_splits));
  return launch_status(fa::launch_fwd_bf16_splitkv(p, d, causal != 0, stream));
}

int fa_fwd_blocksparse(const void* q, const void* k, const void* v, void* o, float* lse,
                       const unsigned char* block_mask, long long mask_stride_b, long long mask_stride_h, int B, int Hq,
                       int Hkv, int N, int d, int causal, float scale, hipStream_t stream) {
  static_assert(FA_SPARSE_BLOCK == fa::kSparseBlock && FA_SPARSE_MAX_N == fa::kSparseMaxN, "block-mask limits");
  int st = check_shapes(B, Hq, Hkv, N, d, causal, scale, true);
  if (st != FA_OK) return st;
  if (mask_stride_b < 0 || mask_stride_h < 0) return FA_ERR_INVALID_ARG;
  if (N > FA_SPARSE_MAX_N) return FA_ERR_UNSUPPORTED;
  if (B == 0 || N == 0) return FA_OK;
  st = check_ptrs({q, k, v, o, lse});
  if (st != FA_OK) return st;
  if (block_mask == nullptr) return FA_ERR_INVALID_ARG;
  st = check_device();
  if (st != FA_OK) return st;
  fa::FwdParams p{};
  p.q = q;
  p.k = k;
  p.v = v;
  p.o = o;
  p.lse = lse;
  p.B = B;
  p.Hq = Hq;
  p.Hkv = Hkv;
  p.N = N;
  p.scale_log2 = scale * kLog2e;
  p.block_mask = block_mask;
  p.mask_stride_b = mask_stride_b;
  p.mask_stride_h = mask_stride_h;
  return launch_status(fa::launch_fwd_bf16_blocksparse(p, d, causal != 0, stream));
}

int fa_quantize_fp8(const void* x, unsigned char* codes, float* scale, int B, int H, int N, int d,
                    hipStream_t stream) {
  static_assert(FA_FP8_BLOCK == fa::kFp8Block, "FP8 block");
  int st = check_shapes(B, H, H, N, d, 0, 1.0f, true);
  if (st != FA_OK) return st;
  if (B == 0 || N == 0) return FA_OK;
  st = check_ptrs({x, codes, scale});
  if (st != FA_OK) return st;
  st = check_device();
  if (st != FA_OK) return st;
  return launch_status(fa::launch_quantize_fp8(x, codes, scale, B * H, N, d, stream));
}

int fa_fwd_fp8(const unsigned char* q_codes, const unsigned char* k_codes, const void* v, const float* q_scale,
               const float* k_scale, void* o, float* lse, int B, int Hq, int Hkv, int N, int d, int causal, float scale,
               hipStream_t stream) {
  int st = check_shapes(B, Hq, Hkv, N, d, causal, scale, true);
  if (st != FA_OK) return st;
  if (d != 128 && d != 256) return FA_ERR_UNSUPPORTED;
  if (B == 0 || N == 0) return FA_OK;
  st = check_ptrs({q_codes, k_codes, v, o, lse});
  if (st != FA_OK) return st;
  if (q_scale == nullptr || k_scale == nullptr) return FA_ERR_INVALID_ARG;
  st = check_device();
  if (st != FA_OK) return st;
  fa::FwdParams p{};
  p.q = q_codes;
  p.k = k_codes;
  p.v = v;
  p.o = o;
  p.lse = lse;
  p.B = B;
  p.Hq = Hq;
  p.Hkv = Hkv;
  p.N = N;
  p.scale_log2 = scale * kLog2e;
  p.q_descale = q_scale;
  p.k_descale = k_scale;
  return launch_status(fa::launch_fwd_fp8(p, d, causal != 0, stream));
}

size_t fa_bwd_workspace_bytes(int B, int Hq, int Hkv, int N, int d) {
  if (check_shapes(B, Hq, Hkv, N, d, 0, 1.0f, true) != FA_OK) return 0;
  return bwd_workspace(B, Hq, Hkv, N, d);
}

int fa_bwd_timed(const void* q, const void* k, const void* v, const void* o, const void* dout, const float* lse,
                 void* dq, void* dk, void* dv, void* workspace, size_t workspace_bytes, int B, int Hq, int Hkv, int N,
                 int d, int causal, float scale, hipStream_t stream, hipEvent_t* events) {
  int st = check_shapes(B, Hq, Hkv, N, d, causal, scale, true);
  if (st != FA_OK) return st;
  if (B == 0 || N == 0) return FA_OK;
  st = check_ptrs({q, k, v, o, dout, lse, dq, dk, dv, workspace});
  if (st != FA_OK) return st;
  if (workspace_bytes < bwd_workspace(B, Hq, Hkv, N, d)) return FA_ERR_INVALID_ARG;
  if (events != nullptr) {
    for (int i = 0; i < 3; ++i)
      if (events[i] == nullptr) return FA_ERR_INVALID_ARG;
  }
  st = check_device();
  if (st != FA_OK) return st;
  fa::BwdParams p{};
  p.q = q;
  p.k = k;
  p.v = v;
  p.o = o;
  p.dout = dout;
  p.lse = lse;
  p.dq = dq;
  p.dk = dk;
  p.dv = dv;
  p.delta = (float*)workspace;
  p.lse2 = (float*)((char*)workspace + bwd_row_bytes(B, Hq, N));
  p.n_gsplit = bwd_group_splits(B, Hq, Hkv, N, d);
  p.dkv_part = p.n_gsplit > 1 ? (float*)((char*)workspace + 2 * bwd_row_bytes(B, Hq, N)) : nullptr;
  p.B = B;
  p.Hq = Hq;
  p.Hkv = Hkv;
  p.N = N;
  p.scale = scale;
  p.scale_log2 = scale * kLog2e;
  return launch_status(fa::launch_bwd_bf16(p, d, causal != 0, stream, events));
}

int fa_bwd(const void* q, const void* k, const void* v, const void* o, const void* dout, const float* lse, void* dq,
           void* dk, void* dv, void* workspace, size_t workspace_bytes, int B, int Hq, int Hkv, int N, int d,
           int causal, float scale, hipStream_t stream) {
  return fa_bwd_timed(q, k, v, o, dout, lse, dq, dk, dv, workspace, workspace_bytes, B, Hq, Hkv, N, d, causal, scale,
                      stream, nullptr);
}

int fa_bwd_noalloc(const void* q, const void* k, const void* v, const void* o, const void* dout, const float* lse,
                   void* dq, void* dk, void* dv, int B, int Hq, int Hkv, int N, int d, int causal, float scale,
                   hipStream_t stream) {
  int st = check_shapes(B, Hq, Hkv, N, d, causal, scale, true);
  if (st != FA_OK) return st;
  if (B == 0 || N == 0) return FA_OK;
  st = check_ptrs({q, k, v, o, dout, lse, dq, dk, dv});
  if (st != FA_OK) return st;
  const size_t need = bwd_workspace(B, Hq, Hkv, N, d);
  if (need > (size_t)FA_BWD_NOALLOC_SCRATCH_BYTES) return FA_ERR_TOO_LARGE;
  st = check_device();
  if (st != FA_OK) return st;
  void* scratch = nullptr;
  if (fa::bwd_noalloc_scratch(&scratch) != hipSuccess) return FA_ERR_DEVICE;
  return fa_bwd_timed(q, k, v, o, dout, lse, dq, dk, dv, scratch, need, B, Hq, Hkv, N, d, causal, scale, stream,
                      nullptr);
}

const char* fa_status_string(int status) {
  switch (status) {
    case FA_OK: return "ok";
    case FA_ERR_INVALID_ARG: return "invalid argument (null/misaligned pointer, bad size, flag or scale)";
    case FA_ERR_UNSUPPORTED: return "unsupported (head dim not 64/128/256, or 256 with fp32 storage; or device is not gfx950)";
    case FA_ERR_DEVICE: return "no usable HIP device";
    case FA_ERR_LAUNCH: return "kernel launch failed";
    case FA_ERR_INTERNAL: return "internal error";
    case FA_ERR_TOO_LARGE: return "problem needs more scratch than fa_bwd_noalloc holds (FA_BWD_NOALLOC_SCRATCH_BYTES)";
    default: return "unknown status";
  }
}

}  // extern "C"

// Forward attention, fp32 storage and fp32 arithmetic throughout (gfx950).
//
// Same computation as the bf16 kernel (attention formula of "FlashAttention
// v2相比于v1有哪些更新" section 1, online softmax of "FlashAttention技术解析"
// sections 2.1-2.2, deferred normalisation), with no bf16 rounding anywhere:
// S^T = K Q^T and O^T += V^T P^T run on v_mfma_f32_16x16x4_f32.
//
// This path serves short, latency-bound problems (its measured case is one
// head of 256 keys), so it favours simplicity: 4 waves x 16 query rows per
// workgroup (the 64-row query block of the mhpq.cn page, section 3.1),
// 32-key K/V tiles staged through two LDS buffers (each tile's global loads
// are issued one tile ahead, into registers), and rows padded to d + 4
// floats so the fragment reads of 16 consecutive rows fall in different
// banks (the row padding of mhpq.cn section 5.2).
//
// The P^T accumulator registers feed O^T += V^T P^T directly: for the r-th
// 4-key step of a 16-key block, lane l's register r holds key 4(l/16) + r,
// which is exactly the k-slot l/16 the instruction reads from lane l.
#include "fa_common.hpp"
#include "fa_launch.hpp"

namespace fa {

constexpr float kRescaleSlackF32 = 8.0f;

template <int D, bool CAUSAL>
__global__ __launch_bounds__(256, 1) void fa_fwd_f32_kernel(FwdParams p) {
  constexpr int QPW = 16, NW = 4, BM = QPW * NW, BN = 32;
  constexpr int KB = BN / 16;
  constexpr int DS = D / 4;   // k-steps of S^T
  constexpr int DB = D / 16;  // 16-row blocks of O^T
  constexpr int LD = D + 4;   // padded LDS row (floats)
  // two K/V tile buffers: tile t+1 is written while tile t is read
  __shared__ __attribute__((aligned(16))) float ks2[2][BN * LD];
  __shared__ __attribute__((aligned(16))) float vs2[2][BN * LD];

  const int N = p.N;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = uniform(tid >> 6);
  const int g = lane >> 4, L = lane & 15;

  const TileCoord tc = map_workgroup(blockIdx.x, p.B * p.Hq, p.n_tiles, CAUSAL);
  const int b = tc.head / p.Hq;
  const int h = tc.head - b * p.Hq;
  const int hk = h / (p.Hq / p.Hkv);
  const float* __restrict__ qg = (const float*)p.q + ((size_t)(b * p.Hq + h) * N) * D;
  const float* __restrict__ kg = (const float*)p.k + ((size_t)(b * p.Hkv + hk) * N) * D;
  const float* __restrict__ vg = (const float*)p.v + ((size_t)(b * p.Hkv + hk) * N) * D;
  float* __restrict__ og = (float*)p.o + ((size_t)(b * p.Hq + h) * N) * D;
  float* __restrict__ lseg = p.lse + (size_t)(b * p.Hq + h) * N;

  const int q0 = tc.tile * BM;
  const int qw0 = q0 + wave * QPW;
  const int kv_end = CAUSAL ? min(N, q0 + BM) : N;
  const int n_kv = (kv_end + BN - 1) / BN;
  const int n_kv_wave = (qw0 < N) ? ((CAUSAL ? min(N, qw0 + QPW) : N) + BN - 1) / BN : 0;

  float qf[DS];
  {
    const int row = min(qw0 + L, N - 1);
#pragma unroll
    for (int ds = 0; ds < DS; ++ds) qf[ds] = qg[(size_t)row * D + ds * 4 + g];
  }
  f32x4 acc[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) acc[db] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_ref = kNegInf, l_part = 0.f;
  const float c = p.scale_log2;

  // Tile loads go global -> registers one tile ahead (their latency overlaps
  // the math of the current tile), then registers -> LDS at the top of the
  // next iteration; one barrier per tile publishes the tile and, with two
  // buffers, also guarantees the buffer written next is no longer read.
  constexpr int VEC = BN * D / 4;             // float4 pieces per tensor
  constexpr int PER = VEC / (NW * 64);        // pieces per thread
  static_assert(VEC % (NW * 64) == 0, "tile split");
  f32x4 kreg[PER], vreg[PER];
  auto load_tile = [&](int t) {
#pragma unroll
    for (int j = 0; j < PER; ++j) {
      const int i = tid + j * NW * 64;
      const int row = i / (D / 4), c4 = i % (D / 4);
      const int grow = min(t * BN + row, N - 1);
      kreg[j] = *(const f32x4*)(kg + (size_t)grow * D + c4 * 4);
      vreg[j] = *(const f32x4*)(vg + (size_t)grow * D + c4 * 4);
    }
  };
  if (n_kv > 0) load_tile(0);
  for (int t = 0; t < n_kv; ++t) {
    const int kv0 = t * BN;
    float* ks = ks2[t & 1];
    float* vs = vs2[t & 1];
#pragma unroll
    for (int j = 0; j < PER; ++j) {
      const int i = tid + j * NW * 64;
      const int row = i / (D / 4), c4 = i % (D / 4);
      *(f32x4*)(ks + row * LD + c4 * 4) = kreg[j];
      *(f32x4*)(vs + row * LD + c4 * 4) = vreg[j];
    }
    if (t + 1 < n_kv) load_tile(t + 1);
    __syncthreads();
    if (t >= n_kv_wave) continue;

    f32x4 s[KB];
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
      f32x4 a = f32x4{0.f, 0.f, 0.f, 0.f};
      const float* krow = ks + (kb * 16 + L) * LD + g;
#pragma unroll
      for (int ds = 0; ds < DS; ++ds) a = mfma_f32_16x16x4(krow[ds * 4], qf[ds], a);
      s[kb] = a;
    }
    const bool need_mask = (kv0 + BN > N) || (CAUSAL && kv0 + BN - 1 > qw0);
    if (need_mask) {
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int key = kv0 + kb * 16 + g * 4 + r;
          const bool visible = key < N && (!CAUSAL || key <= qw0 + L);
          s[kb][r] = visible ? s[kb][r] : kNegInf;
        }
    }
    float mx = s[0][0];
#pragma unroll
    for (int kb = 0; kb < KB; ++kb)
#pragma unroll
      for (int r = 0; r < 4; ++r) mx = fmaxf(mx, s[kb][r]);
    const float tmax = mx * c;
    if (wave_any(tmax > m_ref + kRescaleSlackF32)) {
      const float m_new = fmaxf(m_ref, max_over_row_groups(tmax));
      const float alpha = (m_ref == kNegInf) ? 0.f : exp2_fast(m_ref - m_new);
      m_ref = m_new;
      l_part *= alpha;
#pragma unroll
      for (int db = 0; db < DB; ++db) acc[db] *= alpha;
    }
    const float neg_m = -m_ref;
#pragma unroll
    for (int kb = 0; kb < KB; ++kb)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        s[kb][r] = exp2_fast(fmaf(s[kb][r], c, neg_m));
        l_part += s[kb][r];
      }
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          acc[db] = mfma_f32_16x16x4(vs[(kb * 16 + 4 * g + r) * LD + db * 16 + L], s[kb][r], acc[db]);
  }

  const float l = sum_over_row_groups(l_part);
  const int row = qw0 + L;
  if (row < N) {
    const float inv = 1.0f / l;
#pragma unroll
    for (int db = 0; db < DB; ++db) *(f32x4*)(og + (size_t)row * D + db * 16 + g * 4) = acc[db] * inv;
    if (g == 0) lseg[row] = (m_ref + log2_fast(l)) * kLn2;
  }
}

template <int D, bool CAUSAL>
static hipError_t launch_fwd_f32_cfg(const FwdParams& p_in, hipStream_t stream) {
  FwdParams p = p_in;
  p.n_tiles = (p.N + 63) / 64;
  const unsigned grid = (unsigned)(p.n_tiles * p.B * p.Hq);
  hipLaunchKernelGGL((fa_fwd_f32_kernel<D, CAUSAL>), dim3(grid), dim3(256), 0, stream, p);
  return hipGetLastError();
}

hipError_t launch_fwd_f32(const FwdParams& p, int d, bool causal, hipStream_t stream) {
  if (d == 128) return causal ? launch_fwd_f32_cfg<128, true>(p, stream) : launch_fwd_f32_cfg<128, false>(p, stream);
  if (d == 64) return causal ? launch_fwd_f32_cfg<64, true>(p, stream) : launch_fwd_f32_cfg<64, false>(p, stream);
  return hipErrorInvalidValue;
}

}  // namespace fa

// Forward attention, fp32 storage and fp32 arithmetic throughout (gfx950).
//
// Same computation as the bf16 kernel (attention formula of "FlashAttention
// v2相比于v1有哪些更新" section 1, online softmax of "FlashAttention技术解析"
// sections 2.1-2.2, deferred normalisation), with no bf16 rounding anywhere:
// S^T = K Q^T and O^T += V^T P^T run on v_mfma_f32_16x16x4_f32.
//
// This path serves short, latency-bound problems (its measured case is one
// head of 256 keys), where a query-parallel grid alone leaves each wave a
// long chain of dependent key tiles. So the keys are split too: one
// workgroup of 8 waves per 16-row query block, wave w takes key tiles w,
// w + 8, w + 16, ... (16 keys each) with its own running max, sum and
// accumulator, and the 8 partial results are merged at the end with the
// online-softmax rule one level up (the merge of partial results over key
// ranges, "FlashAttention技术解析" section 4.2):
//   M = max_w m_w,  O = sum_w 2^(m_w - M) acc_w / sum_w 2^(m_w - M) l_w.
// Each wave loads its K and V tiles from global memory straight into the
// operand registers of the matrix instruction, one tile ahead, so the key
// loop needs no LDS and no barrier; LDS is used once, for the merge.
//
// Operand layouts (fragment layouts in fa_common.hpp): for S^T the lane with
// query column L and k-slot g takes head-dim entries g * D/4 .. g * D/4 +
// D/4 - 1, one per k-step, for both K and Q (any common order of the head
// dim contracts correctly); for O^T += V^T P^T, at the r-th 4-key step lane
// (L, g) holds P^T of key 4g + r, which is the instruction's k-slot g, so
// it supplies V[4g + r][16 db + L] as the A operand.
#include "fa_common.hpp"
#include "fa_launch.hpp"

namespace fa {

constexpr float kRescaleSlackF32 = 8.0f;

template <int D, bool CAUSAL>
__global__ __launch_bounds__(512, 1) void fa_fwd_f32_kernel(FwdParams p) {
  constexpr int NW = 8;      // waves per workgroup = key-range parts of one query block
  constexpr int BM = 16;     // query rows per workgroup
  constexpr int BN = 16;     // keys per tile
  constexpr int DS = D / 4;  // k-steps of S^T
  constexpr int DB = D / 16; // 16-row blocks of O^T
  constexpr int LDO = D + 4; // padded merge row (floats)
  __shared__ float sm_m[NW][BM];
  __shared__ float sm_l[NW][BM];
  __shared__ __attribute__((aligned(16))) float sm_o[NW][BM * LDO];

  const int N = p.N;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = uniform(tid >> 6);
  const int g = lane >> 4, L = lane & 15;

  const TileCoord tc = map_workgroup(workgroup_index(), p.B * p.Hq, p.n_tiles, CAUSAL);
  const int b = tc.head / p.Hq;
  const int h = tc.head - b * p.Hq;
  const int hk = h / (p.Hq / p.Hkv);
  const float* __restrict__ qg = (const float*)p.q + ((size_t)(b * p.Hq + h) * N) * D;
  const float* __restrict__ kg = (const float*)p.k + ((size_t)(b * p.Hkv + hk) * N) * D;
  const float* __restrict__ vg = (const float*)p.v + ((size_t)(b * p.Hkv + hk) * N) * D;
  float* __restrict__ og = (float*)p.o + ((size_t)(b * p.Hq + h) * N) * D;
  float* __restrict__ lseg = p.lse + (size_t)(b * p.Hq + h) * N;

  const int q0 = tc.tile * BM;
  const int kv_end = CAUSAL ? min(N, q0 + BM) : N;
  const int n_kv = (kv_end + BN - 1) / BN;  // key tiles with a visible key for the block

  // K and V operands of one tile, and the loads that fill them
  struct Tile {
    float k[DS];
    float v[4][DB];
  };
  auto load_tile = [&](int t, Tile& x) __attribute__((always_inline)) {
    const int krow = min(t * BN + L, N - 1);  // rows past the end: any valid row, masked below
    const f32x4* ks = (const f32x4*)(kg + (size_t)krow * D + g * DS);
#pragma unroll
    for (int j = 0; j < DS / 4; ++j) {
      const f32x4 v4 = ks[j];
      x.k[4 * j] = v4[0];
      x.k[4 * j + 1] = v4[1];
      x.k[4 * j + 2] = v4[2];
      x.k[4 * j + 3] = v4[3];
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int vrow = min(t * BN + 4 * g + r, N - 1);
#pragma unroll
      for (int db = 0; db < DB; ++db) x.v[r][db] = vg[(size_t)vrow * D + db * 16 + L];
    }
  };

  float qf[DS];
  {
    const int row = min(q0 + L, N - 1);
    const f32x4* qs = (const f32x4*)(qg + (size_t)row * D + g * DS);
#pragma unroll
    for (int j = 0; j < DS / 4; ++j) {
      const f32x4 v4 = qs[j];
      qf[4 * j] = v4[0];
      qf[4 * j + 1] = v4[1];
      qf[4 * j + 2] = v4[2];
      qf[4 * j + 3] = v4[3];
    }
  }
  f32x4 acc[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) acc[db] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_ref = kNegInf, l_part = 0.f;
  const float c = p.scale_log2;

  Tile cur, nxt;
  if (wave < n_kv) load_tile(wave, cur);
  for (int t = wave; t < n_kv; t += NW) {
    if (t + NW < n_kv) load_tile(t + NW, nxt);
    const int kv0 = t * BN;
    f32x4 s = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ds = 0; ds < DS; ++ds) s = mfma_f32_16x16x4(cur.k[ds], qf[ds], s);
    if ((kv0 + BN > N) || (CAUSAL && kv0 + BN - 1 > q0)) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int key = kv0 + 4 * g + r;
        const bool visible = key < N && (!CAUSAL || key <= q0 + L);
        s[r] = visible ? s[r] : kNegInf;
      }
    }
    const float tmax = fmaxf(fmaxf(s[0], s[1]), fmaxf(s[2], s[3])) * c;
    if (wave_any(tmax > m_ref + kRescaleSlackF32)) {
      const float m_new = fmaxf(m_ref, max_over_row_groups(tmax));
      const float alpha = (m_ref == kNegInf) ? 0.f : exp2_fast(m_ref - m_new);
      m_ref = m_new;
      l_part *= alpha;
#pragma unroll
      for (int db = 0; db < DB; ++db) acc[db] *= alpha;
    }
    // a row that has seen only masked keys keeps m = -inf; its exponentials are 2^-inf = 0
    const float neg_m = (m_ref == kNegInf) ? 0.f : -m_ref;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      s[r] = exp2_fast(fmaf(s[r], c, neg_m));
      l_part += s[r];
    }
#pragma unroll
    for (int r = 0; r < 4; ++r)
#pragma unroll
      for (int db = 0; db < DB; ++db) acc[db] = mfma_f32_16x16x4(cur.v[r][db], s[r], acc[db]);
    cur = nxt;
  }

  // ---- merge the NW partial results of each query row
  const float l_w = sum_over_row_groups(l_part);
  if (g == 0) {
    sm_m[wave][L] = m_ref;
    sm_l[wave][L] = l_w;
  }
#pragma unroll
  for (int db = 0; db < DB; ++db) *(f32x4*)(&sm_o[wave][L * LDO + db * 16 + 4 * g]) = acc[db];
  __syncthreads();
  constexpr int C4 = D / 4;  // 4-column groups per row
  for (int i = tid; i < BM * C4; i += NW * 64) {
    const int r = i / C4, c4 = i - r * C4;
    const int row = q0 + r;
    if (row >= N) continue;
    float M = kNegInf;
#pragma unroll
    for (int w = 0; w < NW; ++w) M = fmaxf(M, sm_m[w][r]);
    f32x4 o = f32x4{0.f, 0.f, 0.f, 0.f};
    float lsum = 0.f;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      const float mw = sm_m[w][r];
      const float wt = (mw == kNegInf) ? 0.f : exp2_fast(mw - M);  // parts without keys weigh 0
      lsum += wt * sm_l[w][r];
      o += wt * *(const f32x4*)(&sm_o[w][r * LDO + c4 * 4]);
    }
    *(f32x4*)(og + (size_t)row * D + c4 * 4) = o * (1.0f / lsum);
    if (c4 == 0) lseg[row] = (M + log2_fast(lsum)) * kLn2;
  }
}

template <int D, bool CAUSAL>
static hipError_t launch_fwd_f32_cfg(const FwdParams& p_in, hipStream_t stream) {
  FwdParams p = p_in;
  p.n_tiles = (p.N + 15) / 16;
  const unsigned grid = (unsigned)(p.n_tiles * p.B * p.Hq);
  hipLaunchKernelGGL((fa_fwd_f32_kernel<D, CAUSAL>), dim3(grid), dim3(512), 0, stream, p);
  return hipGetLastError();
}

hipError_t launch_fwd_f32(const FwdParams& p, int d, bool causal, hipStream_t stream) {
  if (d == 128) return causal ? launch_fwd_f32_cfg<128, true>(p, stream) : launch_fwd_f32_cfg<128, false>(p, stream);
  if (d == 64) return causal ? launch_fwd_f32_cfg<64, true>(p, stream) : launch_fwd_f32_cfg<64, false>(p, stream);
  return hipErrorInvalidValue;
}

}  // namespace fa

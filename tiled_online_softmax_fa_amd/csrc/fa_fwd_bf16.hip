// Forward attention, bf16 storage, fp32 softmax and accumulators (gfx950).
//
// What is computed: O = softmax(scale * Q K^T [causal mask]) V and the row
// logsumexp, per (batch, query head), as in the attention formula of
// "FlashAttention v2相比于v1有哪些更新" (blogweb.cn) section 1, by the tiled
// online softmax of "FlashAttention技术解析" (mhpq.cn) sections 2.1-2.2 with
// the division by the row sum deferred to the end of the key loop (blogweb.cn
// section 3, "Rescale操作").
//
// Work decomposition (blogweb.cn sections 4-5: parallel over query blocks,
// query block outer, key/value blocks inner; deepschool.ru "Flash Attention-2",
// work partitioning: each warp owns its own rows):
//   * one workgroup per (query tile of BM = NW * QPW rows, batch * head);
//   * each of the NW waves owns QPW consecutive query rows and never exchanges
//     partial results with another wave;
//   * K/V tiles of BN keys are copied global -> LDS with 16-byte direct loads
//     into a double buffer; the copy of tile j+1 is issued right after the
//     single barrier of iteration j and overlaps the math of tile j.
//
// Orientation. Each wave computes S^T = K Q^T (keys on the accumulator's rows,
// queries on its columns) with v_mfma_f32_16x16x32_bf16, so every lane owns
// one query column and holds 4 keys per 16x16 block: the row maximum is an
// in-lane reduction, and the probabilities P^T sit in registers in exactly the
// B-operand layout of O^T += V^T P^T (after a bf16 pack), so P never touches
// LDS. V^T fragments come from the row-major V tile through ds_read_b64_tr_b16.
// K and V tiles are stored with an XOR swizzle of 16-byte (K) and 32-byte (V)
// chunks against LDS bank conflicts (the padding idea of mhpq.cn section 5.2,
// done by permuting chunks instead of padding rows).
//
// Softmax bookkeeping, per query row, in the log2 domain (c = scale*log2 e):
//   m  = reference maximum used for the exponentials,
//   l  = per-lane partial sum of 2^(c s - m) (reduced over lanes at the end),
//   acc = sum of 2^(c s - m) v (unnormalised).
// A new tile only moves the reference maximum (and rescales l and acc by
// 2^(m_old - m_new), the correction of mhpq.cn section 2.2) when some score
// exceeds m + kRescaleSlack. Otherwise the old reference is kept: every
// exponential is then at most 2^kRescaleSlack, and because acc and l share
// the same reference the ratio acc / l, i.e. O, is the same number. The check
// is one compare per row and a wave vote, so the per-tile rescale of acc
// (64-128 multiplies per lane) is skipped on almost every tile.
//
// Causal (key j visible to query i iff j <= i): the key loop stops at the
// last key tile holding a visible key for the workgroup's last query (tiles
// wholly above the diagonal are never loaded, "Flash Attention V3技术解析"
// section 2.1), each wave skips tiles above its own rows, and the element mask
// is applied only on tiles that straddle the diagonal or the end of the
// sequence.
#include <type_traits>

#include "fa_common.hpp"
#include "fa_launch.hpp"

namespace fa {

constexpr float kRescaleSlack = 8.0f;  // log2 units: exponentials stay <= 256

template <int D>
struct KVSwizzle {
  static constexpr int kRowBytes = 2 * D;
  static constexpr int kChunks16 = kRowBytes / 16;        // 16-byte chunks per row
  static constexpr int kRowsPer256 = 256 / kRowBytes;     // rows sharing one 256-byte bank sweep
  // K: physical 16-byte chunk = logical chunk ^ k_swz(row)
  __device__ static __forceinline__ int k_swz(int row) { return (row / kRowsPer256) % kChunks16; }
  // V: physical 32-byte chunk = logical 32-byte chunk ^ v_swz(row)
  __device__ static __forceinline__ int v_swz(int row) { return (row / kRowsPer256) % (kChunks16 / 2); }
};

template <int D, int QPW, int NW, int BN, bool CAUSAL>
__global__ __launch_bounds__(NW * 64, 1) void fa_fwd_bf16_kernel(FwdParams p) {
  constexpr int BM = QPW * NW;
  constexpr int QB = QPW / 16;           // 16-query blocks per wave
  constexpr int DC = D / 32;             // k-steps of S^T = K Q^T
  constexpr int KC = BN / 32;            // 32-key chunks per tile (= k-steps of O^T += V^T P^T)
  constexpr int DB = D / 16;             // 16-row blocks of O^T
  constexpr int TILE_BYTES = BN * D * 2;
  constexpr int COPIES = TILE_BYTES / 1024;       // 1 KiB (64 lanes x 16 B) per copy instruction
  constexpr int COPIES_PER_WAVE = COPIES / NW;
  constexpr int ROWS_PER_COPY = 1024 / (2 * D);
  constexpr int CH = 2 * D / 16;
  using Swz = KVSwizzle<D>;
  static_assert(QPW % 16 == 0 && BN % 32 == 0 && D % 32 == 0, "tile shape");
  static_assert(COPIES % NW == 0, "K/V copy must split evenly over the waves");

  // Two stages of (K, V). Four distinct arrays (not one indexed buffer) let
  // the compiler see that the copy into one stage never aliases the reads of
  // the other, so it does not wait for the in-flight copy before reading.
  __shared__ __attribute__((aligned(1024))) unsigned char k_stage0[TILE_BYTES];
  __shared__ __attribute__((aligned(1024))) unsigned char v_stage0[TILE_BYTES];
  __shared__ __attribute__((aligned(1024))) unsigned char k_stage1[TILE_BYTES];
  __shared__ __attribute__((aligned(1024))) unsigned char v_stage1[TILE_BYTES];

  const int N = p.N;
  const int lane = threadIdx.x & 63;
  const int wave = uniform(threadIdx.x >> 6);
  const int g = lane >> 4;   // row group of an accumulator block
  const int L = lane & 15;   // column of an accumulator block (this lane's query)

  const TileCoord tc = map_workgroup(blockIdx.x, p.B * p.Hq, p.n_tiles, CAUSAL);
  const int b = tc.head / p.Hq;
  const int h = tc.head - b * p.Hq;
  const int hk = h / (p.Hq / p.Hkv);
  const __bf16* __restrict__ qg = (const __bf16*)p.q + ((size_t)(b * p.Hq + h) * N) * D;
  const __bf16* __restrict__ kg = (const __bf16*)p.k + ((size_t)(b * p.Hkv + hk) * N) * D;
  const __bf16* __restrict__ vg = (const __bf16*)p.v + ((size_t)(b * p.Hkv + hk) * N) * D;
  __bf16* __restrict__ og = (__bf16*)p.o + ((size_t)(b * p.Hq + h) * N) * D;
  float* __restrict__ lseg = p.lse + (size_t)(b * p.Hq + h) * N;

  const int q0 = tc.tile * BM;
  const int qw0 = q0 + wave * QPW;  // first query row of this wave
  const int qw_last = qw0 + QPW - 1;
  const int kv_end = CAUSAL ? min(N, q0 + BM) : N;
  const int n_kv = (kv_end + BN - 1) / BN;
  const int n_kv_wave = (qw0 < N) ? ((CAUSAL ? min(N, qw0 + QPW) : N) + BN - 1) / BN : 0;

  // Copy K/V tile `t`: this wave's COPIES_PER_WAVE pieces of 1 KiB each.
  auto issue_tile_copy = [&](int t, lds_u8* kdst, lds_u8* vdst) __attribute__((always_inline)) {
    const int kv0 = t * BN;
#pragma unroll
    for (int c = 0; c < COPIES_PER_WAVE; ++c) {
      const int piece = wave * COPIES_PER_WAVE + c;
      const int prow = piece * ROWS_PER_COPY + lane / CH;  // physical row in the tile
      const int pch = lane % CH;                            // physical 16-byte chunk
      const int grow = min(kv0 + prow, N - 1);              // rows past the end: any valid row, masked later
      const int kch = pch ^ Swz::k_swz(prow);
      const int vch = (((pch >> 1) ^ Swz::v_swz(prow)) << 1) | (pch & 1);
      copy16_global_to_lds(kg + (size_t)grow * D + kch * 8, kdst + piece * 1024);
      copy16_global_to_lds(vg + (size_t)grow * D + vch * 8, vdst + piece * 1024);
    }
  };

  if (n_kv > 0) issue_tile_copy(0, (lds_u8*)k_stage0, (lds_u8*)v_stage0);

  // Q^T fragments (B operand of S^T = K Q^T), held for the whole key loop.
  bf16x8 qf[QB][DC];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const int row = min(qw0 + qb * 16 + L, N - 1);
    const u32x4* src = (const u32x4*)(qg + (size_t)row * D + g * 8);
#pragma unroll
    for (int dc = 0; dc < DC; ++dc) qf[qb][dc] = __builtin_bit_cast(bf16x8, src[dc * 4]);
  }

  f32x4 acc[DB][QB];
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) acc[db][qb] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_ref[QB], l_part[QB];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    m_ref[qb] = kNegInf;
    l_part[qb] = 0.f;
  }
  const float c = p.scale_log2;

  // One 32-key chunk of tile t: S^T, mask, online softmax, O^T += V^T P^T.
  auto chunk = [&](const lds_u8* kt, const lds_u8* vt, int kv0, int kc) __attribute__((always_inline)) {
    const int key0 = kv0 + kc * 32;
    if (CAUSAL && key0 > qw_last) return;  // chunk wholly above this wave's rows

    // ---- S^T for the two 16-key blocks of the chunk
    f32x4 s[2][QB];
#pragma unroll
    for (int hb = 0; hb < 2; ++hb) {
      const int row = kc * 32 + hb * 16 + L;
      bf16x8 kf[DC];
#pragma unroll
      for (int dc = 0; dc < DC; ++dc) {
        const int ch = (dc * 4 + g) ^ Swz::k_swz(row);
        kf[dc] = lds_read_b128(kt + row * (2 * D) + ch * 16);
      }
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) s[hb][qb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int dc = 0; dc < DC; ++dc)
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) s[hb][qb] = mfma_bf16_16x16x32(kf[dc], qf[qb][dc], s[hb][qb]);
    }

    // ---- mask: only chunks crossing the diagonal or the sequence end
    if ((key0 + 32 > N) || (CAUSAL && key0 + 31 > qw0)) {
#pragma unroll
      for (int hb = 0; hb < 2; ++hb)
#pragma unroll
        for (int qb = 0; qb < QB; ++qb)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int key = key0 + hb * 16 + g * 4 + r;
            const int qi = qw0 + qb * 16 + L;
            const bool visible = key < N && (!CAUSAL || key <= qi);
            s[hb][qb][r] = visible ? s[hb][qb][r] : kNegInf;
          }
    }

    // ---- online softmax: move the reference maximum only when needed
    float tmax[QB];
    bool grow = false;
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      float mx = fmaxf(fmaxf(s[0][qb][0], s[0][qb][1]), fmaxf(s[0][qb][2], s[0][qb][3]));
      mx = fmaxf(mx, fmaxf(fmaxf(s[1][qb][0], s[1][qb][1]), fmaxf(s[1][qb][2], s[1][qb][3])));
      tmax[qb] = mx * c;
      grow |= tmax[qb] > m_ref[qb] + kRescaleSlack;
    }
    if (wave_any(grow)) {
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) {
        const float m_new = fmaxf(m_ref[qb], max_over_row_groups(tmax[qb]));
        const float alpha = (m_ref[qb] == kNegInf) ? 0.f : exp2_fast(m_ref[qb] - m_new);
        m_ref[qb] = m_new;
        l_part[qb] *= alpha;
#pragma unroll
        for (int db = 0; db < DB; ++db) acc[db][qb] *= alpha;
      }
    }

    // ---- P^T = 2^(c S^T - m) packed to bf16 in the B-operand layout of O^T += V^T P^T:
    // element e < 4 -> key key0 + 4g + e, element e >= 4 -> key key0 + 16 + 4g + e - 4.
    bf16x8 pf[QB];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      const float neg_m = -m_ref[qb];
      float e[8];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        e[r] = exp2_fast(fmaf(s[0][qb][r], c, neg_m));
        e[4 + r] = exp2_fast(fmaf(s[1][qb][r], c, neg_m));
      }
      l_part[qb] += ((e[0] + e[1]) + (e[2] + e[3])) + ((e[4] + e[5]) + (e[6] + e[7]));
      u32x4 packed = {pack_bf16x2(e[0], e[1]), pack_bf16x2(e[2], e[3]), pack_bf16x2(e[4], e[5]),
                      pack_bf16x2(e[6], e[7])};
      pf[qb] = __builtin_bit_cast(bf16x8, packed);
    }

    // ---- O^T += V^T P^T; A operand rows d = 16db + (lane % 16), keys ordered as in pf
    const int vrow0 = kc * 32 + 4 * g + (L >> 2);
    const int vrow1 = vrow0 + 16;
    const int within = 8 * (L & 3);
#pragma unroll
    for (int db = 0; db < DB; ++db) {
      const i16x4 lo = lds_read_tr16_b64(vt + vrow0 * (2 * D) + ((db ^ Swz::v_swz(vrow0)) * 32) + within);
      const i16x4 hi = lds_read_tr16_b64(vt + vrow1 * (2 * D) + ((db ^ Swz::v_swz(vrow1)) * 32) + within);
      const bf16x8 vf = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) acc[db][qb] = mfma_bf16_16x16x32(vf, pf[qb], acc[db][qb]);
    }
  };

  // One key tile: one barrier, prefetch of the next tile into the other stage, math.
  auto tile = [&](auto stage, int t) __attribute__((always_inline)) {
    constexpr int S = decltype(stage)::value;
    lds_u8* kcur = (lds_u8*)(S == 0 ? k_stage0 : k_stage1);
    lds_u8* vcur = (lds_u8*)(S == 0 ? v_stage0 : v_stage1);
    lds_u8* knext = (lds_u8*)(S == 0 ? k_stage1 : k_stage0);
    lds_u8* vnext = (lds_u8*)(S == 0 ? v_stage1 : v_stage0);
    wait_vmcnt0();     // this wave's copies of tile t have landed
    __syncthreads();   // ... and every other wave's; all reads of tile t-1 are done
    if (t + 1 < n_kv) issue_tile_copy(t + 1, knext, vnext);
    if (t >= n_kv_wave) return;  // tile lies wholly above this wave's rows
#pragma unroll
    for (int kc = 0; kc < KC; ++kc) chunk(kcur, vcur, t * BN, kc);
  };

  for (int t = 0; t < n_kv; t += 2) {
    tile(std::integral_constant<int, 0>{}, t);
    if (t + 1 < n_kv) tile(std::integral_constant<int, 1>{}, t + 1);
  }

  // ---- epilogue: O = acc / l, lse = (m + log2 l) ln 2
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const float l = sum_over_row_groups(l_part[qb]);
    const int row = qw0 + qb * 16 + L;
    if (row < N) {
      const float inv = 1.0f / l;
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        const f32x4 o4 = acc[db][qb] * inv;
        u32x2 packed = {pack_bf16x2(o4[0], o4[1]), pack_bf16x2(o4[2], o4[3])};
        *(u32x2*)(og + (size_t)row * D + db * 16 + g * 4) = packed;
      }
      if (g == 0) lseg[row] = (m_ref[qb] + log2_fast(l)) * kLn2;
    }
  }
}

// ------------------------------------------------------------------ launch
template <int D, int QPW, int NW, int BN, bool CAUSAL>
static hipError_t launch_fwd_bf16_cfg(const FwdParams& p_in, hipStream_t stream) {
  constexpr int BM = QPW * NW;
  FwdParams p = p_in;
  p.n_tiles = (p.N + BM - 1) / BM;
  const unsigned grid = (unsigned)(p.n_tiles * p.B * p.Hq);
  hipLaunchKernelGGL((fa_fwd_bf16_kernel<D, QPW, NW, BN, CAUSAL>), dim3(grid), dim3(NW * 64), 0, stream, p);
  return hipGetLastError();
}

hipError_t launch_fwd_bf16(const FwdParams& p, int d, bool causal, hipStream_t stream) {
  if (d == 128) {
    return causal ? launch_fwd_bf16_cfg<128, 64, 4, 64, true>(p, stream)
                  : launch_fwd_bf16_cfg<128, 64, 4, 64, false>(p, stream);
  }
  if (d == 64) {
    return causal ? launch_fwd_bf16_cfg<64, 64, 4, 64, true>(p, stream)
                  : launch_fwd_bf16_cfg<64, 64, 4, 64, false>(p, stream);
  }
  return hipErrorInvalidValue;
}

}  // namespace fa

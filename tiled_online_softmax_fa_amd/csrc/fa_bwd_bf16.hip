// Backward attention, bf16 storage, fp32 arithmetic (gfx950).
//
// The probabilities are recomputed from the row logsumexp stored by the
// forward pass instead of being kept (the recomputation strategy of the page
// "4.3 FlashAttention-2与FlashAttention-3演进", FlashAttention-3 section 3).
// The pages give no formulas for the gradients; these follow from
// differentiating O = softmax(scale * Q K^T) V, per (batch, query head):
//   P = exp(scale * Q K^T - lse),  dV = P^T dO,  dP = dO V^T,
//   D_i = sum_c dO_ic O_ic,  dS = P o (dP - D),
//   dQ = scale * dS K,  dK = scale * dS^T Q.
// Grouped heads: the dK and dV of a key/value head sum over its query heads.
//
// Three kernels on the caller's stream:
//   1. row term D (fp32) and zeroing of the fp32 dQ accumulator;
//   2. one workgroup per (key tile of 128 keys, batch * key/value head): K, V
//      of the tile stay in registers, each of the 4 waves owns 32 keys and
//      accumulates their dK^T, dV^T; query tiles of 64 rows (Q, dO) stream
//      through LDS (the tiled backward of the page "Flash Attention-2"
//      (deepschool.ru), "Улучшение backward pass", and blogweb.cn section 5).
//      S = Q K^T is computed with keys on the accumulator's columns, so P and
//      dS come out of the MFMA in the B-operand layout of dV^T += dO^T P and
//      dK^T += Q^T dS, whose dO^T / Q^T fragments are transposing LDS reads.
//      dQ needs the contraction over keys, so dS goes through LDS once and
//      dQ += dS K is added to the fp32 accumulator with atomic adds (the dQ
//      atomics of "Flash Attention V3技术解析" section 2.1);
//   3. dQ = bf16(scale * accumulator).
#include "fa_common.hpp"
#include "fa_launch.hpp"

namespace fa {

// ------------------------------------------------------------------ kernel 1: D and zeroed dQ accumulator
// 16 lanes per row, 16 rows per workgroup of 256 threads.
template <int D>
__global__ __launch_bounds__(256) void fa_bwd_pre_kernel(const __bf16* __restrict__ o, const __bf16* __restrict__ dout,
                                                         float* __restrict__ delta, float* __restrict__ dq_acc,
                                                         long long rows) {
  constexpr int PER_LANE = D / 16;  // 8 (d=128) or 4 (d=64) elements
  const long long row = (long long)blockIdx.x * 16 + (threadIdx.x >> 4);
  const int sub = threadIdx.x & 15;
  float s = 0.f;
  if (row < rows) {
    const __bf16* po = o + row * D + sub * PER_LANE;
    const __bf16* pd = dout + row * D + sub * PER_LANE;
#pragma unroll
    for (int i = 0; i < PER_LANE; ++i) s = fmaf((float)po[i], (float)pd[i], s);
    float* z = dq_acc + row * D + sub * PER_LANE;
#pragma unroll
    for (int i = 0; i < PER_LANE; i += 4) *(f32x4*)(z + i) = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  s += __shfl_xor(s, 8, 16);
  s += __shfl_xor(s, 4, 16);
  s += __shfl_xor(s, 2, 16);
  s += __shfl_xor(s, 1, 16);
  if (row < rows && sub == 0) delta[row] = s;
}

// ------------------------------------------------------------------ kernel 3: dQ = bf16(scale * acc)
__global__ __launch_bounds__(256) void fa_bwd_dq_convert_kernel(const float* __restrict__ acc, __bf16* __restrict__ dq,
                                                                float scale, long long n4) {
  const long long i = (long long)blockIdx.x * 256 + threadIdx.x;
  if (i >= n4) return;
  const f32x4 a = ((const f32x4*)acc)[i] * scale;
  u32x2 packed = {pack_bf16x2(a[0], a[1]), pack_bf16x2(a[2], a[3])};
  ((u32x2*)dq)[i] = packed;
}

// ------------------------------------------------------------------ kernel 2: main
template <int D>
struct TileSwizzle {  // 16-byte chunk XOR swizzle of a row-major [rows][D] bf16 tile
  static constexpr int kRowBytes = 2 * D;
  static constexpr int kChunks16 = kRowBytes / 16;
  static constexpr int kRowsPer256 = 256 / kRowBytes;
  __device__ static __forceinline__ int swz(int row) { return (row / kRowsPer256) % kChunks16; }
  // byte offset of element (row, col) for an 8-byte aligned col group
  __device__ static __forceinline__ int offset(int row, int col) {
    const int chunk = (col >> 3) ^ swz(row);
    return row * kRowBytes + chunk * 16 + (col & 7) * 2;
  }
};

template <int D, bool CAUSAL>
__global__ __launch_bounds__(256, 1) void fa_bwd_main_kernel(BwdParams p) {
  constexpr int NW = 4, KPW = 32, BNK = NW * KPW;  // 128 keys per workgroup
  constexpr int BMQ = 64;                          // query rows per step
  constexpr int QB = BMQ / 16, KB = KPW / 16, QC = BMQ / 32, KC = BNK / 32;
  constexpr int DC = D / 32, DB = D / 16;
  constexpr int QTILE_BYTES = BMQ * D * 2;
  constexpr int COPIES_PER_WAVE = QTILE_BYTES / 1024 / NW;
  constexpr int ROWS_PER_COPY = 1024 / (2 * D);
  constexpr int CH = 2 * D / 16;
  constexpr int DST_ROW_BYTES = BMQ * 2;  // dS^T tile row: 64 queries
  using Swz = TileSwizzle<D>;
  static_assert(COPIES_PER_WAVE >= 1, "tile copy split");

  __shared__ __attribute__((aligned(1024))) unsigned char q_stage0[QTILE_BYTES];
  __shared__ __attribute__((aligned(1024))) unsigned char do_stage0[QTILE_BYTES];
  __shared__ __attribute__((aligned(1024))) unsigned char q_stage1[QTILE_BYTES];
  __shared__ __attribute__((aligned(1024))) unsigned char do_stage1[QTILE_BYTES];
  __shared__ __attribute__((aligned(1024))) unsigned char k_tile[BNK * D * 2];
  __shared__ __attribute__((aligned(1024))) unsigned char dst_tile[BNK * DST_ROW_BYTES];

  const int N = p.N;
  const int lane = threadIdx.x & 63;
  const int wave = uniform(threadIdx.x >> 6);
  const int g = lane >> 4, L = lane & 15;
  const int G = p.Hq / p.Hkv;

  const TileCoord tc = map_workgroup(blockIdx.x, p.B * p.Hkv, p.n_tiles, false);  // low key tiles (most work) first
  const int b = tc.head / p.Hkv;
  const int hk = tc.head - b * p.Hkv;
  const int kv0 = tc.tile * BNK;
  const int kw0 = kv0 + wave * KPW;  // this wave's first key
  const size_t kv_head = (size_t)(b * p.Hkv + hk) * N;
  const __bf16* __restrict__ kg = (const __bf16*)p.k + kv_head * D;
  const __bf16* __restrict__ vg = (const __bf16*)p.v + kv_head * D;

  // K tile (all 128 keys) into LDS for dQ += dS K; K^T, V^T fragments of this
  // wave's keys into registers (B operands of S = Q K^T and dP = dO V^T).
  for (int i = threadIdx.x; i < BNK * D / 8; i += NW * 64) {
    const int row = i / (D / 8), c8 = i % (D / 8);
    const int grow = min(kv0 + row, N - 1);
    *(FA_LDS u32x4*)((lds_u8*)k_tile + Swz::offset(row, c8 * 8)) = *(const u32x4*)(kg + (size_t)grow * D + c8 * 8);
  }
  bf16x8 kf[KB][DC], vf[KB][DC];
#pragma unroll
  for (int kb = 0; kb < KB; ++kb) {
    const int row = min(kw0 + kb * 16 + L, N - 1);
#pragma unroll
    for (int dc = 0; dc < DC; ++dc) {
      kf[kb][dc] = __builtin_bit_cast(bf16x8, *(const u32x4*)(kg + (size_t)row * D + dc * 32 + g * 8));
      vf[kb][dc] = __builtin_bit_cast(bf16x8, *(const u32x4*)(vg + (size_t)row * D + dc * 32 + g * 8));
    }
  }

  f32x4 dv_acc[DB][KB], dk_acc[DB][KB];
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
      dv_acc[db][kb] = f32x4{0.f, 0.f, 0.f, 0.f};
      dk_acc[db][kb] = f32x4{0.f, 0.f, 0.f, 0.f};
    }

  const int nq = (N + BMQ - 1) / BMQ;
  const int i_begin = CAUSAL ? (kv0 / BMQ) : 0;  // first query tile with a visible key
  const int steps_per_head = nq - i_begin;
  const int n_steps = steps_per_head * G;
  const float c = p.scale_log2;
  constexpr float kLog2e = 1.4426950408889634f;

  auto step_coords = [&](int s, int& h, int& i) __attribute__((always_inline)) {
    const int gi = s / steps_per_head;
    h = hk * G + gi;
    i = i_begin + (s - gi * steps_per_head);
  };
  auto issue_copy = [&](int s, lds_u8* qdst, lds_u8* ddst) __attribute__((always_inline)) {
    int h, i;
    step_coords(s, h, i);
    const size_t qh = (size_t)(b * p.Hq + h) * N;
    const __bf16* qsrc = (const __bf16*)p.q + qh * D;
    const __bf16* dsrc = (const __bf16*)p.dout + qh * D;
#pragma unroll
    for (int cp = 0; cp < COPIES_PER_WAVE; ++cp) {
      const int piece = wave * COPIES_PER_WAVE + cp;
      const int prow = piece * ROWS_PER_COPY + lane / CH;
      const int pch = lane % CH;
      const int grow = min(i * BMQ + prow, N - 1);
      const int lch = pch ^ Swz::swz(prow);
      copy16_global_to_lds(qsrc + (size_t)grow * D + lch * 8, qdst + piece * 1024);
      copy16_global_to_lds(dsrc + (size_t)grow * D + lch * 8, ddst + piece * 1024);
    }
  };

  auto step = [&](auto stage, int s) __attribute__((always_inline)) {
    constexpr int ST = decltype(stage)::value;
    lds_u8* qt = (lds_u8*)(ST == 0 ? q_stage0 : q_stage1);
    lds_u8* dt = (lds_u8*)(ST == 0 ? do_stage0 : do_stage1);
    wait_vmcnt0();
    __syncthreads();  // tile s landed; dS^T of step s-1 fully consumed
    if (s + 1 < n_steps) issue_copy(s + 1, (lds_u8*)(ST == 0 ? q_stage1 : q_stage0),
                                    (lds_u8*)(ST == 0 ? do_stage1 : do_stage0));
    int h, i;
    step_coords(s, h, i);
    const int q0 = i * BMQ;
    const size_t qh = (size_t)(b * p.Hq + h) * N;

    // ---- S = Q K^T and dP = dO V^T: blocks of 16 queries x 16 keys (keys on columns)
    f32x4 sacc[QB][KB], pacc[QB][KB];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb)
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) {
        sacc[qb][kb] = f32x4{0.f, 0.f, 0.f, 0.f};
        pacc[qb][kb] = f32x4{0.f, 0.f, 0.f, 0.f};
      }
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      const int row = qb * 16 + L;
#pragma unroll
      for (int dc = 0; dc < DC; ++dc) {
        const int off = Swz::offset(row, dc * 32 + g * 8);
        const bf16x8 qa = lds_read_b128(qt + off);
        const bf16x8 da = lds_read_b128(dt + off);
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) {
          sacc[qb][kb] = mfma_bf16_16x16x32(qa, kf[kb][dc], sacc[qb][kb]);
          pacc[qb][kb] = mfma_bf16_16x16x32(da, vf[kb][dc], pacc[qb][kb]);
        }
      }
    }

    // ---- P = 2^(c S - lse log2 e) (0 where masked), dS = P (dP - D)
    const bool need_mask = (q0 + BMQ > N) || (kw0 + KPW > N) || (CAUSAL && kw0 + KPW - 1 > q0);
    bf16x8 pfr[QC][KB], dsfr[QC][KB];
#pragma unroll
    for (int qc = 0; qc < QC; ++qc) {
      u32x2 pp[2][KB], dd[2][KB];
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        const int qb = 2 * qc + half;
        const int qrow = q0 + qb * 16 + 4 * g;  // this lane's queries: qrow + r, r = 0..3
        float lse2[4], dl[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int qq = min(qrow + r, N - 1);
          lse2[r] = p.lse[qh + qq] * kLog2e;
          dl[r] = p.delta[qh + qq];
        }
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) {
          float pv[4], dsv[4];
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            float pr = exp2_fast(fmaf(sacc[qb][kb][r], c, -lse2[r]));
            if (need_mask) {
              const int key = kw0 + kb * 16 + L, qi = qrow + r;
              const bool visible = key < N && qi < N && (!CAUSAL || key <= qi);
              pr = visible ? pr : 0.f;
            }
            pv[r] = pr;
            dsv[r] = pr * (pacc[qb][kb][r] - dl[r]);
          }
          pp[half][kb] = u32x2{pack_bf16x2(pv[0], pv[1]), pack_bf16x2(pv[2], pv[3])};
          dd[half][kb] = u32x2{pack_bf16x2(dsv[0], dsv[1]), pack_bf16x2(dsv[2], dsv[3])};
          // dS^T tile for dQ: row = key within the workgroup tile, 4 consecutive queries
          *(FA_LDS u32x2*)((lds_u8*)dst_tile + (wave * KPW + kb * 16 + L) * DST_ROW_BYTES + (qb * 16 + 4 * g) * 2) =
              dd[half][kb];
        }
      }
      // B-operand packing: elements 0..3 <- query block 2qc (rows 4g + e), 4..7 <- block 2qc + 1
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) {
        pfr[qc][kb] = __builtin_bit_cast(bf16x8, u32x4{pp[0][kb][0], pp[0][kb][1], pp[1][kb][0], pp[1][kb][1]});
        dsfr[qc][kb] = __builtin_bit_cast(bf16x8, u32x4{dd[0][kb][0], dd[0][kb][1], dd[1][kb][0], dd[1][kb][1]});
      }
    }

    // ---- dV^T += dO^T P, dK^T += Q^T dS (A operands: transposing reads of the dO / Q tiles)
#pragma unroll
    for (int qc = 0; qc < QC; ++qc) {
      const int r0 = qc * 32 + 4 * g + (L >> 2), r1 = r0 + 16;
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        const int col = db * 16 + 4 * (L & 3);
        const i16x4 d_lo = lds_read_tr16_b64(dt + Swz::offset(r0, col));
        const i16x4 d_hi = lds_read_tr16_b64(dt + Swz::offset(r1, col));
        const i16x4 q_lo = lds_read_tr16_b64(qt + Swz::offset(r0, col));
        const i16x4 q_hi = lds_read_tr16_b64(qt + Swz::offset(r1, col));
        const bf16x8 dTa = __builtin_bit_cast(bf16x8, __builtin_shufflevector(d_lo, d_hi, 0, 1, 2, 3, 4, 5, 6, 7));
        const bf16x8 qTa = __builtin_bit_cast(bf16x8, __builtin_shufflevector(q_lo, q_hi, 0, 1, 2, 3, 4, 5, 6, 7));
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) {
          dv_acc[db][kb] = mfma_bf16_16x16x32(dTa, pfr[qc][kb], dv_acc[db][kb]);
          dk_acc[db][kb] = mfma_bf16_16x16x32(qTa, dsfr[qc][kb], dk_acc[db][kb]);
        }
      }
    }

    __syncthreads();  // dS^T complete

    // ---- dQ[q, d] += sum over the tile's keys of dS[q, key] K[key, d]; wave w owns d-blocks {2w, 2w+1} (d=128)
    constexpr int DBW = DB / NW;  // d-blocks per wave
    f32x4 dq[QB][DBW];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb)
#pragma unroll
      for (int j = 0; j < DBW; ++j) dq[qb][j] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kc = 0; kc < KC; ++kc) {
      const int r0 = kc * 32 + 4 * g + (L >> 2), r1 = r0 + 16;
      bf16x8 kB[DBW];
#pragma unroll
      for (int j = 0; j < DBW; ++j) {
        const int col = (wave * DBW + j) * 16 + 4 * (L & 3);
        const i16x4 lo = lds_read_tr16_b64((lds_u8*)k_tile + Swz::offset(r0, col));
        const i16x4 hi = lds_read_tr16_b64((lds_u8*)k_tile + Swz::offset(r1, col));
        kB[j] = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
      }
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) {
        const int col = qb * 16 + 4 * (L & 3);
        const i16x4 lo = lds_read_tr16_b64((lds_u8*)dst_tile + r0 * DST_ROW_BYTES + col * 2);
        const i16x4 hi = lds_read_tr16_b64((lds_u8*)dst_tile + r1 * DST_ROW_BYTES + col * 2);
        const bf16x8 sA = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
#pragma unroll
        for (int j = 0; j < DBW; ++j) dq[qb][j] = mfma_bf16_16x16x32(sA, kB[j], dq[qb][j]);
      }
    }
    float* dqa = p.dq_acc + qh * D;
#pragma unroll
    for (int qb = 0; qb < QB; ++qb)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int qi = q0 + qb * 16 + 4 * g + r;
        if (qi < N) {
#pragma unroll
          for (int j = 0; j < DBW; ++j)
            unsafeAtomicAdd(dqa + (size_t)qi * D + (wave * DBW + j) * 16 + L, dq[qb][j][r]);
        }
      }
  };

  if (n_steps > 0) issue_copy(0, (lds_u8*)q_stage0, (lds_u8*)do_stage0);
  for (int s = 0; s < n_steps; s += 2) {
    step(std::integral_constant<int, 0>{}, s);
    if (s + 1 < n_steps) step(std::integral_constant<int, 1>{}, s + 1);
  }

  // ---- dK = scale * dK^T acc, dV = dV^T acc (lane: key column, rows d = 16db + 4g + r)
  __bf16* dkg = (__bf16*)p.dk + kv_head * D;
  __bf16* dvg = (__bf16*)p.dv + kv_head * D;
#pragma unroll
  for (int kb = 0; kb < KB; ++kb) {
    const int key = kw0 + kb * 16 + L;
    if (key < N) {
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        const f32x4 k4 = dk_acc[db][kb] * p.scale;
        const f32x4 v4 = dv_acc[db][kb];
        u32x2 kp = {pack_bf16x2(k4[0], k4[1]), pack_bf16x2(k4[2], k4[3])};
        u32x2 vp = {pack_bf16x2(v4[0], v4[1]), pack_bf16x2(v4[2], v4[3])};
        *(u32x2*)(dkg + (size_t)key * D + db * 16 + 4 * g) = kp;
        *(u32x2*)(dvg + (size_t)key * D + db * 16 + 4 * g) = vp;
      }
    }
  }
}

// ------------------------------------------------------------------ launch
template <int D, bool CAUSAL>
static hipError_t launch_bwd_cfg(const BwdParams& p_in, hipStream_t stream, hipEvent_t* ev) {
  BwdParams p = p_in;
  const long long rows = (long long)p.B * p.Hq * p.N;
  hipError_t e;
  if (ev && (e = hipEventRecord(ev[0], stream)) != hipSuccess) return e;
  hipLaunchKernelGGL((fa_bwd_pre_kernel<D>), dim3((unsigned)((rows + 15) / 16)), dim3(256), 0, stream,
                     (const __bf16*)p.o, (const __bf16*)p.dout, p.delta, p.dq_acc, rows);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  if (ev && (e = hipEventRecord(ev[1], stream)) != hipSuccess) return e;
  p.n_tiles = (p.N + 127) / 128;
  hipLaunchKernelGGL((fa_bwd_main_kernel<D, CAUSAL>), dim3((unsigned)(p.n_tiles * p.B * p.Hkv)), dim3(256), 0, stream,
                     p);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  if (ev && (e = hipEventRecord(ev[2], stream)) != hipSuccess) return e;
  const long long n4 = rows * D / 4;
  hipLaunchKernelGGL(fa_bwd_dq_convert_kernel, dim3((unsigned)((n4 + 255) / 256)), dim3(256), 0, stream, p.dq_acc,
                     (__bf16*)p.dq, p.scale, n4);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  if (ev && (e = hipEventRecord(ev[3], stream)) != hipSuccess) return e;
  return hipSuccess;
}

hipError_t launch_bwd_bf16(const BwdParams& p, int d, bool causal, hipStream_t stream, hipEvent_t* ev) {
  if (d == 128) return causal ? launch_bwd_cfg<128, true>(p, stream, ev) : launch_bwd_cfg<128, false>(p, stream, ev);
  if (d == 64) return causal ? launch_bwd_cfg<64, true>(p, stream, ev) : launch_bwd_cfg<64, false>(p, stream, ev);
  return hipErrorInvalidValue;
}

}  // namespace fa

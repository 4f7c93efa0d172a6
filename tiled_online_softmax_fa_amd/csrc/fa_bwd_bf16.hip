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
// Two kernels on the caller's stream, in this order:
//   1. dQ: one workgroup per (query tile, batch * query head), built like the
//      forward kernel: Q and dO stay in registers and K, V tiles stream
//      through an LDS ring; per 32-key chunk it recomputes S^T and dP^T and
//      accumulates dQ^T += K^T dS^T. Its prologue also forms the row term D
//      of its rows (fp32) and writes -D, with lse in log2 units, for kernel 2. Recomputing S and dP
//      here costs two more matrix products per tile than accumulating dQ
//      inside kernel 2, but kernel 2 would have to add every key tile's
//      contribution to dQ in memory (the atomics of "Flash Attention V3技术
//      解析" section 2.1); the separate pass needs no atomics, no fp32
//      accumulator, and gives a bitwise repeatable dQ;
//   2. dK, dV: one workgroup per (key tile of 128 keys, batch * key/value
//      head); query tiles of 64 rows (Q, dO, lse, D) stream through LDS (the
//      tiled backward of the page "Flash Attention-2" (deepschool.ru),
//      "Улучшение backward pass", and blogweb.cn section 5). Two waves per
//      32-key slice split the work: one computes P and dV, the other dP, dS
//      and dK (details at the kernel).
#include <mutex>

#include "fa.h"
#include "fa_common.hpp"
#include "fa_launch.hpp"

namespace fa {

// ------------------------------------------------------------------ LDS layout shared by both kernels
//
// Tiles here are read both row-wise (16-byte reads of one row's chunk, by the
// 16 lanes of a lane group: rows 0..15) and transposed (ds_read_b64_tr_b16:
// rows 4g..4g+3 of lane group g, 32 bytes per row), so the 16-byte chunk c
// of row r is stored at chunk c ^ f(r). Measured on gfx950 (LDS bank-conflict
// counter over masks that satisfy one rule or the other): the 16-byte reads
// are served 8 lanes at a time from 128 bytes, the transposing reads 32 lanes
// at a time from 256 bytes. So over any 8 consecutive rows, bits 0-2 of f
// must differ (row-wise: 8 chunks in distinct 16-byte slots of 128 bytes) and
// bits 1-3 must differ (transposed: 8 rows of two adjacent chunks, pair index
// c/2 ^ f(r)/2, in distinct 32-byte slots of 256 bytes).
// f(r) = (r mod 8) + 8 (r mod 2) does both; at d = 64 (8 chunks per
// 128-byte row, two rows per 256 bytes, so the row's half is fixed by
// r mod 2) f(r) = r mod 8 does. f < 16 only permutes chunks inside one
// 256-byte sweep, so with 512-byte rows (d = 256) chunk c + 16 sits 256 bytes
// after chunk c: the fragment offsets of the second half of a row are those of
// the first plus 256 (r_half, t_half below), a constant. f repeats every 8 rows, as
// the fragment reads add whole 16-row blocks.
template <int D>
struct DualSwizzle {
  static constexpr int kRowBytes = 2 * D;
  static constexpr int kChunks = kRowBytes / 16;
  __device__ static __forceinline__ int f(int row) {
    return kChunks >= 16 ? ((row & 7) | ((row & 1) << 3)) : (row & 7);
  }
  // lane offsets kept per 32-column step (row-wise reads) and per 16-column
  // block (transposed reads) within one 256-byte half row
  static constexpr int kDC = D / 32 < 4 ? D / 32 : 4;
  static constexpr int kDB = D / 16 < 8 ? D / 16 : 8;
  __device__ static __forceinline__ int r_half(int dc) { return (dc / kDC) * 256; }
  __device__ static __forceinline__ int t_half(int db) { return (db / kDB) * 256; }
};

// ------------------------------------------------------------------ kernel 2: dK, dV
//
// One workgroup of 8 waves per (key tile of 128 keys, 64 at d = 256,
// batch * key/value head). The waves form 4 pairs; pair p owns keys
// kv0 + KPW p .. + KPW - 1 (KPW = 32, 16 at d = 256) and its two waves share
// one SIMD (waves p and p + 4):
//   wave A (p):     S = Q K^T, P = 2^(c S - lse log2 e) (masked), dV^T += dO^T P
//   wave B (p + 4): dP = dO V^T, dS = P o (dP - D), dK^T += Q^T dS
// (both kernels start the dP accumulators at -D, so the matrix unit forms
// dP - D and the vector unit only multiplies by P)
// so each wave keeps one of K^T / V^T and one accumulator in registers.
// Keys sit on the accumulator's columns: P and dS come out of the MFMA in
// the B-operand layout of dV^T += dO^T P and dK^T += Q^T dS, whose A
// operands dO^T, Q^T are transposing LDS reads of the row-major tiles.
// Wave A hands P (bf16) to wave B through LDS; wave B runs one query tile
// behind, so one workgroup barrier per tile publishes both the next Q/dO
// tile and the previous tile's P. Query tiles of 64 rows (32 at d = 256; Q, dO, lse, D)
// stream through a 3-stage ring of asynchronous copies: at step s tile s is
// read by A, tile s-1 by B, and the stage of tile s-2 receives tile s+1.
// For grouped heads the sequence of tiles covers every query head of the
// group, so dK and dV are summed in registers. When the grid of (key tile,
// batch * K/V head) workgroups is too small to reach every compute unit, the
// sequence of (query head, query tile) steps is split into p.n_gsplit
// contiguous parts (part = blockIdx.x / grid), each part writes its fp32
// partial sums, and fa_bwd_dkdv_reduce_kernel adds them up.
template <int D, bool CAUSAL>
__global__ __attribute__((amdgpu_flat_work_group_size(1, 512), amdgpu_waves_per_eu(2)))
void fa_bwd_dkdv_kernel(BwdParams p) {
  constexpr int NP = 4, KPW = D == 256 ? 16 : 32, BNK = NP * KPW;  // keys per workgroup
  constexpr int BMQ = D == 256 ? 32 : 64, STAGES = 3;             // query rows per tile
  constexpr int CPQ = BMQ / 32;                                   // 32-row chunks per query tile
  constexpr int KB = KPW / 16, QB = 2, DC = D / 32, DB = D / 16;
  constexpr int RB = 2 * D;
  constexpr int QT_BYTES = BMQ * RB;                       // one Q (or dO) tile
  constexpr int LSE_OFF = 2 * QT_BYTES, DEL_OFF = LSE_OFF + BMQ * 4;
  constexpr int STAGE_BYTES = 2 * QT_BYTES + 2 * BMQ * 4;  // Q, dO, lse, D
  constexpr int PIECES = 2 * QT_BYTES / 1024;              // 1 KiB copies per tile (Q and dO)
  constexpr int PIECES_PER_WAVE = PIECES / 8;
  constexpr int ROWS_PER_PIECE = 1024 / RB;
  constexpr int CH = RB / 16;
  constexpr int P_BYTES = CPQ * KB * 64 * 16;              // one pair's P of one tile: chunks x key blocks
  constexpr int LPW = BMQ / NP;                            // lse (D) rows copied per wave
  using Swz = DualSwizzle<D>;
  static_assert(PIECES % 8 == 0 && PIECES_PER_WAVE >= 1, "copy split");
  static_assert(STAGE_BYTES % 256 == 0, "stage alignment");

  __shared__ __attribute__((aligned(1024))) unsigned char smem_raw[STAGES * STAGE_BYTES + 2 * NP * P_BYTES];
  lds_u8* const smem = (lds_u8*)smem_raw;

  const int N = p.N;
  const int lane = threadIdx.x & 63;
  const int wave = uniform(threadIdx.x >> 6);
  const int role = wave >> 2, pair = wave & 3;
  const int g = lane >> 4, L = lane & 15;
  const int G = p.Hq / p.Hkv;

  const int n_wg = p.n_tiles * p.B * p.Hkv;  // workgroups per part of the head group
  const int part = workgroup_index() / n_wg;
  const TileCoord tc = map_workgroup(workgroup_index() - part * n_wg, p.B * p.Hkv, p.n_tiles, false);  // low key tiles (most work) first
  const int b = tc.head / p.Hkv;
  const int hk = tc.head - b * p.Hkv;
  const int kv0 = tc.tile * BNK;
  const int kw0 = kv0 + pair * KPW;  // this pair's first key
  const size_t kv_head = (size_t)(b * p.Hkv + hk) * N;

  const int nq = (N + BMQ - 1) / BMQ;
  const int t_first = CAUSAL ? kv0 / BMQ : 0;  // first query tile with a visible key
  const int per_head = nq - t_first;
  const int n_all = per_head * G;             // steps of the whole sequence (all heads of the group)
  const int j0 = (int)((long long)part * n_all / p.n_gsplit);  // this part's steps: j0 .. j0 + n_seq - 1
  const int n_seq = (int)((long long)(part + 1) * n_all / p.n_gsplit) - j0;

  // ---- copies of step jl of this part (sequence step j = j0 + jl: query head
  // hk*G + j / per_head, query tile t_first + j % per_head) into stage jl % STAGES
  auto issue_tile_copy = [&](int jl) __attribute__((always_inline)) {
    const int j = j0 + jl;
    const int gi = j / per_head;
    const int tq = t_first + (j - gi * per_head);
    const size_t qh = (size_t)(b * p.Hq + hk * G + gi) * N;
    const uint32_t dst = lds_address(smem) + (jl % STAGES) * STAGE_BYTES;
#pragma unroll
    for (int c = 0; c < PIECES_PER_WAVE; ++c) {
      const int piece = wave * PIECES_PER_WAVE + c;
      const int which = piece / (PIECES / 2);  // 0: Q, 1: dO
      const int pp = piece - which * (PIECES / 2);
      const int prow = pp * ROWS_PER_PIECE + lane / CH;
      const int lch = (lane % CH) ^ Swz::f(prow);
      const int grow = min(tq * BMQ + prow, N - 1);  // rows past the end: any valid row, masked later
      const void* base = which ? (const void*)((const __bf16*)p.dout + qh * D) : (const void*)((const __bf16*)p.q + qh * D);
      copy16_global_to_lds_async(base, (uint32_t)(grow * D + lch * 8) * 2, dst + which * QT_BYTES + pp * 1024);
    }
    // lse * log2(e) (waves 0-3) or D (waves 4-7): LPW rows per wave, one dword per lane
    if (lane < LPW) {
      const int row = min(tq * BMQ + LPW * pair + lane, N - 1);
      const float* src = (role == 0 ? p.lse2 : p.delta) + qh;
      copy4_global_to_lds_async(src, (uint32_t)row * 4, dst + (role == 0 ? LSE_OFF : DEL_OFF) + 4 * LPW * pair);
    }
  };
  constexpr int OPS = PIECES_PER_WAVE + 1;  // copy instructions per wave per tile
  (void)OPS;

  if (n_seq > 0) issue_tile_copy(0);

  // K^T (wave A) or V^T (wave B) fragments of the pair's keys: B operands
  // (column = key kw0 + 16 kb + L, k = d)
  bf16x8 kvf[KB][DC];
  {
    const __bf16* src = (const __bf16*)(role == 0 ? p.k : p.v) + kv_head * D;
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
      const int row = min(kw0 + kb * 16 + L, N - 1);
#pragma unroll
      for (int dc = 0; dc < DC; ++dc)
        kvf[kb][dc] = __builtin_bit_cast(bf16x8, *(const u32x4*)(src + (size_t)row * D + dc * 32 + g * 8));
    }
  }
  f32x4 acc[DB][KB];  // dV^T (wave A) or dK^T (wave B): rows d, columns keys
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) acc[db][kb] = f32x4{0.f, 0.f, 0.f, 0.f};

  const float c = p.scale_log2;
  int r_off[Swz::kDC];  // row-wise read: row L of a 16-row block, chunk dc*4 + g
#pragma unroll
  for (int dc = 0; dc < Swz::kDC; ++dc) r_off[dc] = L * RB + (((dc * 4 + g) ^ Swz::f(L)) << 4);
  int t_off[Swz::kDB];  // transposed read: row 4g + L/4 of a 32-row chunk, columns 16 db + 4 (L & 3) .. +3
  {
    const int trow = 4 * g + (L >> 2);
#pragma unroll
    for (int db = 0; db < Swz::kDB; ++db)
      t_off[db] = trow * RB + (((2 * db + ((L & 3) >> 1)) ^ Swz::f(trow)) << 4) + 8 * (L & 1);
  }
  auto roff = [&](int dc) __attribute__((always_inline)) { return r_off[dc % Swz::kDC] + Swz::r_half(dc); };
  auto toff = [&](int db) __attribute__((always_inline)) { return t_off[db % Swz::kDB] + Swz::t_half(db); };
  // P buffer of this pair: [tile parity][chunk][key block][lane] x 16 bytes
  lds_u8* const pbuf = smem + STAGES * STAGE_BYTES + pair * 2 * P_BYTES + lane * 16;

  // ---- one step: wait for tile s, publish it (and P of tile s-1), refill
  auto begin_step = [&](int s) __attribute__((always_inline)) {
    wait_vmcnt0();  // tile s landed (the only copies in flight)
    __syncthreads();
    if (s + 1 < n_seq) issue_tile_copy(s + 1);
  };

  // mask for wave A: key kw0 + 16 kb + L is visible to query q iff
  // lo[kb] <= q - 4g and q - 4g <= hi (q = the lane's query 4g + r of a block)
  int lo[KB];
#pragma unroll
  for (int kb = 0; kb < KB; ++kb) lo[kb] = (CAUSAL ? kw0 + kb * 16 + L : 0) - 4 * g;
  const int hi = N - 1 - 4 * g;

  // wave A, query chunk cc of tile j (query rows q0 + 32 cc ..). Every
  // fragment a block of matrix instructions needs is read into registers
  // before the block: the reads of one block are in flight together, and the
  // dO^T reads of the second product are issued ahead of the exponentials.
  auto chunk_a = [&](const lds_u8* st, int q0, int cc, lds_u8* pb, auto mask) __attribute__((always_inline)) {
    const lds_u8* qt = st;
    const lds_u8* dt = st + QT_BYTES;
    bf16x8 qa[DC][QB];
#pragma unroll
    for (int dc = 0; dc < DC; ++dc)
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) qa[dc][qb] = lds_read_b128(qt + (cc * 32 + qb * 16) * RB + roff(dc));
    f32x4 l4[QB];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) l4[qb] = *(const FA_LDS f32x4*)(st + LSE_OFF + (cc * 32 + qb * 16 + 4 * g) * 4);
    f32x4 s[QB][KB];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb)
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) s[qb][kb] = f32x4{0.f, 0.f, 0.f, 0.f};
    __builtin_amdgcn_s_setprio(1);
#pragma unroll
    for (int dc = 0; dc < DC; ++dc)
#pragma unroll
      for (int qb = 0; qb < QB; ++qb)
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) s[qb][kb] = mfma_bf16_16x16x32(qa[dc][qb], kvf[kb][dc], s[qb][kb]);
    __builtin_amdgcn_s_setprio(0);
    bf16x8 da[DB];
#pragma unroll
    for (int db = 0; db < DB; ++db) {
      const i16x4 lo4 = lds_read_tr16_b64(dt + cc * 32 * RB + toff(db));
      const i16x4 hi4 = lds_read_tr16_b64(dt + (cc * 32 + 16) * RB + toff(db));
      da[db] = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo4, hi4, 0, 1, 2, 3, 4, 5, 6, 7));
    }
    // P = 2^(c S - lse log2 e); B-operand packing: e < 4 -> query block 0
    // (rows 4g + e), e >= 4 -> block 1 (rows 16 + 4g + e - 4)
    u32x4 pw[KB];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) {
        float e[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          float x = s[qb][kb][r];
          if (decltype(mask)::value) {
            const int qq = q0 + cc * 32 + qb * 16 + r;  // query - 4g
            x = (qq >= lo[kb] && qq <= hi) ? x : kNegInf;
          }
          e[r] = exp2_fast(fmaf(x, c, -l4[qb][r]));
        }
        pw[kb][2 * qb] = pack_bf16x2(e[0], e[1]);
        pw[kb][2 * qb + 1] = pack_bf16x2(e[2], e[3]);
      }
    }
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) *(FA_LDS u32x4*)(pb + (cc * KB + kb) * 1024) = pw[kb];
    __builtin_amdgcn_s_setprio(1);
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) acc[db][kb] = mfma_bf16_16x16x32(da[db], __builtin_bit_cast(bf16x8, pw[kb]), acc[db][kb]);
    __builtin_amdgcn_s_setprio(0);
  };

  // wave B, query chunk cc of the previous tile (fragments read ahead of
  // their block, as for wave A)
  auto chunk_b = [&](const lds_u8* st, int cc, const lds_u8* pb) __attribute__((always_inline)) {
    const lds_u8* qt = st;
    const lds_u8* dt = st + QT_BYTES;
    bf16x8 oa[DC][QB];
#pragma unroll
    for (int dc = 0; dc < DC; ++dc)
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) oa[dc][qb] = lds_read_b128(dt + (cc * 32 + qb * 16) * RB + roff(dc));
    f32x4 dp[QB][KB];  // dP - D: the accumulators start at -D of their rows
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      const f32x4 nd4 = *(const FA_LDS f32x4*)(st + DEL_OFF + (cc * 32 + qb * 16 + 4 * g) * 4);
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) dp[qb][kb] = nd4;
    }
    u32x4 pr[KB];
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) pr[kb] = *(const FA_LDS u32x4*)(pb + (cc * KB + kb) * 1024);
    __builtin_amdgcn_s_setprio(1);
#pragma unroll
    for (int dc = 0; dc < DC; ++dc)
#pragma unroll
      for (int qb = 0; qb < QB; ++qb)
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) dp[qb][kb] = mfma_bf16_16x16x32(oa[dc][qb], kvf[kb][dc], dp[qb][kb]);
    __builtin_amdgcn_s_setprio(0);
    bf16x8 qa[DB];
#pragma unroll
    for (int db = 0; db < DB; ++db) {
      const i16x4 lo4 = lds_read_tr16_b64(qt + cc * 32 * RB + toff(db));
      const i16x4 hi4 = lds_read_tr16_b64(qt + (cc * 32 + 16) * RB + toff(db));
      qa[db] = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo4, hi4, 0, 1, 2, 3, 4, 5, 6, 7));
    }
    u32x4 dw[KB];
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) {
        float e[4];
#pragma unroll
        for (int h2 = 0; h2 < 2; ++h2) {
          const uint32_t w = pr[kb][2 * qb + h2];
          const float p0 = __builtin_bit_cast(float, w << 16);
          const float p1 = __builtin_bit_cast(float, w & 0xFFFF0000u);
          e[2 * h2] = p0 * dp[qb][kb][2 * h2];
          e[2 * h2 + 1] = p1 * dp[qb][kb][2 * h2 + 1];
        }
        dw[kb][2 * qb] = pack_bf16x2(e[0], e[1]);
        dw[kb][2 * qb + 1] = pack_bf16x2(e[2], e[3]);
      }
    }
    __builtin_amdgcn_s_setprio(1);
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) acc[db][kb] = mfma_bf16_16x16x32(qa[db], __builtin_bit_cast(bf16x8, dw[kb]), acc[db][kb]);
    __builtin_amdgcn_s_setprio(0);
  };

  auto stage_of = [&](int j) __attribute__((always_inline)) { return smem + uniform((j % STAGES) * STAGE_BYTES); };
  auto pbuf_of = [&](int j) __attribute__((always_inline)) { return pbuf + uniform((j & 1) * P_BYTES); };

  if (role == 0) {
    // wave A: steps 0 .. n_seq-1 process tile s; a last step keeps the
    // barrier count equal to wave B's. Per head: the tiles that reach above
    // the workgroup's last key (the diagonal under causal) and a partial
    // last tile take the masked path.
    const int t_clean0 = CAUSAL ? t_first + (BNK + BMQ - 2) / BMQ : 0;  // first tile no wave of the workgroup masks
    const int t_clean1 = N / BMQ;                                        // end of the full tiles
    int s = 0;
    while (s < n_seq) {  // one query head's run of this part's steps
      const int j = j0 + s;
      const int gi = j / per_head;
      const int tq_end = t_first + min(per_head, j0 + n_seq - gi * per_head);
      int tq = t_first + (j - gi * per_head);
      for (; tq < min(t_clean0, tq_end); ++tq, ++s) {
        begin_step(s);
#pragma unroll
        for (int cc = 0; cc < CPQ; ++cc) chunk_a(stage_of(s), tq * BMQ, cc, pbuf_of(s), std::true_type{});
      }
      for (; tq < min(t_clean1, tq_end); ++tq, ++s) {
        begin_step(s);
#pragma unroll
        for (int cc = 0; cc < CPQ; ++cc) chunk_a(stage_of(s), tq * BMQ, cc, pbuf_of(s), std::false_type{});
      }
      for (; tq < tq_end; ++tq, ++s) {
        begin_step(s);
#pragma unroll
        for (int cc = 0; cc < CPQ; ++cc) chunk_a(stage_of(s), tq * BMQ, cc, pbuf_of(s), std::true_type{});
      }
    }
    if (n_seq > 0) begin_step(n_seq);
  } else {
    // wave B: step s processes tile s-1
    if (n_seq > 0) begin_step(0);
    for (int s = 1; s <= n_seq; ++s) {
      begin_step(s);
#pragma unroll
      for (int cc = 0; cc < CPQ; ++cc) chunk_b(stage_of(s - 1), cc, pbuf_of(s - 1));
    }
  }

  // ---- dV = dV^T acc (wave A), dK = scale * dK^T acc (wave B); lane: key
  // column, rows d = 16 db + 4 g + r
  if (p.n_gsplit > 1) {  // this part's fp32 sums, unscaled
    float* part_out = p.dkv_part + ((size_t)(role * p.n_gsplit + part) * p.B * p.Hkv * N + kv_head) * D;
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
      const int key = kw0 + kb * 16 + L;
      if (key < N) {
#pragma unroll
        for (int db = 0; db < DB; ++db) *(f32x4*)(part_out + (size_t)key * D + db * 16 + 4 * g) = acc[db][kb];
      }
    }
    return;
  }
  // whole rows through each wave's region of the now idle LDS
  static_assert(8 * staged_rows_bytes<D>(KPW) <= STAGES * STAGE_BYTES, "dK/dV staging must fit in the ring");
  wait_vmcnt0();
  __syncthreads();  // every wave is done with the ring and the P buffers
  __bf16* out = (__bf16*)(role == 0 ? p.dv : p.dk) + kv_head * D;
  float osc[KB];
#pragma unroll
  for (int kb = 0; kb < KB; ++kb) osc[kb] = role == 0 ? 1.0f : p.scale;
  store_rows_through_lds<D, KB>(smem + wave * staged_rows_bytes<D>(KPW), acc, osc, out, kw0, N, lane);
}

// Split head groups: dV = sum of the parts' dV^T, dK = scale * sum of the
// parts' dK^T, per key row (rows = B * Hkv * N), D / 4 lanes per row.
template <int D>
__global__ __launch_bounds__(256) void fa_bwd_dkdv_reduce_kernel(BwdParams p, long long rows) {
  constexpr int LPR = D / 4;  // lanes per row
  const long long row = (long long)workgroup_index() * (256 / LPR) + threadIdx.x / LPR;
  const int c4 = threadIdx.x % LPR;
  if (row >= rows) return;
  const int S = p.n_gsplit;
  f32x4 sv = {0.f, 0.f, 0.f, 0.f}, sk = {0.f, 0.f, 0.f, 0.f};
  for (int s = 0; s < S; ++s) {
    sv += *(const f32x4*)(p.dkv_part + ((size_t)s * rows + row) * D + c4 * 4);
    sk += *(const f32x4*)(p.dkv_part + ((size_t)(S + s) * rows + row) * D + c4 * 4);
  }
  sk *= p.scale;
  *(u32x2*)((__bf16*)p.dv + row * D + c4 * 4) = u32x2{pack_bf16x2(sv[0], sv[1]), pack_bf16x2(sv[2], sv[3])};
  *(u32x2*)((__bf16*)p.dk + row * D + c4 * 4) = u32x2{pack_bf16x2(sk[0], sk[1]), pack_bf16x2(sk[2], sk[3])};
}

// ------------------------------------------------------------------ kernel 1: dQ (and D)
//
// One workgroup of 8 waves per (query tile of 256 rows, 128 at d = 256,
// batch * query head); each wave owns 32 query rows (16 at d = 256). Per
// 32-key chunk, with keys on the
// accumulator rows and queries on its columns (as in the forward kernel):
//   S^T = K Q^T, dP^T = V dO^T                         (A: K, V rows from LDS)
//   P^T = 2^(c S^T - lse log2 e), dS^T = P^T o (dP^T - D)   (per lane: one query)
//   dQ^T += K^T dS^T          (A: transposing reads of the K tile, B: dS^T packed)
// dQ = scale * dQ^T at the end. K/V tiles of 64 keys (32 at d = 256) stream
// through a ring of STAGES stages with asynchronous direct copies, one
// barrier per tile.
// NW, BN: 8 waves (256-row query tiles) with 64-key tiles, or, for short
// sequences and small grids, 4 waves (128 rows) with 32-key tiles, 48 KiB of
// LDS at head dim 128, so that two workgroups share a compute unit.
template <int D, bool CAUSAL, int STAGES = 3, int NW = 8, int BN = (D == 256 ? 32 : 64)>
__global__ __attribute__((amdgpu_flat_work_group_size(1, NW * 64), amdgpu_waves_per_eu(2)))
void fa_bwd_dq_kernel(BwdParams p) {
  constexpr int QPW = D == 256 ? 16 : 32, BM = QPW * NW;
  constexpr int QB = QPW / 16, DC = D / 32, DB = D / 16, CPT = BN / 32;
  constexpr int RB = 2 * D;  // bytes per tile row
  constexpr int TILE_BYTES = BN * RB;
  constexpr int COPIES_PER_WAVE = TILE_BYTES / 1024 / NW;
  constexpr int OPS = 2 * COPIES_PER_WAVE;  // copy instructions per wave per tile (K and V)
  constexpr int ROWS_PER_COPY = 1024 / RB;
  constexpr int CH = RB / 16;
  using Swz = DualSwizzle<D>;
  static_assert(COPIES_PER_WAVE >= 1 && TILE_BYTES % (1024 * NW) == 0, "K/V copy must split evenly over the waves");

  __shared__ __attribute__((aligned(1024))) unsigned char smem_raw[STAGES * 2 * TILE_BYTES];
  lds_u8* const smem = (lds_u8*)smem_raw;

  const int N = p.N;
  const int lane = threadIdx.x & 63;
  const int wave = uniform(threadIdx.x >> 6);
  const int g = lane >> 4, L = lane & 15;

  const TileCoord tc = map_workgroup(workgroup_index(), p.B * p.Hq, p.n_tiles, CAUSAL);
  const int b = tc.head / p.Hq;
  const int h = tc.head - b * p.Hq;
  const int hk = h / (p.Hq / p.Hkv);
  const size_t qh = (size_t)(b * p.Hq + h) * N;
  const __bf16* kg = (const __bf16*)p.k + (size_t)(b * p.Hkv + hk) * N * D;
  const __bf16* vg = (const __bf16*)p.v + (size_t)(b * p.Hkv + hk) * N * D;

  const int q0 = tc.tile * BM;
  const int qw0 = q0 + wave * QPW;
  const int kv_end = CAUSAL ? min(N, q0 + BM) : N;
  const int n_kv = (kv_end + BN - 1) / BN;
  const int n_ch = (qw0 < N) ? ((CAUSAL ? min(N, qw0 + QPW) : N) + 31) / 32 : 0;

  auto issue_tile_copy = [&](int t) __attribute__((always_inline)) {
    const int kv0 = t * BN;
    const uint32_t dst = lds_address(smem) + (t % STAGES) * 2 * TILE_BYTES;
#pragma unroll
    for (int c = 0; c < COPIES_PER_WAVE; ++c) {
      const int piece = wave * COPIES_PER_WAVE + c;
      const int prow = piece * ROWS_PER_COPY + lane / CH;
      const int lch = (lane % CH) ^ Swz::f(prow);  // logical chunk stored at this lane's physical chunk
      const int grow = min(kv0 + prow, N - 1);    // rows past the end: any valid row, masked later
      const uint32_t src = (uint32_t)(grow * D + lch * 8) * 2;
      copy16_global_to_lds_async(kg, src, dst + piece * 1024);
      copy16_global_to_lds_async(vg, src, dst + TILE_BYTES + piece * 1024);
    }
  };
  for (int t = 0; t < STAGES - 1 && t < n_kv; ++t) issue_tile_copy(t);

  // Q^T and dO^T fragments (B operands), the row's lse (log2 units) and D
  bf16x8 qf[QB][DC], df[QB][DC];
  float lse2[QB], dl[QB];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const int row = min(qw0 + qb * 16 + L, N - 1);
    const u32x4* qs = (const u32x4*)((const __bf16*)p.q + (qh + row) * D + g * 8);
    const u32x4* ds = (const u32x4*)((const __bf16*)p.dout + (qh + row) * D + g * 8);
    const u32x4* os = (const u32x4*)((const __bf16*)p.o + (qh + row) * D + g * 8);
    float dsum = 0.f;  // this lane's part of D = sum_c dO_c O_c (d = 32 dc + 8 g + e)
#pragma unroll
    for (int dc = 0; dc < DC; ++dc) {
      qf[qb][dc] = __builtin_bit_cast(bf16x8, qs[dc * 4]);
      df[qb][dc] = __builtin_bit_cast(bf16x8, ds[dc * 4]);
      const bf16x8 ov = __builtin_bit_cast(bf16x8, os[dc * 4]);
#pragma unroll
      for (int e = 0; e < 8; ++e) dsum = fmaf((float)df[qb][dc][e], (float)ov[e], dsum);
    }
    lse2[qb] = p.lse[qh + row] * 1.4426950408889634f;
    dl[qb] = sum_over_row_groups(dsum);  // the four lanes of the row hold its four d-slices
    if (g == 0 && qw0 + qb * 16 + L < N) {  // for the dK/dV kernel
      p.delta[qh + row] = -dl[qb];
      p.lse2[qh + row] = lse2[qb];
    }
  }
  f32x4 acc[DB][QB];
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) acc[db][qb] = f32x4{0.f, 0.f, 0.f, 0.f};
  const float c = p.scale_log2;
  // key k of a chunk is visible to this lane's query iff k <= lim; on masked
  // chunks the test is hb * 16 + r <= lim - (chunk start + 4g)
  int lim[QB];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) lim[qb] = (CAUSAL ? min(qw0 + qb * 16 + L, N - 1) : N - 1) - 4 * g;

  // lane parts of the LDS fragment offsets
  int r_off[Swz::kDC];  // row L of a 16-row block, chunk dc*4 + g
#pragma unroll
  for (int dc = 0; dc < Swz::kDC; ++dc) r_off[dc] = L * RB + (((dc * 4 + g) ^ Swz::f(L)) << 4);
  int t_off[Swz::kDB];  // transposed read: row 4g + L/4 of a 32-row chunk, columns 16 db + 4 (L & 3) .. +3
  {
    const int trow = 4 * g + (L >> 2);
#pragma unroll
    for (int db = 0; db < Swz::kDB; ++db)
      t_off[db] = trow * RB + (((2 * db + ((L & 3) >> 1)) ^ Swz::f(trow)) << 4) + 8 * (L & 1);
  }
  auto roff = [&](int dc) __attribute__((always_inline)) { return r_off[dc % Swz::kDC] + Swz::r_half(dc); };
  auto toff = [&](int db) __attribute__((always_inline)) { return t_off[db % Swz::kDB] + Swz::t_half(db); };

  // One 32-key chunk (K rows at kt, V rows at kt + TILE_BYTES, chunk index ch).
  auto chunk = [&](const lds_u8* kt, int ch, auto mask) __attribute__((always_inline)) {
    const lds_u8* vt = kt + TILE_BYTES;
    // S^T = K Q^T and dP^T = V dO^T, one 16-key half at a time, each half
    // turned into dS^T = P^T o (dP^T - D) and packed to bf16 right away
    u32x2 half_pk[2][QB];
#pragma unroll
    for (int hb = 0; hb < 2; ++hb) {
      f32x4 s[QB], dp[QB];
      {
        bf16x8 kf[DC], vf[DC];
#pragma unroll
        for (int dc = 0; dc < DC; ++dc) {
          kf[dc] = lds_read_b128(kt + hb * 16 * RB + roff(dc));
          vf[dc] = lds_read_b128(vt + hb * 16 * RB + roff(dc));
        }
        __builtin_amdgcn_s_setprio(1);
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) {
          s[qb] = f32x4{0.f, 0.f, 0.f, 0.f};
          dp[qb] = f32x4{-dl[qb], -dl[qb], -dl[qb], -dl[qb]};  // dP^T - D
        }
#pragma unroll
        for (int dc = 0; dc < DC; ++dc)
#pragma unroll
          for (int qb = 0; qb < QB; ++qb) {
            s[qb] = mfma_bf16_16x16x32(kf[dc], qf[qb][dc], s[qb]);
            dp[qb] = mfma_bf16_16x16x32(vf[dc], df[qb][dc], dp[qb]);
          }
        __builtin_amdgcn_s_setprio(0);
      }
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) {
        float e[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          float x = s[qb][r];
          if (decltype(mask)::value) x = (hb * 16 + r <= lim[qb] - ch * 32) ? x : kNegInf;
          e[r] = exp2_fast(fmaf(x, c, -lse2[qb])) * dp[qb][r];
        }
        half_pk[hb][qb] = u32x2{pack_bf16x2(e[0], e[1]), pack_bf16x2(e[2], e[3])};
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    // dS^T as the B operand of dQ^T += K^T dS^T: element e < 4 -> key 4g + e,
    // e >= 4 -> key 16 + 4g + e - 4 of the chunk
    bf16x8 dsf[QB];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb)
      dsf[qb] = __builtin_bit_cast(bf16x8, u32x4{half_pk[0][qb][0], half_pk[0][qb][1], half_pk[1][qb][0],
                                                half_pk[1][qb][1]});
    __builtin_amdgcn_s_setprio(1);
#pragma unroll
    for (int db = 0; db < DB; ++db) {
      const i16x4 lo = lds_read_tr16_b64(kt + toff(db));
      const i16x4 hi = lds_read_tr16_b64(kt + 16 * RB + toff(db));
      const bf16x8 ka = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) acc[db][qb] = mfma_bf16_16x16x32(ka, dsf[qb], acc[db][qb]);
    }
    __builtin_amdgcn_s_setprio(0);
  };

  // key loop: tile t is published by the barrier at its start; at that point
  // every wave is done with tile t-1, whose stage receives tile t+STAGES-1.
  // (the stage base is a run-time value, so the address arithmetic of the
  // three stages is not hoisted into registers of its own)
  // Two loops: tiles before t_mask need no mask in any wave (straight-line
  // bodies), the rest (the workgroup's diagonal and the end of the sequence)
  // take the masked path per wave.
  // Every load of the prologue landed before the key loop. The compiler counts
  // the Q/dO/O/lse loads but not the tile copies (inline assembly), so unless
  // a full wait covers them on every path into the loop it waits for them
  // inside the loop, which in fact holds each wave, on every tile, until its
  // newest copy has landed. (The D computation above has waited for nearly
  // all of them already.)
  wait_vmcnt0();
  int stage = 0;
  auto begin_tile = [&](int t) __attribute__((always_inline)) {
    if (t + STAGES - 2 < n_kv) {
      wait_vmcnt_le<(STAGES - 2) * OPS>();  // tile t landed; tiles up to t+STAGES-2 may fly
    } else {
      wait_vmcnt0();
    }
    __syncthreads();
    if (t + STAGES - 1 < n_kv) issue_tile_copy(t + STAGES - 1);
    const lds_u8* kt = smem + uniform(stage * 2 * TILE_BYTES);
    stage = (stage == STAGES - 1) ? 0 : stage + 1;
    return kt;
  };
  const int t_mask = min(n_kv, (CAUSAL ? min(q0, N) : N) / BN);
  int t = 0;
  for (; t < t_mask; ++t) {
    const lds_u8* kt = begin_tile(t);
#pragma unroll
    for (int cc = 0; cc < CPT; ++cc) chunk(kt + cc * 32 * RB, CPT * t + cc, std::false_type{});
  }
  for (; t < n_kv; ++t) {
    const lds_u8* kt = begin_tile(t);
#pragma unroll
    for (int cc = 0; cc < CPT; ++cc)
      if (CPT * t + cc < n_ch) chunk(kt + cc * 32 * RB, CPT * t + cc, std::true_type{});
  }

  // dQ = scale * dQ^T: lane holds query L + 16 qb, d = 16 db + 4 g + r;
  // whole rows through each wave's region of the now idle K/V ring
  static_assert(NW * staged_rows_bytes<D>(QPW) <= STAGES * 2 * TILE_BYTES, "dQ staging must fit in the ring");
  wait_vmcnt0();
  __syncthreads();  // every wave is done with the K/V ring
  float sc[QB];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) sc[qb] = p.scale;
  store_rows_through_lds<D, QB>(smem + wave * staged_rows_bytes<D>(QPW), acc, sc, (__bf16*)p.dq + qh * D, qw0, N, lane);
}

// ------------------------------------------------------------------ launch
template <int D, bool CAUSAL>
static hipError_t launch_bwd_cfg(const BwdParams& p_in, hipStream_t stream, hipEvent_t* ev) {
  constexpr int BM_DQ = D == 256 ? 128 : 256, BN_DKDV = D == 256 ? 64 : 128;  // as in the kernels
  BwdParams p = p_in;
  hipError_t e;
  // dQ first: it also writes -D (the row term, negated) that the dK/dV kernel reads
  if (ev && (e = hipEventRecord(ev[0], stream)) != hipSuccess) return e;
  // short sequences, fewer than two 256-row workgroups per compute unit, or
  // causal at head dim 64 (four 128-row workgroups per compute unit)
  bool small = false;
  if constexpr (D <= 128)
    small = p.N <= 512 || (long long)((p.N + BM_DQ - 1) / BM_DQ) * p.B * p.Hq < 2 * 256 || (D == 64 && CAUSAL);
  if (small) {
    if constexpr (D <= 128) {
      p.n_tiles = (p.N + 127) / 128;
      hipLaunchKernelGGL((fa_bwd_dq_kernel<D, CAUSAL, 3, 4, 32>), dim3((unsigned)(p.n_tiles * p.B * p.Hq)), dim3(256),
                         0, stream, p);
    }
  } else {
    p.n_tiles = (p.N + BM_DQ - 1) / BM_DQ;
    hipLaunchKernelGGL((fa_bwd_dq_kernel<D, CAUSAL>), dim3((unsigned)(p.n_tiles * p.B * p.Hq)), dim3(512), 0, stream,
                       p);
  }
  if ((e = hipGetLastError()) != hipSuccess) return e;
  if (ev && (e = hipEventRecord(ev[1], stream)) != hipSuccess) return e;
  p.n_tiles = (p.N + BN_DKDV - 1) / BN_DKDV;
  hipLaunchKernelGGL((fa_bwd_dkdv_kernel<D, CAUSAL>), dim3((unsigned)(p.n_tiles * p.B * p.Hkv * p.n_gsplit)), dim3(512),
                     0, stream, p);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  if (p.n_gsplit > 1) {
    const long long rows = (long long)p.B * p.Hkv * p.N;
    const long long rows_per_block = 256 / (D / 4);
    hipLaunchKernelGGL((fa_bwd_dkdv_reduce_kernel<D>), dim3((unsigned)((rows + rows_per_block - 1) / rows_per_block)),
                       dim3(256), 0, stream, p, rows);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  if (ev && (e = hipEventRecord(ev[2], stream)) != hipSuccess) return e;
  return hipSuccess;
}

hipError_t launch_bwd_bf16(const BwdParams& p, int d, bool causal, hipStream_t stream, hipEvent_t* ev) {
  if (d == 256) return causal ? launch_bwd_cfg<256, true>(p, stream, ev) : launch_bwd_cfg<256, false>(p, stream, ev);
  if (d == 128) return causal ? launch_bwd_cfg<128, true>(p, stream, ev) : launch_bwd_cfg<128, false>(p, stream, ev);
  if (d == 64) return causal ? launch_bwd_cfg<64, true>(p, stream, ev) : launch_bwd_cfg<64, false>(p, stream, ev);
  return hipErrorInvalidValue;
}

// ------------------------------------------------------------------ scratch of fa_bwd_noalloc
//
// The allocation-free backward keeps its workspace (the row terms and the
// split dK/dV partial sums) in this array instead of caller memory. Every
// GPU the library runs on holds its own copy, at its own address, until the
// process ends. In host code the array's name stands for a host-side
// shadow, not for device memory: kernels and copies get the address that
// hipGetSymbolAddress returns for the current device, looked up once per
// device on that device's first call and cached here. Every byte a call
// reads is first written by the same call (D and lse * log2 e by the dQ
// kernel, each split part's sums for all of its rows), so nothing needs
// clearing between calls; calls that overlap on one GPU share the array and
// race.
static __device__ __align__(256) unsigned char scratch[FA_BWD_NOALLOC_SCRATCH_BYTES];

namespace {
constexpr int kScratchDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kScratchDevices] = {};
}  // namespace

hipError_t bwd_noalloc_scratch(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kScratchDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (ptr == nullptr) return hipErrorInvalidSymbol;
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return hipSuccess;
}

}  // namespace fa

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
//   * one workgroup of 8 waves per (query tile of 256 rows, batch * head), two
//     waves per SIMD; each wave owns 32 consecutive query rows and never
//     exchanges partial results with another wave (head dim 256: 128-row
//     tiles, 16 rows per wave, so the accumulator keeps its register size);
//   * short sequences (N <= 512), small grids (fewer than two 256-row
//     workgroups per CU) and causal head dim 64, at head dim <= 128:
//     workgroups of 4 waves (128 rows) with 32-key tiles, 48 KiB of LDS at
//     head dim 128, so two (four at head dim 64) share a CU and one's loads
//     or diagonal overlap another's math;
//   * K/V tiles of 64 keys (32 at head dim 256) are copied global -> LDS with 16-byte direct loads
//     into a ring of STAGES stages. The copy of tile t+STAGES-1 is issued
//     right after the single barrier that publishes tile t+1, so it overlaps
//     the math of STAGES-2 tiles ("Flash Attention V3技术解析" section 2.1,
//     double buffering; one barrier per tile as in the aiknowledge.cn page,
//     FA2 section 1).
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
// Software pipeline. A wave walks its keys in 32-key chunks. The steady-state
// step for chunk c is one straight-line block holding the exponentials of c,
// the S^T MFMAs of chunk c+1, the O^T += V^T P^T MFMAs of chunk c and the
// row maximum of chunk c+1, so the matrix unit works on c+1 while the vector
// unit finishes c (the softmax/GEMM overlap that "Flash Attention V3技术解析"
// section 1.2 obtains with ping-pong warp groups, here inside one wave).
// Chunks that need a mask (diagonal, end of sequence) take a plain path.
//
// Softmax bookkeeping, per query row, in the log2 domain (c = scale*log2 e):
//   m  = reference maximum used for the exponentials,
//   l  = per-lane partial sum of 2^(c s - m) (reduced over lanes at the end),
//   acc = sum of 2^(c s - m) v (unnormalised).
// A new chunk only moves the reference maximum (and rescales l and acc by
// 2^(m_old - m_new), the correction of mhpq.cn section 2.2) when some score
// exceeds m + kRescaleSlack. Otherwise the old reference is kept: every
// exponential is then at most 2^kRescaleSlack, and because acc and l share
// the same reference the ratio acc / l, i.e. O, is the same number. The check
// is one compare per row and a wave vote, so the per-chunk rescale of acc
// (64 multiplies per lane at head dim 128) is skipped on almost every chunk.
//
// Causal (key j visible to query i iff j <= i): the key loop stops at the
// last key tile holding a visible key for the workgroup's last query (tiles
// wholly above the diagonal are never loaded, "Flash Attention V3技术解析"
// section 2.1), each wave stops at its own diagonal, and the element mask is
// applied only on chunks that straddle the diagonal or the end of the
// sequence.
//
// The same kernel, through template flags described at its definition, also
// runs split-KV (key-range parts of a query tile plus a merge kernel), a
// block mask (block-sparse) and FP8 queries and keys.
#include <type_traits>

#include "fa_common.hpp"
#include "fa_launch.hpp"

namespace fa {

constexpr float kRescaleSlack = 8.0f;  // log2 units: exponentials stay <= 256

template <int D>
struct KVSwizzle {
  static constexpr int kRowBytes = 2 * D;
  static constexpr int kChunks16 = kRowBytes / 16;        // 16-byte chunks per row
  static constexpr int kRowsPer256 = kRowBytes >= 256 ? 1 : 256 / kRowBytes;  // rows sharing one 256-byte bank sweep
  // XOR masks span one 256-byte sweep (16 chunks of 16 bytes, 8 of 32 bytes) at most
  static constexpr int kKMod = kChunks16 < 16 ? kChunks16 : 16;
  static constexpr int kVMod = kChunks16 / 2 < 8 ? kChunks16 / 2 : 8;
  // K: physical 16-byte chunk = logical chunk ^ k_swz(row)
  __device__ static __forceinline__ int k_swz(int row) { return (row / kRowsPer256) % kKMod; }
  // V: physical 32-byte chunk = logical 32-byte chunk ^ v_swz(row)
  __device__ static __forceinline__ int v_swz(int row) { return (row / kRowsPer256) % kVMod; }
  // the fragment reads add whole 16-row blocks to a lane's row: the masks
  // must repeat every 16 rows
  static_assert(16 % (kRowsPer256 * kKMod) == 0 && 16 % (kRowsPer256 * kVMod) == 0, "swizzle period");
};

// Tuning knobs (instantiated by the launcher): QPW query rows per wave, NW
// waves per workgroup, STAGES K/V tiles in the LDS ring. The register budget
// follows from the waves per CU: 8 waves (one workgroup) put two on every
// SIMD, and the vector phase of one overlaps the matrix phase of the other;
// 4-wave workgroups are held to 256 registers per wave so that two of them
// share a CU (waves_per_eu(2)). PRIO raises the
// wave's issue priority around its runs of matrix instructions, so the wave
// that has MFMA work ready wins the issue slot and the other wave's vector
// work fills the gaps.
// SPLIT: the workgroup processes part blockIdx.x / (n_tiles * B * Hq) of the
// query tile's key tiles and writes that part's O (fp32) and lse to
// p.o_part / p.lse_part for the merge kernel, instead of O and lse.
// SPARSE: a block mask of 128 x 128 blocks says which key blocks each query
// block sees ("FlashAttention技术解析" (mhpq.cn) section 6.2, block-sparse
// integration). The workgroup first compacts the key blocks that any of its
// query blocks sees (the union; causal drops blocks wholly above the
// diagonal) into a list in LDS and then streams only those tiles, exactly
// as the causal skip streams only the tiles below the diagonal. A wave
// skips the chunks of listed blocks that its own query block does not see
// (and chunks above its diagonal or past the end). Rows that see no key get
// O = 0 and lse = -inf.
// F8: q and k hold e4m3 codes with one fp32 scale per 64 rows (block-wise
// quantisation of the inputs of Q K^T, "Flash Attention V3技术解析" (mlqm.cn)
// sections 1.3 and 3.2); S^T = K Q^T runs on the FP8 matrix instruction
// (16x16x128, the whole head dim of a 16 x 16 block in one or two steps),
// and the block scales fold into the per-chunk exponent factor. V, P, the
// softmax and O are as in the bf16 path (BF16 where precision matters, as in
// "4.3 FlashAttention-2与FlashAttention-3演进", FlashAttention-3 section 2).
template <int D, bool CAUSAL, int QPW, int NW, bool PRIO, int STAGES, bool SPLIT = false, int BN = 64,
          bool SPARSE = false, bool F8 = false>
__global__ __attribute__((amdgpu_flat_work_group_size(1, NW * 64), amdgpu_waves_per_eu(NW <= 4 ? 2 : 1)))
void fa_fwd_bf16_kernel(FwdParams p) {
  constexpr int BM = QPW * NW;
  static_assert(BN == 32 || BN == 64, "one or two 32-key chunks per tile");
  // copy instructions per wave per tile (K and V[, the K scale])
  constexpr int OPS = F8 ? (BN * D / 1024) / NW + (BN * D * 2 / 1024) / NW + 1 : 2 * (BN * D * 2 / 1024) / NW;
  static_assert(STAGES >= 3, "the copy of tile t+STAGES-1 is issued while tile t is read");
  constexpr int QB = QPW / 16;           // 16-query blocks per wave
  constexpr int DC = D / 32;             // k-steps of S^T = K Q^T
  constexpr int DB = D / 16;             // 16-row blocks of O^T
  constexpr int CPT = BN / 32;           // 32-key chunks per tile
  constexpr int TILE_BYTES = BN * D * 2;
  constexpr int COPIES = TILE_BYTES / 1024;       // 1 KiB (64 lanes x 16 B) per copy instruction
  constexpr int COPIES_PER_WAVE = COPIES / NW;
  constexpr int ROWS_PER_COPY = 1024 / (2 * D);
  constexpr int CH = 2 * D / 16;
  using Swz = KVSwizzle<D>;
  static_assert(COPIES % NW == 0, "K/V copy must split evenly over the waves");
  // stage = K tile (bf16 rows, or e4m3 rows of D bytes), V tile, and (F8) the tile's K scale
  constexpr int KROW = F8 ? D : 2 * D;
  constexpr int K_TILE_BYTES = BN * KROW;
  constexpr int V_OFF = K_TILE_BYTES;
  constexpr int SCALE_OFF = K_TILE_BYTES + TILE_BYTES;
  constexpr int STAGE_BYTES = SCALE_OFF + (F8 ? 256 : 0);
  constexpr int DC8 = D / 128;                                  // F8: 128-byte k-steps of S^T
  constexpr int K8_COPIES_PER_WAVE = K_TILE_BYTES / 1024 / NW;  // F8 copies of K per wave
  constexpr int K8_ROWS = 1024 / KROW, K8_CH = KROW / 16;
  using Swz8 = KVSwizzle<D / 2>;                                // F8 K rows: D bytes
  static_assert(!F8 || ((D == 128 || D == 256) && !SPARSE && !SPLIT && K_TILE_BYTES % (1024 * NW) == 0),
                "FP8: head dim 128 or 256, plain forward");
  constexpr int SB = kSparseBlock;  // block-mask block (queries and keys)
  constexpr int TPB = SB / BN;      // key tiles per mask block
  static_assert(!SPARSE || (BM % SB == 0 && BM / SB <= 2 && !SPLIT), "sparse: 1 or 2 query blocks per workgroup");

  // ring of STAGES x (K tile, V tile[, K scale])
  __shared__ __attribute__((aligned(1024))) unsigned char smem_raw[STAGES * STAGE_BYTES];
  lds_u8* const smem = (lds_u8*)smem_raw;
  // sparse: listed key blocks, bits 0-13 block index, bit 14 + i: query block i of the workgroup sees it
  __shared__ uint16_t blk_list[SPARSE ? kSparseMaxBlocks : 1];
  __shared__ int blk_count[SPARSE ? NW : 1];

  const int N = p.N;
  const int lane = threadIdx.x & 63;
  const int wave = uniform(threadIdx.x >> 6);
  const int g = lane >> 4;   // row group of an accumulator block
  const int L = lane & 15;   // column of an accumulator block (this lane's query)

  const int n_wg = p.n_tiles * p.B * p.Hq;  // workgroups per part
  const int part = SPLIT ? workgroup_index() / n_wg : 0;
  const TileCoord tc = map_workgroup(SPLIT ? workgroup_index() - part * n_wg : workgroup_index(), p.B * p.Hq, p.n_tiles, CAUSAL);
  const int b = tc.head / p.Hq;
  const int h = tc.head - b * p.Hq;
  const int hk = h / (p.Hq / p.Hkv);
  const __bf16* __restrict__ qg = (const __bf16*)p.q + ((size_t)(b * p.Hq + h) * N) * D;
  const __bf16* kg = (const __bf16*)p.k + ((size_t)(b * p.Hkv + hk) * N) * D;
  const __bf16* vg = (const __bf16*)p.v + ((size_t)(b * p.Hkv + hk) * N) * D;
  __bf16* __restrict__ og = (__bf16*)p.o + ((size_t)(b * p.Hq + h) * N) * D;
  float* __restrict__ lseg = p.lse + (size_t)(b * p.Hq + h) * N;

  const int q0 = tc.tile * BM;
  const int qw0 = q0 + wave * QPW;  // first query row of this wave

  // Q^T fragments (B operand of S^T = K Q^T), held for the whole key loop.
  bf16x8 qf[F8 ? 1 : QB][F8 ? 1 : DC];
  i32x8 qf8[F8 ? QB : 1][F8 ? DC8 : 1];  // F8: bytes 32 g .. 32 g + 31 of each 128-byte k-step
  auto load_q = [&]() __attribute__((always_inline)) {
    if constexpr (F8) {
      const unsigned char* q8 = (const unsigned char*)p.q + ((size_t)(b * p.Hq + h) * N) * D;
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) {
        const int row = min(qw0 + qb * 16 + L, N - 1);
#pragma unroll
        for (int dc = 0; dc < DC8; ++dc) {
          const u32x4* src = (const u32x4*)(q8 + (size_t)row * D + dc * 128 + g * 32);
          const u32x4 lo = src[0], hi = src[1];
          qf8[qb][dc] = i32x8{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
        }
      }
    } else {
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) {
        const int row = min(qw0 + qb * 16 + L, N - 1);
        const u32x4* src = (const u32x4*)(qg + (size_t)row * D + g * 8);
#pragma unroll
        for (int dc = 0; dc < DC; ++dc) qf[qb][dc] = __builtin_bit_cast(bf16x8, src[dc * 4]);
      }
    }
  };
  // sparse: the Q loads go out first, so their latency overlaps the mask scan
  if constexpr (SPARSE) load_q();

  // sparse: compact the listed key blocks (ballot + prefix over the waves)
  int n_list = 0;
  if constexpr (SPARSE) {
    const int n_kb = (N + SB - 1) / SB;
    const int qb0 = q0 / SB;
    const int nqb = min(BM / SB, n_kb - qb0);
    const unsigned char* mrow =
        p.block_mask + (long long)b * p.mask_stride_b + (long long)h * p.mask_stride_h + (long long)qb0 * n_kb;
    const int n_scan = CAUSAL ? min(n_kb, qb0 + nqb) : n_kb;
    for (int j0 = 0; j0 < n_scan; j0 += NW * 64) {
      const int j = j0 + (int)threadIdx.x;
      bool v0 = false, v1 = false;
      if (j < n_scan) {
        v0 = mrow[j] != 0 && (!CAUSAL || j <= qb0);
        v1 = nqb > 1 && mrow[n_kb + j] != 0 && (!CAUSAL || j <= qb0 + 1);
      }
      const uint64_t bal = __builtin_amdgcn_ballot_w64(v0 || v1);
      if (lane == 0) blk_count[wave] = __builtin_popcountll(bal);
      __syncthreads();
      int before = 0, total = 0;
#pragma unroll
      for (int w = 0; w < NW; ++w) {
        const int cnt = blk_count[w];
        before += w < wave ? cnt : 0;
        total += cnt;
      }
      if (v0 || v1) {
        const int pos = n_list + before + __builtin_popcountll(bal & ((1ull << lane) - 1ull));
        blk_list[pos] = (uint16_t)(j | (v0 ? 1 << 14 : 0) | (v1 ? 1 << 15 : 0));
      }
      n_list += total;
      __syncthreads();  // the list is complete; blk_count may be reused
    }
  }
  // sparse: sequence position t -> key tile, and whether this wave's query block sees it
  auto kv_tile_of = [&](int t) __attribute__((always_inline)) {
    if constexpr (SPARSE) return uniform((blk_list[t / TPB] & 0x3FFF) * TPB + t % TPB);
    else return t;
  };
  const int wave_qblock = (wave * QPW) / SB;
  auto sees_tile = [&](int t) __attribute__((always_inline)) {
    return ((uniform(blk_list[t / TPB]) >> (14 + wave_qblock)) & 1) != 0;
  };

  const int kv_end = CAUSAL ? min(N, q0 + BM) : N;
  const int n_kv_all = SPARSE ? n_list * TPB : (kv_end + BN - 1) / BN;  // key tiles the workgroup visits
  // this workgroup's key tiles [t_lo, n_kv) (all of them without SPLIT)
  const int t_lo = SPLIT ? (int)(((long long)part * n_kv_all) / p.n_splits) : 0;
  const int n_kv = SPLIT ? (int)(((long long)(part + 1) * n_kv_all) / p.n_splits) : n_kv_all;
  // chunks this wave processes [c_lo, n_ch), and the first one that needs an element mask
  const int n_ch_all = (qw0 < N) ? ((CAUSAL ? min(N, qw0 + QPW) : N) + 31) / 32 : 0;
  const int n_ch = min(n_ch_all, CPT * n_kv);
  const int c_lo = CPT * t_lo;
  const int first_mask = min(n_ch_all, CAUSAL ? min((qw0 + 1) / 32, N / 32) : N / 32);

  // ---- K/V tile copies (asynchronous; published by the barrier of the tile)
  auto issue_tile_copy = [&](int t) __attribute__((always_inline)) {
    const int kv0 = kv_tile_of(t) * BN;
    const uint32_t kdst = lds_address(smem) + ((t - t_lo) % STAGES) * STAGE_BYTES;
    if constexpr (F8) {
      const unsigned char* k8 = (const unsigned char*)p.k + ((size_t)(b * p.Hkv + hk) * N) * D;
#pragma unroll
      for (int c = 0; c < K8_COPIES_PER_WAVE; ++c) {
        const int piece = wave * K8_COPIES_PER_WAVE + c;
        const int prow = piece * K8_ROWS + lane / K8_CH;
        const int pch = lane % K8_CH;
        const int grow = min(kv0 + prow, N - 1);
        copy16_global_to_lds_async(k8, (uint32_t)(grow * D + (pch ^ Swz8::k_swz(prow)) * 16), kdst + piece * 1024);
      }
#pragma unroll
      for (int c = 0; c < COPIES_PER_WAVE; ++c) {
        const int piece = wave * COPIES_PER_WAVE + c;
        const int prow = piece * ROWS_PER_COPY + lane / CH;
        const int pch = lane % CH;
        const int grow = min(kv0 + prow, N - 1);
        const int vch = (((pch >> 1) ^ Swz::v_swz(prow)) << 1) | (pch & 1);
        copy16_global_to_lds_async(vg, (uint32_t)(grow * D + vch * 8) * 2, kdst + V_OFF + piece * 1024);
      }
      // the tile's K scale (every wave copies it, so all waves count the same copies)
      if (lane == 0) {
        const float* ks = p.k_descale + (size_t)(b * p.Hkv + hk) * ((N + kFp8Block - 1) / kFp8Block);
        copy4_global_to_lds_async(ks, (uint32_t)(min(kv0, N - 1) / kFp8Block) * 4, kdst + SCALE_OFF);
      }
      return;
    }
#pragma unroll
    for (int c = 0; c < COPIES_PER_WAVE; ++c) {
      const int piece = wave * COPIES_PER_WAVE + c;
      const int prow = piece * ROWS_PER_COPY + lane / CH;  // physical row in the tile
      const int pch = lane % CH;                            // physical 16-byte chunk
      const int grow = min(kv0 + prow, N - 1);              // rows past the end: any valid row, masked later
      const int kch = pch ^ Swz::k_swz(prow);
      const int vch = (((pch >> 1) ^ Swz::v_swz(prow)) << 1) | (pch & 1);
      copy16_global_to_lds_async(kg, (uint32_t)(grow * D + kch * 8) * 2, kdst + piece * 1024);
      copy16_global_to_lds_async(vg, (uint32_t)(grow * D + vch * 8) * 2, kdst + TILE_BYTES + piece * 1024);
    }
  };

  for (int t = t_lo; t < t_lo + STAGES - 1 && t < n_kv; ++t) issue_tile_copy(t);
  if constexpr (!SPARSE) load_q();

  f32x4 acc[DB][QB];
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) acc[db][qb] = f32x4{0.f, 0.f, 0.f, 0.f};
  // Row sums l. At head dim 64 a chunk has half the matrix work per score
  // of d = 128 and the vector unit bounds the loop, so there the sums come
  // from the matrix unit: one more MFMA per query block and chunk, an
  // all-ones A operand times P^T, leaves in every element of lsum[qb] the
  // sum of the bf16 probabilities of its query (the same values that weight
  // V). Elsewhere each lane adds its fp32 probabilities into l_part, and the
  // four row groups are summed at the end.
  constexpr bool kRowSumOnMatrix = D == 64;
  float m_ref[QB], l_part[QB];
  f32x4 lsum[QB];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    m_ref[qb] = kNegInf;
    l_part[qb] = 0.f;
    lsum[qb] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  const float c = p.scale_log2;
  // exponent factor of the scores in s_cur (F8: times the Q and K block scales)
  float c_s = c;
  float c_q = c;  // F8: c times this wave's Q block scale (its rows lie in one 64-row block)
  if constexpr (F8) {
    const int n_qblk = (N + kFp8Block - 1) / kFp8Block;
    c_q = c * p.q_descale[(size_t)(b * p.Hq + h) * n_qblk + min(qw0, N - 1) / kFp8Block];
  }

  // Lane parts of the LDS fragment addresses (the stage and chunk parts are
  // compile-time constants at every use, so they fold into the instruction
  // offsets and no address arithmetic runs per chunk).
  int k_off[F8 ? 1 : DC];  // K row L of a 16-key block, 16-byte chunk dc*4 + g (swizzled)
  int k8_off[F8 ? DC8 : 1][2];  // F8: K row L, 16-byte chunks 8 dc + 2 g and 8 dc + 2 g + 1 (swizzled)
  if constexpr (F8) {
#pragma unroll
    for (int dc = 0; dc < DC8; ++dc)
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) k8_off[dc][hh] = L * KROW + (((dc * 8 + 2 * g + hh) ^ Swz8::k_swz(L)) * 16);
  } else {
#pragma unroll
    for (int dc = 0; dc < DC; ++dc) k_off[dc] = L * (2 * D) + (((dc * 4 + g) ^ Swz::k_swz(L)) * 16);
  }
  int v_off[DB];  // V row 4g + L/4 of a 32-key chunk, 32-byte chunk db (swizzled), 8 bytes at 8 (L & 3)
  {
    const int vrow = 4 * g + (L >> 2);
#pragma unroll
    for (int db = 0; db < DB; ++db) v_off[db] = vrow * (2 * D) + ((db ^ Swz::v_swz(vrow)) * 32) + 8 * (L & 3);
  }

  // K fragments (A operand of S^T) of chunk cc (0..CPT-1) of the K tile at kt
  auto read_k = [&](const lds_u8* kt, int cc, bf16x8 (&kf)[2][DC]) __attribute__((always_inline)) {
#pragma unroll
    for (int hb = 0; hb < 2; ++hb)
#pragma unroll
      for (int dc = 0; dc < DC; ++dc)
        kf[hb][dc] = lds_read_b128(kt + (cc * 32 + hb * 16) * (2 * D) + k_off[dc]);
  };
  // V^T fragments (A operand of O^T += V^T P^T): rows d = 16 db + lane % 16,
  // element e < 4 -> key 4g + e, e >= 4 -> key 16 + 4g + e - 4 of the chunk
  // F8: K fragments of chunk cc, 32 bytes per lane per 128-byte k-step
  auto read_k8 = [&](const lds_u8* kt, int cc, i32x8 (&kf)[2][DC8 > 0 ? DC8 : 1]) __attribute__((always_inline)) {
#pragma unroll
    for (int hb = 0; hb < 2; ++hb)
#pragma unroll
      for (int dc = 0; dc < DC8; ++dc) {
        const lds_u8* rowp = kt + (cc * 32 + hb * 16) * KROW;
        const u32x4 lo = *(const FA_LDS u32x4*)(rowp + k8_off[dc][0]);
        const u32x4 hi = *(const FA_LDS u32x4*)(rowp + k8_off[dc][1]);
        kf[hb][dc] = i32x8{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
      }
  };
  auto read_v = [&](const lds_u8* kt, int cc, bf16x8 (&vf)[DB]) __attribute__((always_inline)) {
    const lds_u8* vt = kt + V_OFF + cc * 32 * (2 * D);
#pragma unroll
    for (int db = 0; db < DB; ++db) {
      const i16x4 lo = lds_read_tr16_b64(vt + v_off[db]);
      const i16x4 hi = lds_read_tr16_b64(vt + 16 * (2 * D) + v_off[db]);
      vf[db] = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
    }
  };
  auto compute_s = [&](const bf16x8 (&kf)[2][DC], f32x4 (&s)[2][QB]) __attribute__((always_inline)) {
    if (PRIO) __builtin_amdgcn_s_setprio(1);
#pragma unroll
    for (int hb = 0; hb < 2; ++hb) {
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) s[hb][qb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int dc = 0; dc < DC; ++dc)
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) s[hb][qb] = mfma_bf16_16x16x32(kf[hb][dc], qf[qb][dc], s[hb][qb]);
    }
    if (PRIO) __builtin_amdgcn_s_setprio(0);
  };
  auto apply_mask = [&](int ch, f32x4 (&s)[2][QB], bool sees = true) __attribute__((always_inline)) {
    const int key0 = ch * 32;
#pragma unroll
    for (int hb = 0; hb < 2; ++hb)
#pragma unroll
      for (int qb = 0; qb < QB; ++qb)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int key = key0 + hb * 16 + g * 4 + r;
          const int qi = qw0 + qb * 16 + L;
          const bool visible = (!SPARSE || sees) && key < N && (!CAUSAL || key <= qi);
          s[hb][qb][r] = visible ? s[hb][qb][r] : kNegInf;
        }
  };
  // in-lane maximum of the chunk per query block, scaled to log2 units
  auto chunk_max = [&](const f32x4 (&s)[2][QB], float (&tmax)[QB]) __attribute__((always_inline)) {
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      float mx = fmaxf(fmaxf(s[0][qb][0], s[0][qb][1]), s[0][qb][2]);
      mx = fmaxf(fmaxf(mx, s[0][qb][3]), s[1][qb][0]);
      mx = fmaxf(fmaxf(mx, s[1][qb][1]), s[1][qb][2]);
      tmax[qb] = fmaxf(mx, s[1][qb][3]) * c_s;
    }
  };
  // move the reference maximum if some score exceeds it by more than the slack
  auto update_reference = [&](const float (&tmax)[QB]) __attribute__((always_inline)) {
    bool grow = false;
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) grow |= tmax[qb] > m_ref[qb] + kRescaleSlack;
    if (wave_any(grow)) {
      // rare path: the marker keeps the compiler from turning this branch
      // into unconditional selects executed on every chunk
      asm volatile("; reference maximum moves" ::: "memory");
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) {
        const float m_new = fmaxf(m_ref[qb], max_over_row_groups(tmax[qb]));
        const float alpha = (m_ref[qb] == kNegInf) ? 0.f : exp2_fast(m_ref[qb] - m_new);
        m_ref[qb] = m_new;
        if constexpr (kRowSumOnMatrix) {
          lsum[qb] *= alpha;
        } else {
          l_part[qb] *= alpha;
        }
#pragma unroll
        for (int db = 0; db < DB; ++db) acc[db][qb] *= alpha;
      }
    }
  };
  // P^T = 2^(c S^T - m), packed to bf16 in the B-operand layout of O^T += V^T P^T
  auto exponentiate = [&](const f32x4 (&s)[2][QB], bf16x8 (&pf)[QB]) __attribute__((always_inline)) {
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      // sparse: a row may have seen no key yet (m = -inf); its masked scores give 2^-inf = 0
      const float neg_m = (SPARSE && m_ref[qb] == kNegInf) ? 0.f : -m_ref[qb];
      float e[8];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        e[r] = exp2_fast(fmaf(s[0][qb][r], c_s, neg_m));
        e[4 + r] = exp2_fast(fmaf(s[1][qb][r], c_s, neg_m));
      }
      u32x4 packed = {pack_bf16x2(e[0], e[1]), pack_bf16x2(e[2], e[3]), pack_bf16x2(e[4], e[5]),
                      pack_bf16x2(e[6], e[7])};
      if constexpr (!kRowSumOnMatrix) l_part[qb] += ((e[0] + e[1]) + (e[2] + e[3])) + ((e[4] + e[5]) + (e[6] + e[7]));
      pf[qb] = __builtin_bit_cast(bf16x8, packed);
    }
  };
  auto accumulate_pv = [&](const bf16x8 (&vf)[DB], const bf16x8 (&pf)[QB]) __attribute__((always_inline)) {
    if (PRIO) __builtin_amdgcn_s_setprio(1);
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) acc[db][qb] = mfma_bf16_16x16x32(vf[db], pf[qb], acc[db][qb]);
    if constexpr (kRowSumOnMatrix) {
      const bf16x8 ones = __builtin_bit_cast(bf16x8, u32x4{0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u});
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) lsum[qb] = mfma_bf16_16x16x32(ones, pf[qb], lsum[qb]);
    }
    if (PRIO) __builtin_amdgcn_s_setprio(0);
  };

  // S^T of the chunk about to be exponentiated (masked, maximum folded in)
  f32x4 s_cur[2][QB];

  // S^T of chunk ch (K tile at kt, position cc), masked when MASK, and the reference update.
  auto scores = [&](const lds_u8* kt, int cc, int ch, auto mask, bool sees = true) __attribute__((always_inline)) {
    if constexpr (F8) {
      i32x8 kf[2][DC8 > 0 ? DC8 : 1];
      read_k8(kt, cc, kf);
      if (PRIO) __builtin_amdgcn_s_setprio(1);
#pragma unroll
      for (int hb = 0; hb < 2; ++hb)
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) {
          s_cur[hb][qb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int dc = 0; dc < DC8; ++dc) s_cur[hb][qb] = mfma_fp8_16x16x128(kf[hb][dc], qf8[qb][dc], s_cur[hb][qb]);
        }
      if (PRIO) __builtin_amdgcn_s_setprio(0);
      c_s = c_q * *(const FA_LDS float*)(kt + SCALE_OFF);
    } else {
      bf16x8 kf[2][DC];
      read_k(kt, cc, kf);
      compute_s(kf, s_cur);
    }
    if (decltype(mask)::value) apply_mask(ch, s_cur, sees);
    float tmax[QB];
    chunk_max(s_cur, tmax);
    update_reference(tmax);
  };

  // Chunk ch (S^T in s_cur, reference current): exponentials and O^T += V^T P^T
  // of ch, then S^T and the maximum of chunk ch+1 (K tile at ktn, position
  // ccn). Up to the vote on ch+1 this is one straight-line block, so the
  // scheduler overlaps the exponentials of ch with the matrix work of ch+1.
  auto chunk_step = [&](const lds_u8* kt, int cc, const lds_u8* ktn, int ccn, int ch, auto mask)
                        __attribute__((always_inline)) {
    bf16x8 vf[DB], pf[QB];
    read_v(kt, cc, vf);
    exponentiate(s_cur, pf);
    accumulate_pv(vf, pf);
    if (!decltype(mask)::value || ch + 1 < n_ch) scores(ktn, ccn, ch + 1, mask);
  };
  // sparse: one step of this wave's own chunk sequence. A chunk the wave
  // does not see (block off, wholly above its diagonal, or past the end) is
  // skipped; s_cur is live (cur_live) when the previous step computed the
  // scores of a seen chunk. Both live: the straight-line step of the dense
  // loop (masked only where the diagonal or the end of the sequence cuts
  // the next chunk); otherwise only the half that exists.
  auto chunk_seen = [&](int ch, bool block_seen) __attribute__((always_inline)) {
    return block_seen && ch * 32 < N && !(CAUSAL && ch * 32 > qw0 + QPW - 1);
  };
  auto finish_chunk = [&](const lds_u8* kt, int cc) __attribute__((always_inline)) {
    bf16x8 vf[DB], pf[QB];
    read_v(kt, cc, vf);
    exponentiate(s_cur, pf);
    accumulate_pv(vf, pf);
  };
  auto sparse_step = [&](const lds_u8* kt, int cc, const lds_u8* ktn, int ccn, int next_ch, bool next_live,
                         bool& cur_live, auto mask) __attribute__((always_inline)) {
    if (cur_live && next_live) {
      finish_chunk(kt, cc);
      scores(ktn, ccn, next_ch, mask);
    } else if (cur_live) {
      finish_chunk(kt, cc);
    } else if (next_live) {
      scores(ktn, ccn, next_ch, mask);
    }
    cur_live = next_live;
  };

  // ---- key loop: tiles in workgroup lock-step, chunks per wave. The last
  // chunk of tile t reads K of tile t+1, so tile t+1 is published by the
  // barrier just before it; at that point every wave is done with tile t-1,
  // whose stage receives tile t+STAGES-1. Tiles before t_steady need no mask
  // in any wave (this tile's chunks and the first chunk of the next): they
  // run in a loop of their own with branch-free bodies; the diagonal and the
  // end of the sequence take the masked path. Stage bases are run-time values.
  auto stage_base = [&](int t) __attribute__((always_inline)) {
    return smem + uniform(((t - t_lo) % STAGES) * STAGE_BYTES);
  };
  auto publish_next = [&](int t) __attribute__((always_inline)) {
    if (t + STAGES - 2 < n_kv) {
      wait_vmcnt_le<(STAGES - 3) * OPS>();  // tile t+1 landed; tiles up to t+STAGES-2 may fly
    } else {
      wait_vmcnt0();
    }
    __syncthreads();
    if (t + STAGES - 1 < n_kv) issue_tile_copy(t + STAGES - 1);
  };
  // Q and the first STAGES-1 tiles landed, on every path into the key loop.
  // The compiler counts the Q loads but not the copies (inline assembly), so
  // to it the Q loads are the newest ones, covered only by a full wait; a
  // path left without one (even an infeasible one of its control flow) makes
  // it wait for Q inside the loop, which in fact holds each wave, on every
  // tile, until its newest copy has landed. The prologue tiles are issued
  // together, so waiting for the second costs little.
  wait_vmcnt0();
  if (n_kv > t_lo) {
    __syncthreads();
    if constexpr (SPARSE) {
      // (the first chunk's scores; the loop below consumes them)
    } else if (n_ch > c_lo) {
      if (first_mask > c_lo) {
        scores(smem, 0, c_lo, std::false_type{});
      } else {
        scores(smem, 0, c_lo, std::true_type{});
      }
    }
  }
  // every wave's first masked chunk is at or after F
  const int F = CAUSAL ? min(q0, N) / 32 : N / 32;
  // (a tile is mask-free for every wave when its chunks, and the first chunk
  // of the next tile, all come before F)
  const int t_steady = min(n_kv - 1, F >= 1 ? (F - 1) / CPT : 0);
  int t = t_lo;
  if constexpr (SPARSE) {
    // Listed tiles before t_clean need no element mask in any wave (below
    // every diagonal of the workgroup and inside the sequence; the list is
    // in key order, so they come first): an unmasked region, then a masked
    // one, as in the dense loop.
    // (head dim 256: one masked region only; the second copy of the chunk
    // code does not fit the register budget there)
    int t_clean = 0;
    if constexpr (D <= 128) {
      const int clean_end = min(CAUSAL ? q0 : N, N - N % BN);  // tiles wholly before this key need no mask
      while (t_clean < n_kv && (kv_tile_of(t_clean) + 1) * BN <= clean_end) ++t_clean;
    }
    bool cur_live = false;
    auto run = [&](int t_end, auto mask) __attribute__((always_inline)) {
      for (; t < t_end; ++t) {
        const lds_u8* kt = stage_base(t);
        const bool more = t + 1 < n_kv;
        const int tile = kv_tile_of(t);
        // the next chunk of the last tile of the unmasked region belongs to the masked one
        const bool next_tile_clean = !decltype(mask)::value && t + 1 < t_clean;
        if constexpr (CPT == 2) {
          sparse_step(kt, 0, kt, 1, tile * 2 + 1, chunk_seen(tile * 2 + 1, sees_tile(t)), cur_live, mask);
          if (more) publish_next(t);
          const int nch = more ? kv_tile_of(t + 1) * 2 : 0;
          const bool nl = more && chunk_seen(nch, sees_tile(t + 1));
          if (decltype(mask)::value || next_tile_clean) {
            sparse_step(kt, 1, stage_base(t + 1), 0, nch, nl, cur_live, mask);
          } else {
            sparse_step(kt, 1, stage_base(t + 1), 0, nch, nl, cur_live, std::true_type{});
          }
        } else {
          if (more) publish_next(t);
          const int nch = more ? kv_tile_of(t + 1) : 0;
          const bool nl = more && chunk_seen(nch, sees_tile(t + 1));
          if (decltype(mask)::value || next_tile_clean) {
            sparse_step(kt, 0, stage_base(t + 1), 0, nch, nl, cur_live, mask);
          } else {
            sparse_step(kt, 0, stage_base(t + 1), 0, nch, nl, cur_live, std::true_type{});
          }
        }
      }
    };
    if (n_kv > 0) {  // scores of the first chunk (tile 0, published above)
      const int ch0 = kv_tile_of(0) * CPT;
      const bool live0 = chunk_seen(ch0, sees_tile(0));
      if (t_clean > 0) {
        sparse_step(smem, 0, smem, 0, ch0, live0, cur_live, std::false_type{});
      } else {
        sparse_step(smem, 0, smem, 0, ch0, live0, cur_live, std::true_type{});
      }
    }
    run(t_clean, std::false_type{});
    run(n_kv, std::true_type{});
  } else if constexpr (CPT == 2) {
    for (; t < t_steady; ++t) {
      const lds_u8* kt = stage_base(t);
      chunk_step(kt, 0, kt, 1, 2 * t, std::false_type{});
      publish_next(t);
      chunk_step(kt, 1, stage_base(t + 1), 0, 2 * t + 1, std::false_type{});
    }
    for (; t < n_kv; ++t) {
      const lds_u8* kt = stage_base(t);
      if (2 * t < n_ch) chunk_step(kt, 0, kt, 1, 2 * t, std::true_type{});
      if (t + 1 < n_kv) publish_next(t);
      if (2 * t + 1 < n_ch) chunk_step(kt, 1, stage_base(t + 1), 0, 2 * t + 1, std::true_type{});
    }
  } else {
    // one chunk per tile: chunk t reads K of tile t+1, published first
    for (; t < t_steady; ++t) {
      publish_next(t);
      chunk_step(stage_base(t), 0, stage_base(t + 1), 0, t, std::false_type{});
    }
    for (; t < n_kv; ++t) {
      if (t + 1 < n_kv) publish_next(t);
      if (t < n_ch) chunk_step(stage_base(t), 0, stage_base(t + 1), 0, t, std::true_type{});
    }
  }

  // ---- epilogue: O = acc / l, lse = (m + log2 l) ln 2
  if constexpr (SPLIT) {
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      const float l = kRowSumOnMatrix ? lsum[qb][0] : sum_over_row_groups(l_part[qb]);
      const int row = qw0 + qb * 16 + L;
      if (row < N) {
        // this part's O (fp32) and lse; a row with no key in the part (l = 0)
        // gets O = 0, lse = -inf, which the merge weighs by exp(-inf) = 0
        const size_t prow = ((size_t)part * p.B * p.Hq + (size_t)(b * p.Hq + h)) * N + row;
        const float inv = l > 0.f ? 1.0f / l : 0.f;
#pragma unroll
        for (int db = 0; db < DB; ++db) *(f32x4*)(p.o_part + prow * D + db * 16 + g * 4) = acc[db][qb] * inv;
        if (g == 0) p.lse_part[prow] = l > 0.f ? (m_ref[qb] + log2_fast(l)) * kLn2 : kNegInf;
      }
    }
  } else {
    // O leaves as whole rows through each wave's region of the now idle K/V
    // ring (store_rows_through_lds). All workgroups finish at nearly the
    // same time, so this final write-back of O is a burst, which drains
    // faster in whole cache lines.
    static_assert(NW * staged_rows_bytes<D>(QPW) <= STAGES * STAGE_BYTES, "O staging must fit in the K/V ring");
    __syncthreads();  // every wave is done with the K/V ring (no copy is in flight)
    float inv[QB];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      const float l = kRowSumOnMatrix ? lsum[qb][0] : sum_over_row_groups(l_part[qb]);
      const int row = qw0 + qb * 16 + L;
      // (sparse: a row that saw no key has l = 0 and gets O = 0, lse = -inf)
      inv[qb] = (!SPARSE || l > 0.f) ? 1.0f / l : 0.f;
      if (g == 0 && row < N) lseg[row] = (!SPARSE || l > 0.f) ? (m_ref[qb] + log2_fast(l)) * kLn2 : kNegInf;
    }
    store_rows_through_lds<D, QB>(smem + wave * staged_rows_bytes<D>(QPW), acc, inv, og, qw0, N, lane);
  }
}

// ------------------------------------------------------------------ split-KV merge
//
// The partial results of the key-range parts of a row are combined with the
// online-softmax rule one level up (the merge of per-device partial results
// in "FlashAttention技术解析" section 4.2): lse = log sum_s exp(lse_s),
// O = sum_s exp(lse_s - lse) O_s. D / 4 lanes per row, 4 columns each.
template <int D>
__global__ __launch_bounds__(256) void fa_fwd_merge_kernel(FwdParams p, long long rows) {
  constexpr int LPR = D / 4;  // lanes per row
  const long long row = (long long)workgroup_index() * (256 / LPR) + threadIdx.x / LPR;
  const int c4 = threadIdx.x % LPR;
  if (row >= rows) return;
  const int S = p.n_splits;
  float m = kNegInf;
  for (int s = 0; s < S; ++s) m = fmaxf(m, p.lse_part[(size_t)s * rows + row]);
  f32x4 o = {0.f, 0.f, 0.f, 0.f};
  float wsum = 0.f;
  if (m != kNegInf) {  // always true for a valid row (key 0 is visible to every query)
    for (int s = 0; s < S; ++s) {
      const float w = __expf(p.lse_part[(size_t)s * rows + row] - m);
      wsum += w;
      o += w * *(const f32x4*)(p.o_part + ((size_t)s * rows + row) * D + c4 * 4);
    }
  }
  const float inv = wsum > 0.f ? 1.0f / wsum : 0.f;
  o *= inv;
  *(u32x2*)((__bf16*)p.o + row * D + c4 * 4) = u32x2{pack_bf16x2(o[0], o[1]), pack_bf16x2(o[2], o[3])};
  if (c4 == 0) p.lse[row] = m + __logf(wsum);
}

// ------------------------------------------------------------------ launch
// Head dim 256: 16 query rows per wave (the accumulator and Q^T keep the
// register footprint of d = 128) and 32-key tiles (a 3-stage K/V ring of
// 96 KiB).
template <int D>
struct FwdCfg {
  static constexpr int QPW = D == 256 ? 16 : 32, NW = 8, STAGES = 3, BN = D == 256 ? 32 : 64;
};

// 4-wave workgroups of 128 rows with 32-key tiles and registers kept within
// 256 per wave, so two workgroups share a CU (four at head dim 64), for the
// shapes where the 256-row workgroups leave the compute units waiting:
//   * short sequences (a head's queries fill one or two tiles, little work
//     per byte): one workgroup's loads overlap another's math;
//   * grids of fewer than two 256-row workgroups per compute unit: twice as
//     many workgroups;
//   * causal at head dim 64: four resident workgroups cover the waves that
//     stop early at the diagonal.
constexpr int kShortSeqMaxN = 512;
constexpr long long kFullGridWorkgroups = 2 * 256;  // two per compute unit on the 256 CUs of gfx950
struct FwdShortCfg {
  static constexpr int QPW = 32, NW = 4, STAGES = 3, BN = 32;
};

template <int D, bool CAUSAL>
static hipError_t launch_fwd_bf16_short(const FwdParams& p_in, hipStream_t stream) {
  using C = FwdShortCfg;
  FwdParams p = p_in;
  p.n_tiles = (p.N + C::QPW * C::NW - 1) / (C::QPW * C::NW);
  const unsigned grid = (unsigned)(p.n_tiles * p.B * p.Hq);
  hipLaunchKernelGGL((fa_fwd_bf16_kernel<D, CAUSAL, C::QPW, C::NW, true, C::STAGES, false, C::BN>), dim3(grid),
                     dim3(C::NW * 64), 0, stream, p);
  return hipGetLastError();
}

template <int D, bool CAUSAL>
static hipError_t launch_fwd_bf16_cfg(const FwdParams& p_in, hipStream_t stream) {
  if constexpr (D <= 128) {
    const long long wg_full = (long long)((p_in.N + 255) / 256) * p_in.B * p_in.Hq;  // 256-row workgroups
    if (p_in.N <= kShortSeqMaxN || wg_full < kFullGridWorkgroups || (D == 64 && CAUSAL))
      return launch_fwd_bf16_short<D, CAUSAL>(p_in, stream);
  }
  using C = FwdCfg<D>;
  FwdParams p = p_in;
  p.n_tiles = (p.N + C::QPW * C::NW - 1) / (C::QPW * C::NW);
  const unsigned grid = (unsigned)(p.n_tiles * p.B * p.Hq);
  hipLaunchKernelGGL((fa_fwd_bf16_kernel<D, CAUSAL, C::QPW, C::NW, true, C::STAGES, false, C::BN>), dim3(grid),
                     dim3(C::NW * 64), 0, stream, p);
  return hipGetLastError();
}

template <int D, bool CAUSAL>
static hipError_t launch_fwd_bf16_split_cfg(const FwdParams& p_in, hipStream_t stream) {
  using C = FwdCfg<D>;
  FwdParams p = p_in;
  p.n_tiles = (p.N + C::QPW * C::NW - 1) / (C::QPW * C::NW);
  const unsigned grid = (unsigned)(p.n_tiles * p.B * p.Hq * p.n_splits);
  hipLaunchKernelGGL((fa_fwd_bf16_kernel<D, CAUSAL, C::QPW, C::NW, true, C::STAGES, true, C::BN>), dim3(grid),
                     dim3(C::NW * 64), 0, stream, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const long long rows = (long long)p.B * p.Hq * p.N;
  const long long rows_per_block = 256 / (D / 4);
  hipLaunchKernelGGL((fa_fwd_merge_kernel<D>), dim3((unsigned)((rows + rows_per_block - 1) / rows_per_block)), dim3(256), 0,
                     stream, p, rows);
  return hipGetLastError();
}

hipError_t launch_fwd_bf16_splitkv(const FwdParams& p, int d, bool causal, hipStream_t stream) {
  if (d == 256) return causal ? launch_fwd_bf16_split_cfg<256, true>(p, stream) : launch_fwd_bf16_split_cfg<256, false>(p, stream);
  if (d == 128) return causal ? launch_fwd_bf16_split_cfg<128, true>(p, stream) : launch_fwd_bf16_split_cfg<128, false>(p, stream);
  if (d == 64) return causal ? launch_fwd_bf16_split_cfg<64, true>(p, stream) : launch_fwd_bf16_split_cfg<64, false>(p, stream);
  return hipErrorInvalidValue;
}

template <int D, bool CAUSAL>
static hipError_t launch_fwd_bf16_sparse_cfg(const FwdParams& p_in, hipStream_t stream) {
  using C = FwdCfg<D>;
  FwdParams p = p_in;
  p.n_tiles = (p.N + C::QPW * C::NW - 1) / (C::QPW * C::NW);
  const unsigned grid = (unsigned)(p.n_tiles * p.B * p.Hq);
  hipLaunchKernelGGL((fa_fwd_bf16_kernel<D, CAUSAL, C::QPW, C::NW, true, C::STAGES, false, C::BN, true>), dim3(grid),
                     dim3(C::NW * 64), 0, stream, p);
  return hipGetLastError();
}

hipError_t launch_fwd_bf16_blocksparse(const FwdParams& p, int d, bool causal, hipStream_t stream) {
  if (d == 256) return causal ? launch_fwd_bf16_sparse_cfg<256, true>(p, stream) : launch_fwd_bf16_sparse_cfg<256, false>(p, stream);
  if (d == 128) return causal ? launch_fwd_bf16_sparse_cfg<128, true>(p, stream) : launch_fwd_bf16_sparse_cfg<128, false>(p, stream);
  if (d == 64) return causal ? launch_fwd_bf16_sparse_cfg<64, true>(p, stream) : launch_fwd_bf16_sparse_cfg<64, false>(p, stream);
  return hipErrorInvalidValue;
}

template <int D, bool CAUSAL>
static hipError_t launch_fwd_fp8_cfg(const FwdParams& p_in, hipStream_t stream) {
  using C = FwdCfg<D>;
  FwdParams p = p_in;
  p.n_tiles = (p.N + C::QPW * C::NW - 1) / (C::QPW * C::NW);
  const unsigned grid = (unsigned)(p.n_tiles * p.B * p.Hq);
  hipLaunchKernelGGL((fa_fwd_bf16_kernel<D, CAUSAL, C::QPW, C::NW, true, C::STAGES, false, C::BN, false, true>),
                     dim3(grid), dim3(C::NW * 64), 0, stream, p);
  return hipGetLastError();
}

hipError_t launch_fwd_fp8(const FwdParams& p, int d, bool causal, hipStream_t stream) {
  if (d == 256) return causal ? launch_fwd_fp8_cfg<256, true>(p, stream) : launch_fwd_fp8_cfg<256, false>(p, stream);
  if (d == 128) return causal ? launch_fwd_fp8_cfg<128, true>(p, stream) : launch_fwd_fp8_cfg<128, false>(p, stream);
  return hipErrorInvalidValue;
}

hipError_t launch_fwd_bf16(const FwdParams& p, int d, bool causal, hipStream_t stream) {
  if (d == 256) return causal ? launch_fwd_bf16_cfg<256, true>(p, stream) : launch_fwd_bf16_cfg<256, false>(p, stream);
  if (d == 128) return causal ? launch_fwd_bf16_cfg<128, true>(p, stream) : launch_fwd_bf16_cfg<128, false>(p, stream);
  if (d == 64) return causal ? launch_fwd_bf16_cfg<64, true>(p, stream) : launch_fwd_bf16_cfg<64, false>(p, stream);
  return hipErrorInvalidValue;
}

}  // namespace fa

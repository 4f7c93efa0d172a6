// Device helpers shared by the attention kernels (gfx950 / CDNA4, wave64).
//
// Fragment layouts of the matrix instructions used here (checked on the
// device against a host matmul before any kernel relied on them):
//
//  v_mfma_f32_16x16x32_bf16  D[16x16] = A[16x32] * B[32x16] + C
//    A: lane l holds row (l % 16), k = (l / 16) * 8 + e,  e = 0..7  (8 bf16)
//    B: lane l holds col (l % 16), k = (l / 16) * 8 + e,  e = 0..7  (8 bf16)
//    C/D: lane l holds col (l % 16), rows (l / 16) * 4 + r, r = 0..3 (4 f32)
//  v_mfma_f32_16x16x4_f32    D[16x16] = A[16x4] * B[4x16] + C
//    A: lane l holds row (l % 16), k = l / 16;  B: col (l % 16), k = l / 16
//    C/D: as above.
//  ds_read_b64_tr_b16: within each group of 16 lanes, lane L supplies the
//    address of four consecutive 16-bit values D[L][0..3]; output lane
//    o = 4a + b receives D[a][b], D[a+4][b], D[a+8][b], D[a+12][b].
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef int i32x8 __attribute__((ext_vector_type(8)));

#define FA_LDS __attribute__((address_space(3)))
#define FA_GLOBAL __attribute__((address_space(1)))

typedef FA_LDS unsigned char lds_u8;

constexpr float kLn2 = 0.693147180559945309417f;
constexpr float kNegInf = -__builtin_inff();

__device__ __forceinline__ f32x4 mfma_bf16_16x16x32(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma_f32_16x16x4(float a, float b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

// v_mfma_scale_f32_16x16x128_f8f6f4 with both operands e4m3 and unit block
// scales (E8M0 127 = 2^0): D[16x16] = A[16x128] * B[128x16] + C. Each lane
// supplies 32 bytes: A lane l row (l % 16), B lane l column (l % 16), with the
// same k positions for byte e of lane l in A and in B, so operands loaded with
// one common byte order per lane contract over matching k. C/D as above.
__device__ __forceinline__ f32x4 mfma_fp8_16x16x128(i32x8 a, i32x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, 0, 127, 0, 127);
}

// 2^x on the transcendental unit (v_exp_f32): 2^-inf = 0.
__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float log2_fast(float x) { return __builtin_amdgcn_logf(x); }

// Wave-uniform value from lane 0 (keeps LDS base addresses in scalar registers).
__device__ __forceinline__ int uniform(int x) { return __builtin_amdgcn_readfirstlane(x); }

// s_waitcnt encodings for gfx9: vmcnt in [3:0] and [15:14], expcnt [6:4], lgkmcnt [11:8].
__device__ __forceinline__ void wait_vmcnt0() { __builtin_amdgcn_s_waitcnt(0x0F70); }
// wait until at most N vector-memory operations of this wave are outstanding
// (the checking build FA_DEBUG_SYNC waits for all of them: every copy has
// landed before any tile is read, so no result can depend on copy timing)
template <int N>
__device__ __forceinline__ void wait_vmcnt_le() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
#ifdef FA_DEBUG_SYNC
  __builtin_amdgcn_s_waitcnt(0x0F70);
#else
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x0F70);
#endif
}

// This workgroup's place in the grid, for the work maps below. The checking
// build FA_REVERSE_GRID hands the places out in reverse launch order (last
// first), so that a result depending on which workgroups run first or
// together would change between the two builds.
__device__ __forceinline__ int workgroup_index() {
#ifdef FA_REVERSE_GRID
  return (int)gridDim.x - 1 - (int)blockIdx.x;
#else
  return (int)blockIdx.x;
#endif
}

// 16-byte direct global -> LDS copy: lane i writes lds_base + 16 * i.
__device__ __forceinline__ void copy16_global_to_lds(const void* gsrc, lds_u8* lds_base) {
  __builtin_amdgcn_global_load_lds((const FA_GLOBAL void*)gsrc, (FA_LDS void*)lds_base, 16, 0, 0);
}

// The same 16-byte copy issued from inline assembly: `base` is a wave-uniform
// global address, `voffset` this lane's byte offset from it, `lds_addr` the
// wave-uniform LDS byte address written by lane 0 (lane i writes +16 i).
// The compiler does not see the LDS write, so it inserts no wait for it:
// the caller waits with wait_vmcnt0() before the barrier that publishes the
// tile. M0 (the LDS address register of the instruction) is saved and
// restored around the copy.
__device__ __forceinline__ void copy16_global_to_lds_async(const void* base, uint32_t voffset, uint32_t lds_addr) {
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %3\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %2, %1\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "s"(base), "v"(voffset), "s"(lds_addr)
      : "memory");
}

// 4-byte variant: lane i writes lds_addr + 4 i.
__device__ __forceinline__ void copy4_global_to_lds_async(const void* base, uint32_t voffset, uint32_t lds_addr) {
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %3\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dword %2, %1\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "s"(base), "v"(voffset), "s"(lds_addr)
      : "memory");
}

__device__ __forceinline__ uint32_t lds_address(const lds_u8* p) { return (uint32_t)(uintptr_t)p; }

__device__ __forceinline__ bf16x8 lds_read_b128(const lds_u8* p) {
  return __builtin_bit_cast(bf16x8, *(const FA_LDS u32x4*)p);
}

__device__ __forceinline__ i16x4 lds_read_tr16_b64(const lds_u8* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((FA_LDS i16x4*)p);
}

// fp32 pair -> packed bf16 pair, round to nearest even (v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  f32x2 x = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(x, bf16x2));
}

// Max / sum over the four lanes l, l^16, l^32, l^48 (the lanes that share one
// column of a 16x16 accumulator block).
__device__ __forceinline__ float max_over_row_groups(float x) {
  x = fmaxf(x, __shfl_xor(x, 16, 64));
  x = fmaxf(x, __shfl_xor(x, 32, 64));
  return x;
}
__device__ __forceinline__ float sum_over_row_groups(float x) {
  x += __shfl_xor(x, 16, 64);
  x += __shfl_xor(x, 32, 64);
  return x;
}

__device__ __forceinline__ bool wave_any(bool p) { return __builtin_amdgcn_ballot_w64(p) != 0; }

// Workgroup id -> (flattened batch*head, query tile).
//
// Workgroups are handed to the 8 XCDs round-robin (id % 8). When the head
// count divides by 8, each XCD receives a contiguous run of heads, so the
// query tiles that stream one head's K/V (and the query heads of one grouped
// K/V head, which are adjacent) share that XCD's L2. Within an XCD, and in
// the fallback order, tiles go heaviest first when `heavy_first` is set
// (causal: the last query tile sees the most keys), so the light tiles fill
// the tail of the schedule.
struct TileCoord {
  int head;
  int tile;
};
__device__ __forceinline__ TileCoord map_workgroup(int wg, int n_heads, int n_tiles, bool heavy_first) {
  int head, rank;
  if ((n_heads & 7) == 0) {
    const int per_xcd = n_heads >> 3;
    const int xcd = wg & 7;
    const int j = wg >> 3;
    rank = j / per_xcd;
    head = xcd * per_xcd + (j - rank * per_xcd);
  } else {
    rank = wg / n_heads;
    head = wg - rank * n_heads;
  }
  return TileCoord{head, heavy_first ? (n_tiles - 1 - rank) : rank};
}

// Stores a wave's results as whole bf16 rows. An accumulator acc[db][rb]
// holds, in lane (L = lane & 15, g = lane >> 4), row 16 rb + L, columns
// 16 db + 4 g .. 16 db + 4 g + 3, times mul[rb]; stored directly, every
// instruction would write 16 rows in 32-byte pieces. The rows go through
// `region` (16 NRB rows of 2 D + 16 bytes owned by this wave; the padding
// spreads the 16 rows of a block over the LDS banks for the 8-byte writes)
// and leave 16 bytes per lane, so that an instruction writes 64 x 16 bytes of
// consecutive rows, in whole cache lines. Row r goes to out + (row0 + r) D
// when row0 + r < n_rows. The wave reads back only what it wrote itself, and
// its LDS operations complete in order.
template <int D, int NRB>
__device__ __forceinline__ void store_rows_through_lds(lds_u8* region, const f32x4 (&acc)[D / 16][NRB],
                                                       const float (&mul)[NRB], __bf16* out, int row0, int n_rows,
                                                       int lane) {
  constexpr int RS = 2 * D + 16;   // bytes per staged row
  constexpr int LPR = 2 * D / 16;  // lanes per row when storing
  constexpr int RPI = 64 / LPR;    // rows per store instruction
  const int g = lane >> 4, L = lane & 15;
#pragma unroll
  for (int rb = 0; rb < NRB; ++rb)
#pragma unroll
    for (int db = 0; db < D / 16; ++db) {
      const f32x4 v = acc[db][rb] * mul[rb];
      *(FA_LDS u32x2*)(region + (rb * 16 + L) * RS + (db * 16 + g * 4) * 2) =
          u32x2{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
    }
#pragma unroll
  for (int r0 = 0; r0 < NRB * 16; r0 += RPI) {
    const int r = r0 + lane / LPR;
    const u32x4 v = *(const FA_LDS u32x4*)(region + r * RS + (lane % LPR) * 16);
    if (row0 + r < n_rows) *(u32x4*)((char*)(out + (size_t)(row0 + r) * D) + (lane % LPR) * 16) = v;
  }
}
// LDS bytes store_rows_through_lds stages for `rows` rows
template <int D>
constexpr int staged_rows_bytes(int rows) { return rows * (2 * D + 16); }

}  // namespace fa

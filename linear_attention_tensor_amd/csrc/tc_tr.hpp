// tc_tr.hpp — 64-row blocks of bf16 rows (K or V rows as they are in memory)
// in LDS, read back as transposed operands of v_mfma_f32_32x32x16_bf16
// (gfx950), shared by the fused layer's kernels.
//
// Layout of a block: row c (token c of the block) holds that token's D
// features; its 16-byte piece p (features 8p .. 8p+7) sits at position
// p ^ swz<D>(c).  The operand of MFMA k-step KK for the 32 features
// 32 dt .. 32 dt + 31 needs, in lane (col, hh), tokens 16 KK + 8 hh .. +7 of
// feature 32 dt + col, in that order: two ds_read_b64_tr_b16 of 4 rows each.
// Within each 16-lane group such a read gives lane j element j % 4 of the
// 8-byte vectors addressed by lanes 4 r + j / 4 (r = 0..3), i.e. one feature
// of 4 consecutive rows.  Over a wave the 32 pieces read fall exactly twice
// on every 4-bank group (two LDS cycles, no further conflict).
// Kernels that also read whole 16-byte pieces of rows (row-major MFMA
// operands, 16 rows per quarter wave) use the RR variant of the permutation,
// which adds (c / 4) % 4 to it: the transpose reads of a quarter wave keep
// their 8 distinct positions, and 16 consecutive rows at one piece now fall
// on 16 distinct 4-bank groups as well.
#pragma once

#include "tc_common.hpp"
#include "tc_mfma.hpp"

namespace tc {
namespace tr {

template <int D, bool RR = false>
__device__ __forceinline__ int swz(int c) {
  static_assert(D == 64 || D == 128, "rows of 8 or 16 pieces");
  return (D == 128 ? 4 * (c & 3) : 4 * ((c >> 1) & 1)) + (RR ? (c >> 2) & 3 : 0);
}

// Global byte offset, from the block's first row, of the piece that LDS slot
// s (16 bytes at 16 s) of the block holds.  A global -> LDS copy in which
// lane l of an instruction fills slot s0 + l reads from there.
template <int D, bool RR = false>
__device__ __forceinline__ int slot_src(int s) {
  const int row = s / (D / 8), pos = s % (D / 8);
  return (row * D + 8 * (pos ^ swz<D, RR>(row))) * 2;
}

// Byte offset of piece p (features 8p .. 8p+7) of row r.
template <int D, bool RR = false>
__device__ __forceinline__ uint32_t piece_off(int r, int p) {
  return (uint32_t)(r * 2 * D + 16 * (p ^ swz<D, RR>(r)));
}

typedef short s16x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint2 lds_tr(const char* base, uint32_t off) {
  const s16x4 x = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) s16x4*)(base + off));
  return __builtin_bit_cast(uint2, x);
}

// Lane byte offset of the operand reads for feature tile dt: the 16 lanes i
// of a quarter wave (feature half (col / 16) % 2, token half hh) read row
// 8 hh + i / 4 at features 32 dt + 16 ((col / 16) % 2) + 4 (i % 4).
// (radd = 4: the same for the read of rows + 4, whose permutation differs in
// the RR variant; in the other one it is the first offset plus 4 rows.)
template <int D, bool RR = false>
__device__ __forceinline__ uint32_t lane_offset(int dt, int radd = 0) {
  const int l = lane_id(), col = l & 31, hh = l >> 5, i = col & 15;
  const int row = 8 * hh + (i >> 2) + radd;
  const int piece_lo = ((col & 16) >> 3) + ((col & 3) >> 1);  // piece within the 32 features of a tile
  const int half = col & 1;                                    // 8-byte half of that piece
  return (uint32_t)(row * 2 * D + 16 * ((4 * dt + piece_lo) ^ swz<D, RR>(row)) + 8 * half);
}
template <int D, bool RR = false>
__device__ __forceinline__ void lane_offsets(uint32_t* vls) {
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt) vls[dt] = lane_offset<D, RR>(dt);
}

// Operand of k-step KK (tokens 16 KK .. 16 KK + 15) for one feature tile
// (vl = lane_offset(dt)).
template <int D, int KK>
__device__ __forceinline__ bf16x8 ld1(const char* blk, uint32_t vl) {
  constexpr uint32_t RB = 2 * D;  // bytes per row
  const uint2 a = lds_tr(blk, vl + (16 * KK) * RB);
  const uint2 b = lds_tr(blk, vl + (16 * KK + 4) * RB);
  return mf::as_bf16x8(a.x, a.y, b.x, b.y);
}
// ... with separate lane offsets for the two reads (RR layout: vl0 =
// lane_offset<D, true>(dt), vl1 = lane_offset<D, true>(dt, 4)); adding 16 KK
// rows leaves either permutation unchanged
template <int D, int KK>
__device__ __forceinline__ bf16x8 ld1(const char* blk, uint32_t vl0, uint32_t vl1) {
  constexpr uint32_t RB = 2 * D;
  const uint2 a = lds_tr(blk, vl0 + (16 * KK) * RB);
  const uint2 b = lds_tr(blk, vl1 + (16 * KK) * RB);
  return mf::as_bf16x8(a.x, a.y, b.x, b.y);
}
// ... and for all D / 32 feature tiles
template <int D, int KK>
__device__ __forceinline__ void ld(const char* blk, const uint32_t* vls, bf16x8* x) {
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt) x[dt] = ld1<D, KK>(blk, vls[dt]);
}

}  // namespace tr
}  // namespace tc

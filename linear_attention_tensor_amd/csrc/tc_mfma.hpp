// tc_mfma.hpp — bf16 MFMA building blocks shared by the fused-layer kernels
// (gfx950, v_mfma_f32_32x32x16_bf16, 64-lane waves).
//
// Operand layout of v_mfma_f32_32x32x16_bf16 (lane l, col = l % 32,
// hh = l / 32): A(m, k) = lane m + 32 (k / 8), element k % 8; B(k, n) = lane
// n + 32 (k / 8), element k % 8; D(m, n) = lane n + 32 ((m / 4) % 2), element
// 4 (m / 8) + m % 4.  Any permutation of K shared by A and B is harmless.
#pragma once

#include "tc_common.hpp"

namespace tc {
namespace mf {

constexpr int KB = 64;  // keys per block

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) void* lds_ptr_t;

__device__ __forceinline__ floatx16 mfma32(bf16x8 a, bf16x8 b, floatx16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// two floats -> packed bf16 pair (hardware round-to-nearest-even)
__device__ __forceinline__ uint32_t cvt_pk(float lo, float hi) {
  const f32x2 f = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f, bf16x2));
}

__device__ __forceinline__ bf16x8 as_bf16x8(uint32_t a, uint32_t b, uint32_t c, uint32_t d) {
  return __builtin_bit_cast(bf16x8, u32x4{a, b, c, d});
}
__device__ __forceinline__ bf16x8 as_bf16x8(uint4 x) { return as_bf16x8(x.x, x.y, x.z, x.w); }

__device__ __forceinline__ float lo_f(uint32_t u) { return __uint_as_float(u << 16); }
__device__ __forceinline__ float hi_f(uint32_t u) { return __uint_as_float(u & 0xFFFF0000u); }

__device__ __forceinline__ floatx16 zero16() {
  floatx16 z;
#pragma unroll
  for (int i = 0; i < 16; ++i) z[i] = 0.f;
  return z;
}

// s_waitcnt vmcnt(n) with the other counters left alone (gfx9 encoding)
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

// lam^e for an integer e >= 0 (0^0 = 1, 1^e = 1).
struct Decay {
  float lam, log2lam;
  __device__ __forceinline__ explicit Decay(float l) : lam(l), log2lam(l > 0.f ? log2f(l) : 0.f) {}
  __device__ __forceinline__ float operator()(int e) const {
    if (e == 0) return 1.f;
    if (lam == 0.f) return 0.f;
    return __builtin_amdgcn_exp2f(static_cast<float>(e) * log2lam);
  }
};

// ---------------------------------------------------------------------------
// LDS layouts of one 64-key block (bf16, 16-byte slots).
//   K    D/64 halves of [64 rows][8 slots]: slot (c % 8) ^ ((m / 2) % 8) of
//        row m in half c / 8 holds chunk c (dims 8c..8c+7) of the key in row
//        m; row m holds key perm16(m) of the block.
//   V^T  [D rows][8 slots]: slot c ^ ((dv / 2) % 8) of row dv holds keys
//        8c..8c+7 of feature dv.
// In both, the 16-byte operand read of k-step j by lane (col, hh) sits at
// 128 col + 16 ((2 j + hh) ^ ((col / 2) % 8)) plus a constant, so a wave
// needs four address registers per block, and the 16 lanes of every
// quarter-wave hit 16 different slots of a 64-bank row (no conflicts).
__device__ __forceinline__ uint32_t lane_slot(int j) {
  const int l = lane_id(), col = l & 31, hh = l >> 5;
  return 128u * col + 16u * ((2 * j + hh) ^ ((col >> 1) & 7));
}
// Key order inside each 16-row group of a K block: rows 4-7 and 8-11 are
// swapped, so that the eight scores a lane holds for one PV k-step belong to
// eight consecutive keys (one 16-byte V^T read).
__device__ __forceinline__ int perm16(int m) {
  const int t = m & 15;
  return (m & ~15) | (t >= 4 && t < 8 ? t + 4 : (t >= 8 && t < 12 ? t - 4 : t));
}
// key (within a 64-key block) of element e of S^T tile kt held by this lane
__device__ __forceinline__ int key_of(int kt, int e, int hh) {
  return 32 * kt + 16 * (e >> 3) + 8 * hh + (e & 7);
}
// K slot s (0 .. 8 D - 1) -> (row m, chunk c)
template <int D>
__device__ __forceinline__ void k_slot_inv(int s, int& m, int& c) {
  m = (s >> 3) & 63;
  c = 8 * (s >> 9) + ((s & 7) ^ ((m >> 1) & 7));
}
// V^T slot s (0 .. 8 D - 1) -> (row dv, chunk c)
__device__ __forceinline__ void v_slot_inv(int s, int& dv, int& c) {
  dv = s >> 3;
  c = (s & 7) ^ ((dv >> 1) & 7);
}

// 16-byte LDS read at a byte offset from a block base
__device__ __forceinline__ bf16x8 lds16(const char* base, uint32_t off) {
  return as_bf16x8(*reinterpret_cast<const uint4*>(base + off));
}

}  // namespace mf
}  // namespace tc

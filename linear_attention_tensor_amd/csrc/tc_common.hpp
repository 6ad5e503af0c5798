// tc_common.hpp — device helpers shared by the gfx950 kernels of libtc.so.
//
// MFMA operand layouts used throughout (64-lane wavefront, lane = l):
//   v_mfma_f32_16x16x4_f32   A(m,k): lane m + 16k holds A[m][k]      (k < 4)
//                            B(k,n): lane n + 16k holds B[k][n]
//   v_mfma_f32_16x16x32_bf16 A(m,k): lane m + 16*(k/8) slot k%8       (k < 32)
//                            B(k,n): lane n + 16*(k/8) slot k%8
//   both                     D(m,n): lane n + 16*(m/4) element m%4
// Only the M/N placement matters for correctness: any permutation of K is
// harmless as long as A and B use the same one, which the kernels rely on.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace tc {

typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short shortx8 __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ int lane_id() { return threadIdx.x & 63; }
// Wave index as a scalar: tells the compiler that tests on it are wave-uniform.
__device__ __forceinline__ int wave_id() {
  return __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x >> 6));
}

// Workgroup barrier that orders LDS accesses only.  __syncthreads() also
// drains every outstanding global load (s_waitcnt vmcnt(0)), which would
// cancel register prefetching across the barrier.
//
// The wave's own LDS reads and writes are drained explicitly (s_waitcnt
// lgkmcnt(0)) before s_barrier: a fence restricted to LDS lets the compiler
// assume that the LDS of a CU serves every wave's requests in one order and
// leave the wait out, but requests from different waves can be served out of
// order, so a write issued just before the barrier could still be pending
// when another wave reads the same address after it.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// Buffer resource over [base, base + nbytes): raw buffer loads past the end
// (or at a negative offset, which wraps to a huge unsigned one) return zero
// instead of touching memory, so edge tiles need no branches around loads.
// 0x00020000 is the gfx9 word-3 value (raw dword data, no swizzle).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t nbytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), static_cast<short>(0),
                                           static_cast<int>(nbytes), 0x00020000);
}

__device__ __forceinline__ uint4 buf_load16(__amdgpu_buffer_rsrc_t r, int byte_off) {
  const u32x4 x = __builtin_amdgcn_raw_buffer_load_b128(r, byte_off, 0, 0);
  return make_uint4(x[0], x[1], x[2], x[3]);
}

// bfloat16 stored as raw 16-bit patterns (uint16_t) in memory.
__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}
// Round-to-nearest-even float -> bfloat16 bits (inputs here are finite).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return static_cast<uint16_t>(u >> 16);
}

// Two floats -> two round-to-nearest-even bf16 in one 32-bit word (lo first).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return static_cast<uint32_t>(f32_to_bf16(lo)) | (static_cast<uint32_t>(f32_to_bf16(hi)) << 16);
}

template <typename T> struct InT;
template <> struct InT<float> {
  __device__ __forceinline__ static float ld(const float* p, long i) { return p[i]; }
};
template <> struct InT<uint16_t> {
  __device__ __forceinline__ static float ld(const uint16_t* p, long i) { return bf16_to_f32(p[i]); }
};

// lam ** e for an integer e >= 0, with 0 ** 0 = 1 and 1 ** e = 1 exactly.
__device__ __forceinline__ float pow_int(float lam, int e) {
  if (e == 0) return 1.0f;
  if (lam == 0.0f) return 0.0f;
  if (lam == 1.0f) return 1.0f;
  return exp2f(static_cast<float>(e) * log2f(lam));
}

__device__ __forceinline__ floatx4 mfma4(float a, float b, floatx4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ floatx4 mfma_bf16_16x16x32(bf16x8 a, bf16x8 b, floatx4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// One wave accumulates a 16x16 fp32 tile: C += A[16 x K] * B[K x 16] with
// both operands in LDS, addressed through element strides so that either
// operand can be read transposed.  A(m,k) = pa[m*am + k*ak],
// B(k,n) = pb[k*bk + n*bn].
template <int K>
__device__ __forceinline__ floatx4 wave_mma_f32(const float* pa, int am, int ak,
                                                const float* pb, int bk, int bn, floatx4 c) {
  const int l = lane_id();
  const int r = l & 15, kk = l >> 4;
  const float* a = pa + r * am + kk * ak;
  const float* b = pb + kk * bk + r * bn;
#pragma unroll 8
  for (int k0 = 0; k0 < K; k0 += 4) {
    c = mfma4(a[k0 * ak], b[k0 * bk], c);
  }
  return c;
}

__device__ __forceinline__ floatx4 zero4() { return floatx4{0.f, 0.f, 0.f, 0.f}; }

// fp32 MFMA over LDS rows that are contiguous in k:
// acc[t] += A[16 x K] * B_t[K x 16], A rows at a + r sa, B_t given transposed
// (rows = columns of B_t) at bt + t bstep + r sb.
template <int K, int NT>
__device__ __forceinline__ void mma_rows(const float* a, int sa, const float* bt, int bstep, int sb,
                                         floatx4* acc) {
  const int l = lane_id(), r = l & 15, g = l >> 4;
  const float* ap = a + r * sa + 4 * g;
  const float* bp = bt + r * sb + 4 * g;
#pragma unroll
  for (int J = 0; J < K / 16; ++J) {
    const float4 x = *reinterpret_cast<const float4*>(ap + 16 * J);
    float4 y[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t) y[t] = *reinterpret_cast<const float4*>(bp + t * bstep + 16 * J);
#pragma unroll
    for (int t = 0; t < NT; ++t) acc[t] = mfma4(x.x, y[t].x, acc[t]);
#pragma unroll
    for (int t = 0; t < NT; ++t) acc[t] = mfma4(x.y, y[t].y, acc[t]);
#pragma unroll
    for (int t = 0; t < NT; ++t) acc[t] = mfma4(x.z, y[t].z, acc[t]);
#pragma unroll
    for (int t = 0; t < NT; ++t) acc[t] = mfma4(x.w, y[t].w, acc[t]);
  }
}
// (MFMA 4J + s takes k = 16J + 4g + s from lane (row, g), so one 16-byte
// read per operand feeds four MFMAs; the permutation of k is shared by A and
// B and changes nothing.)

}  // namespace tc

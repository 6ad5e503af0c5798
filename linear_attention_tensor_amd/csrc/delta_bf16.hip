// delta_bf16.hip — chunked delta-rule scan for bf16 inputs, d in {64, 128}
// (gfx950, v_mfma_f32_16x16x32_bf16).
//
// "DeltaNet-family linear attention variants", DeltaNet section: the write
// is the prediction error, e_t = beta_t (v_t - S_{t-1} k_t), S_t = S_{t-1} +
// e_t k_t^T, and the read after the write is o_t = S_t q_t (S is d_v x d_k).
//
// Chunked form (derived from that rule; the page gives only the per-token
// form).  In a chunk of 64 tokens entered with state S0, u_r = beta_r (v_r -
// S_{r-1} k_r) and S_{r-1} k_r = S0 k_r + sum_{i<r} <k_r, k_i> u_i, so
//   (I + diag(beta) tril_{-1}(K K^T)) U = diag(beta) (V - K S0^T),
//   U = A (V - K S0^T),  A = (I + diag(beta) tril_{-1}(K K^T))^-1 diag(beta),
//   O = Q S0^T + tril_0(Q K^T) U,      S = S0 + U^T K.
// A depends on K and beta only, so it is computed for every chunk at once:
//   delta_prep   per (chunk, b, h): A by forward substitution (fp32), stored
//                as a bf16 pair A = A_hi + A_lo, and K^T of the chunk;
//   delta_main   per (b, h, 16-row slice of S): walks the chunks in order.
// The rows of S are independent (row j only sees column j of V and U), so
// the slices need no communication.  The terms that feed the recurrence (K
// S0^T, A X, U^T K) use bf16 pairs for their fp32 operands, so each product
// keeps about 16 bits; the read-only terms (Q S0^T, tril(Q K^T) U) use one
// bf16 term, since their rounding does not accumulate.
#include "tc_common.hpp"
#include "tc_kernels.hpp"
#include "tc_mfma.hpp"

#include <math.h>

namespace tc {

namespace {

using namespace mf;

constexpr int CH = 64;   // tokens per chunk
constexpr int DVT = 16;  // rows of S per workgroup
constexpr int NXCD = 8;  // MI355X: 8 accelerator complex dies, dispatched round-robin

typedef int i32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ i32x4 raw_desc(const void* base, uint32_t nbytes) {
  const uint64_t a = reinterpret_cast<uint64_t>(base);
  return i32x4{static_cast<int>(a), static_cast<int>((a >> 32) & 0xFFFF), static_cast<int>(nbytes),
               0x00020000};
}

// 16 bytes per lane global -> LDS (lane i writes lds_base + 16 i), issued as
// inline asm so the compiler adds no wait for it before LDS reads and
// barriers; the kernel orders it with s_waitcnt vmcnt(0) and a barrier.  No
// register is written and the operands are read when the instruction issues.
__device__ __forceinline__ void dma16(i32x4 desc, const void* lds_base, int voffset) {
  const uint32_t lds = (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)lds_base;
  asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
               :
               : "s"(lds), "v"(voffset), "s"(desc)
               : "memory", "m0");
}

// Swizzled bf16 LDS rows of NCH 16-byte chunks: chunk c of row r sits at
// position c ^ swz(r), so 16 lanes reading one chunk of 16 consecutive rows
// (the 16x16x32 operand pattern) hit 16 different 4-bank groups.
template <int NCH>
__device__ __forceinline__ int swz(int r) {
  static_assert(NCH == 8 || NCH == 16, "row width");
  return NCH == 16 ? (r & 15) : ((r >> 1) & 7);
}
template <int NCH>
__device__ __forceinline__ int pos(int r, int c) {
  return (r * NCH + (c ^ swz<NCH>(r))) * 8;  // element offset of the chunk
}
template <int NCH>
__device__ __forceinline__ bf16x8 ldc(const uint16_t* base, int r, int c) {
  return as_bf16x8(*reinterpret_cast<const uint4*>(base + pos<NCH>(r, c)));
}
// element (r, col) of a swizzled array
template <int NCH>
__device__ __forceinline__ int epos(int r, int col) {
  return pos<NCH>(r, col >> 3) + (col & 7);
}

__device__ __forceinline__ floatx4 mma(bf16x8 a, bf16x8 b, floatx4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// x = hi + lo with hi, lo bf16 (about 16 significant bits)
__device__ __forceinline__ void split2(float x0, float x1, uint32_t& hi, uint32_t& lo) {
  hi = cvt_pk(x0, x1);
  lo = cvt_pk(x0 - lo_f(hi), x1 - hi_f(hi));
}

// ---------------------------------------------------------------------------
// delta_prep: one wave per (chunk, b, h).
template <int D>
__global__ __launch_bounds__(64) void delta_prep_kernel(const uint16_t* __restrict__ k,
                                                        const float* __restrict__ beta, int T,
                                                        int n_chunks, uint16_t* __restrict__ a_out,
                                                        uint16_t* __restrict__ kt_out) {
  constexpr int NCH = D / 8;
  constexpr int LS = CH + 4;  // fp32 L rows, 16-byte aligned
  __shared__ __attribute__((aligned(16))) uint16_t sK[CH * D];
  __shared__ __attribute__((aligned(16))) float sL[CH * LS];
  __shared__ float sB[CH];
  const int n = blockIdx.x, bh = blockIdx.y, l = threadIdx.x;
  const int t0 = n * CH;
  const __amdgpu_buffer_rsrc_t rk = make_rsrc(k + (long)bh * T * D, (uint32_t)T * D * 2);
  // lane l: key t0 + l (zero past T)
  uint4 kr[NCH];
#pragma unroll
  for (int c = 0; c < NCH; ++c) kr[c] = buf_load16(rk, ((t0 + l) * D + 8 * c) * 2);
  const float b = t0 + l < T ? beta[(long)bh * T + t0 + l] : 0.f;
  sB[l] = b;
#pragma unroll
  for (int c = 0; c < NCH; ++c) *reinterpret_cast<uint4*>(sK + pos<NCH>(l, c)) = kr[c];
  // K^T of the chunk: row dk holds the 64 keys (lane l writes key l)
  uint16_t* kt = kt_out + ((long)bh * n_chunks + n) * D * CH;
#pragma unroll
  for (int c = 0; c < NCH; ++c) {
    const uint32_t w4[4] = {kr[c].x, kr[c].y, kr[c].z, kr[c].w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      kt[(8 * c + 2 * e) * CH + l] = static_cast<uint16_t>(w4[e] & 0xFFFFu);
      kt[(8 * c + 2 * e + 1) * CH + l] = static_cast<uint16_t>(w4[e] >> 16);
    }
  }
  __syncthreads();
  // L = diag(beta) tril_{-1}(K K^T): tiles (mi, ni) with ni <= mi
  const int lr = l & 15, lg = l >> 4;
#pragma unroll
  for (int mi = 0; mi < 4; ++mi) {
#pragma unroll
    for (int ni = 0; ni < 4; ++ni) {
      if (ni > mi) {
#pragma unroll
        for (int e = 0; e < 4; ++e) sL[(16 * mi + 4 * lg + e) * LS + 16 * ni + lr] = 0.f;
        continue;
      }
      floatx4 acc = zero4();
#pragma unroll
      for (int ks = 0; ks < D / 32; ++ks)
        acc = mma(ldc<NCH>(sK, 16 * mi + lr, 4 * ks + lg), ldc<NCH>(sK, 16 * ni + lr, 4 * ks + lg), acc);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int r = 16 * mi + 4 * lg + e, c = 16 * ni + lr;
        sL[r * LS + c] = c < r ? sB[r] * acc[e] : 0.f;
      }
    }
  }
  __syncthreads();
  // M = (I + L)^-1, one column per lane: M[r] = e_r - sum_{i<r} L[r][i] M[i]
  float m[CH];
#pragma unroll
  for (int r = 0; r < CH; ++r) m[r] = 0.f;
#pragma unroll
  for (int r = 0; r < CH; ++r) {
    float s0 = r == l ? 1.f : 0.f, s1 = 0.f;
#pragma unroll
    for (int i = 0; i < r; i += 4) {  // L[r][i..i+3] is 0 past r - 1
      const float4 lv = *reinterpret_cast<const float4*>(sL + r * LS + i);
      s0 = fmaf(-lv.x, m[i], s0);
      s1 = fmaf(-lv.y, m[i + 1], s1);
      s0 = fmaf(-lv.z, m[i + 2], s0);
      s1 = fmaf(-lv.w, m[i + 3], s1);
    }
    m[r] = s0 + s1;
  }
  // A = M diag(beta): column l scaled by beta_l; out as bf16 pair [hi | lo]
  uint16_t* ao = a_out + ((long)bh * n_chunks + n) * 2 * CH * CH;
#pragma unroll
  for (int r = 0; r < CH; ++r) {
    const float a = m[r] * b;
    const uint16_t hi = f32_to_bf16(a);
    ao[r * CH + l] = hi;
    ao[CH * CH + r * CH + l] = f32_to_bf16(a - bf16_to_f32(hi));
  }
}

// ---------------------------------------------------------------------------
// delta_main: four waves per (b, h, slice); wave w owns tokens 16w..16w+15
// of the chunk in the M = 64 products and d_k columns w D/4 .. of the state.
template <int D>
struct DeltaLds {
  // double-buffered chunk inputs (swizzled rows)
  uint16_t q[2][CH * D];      // [token][dk]
  uint16_t k[2][CH * D];      // [token][dk]
  uint16_t kt[2][D * CH];     // [dk][token]
  uint16_t a[2][2][CH * CH];  // [hi|lo][token r][token c]
  uint16_t v[2][CH * DVT];    // [token][dv] plain
  // per-chunk work
  uint16_t h[2][DVT * D];     // state slice [hi|lo][dv][dk]
  uint16_t xt[2][DVT * CH];   // (V - K S0^T)^T [hi|lo][dv][token]
  uint16_t ut[2][DVT * CH];   // U^T [hi|lo][dv][token]
  uint16_t qk[CH * CH];       // tril_0(Q K^T) [r][c]
};

template <int D>
__global__ __launch_bounds__(256) void delta_main_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
    const uint16_t* __restrict__ a_in, const uint16_t* __restrict__ kt_in, int T, int n_chunks,
    int n_items, const float* __restrict__ S0, float* __restrict__ o, float* __restrict__ S_final) {
  constexpr int NCH = D / 8;  // chunks per q/k/h row
  constexpr int NT = D / 64;  // 16-column state tiles per wave
  __shared__ __attribute__((aligned(16))) DeltaLds<D> lds;

  // the slices of one head take consecutive items on one XCD (shared L2)
  const int per_xcd = (n_items + NXCD - 1) / NXCD;
  const int item = (blockIdx.x % NXCD) * per_xcd + blockIdx.x / NXCD;
  if (item >= n_items) return;
  const int bh = item / (D / DVT), dv0 = (item % (D / DVT)) * DVT;

  const int w = wave_id(), l = lane_id(), lr = l & 15, lg = l >> 4;
  const long tb = (long)bh * T;
  const i32x4 dq = raw_desc(q + tb * D, (uint32_t)T * D * 2);
  const i32x4 dk = raw_desc(k + tb * D, (uint32_t)T * D * 2);
  const i32x4 dv = raw_desc(v + tb * D, (uint32_t)T * D * 2);
  const i32x4 da = raw_desc(a_in + (long)bh * n_chunks * 2 * CH * CH, (uint32_t)n_chunks * 2 * CH * CH * 2);
  const i32x4 dkt = raw_desc(kt_in + (long)bh * n_chunks * D * CH, (uint32_t)n_chunks * D * CH * 2);

  // DMA of chunk n into buffer b: slot s of an array holds the 16-byte
  // chunk that its swizzle maps there.
  auto issue = [&](int n, int b) __attribute__((always_inline)) {
    const int t0 = n * CH;
    constexpr int NQ = CH * D / 8 / 256;  // 16-byte slots per thread per q/k array
#pragma unroll
    for (int i = 0; i < NQ; ++i) {
      const int seg = i * 4 + w, s = seg * 64 + l;
      const int r = s / NCH, c = (s % NCH) ^ swz<NCH>(r);
      dma16(dq, lds.q[b] + seg * 512, ((t0 + r) * D + 8 * c) * 2);
      dma16(dk, lds.k[b] + seg * 512, ((t0 + r) * D + 8 * c) * 2);
    }
#pragma unroll
    for (int i = 0; i < NQ; ++i) {  // K^T: D rows of 8 chunks
      const int seg = i * 4 + w, s = seg * 64 + l;
      const int r = s / 8, c = (s % 8) ^ swz<8>(r);
      dma16(dkt, lds.kt[b] + seg * 512, (((long)n * D + r) * CH + 8 * c) * 2);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {  // A hi, lo: 2 x 64 rows of 8 chunks (16 KiB)
      const int seg = i * 4 + w, s = seg * 64 + l;
      const int h = s / 512, r = (s / 8) % 64, c = (s % 8) ^ swz<8>(r);
      dma16(da, lds.a[b][0] + seg * 512, ((((long)n * 2 + h) * CH + r) * CH + 8 * c) * 2);
    }
    if (w < 2) {  // V slice: 64 rows of two 16-byte chunks
      const int s = w * 64 + l, r = s / 2, c = s % 2;
      dma16(dv, lds.v[b] + w * 512, ((t0 + r) * D + dv0 + 8 * c) * 2);
    }
  };

  // state slice: rows dv0 .. dv0+15; wave w owns columns D/4 w .. (NT tiles
  // of 16); D layout: lane lr + 16 lg holds rows 4 lg + e of column lr.
  floatx4 hs[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int r = 4 * lg + e, c = (D / 4) * w + 16 * t + lr;
      hs[t][e] = S0 != nullptr ? S0[((long)bh * D + dv0 + r) * D + c] : 0.f;
    }
  }
  auto publish_state = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int t = 0; t < NT; ++t) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int r = 4 * lg + e, c = (D / 4) * w + 16 * t + lr;
        const uint16_t hi = f32_to_bf16(hs[t][e]);
        lds.h[0][epos<NCH>(r, c)] = hi;
        lds.h[1][epos<NCH>(r, c)] = f32_to_bf16(hs[t][e] - bf16_to_f32(hi));
      }
    }
  };
  publish_state();
  if (n_chunks > 0) issue(0, 0);

  floatx4 o_prev = zero4();
  int t_prev = -1;  // first token of the chunk whose O is still in registers
  const int r0 = 16 * w;  // this wave's tokens in the chunk
#pragma unroll 1
  for (int n = 0; n < n_chunks; ++n) {
    const int b = n & 1, t0 = n * CH;
    wait_vmcnt<0>();  // chunk n (and the O stores of chunk n - 2) have landed
    lds_barrier();    // ... for every wave; chunk n - 1's buffers and h are free / published
    if (n + 1 < n_chunks) issue(n + 1, b ^ 1);
    // O of the previous chunk (stored now, so its stores overlap this chunk)
    if (t_prev >= 0) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int t = t_prev + r0 + 4 * lg + e;
        if (t < T) o[(tb + t) * D + dv0 + lr] = o_prev[e];
      }
    }

    // phase 1: tril_0(Q K^T) rows of this wave's keys; X = V - K S0^T; Q S0^T
#pragma unroll
    for (int ni = 0; ni < 4; ++ni) {
      // (Q K^T)^T tile: keys c = r0 + 4 lg + e (M), queries 16 ni + lr (N)
      floatx4 acc = zero4();
#pragma unroll
      for (int ks = 0; ks < D / 32; ++ks)
        acc = mma(ldc<NCH>(lds.k[b], r0 + lr, 4 * ks + lg), ldc<NCH>(lds.q[b], 16 * ni + lr, 4 * ks + lg), acc);
      const int rq = 16 * ni + lr, c0 = r0 + 4 * lg;
      uint32_t p0, p1;
      p0 = cvt_pk(c0 <= rq ? acc[0] : 0.f, c0 + 1 <= rq ? acc[1] : 0.f);
      p1 = cvt_pk(c0 + 2 <= rq ? acc[2] : 0.f, c0 + 3 <= rq ? acc[3] : 0.f);
      *reinterpret_cast<uint2*>(lds.qk + epos<8>(rq, c0)) = make_uint2(p0, p1);
    }
    floatx4 kh = zero4(), qh = zero4();
#pragma unroll
    for (int ks = 0; ks < D / 32; ++ks) {
      const bf16x8 hh = ldc<NCH>(lds.h[0], lr, 4 * ks + lg), hl = ldc<NCH>(lds.h[1], lr, 4 * ks + lg);
      const bf16x8 ka = ldc<NCH>(lds.k[b], r0 + lr, 4 * ks + lg);
      kh = mma(ka, hh, kh);
      kh = mma(ka, hl, kh);
      qh = mma(ldc<NCH>(lds.q[b], r0 + lr, 4 * ks + lg), hh, qh);
    }
    {
      // X^T row dv = lr, tokens r0 + 4 lg + e
      float x[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) x[e] = bf16_to_f32(lds.v[b][(r0 + 4 * lg + e) * DVT + lr]) - kh[e];
      uint32_t h0, h1, l0, l1;
      split2(x[0], x[1], h0, l0);
      split2(x[2], x[3], h1, l1);
      *reinterpret_cast<uint2*>(lds.xt[0] + epos<8>(lr, r0 + 4 * lg)) = make_uint2(h0, h1);
      *reinterpret_cast<uint2*>(lds.xt[1] + epos<8>(lr, r0 + 4 * lg)) = make_uint2(l0, l1);
    }
    lds_barrier();

    // phase 2: U = A X for this wave's tokens
    floatx4 u = zero4();
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      const bf16x8 ah = ldc<8>(lds.a[b][0], r0 + lr, 4 * ks + lg), al = ldc<8>(lds.a[b][1], r0 + lr, 4 * ks + lg);
      const bf16x8 xh = ldc<8>(lds.xt[0], lr, 4 * ks + lg), xl = ldc<8>(lds.xt[1], lr, 4 * ks + lg);
      u = mma(ah, xh, u);
      u = mma(ah, xl, u);
      u = mma(al, xh, u);
    }
    {
      uint32_t h0, h1, l0, l1;
      split2(u[0], u[1], h0, l0);
      split2(u[2], u[3], h1, l1);
      *reinterpret_cast<uint2*>(lds.ut[0] + epos<8>(lr, r0 + 4 * lg)) = make_uint2(h0, h1);
      *reinterpret_cast<uint2*>(lds.ut[1] + epos<8>(lr, r0 + 4 * lg)) = make_uint2(l0, l1);
    }
    lds_barrier();

    // phase 3: O = Q S0^T + tril_0(Q K^T) U;  S += U^T K
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
      qh = mma(ldc<8>(lds.qk, r0 + lr, 4 * ks + lg), ldc<8>(lds.ut[0], lr, 4 * ks + lg), qh);
    o_prev = qh;
    t_prev = t0;
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      const int c = (D / 4) * w + 16 * t + lr;  // d_k column (N)
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        const bf16x8 kt = ldc<8>(lds.kt[b], c, 4 * ks + lg);
        hs[t] = mma(ldc<8>(lds.ut[0], lr, 4 * ks + lg), kt, hs[t]);
        hs[t] = mma(ldc<8>(lds.ut[1], lr, 4 * ks + lg), kt, hs[t]);
      }
    }
    publish_state();  // read next after the barrier at the top of the loop
  }
  if (t_prev >= 0) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int t = t_prev + r0 + 4 * lg + e;
      if (t < T) o[(tb + t) * D + dv0 + lr] = o_prev[e];
    }
  }
  if (S_final != nullptr) {
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
      for (int e = 0; e < 4; ++e)
        S_final[((long)bh * D + dv0 + 4 * lg + e) * D + (D / 4) * w + 16 * t + lr] = hs[t][e];
  }
}

template <int D>
hipError_t run_delta_bf16(const uint16_t* q, const uint16_t* k, const uint16_t* v, const float* beta,
                          int BH, int T, const float* S0, float* o, float* S_final, void* ws,
                          hipStream_t s) {
  const int n_chunks = (T + CH - 1) / CH;
  uint16_t* a_ws = static_cast<uint16_t*>(ws);
  uint16_t* kt_ws = a_ws + (size_t)BH * n_chunks * 2 * CH * CH;
  if (n_chunks > 0)
    hipLaunchKernelGGL(delta_prep_kernel<D>, dim3(n_chunks, BH), dim3(64), 0, s, k, beta, T, n_chunks,
                       a_ws, kt_ws);
  const int n_items = BH * (D / DVT);
  const int grid = (n_items + NXCD - 1) / NXCD * NXCD;
  profile_mark_before(s);
  hipLaunchKernelGGL(delta_main_kernel<D>, dim3(grid), dim3(256), 0, s, q, k, v, a_ws, kt_ws, T,
                     n_chunks, n_items, S0, o, S_final);
  profile_mark_after(s);
  return hipGetLastError();
}

}  // namespace

bool delta_bf16_supported(bool bf16, int d) { return bf16 && (d == 64 || d == 128); }

size_t delta_bf16_ws_bytes(int B, int H, int T, int d) {
  const size_t n_chunks = (T + CH - 1) / CH;
  return (size_t)B * H * n_chunks * (2 * CH * CH + (size_t)d * CH) * sizeof(uint16_t);
}

hipError_t launch_delta_bf16(const void* q, const void* k, const void* v, const float* beta, int B,
                             int H, int T, int d, const float* S0, float* o, float* S_final, void* ws,
                             hipStream_t s) {
  const uint16_t* Q = static_cast<const uint16_t*>(q);
  const uint16_t* K = static_cast<const uint16_t*>(k);
  const uint16_t* V = static_cast<const uint16_t*>(v);
  if (d == 128) return run_delta_bf16<128>(Q, K, V, beta, B * H, T, S0, o, S_final, ws, s);
  if (d == 64) return run_delta_bf16<64>(Q, K, V, beta, B * H, T, S0, o, S_final, ws, s);
  return hipErrorInvalidValue;
}

}  // namespace tc

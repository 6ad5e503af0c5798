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
//   delta_prep   per (chunk, b, h): A by blocked inversion (fp32), stored
//                as a bf16 pair A = A_hi + A_lo;
//   delta_main   per (b, h, 16-row slice of S): walks the chunks in order;
//                it forms tril_0(Q K^T) (it depends on q and k only) from
//                the chunk's q and k rows itself, and takes the K^T operands
//                by transpose reads of the K rows, so that a chunk brings
//                only q, k, A and the V slice into LDS.
// The rows of S are independent (row j only sees column j of V and U), so
// the slices need no communication.  The terms that feed the recurrence (K
// S0^T, A X, U^T K) use bf16 pairs for their fp32 operands, so each product
// keeps about 16 bits; the read-only terms (Q S0^T, tril(Q K^T) U) use one
// bf16 term, since their rounding does not accumulate.
#include "tc_common.hpp"
#include "tc_kernels.hpp"
#include "tc_dma.hpp"
#include "tc_mfma.hpp"

#include <math.h>

namespace tc {

namespace {

using namespace mf;
using dma::dma16;
using dma::i32x4;
using dma::raw_desc;

constexpr int CH = 64;   // tokens per chunk
constexpr int DVT = 16;  // rows of S per workgroup
constexpr int NXCD = 8;  // MI355X: 8 accelerator complex dies, dispatched round-robin

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

// scheduling fence: keeps operand reads ahead of the MFMAs that use them
#define TC_SB() __builtin_amdgcn_sched_barrier(0)

__device__ __forceinline__ floatx4 mma(bf16x8 a, bf16x8 b, floatx4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// x = hi + lo with hi, lo bf16 (about 16 significant bits)
__device__ __forceinline__ void split2(float x0, float x1, uint32_t& hi, uint32_t& lo) {
  hi = cvt_pk(x0, x1);
  lo = cvt_pk(x0 - lo_f(hi), x1 - hi_f(hi));
}

// ---------------------------------------------------------------------------
// delta_prep: four waves per (chunk, b, h).  A leaves in 16-byte pieces per
// lane; one buffer holds in turn L and M = (I + L)^-1.
template <int D>
__global__ __launch_bounds__(256) void delta_prep_kernel(const uint16_t* __restrict__ k,
                                                         const float* __restrict__ beta, int T,
                                                         int n_chunks, uint16_t* __restrict__ a_out) {
  constexpr int NCH = D / 8;
  constexpr int LS = CH + 4;                 // fp32 rows of L and M, 16-byte aligned
  constexpr int NP = CH * NCH / 256;         // 16-byte pieces per thread of a [64][D] array
  __shared__ __attribute__((aligned(16))) uint16_t sK[CH * D];
  __shared__ __attribute__((aligned(16))) float sL[CH * LS];  // L, then M
  __shared__ float sT[4][16 * 17];                            // one block product per wave
  __shared__ float sB[CH];
  const int n = blockIdx.x, bh = blockIdx.y, t = threadIdx.x;
  const int w = wave_id(), l = lane_id(), lr = l & 15, lg = l >> 4;
  const int t0 = n * CH;
  const __amdgpu_buffer_rsrc_t rk = make_rsrc(k + (long)bh * T * D, (uint32_t)T * D * 2);

  // rows of K (zero past T); piece i of this thread is row s / NCH, chunk
  // s % NCH with s = 256 i + t
  uint4 kr[NP];
#pragma unroll
  for (int i = 0; i < NP; ++i) {
    const int s = i * 256 + t, row = s / NCH, c = s % NCH;
    kr[i] = buf_load16(rk, ((t0 + row) * D + 8 * c) * 2);
  }
  if (t < CH) sB[t] = t0 + t < T ? beta[(long)bh * T + t0 + t] : 0.f;
#pragma unroll
  for (int i = 0; i < NP; ++i) {
    const int s = i * 256 + t, row = s / NCH, c = s % NCH;
    *reinterpret_cast<uint4*>(sK + pos<NCH>(row, c)) = kr[i];
  }
  __syncthreads();
  // L = diag(beta) tril_{-1}(K K^T): wave w takes rows 16w.. (tiles ni <= w)
  {
    const int mi = w;
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
  // M = (I + L)^-1 by 16 x 16 blocks (L strictly lower triangular), in place:
  //   M_ii = (I + L_ii)^-1 by forward substitution (wave i, one column per
  //   lane; lanes 16.. repeat columns 0..15);
  //   M_ij = -M_ii sum_{k=j}^{i-1} L_ik M_kj (wave j), block row by block row.
  {
    const int c = l & 15;
    float md[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const float* row = sL + (16 * w + r) * LS + 16 * w;
      float s0 = r == c ? 1.f : 0.f, s1 = 0.f;
#pragma unroll
      for (int kk = 0; kk < r; kk += 2) {
        s0 = fmaf(-row[kk], md[kk], s0);
        if (kk + 1 < r) s1 = fmaf(-row[kk + 1], md[kk + 1], s1);
      }
      md[r] = s0 + s1;
    }
    if (l < 16) {
#pragma unroll
      for (int r = 0; r < 16; ++r) sL[(16 * w + r) * LS + 16 * w + c] = md[r];
    }
  }
  __syncthreads();
#pragma unroll
  for (int i = 1; i < 4; ++i) {
    const int j = w;
    floatx4 res = zero4();
    if (j < i) {
      floatx4 tt = zero4();  // sum_{k=j}^{i-1} L_ik M_kj
#pragma unroll
      for (int kb = 0; kb < 3; ++kb) {
        const int kk0 = j + kb;
        if (kk0 >= i) break;
#pragma unroll
        for (int kk = 0; kk < 16; kk += 4)
          tt = mfma4(sL[(16 * i + lr) * LS + 16 * kk0 + kk + lg], sL[(16 * kk0 + kk + lg) * LS + 16 * j + lr], tt);
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) sT[w][(4 * lg + e) * 17 + lr] = tt[e];
      floatx4 mm = zero4();  // M_ii tt (the wave reads back what it wrote)
#pragma unroll
      for (int kk = 0; kk < 16; kk += 4)
        mm = mfma4(sL[(16 * i + lr) * LS + 16 * i + kk + lg], sT[w][(kk + lg) * 17 + lr], mm);
      res = -mm;
    }
    __syncthreads();  // every wave is done reading L's row i
    if (j < i) {
#pragma unroll
      for (int e = 0; e < 4; ++e) sL[(16 * i + 4 * lg + e) * LS + 16 * j + lr] = res[e];
    }
    __syncthreads();
  }
  // A = M diag(beta), written as a bf16 pair A = A_hi + A_lo, [hi | lo] row-major
  uint16_t* ao = a_out + ((long)bh * n_chunks + n) * 2 * CH * CH;
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int s = i * 256 + t, r = s >> 3, c8 = 8 * (s & 7);
    float4 x0 = *reinterpret_cast<const float4*>(sL + r * LS + c8);
    float4 x1 = *reinterpret_cast<const float4*>(sL + r * LS + c8 + 4);
    x0.x *= sB[c8];
    x0.y *= sB[c8 + 1];
    x0.z *= sB[c8 + 2];
    x0.w *= sB[c8 + 3];
    x1.x *= sB[c8 + 4];
    x1.y *= sB[c8 + 5];
    x1.z *= sB[c8 + 6];
    x1.w *= sB[c8 + 7];
    uint32_t h[4], lo[4];
    split2(x0.x, x0.y, h[0], lo[0]);
    split2(x0.z, x0.w, h[1], lo[1]);
    split2(x1.x, x1.y, h[2], lo[2]);
    split2(x1.z, x1.w, h[3], lo[3]);
    *reinterpret_cast<uint4*>(ao + r * CH + c8) = make_uint4(h[0], h[1], h[2], h[3]);
    *reinterpret_cast<uint4*>(ao + CH * CH + r * CH + c8) = make_uint4(lo[0], lo[1], lo[2], lo[3]);
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
  uint16_t a[2][2][CH * CH];  // [hi|lo][token r][token c]
  uint16_t v[2][CH * DVT];    // [token][dv] plain
  // per-chunk work
  uint16_t h[2][DVT * D];     // state slice [hi|lo][dv][dk]
  uint16_t xt[2][DVT * CH];   // (V - K S0^T)^T [hi|lo][dv][token]
  uint16_t ut[2][DVT * CH];   // U^T [hi|lo][dv][token]
};

// ds_read_b64_tr_b16: lane j of each 16-lane group gets element j % 4 of the
// 8-byte pieces addressed by lanes 4 i + j / 4 (i = 0..3)
__device__ __forceinline__ uint2 lds_tr8(const uint16_t* base, int elem) {
  typedef short s16x4 __attribute__((ext_vector_type(4)));
  const s16x4 x = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) s16x4*)(base + elem));
  return __builtin_bit_cast(uint2, x);
}

template <int D>
__global__ __launch_bounds__(256) void delta_main_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
    const uint16_t* __restrict__ a_in, int T, int n_chunks, int n_items, const float* __restrict__ S0,
    float* __restrict__ o, float* __restrict__ S_final) {
  constexpr int NCH = D / 8;  // chunks per q/k/h row
  constexpr int NT = D / 64;  // 16-column state tiles per wave
  constexpr int NK = D / 32;  // k-steps over d_k
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
  const __amdgpu_buffer_rsrc_t ro = make_rsrc(o + tb * D, (uint32_t)T * D * 4);  // rows past T: dropped

  // DMA of chunk n into buffer b, in two parts issued during different
  // phases of the previous chunk (so that the workgroup's copy instructions
  // do not queue all at once).  Slot s of an array holds the 16-byte chunk
  // that its swizzle maps there.
  constexpr int NQ = CH * D / 8 / 256;  // 16-byte slots per thread per q/k array
  auto issue_qkv = [&](int n, int b) __attribute__((always_inline)) {
    const int t0 = n * CH;
#pragma unroll
    for (int i = 0; i < NQ; ++i) {
      const int seg = i * 4 + w, s = seg * 64 + l;
      const int r = s / NCH, c = (s % NCH) ^ swz<NCH>(r);
      dma16(dq, lds.q[b] + seg * 512, ((t0 + r) * D + 8 * c) * 2);
      dma16(dk, lds.k[b] + seg * 512, ((t0 + r) * D + 8 * c) * 2);
    }
    if (w < 2) {  // V slice: 64 rows of two 16-byte chunks
      const int s = w * 64 + l, r = s / 2, c = s % 2;
      dma16(dv, lds.v[b] + w * 512, ((t0 + r) * D + dv0 + 8 * c) * 2);
    }
  };
  auto issue_a = [&](int n, int b) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {  // A hi, lo: 2 x 64 rows of 8 chunks (16 KiB)
      const int seg = i * 4 + w, s = seg * 64 + l;
      const int h = s / 512, r = (s / 8) % 64, c = (s % 8) ^ swz<8>(r);
      dma16(da, lds.a[b][0] + seg * 512, ((((long)n * 2 + h) * CH + r) * CH + 8 * c) * 2);
    }
  };
  // copy instructions per wave and part (the waits below count them): q/k/v
  // 2 NQ, plus one V piece in waves 0 and 1; A 4
  constexpr int N_A = 4;

  // S^T slice: rows dk = (D/4) w + 16 t + 4 lg + e, column dv0 + lr (the
  // accumulator layout of S^T += K^T U); published as bf16 hi/lo rows
  // [dv][dk], four consecutive dk (8 bytes) per lane and tile.
  floatx4 hs[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int c = (D / 4) * w + 16 * t + 4 * lg + e;
      hs[t][e] = S0 != nullptr ? S0[((long)bh * D + dv0 + lr) * D + c] : 0.f;
    }
  }
  auto publish_state = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      const int c = (D / 4) * w + 16 * t + 4 * lg;
      uint32_t h0, h1, l0, l1;
      split2(hs[t][0], hs[t][1], h0, l0);
      split2(hs[t][2], hs[t][3], h1, l1);
      *reinterpret_cast<uint2*>(lds.h[0] + epos<NCH>(lr, c)) = make_uint2(h0, h1);
      *reinterpret_cast<uint2*>(lds.h[1] + epos<NCH>(lr, c)) = make_uint2(l0, l1);
    }
  };
  publish_state();
  if (T % CH != 0) {
    // A ragged last chunk copies rows past T, which the descriptors turn
    // into zeros; the buffers are cleared first as well, so those rows can
    // never hold what an earlier kernel left in LDS (U's rows past T are
    // 0 * X, which a NaN pattern there would poison).
    auto clear = [&](uint16_t* p, int bytes) __attribute__((always_inline)) {
      for (int i = threadIdx.x; i < bytes / 16; i += 256) reinterpret_cast<uint4*>(p)[i] = make_uint4(0, 0, 0, 0);
    };
    clear(&lds.q[0][0], (int)sizeof(lds.q));
    clear(&lds.k[0][0], (int)sizeof(lds.k));
    clear(&lds.v[0][0], (int)sizeof(lds.v));
    lds_barrier();
  }
  if (n_chunks > 0) {
    issue_qkv(0, 0);
    issue_a(0, 0);
  }

  floatx4 o_prev = zero4();
  int t_prev = -1;  // first token of the chunk whose O is still in registers
  const int r0 = 16 * w;  // this wave's tokens in the chunk
  // K^T operand pieces by transpose reads of K rows: lane j of group lg
  // addresses row R + j / 4, columns 4 (j % 4) .. of a 16-column tile, and
  // receives column j of rows R .. R + 3
  const int tr_row = lr >> 2, tr_col = 4 * (lr & 3);
#pragma unroll 1
  for (int n = 0; n < n_chunks; ++n) {
    const int b = n & 1, t0 = n * CH;
    // Copies complete in issue order.  Issued for chunk n during chunk n - 1:
    // q/k/v (phase 1), then A (phase 2).
    wait_vmcnt<N_A>();  // q, k, v of chunk n have landed
    lds_barrier();      // ... for every wave; chunk n - 1's buffers are free, the state is published
    const bool more = n + 1 < n_chunks;  // chunk n + 1 is copied during this one
    if (t_prev >= 0) {  // O of the previous chunk, stored now so the stores overlap this chunk
#pragma unroll
      for (int e = 0; e < 4; ++e)
        __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(o_prev[e]), ro,
                                              ((t_prev + r0 + 4 * lg + e) * D + dv0 + lr) * 4, 0, 0);
    }

    // phase 1: K S0^T, Q S0^T (this wave's tokens); X = V - K S0^T; and,
    // off the chain, tril_0(Q K^T) for this wave's queries
    bf16x8 ka[NK], hh[NK], hl[NK], qa[NK];
    TC_SB();
#pragma unroll
    for (int ks = 0; ks < NK; ++ks) {
      ka[ks] = ldc<NCH>(lds.k[b], r0 + lr, 4 * ks + lg);
      hh[ks] = ldc<NCH>(lds.h[0], lr, 4 * ks + lg);
      hl[ks] = ldc<NCH>(lds.h[1], lr, 4 * ks + lg);
      qa[ks] = ldc<NCH>(lds.q[b], r0 + lr, 4 * ks + lg);
    }
    TC_SB();
    if (more) issue_qkv(n + 1, b ^ 1);
    TC_SB();
    floatx4 kh = zero4(), kl = zero4(), qh = zero4();
#pragma unroll
    for (int ks = 0; ks < NK; ++ks) {
      kh = mma(ka[ks], hh[ks], kh);
      kl = mma(ka[ks], hl[ks], kl);
      qh = mma(qa[ks], hh[ks], qh);
    }
    // (Q K^T)^T tiles: keys 16 mt + 4 lg + e of query r0 + lr (only the
    // tiles with keys <= the wave's last query)
    floatx4 qkt[4];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
      qkt[mt] = zero4();
      if (mt <= w) {
#pragma unroll
        for (int ks = 0; ks < NK; ++ks) qkt[mt] = mma(ldc<NCH>(lds.k[b], 16 * mt + lr, 4 * ks + lg), qa[ks], qkt[mt]);
      }
    }
    {
      // X^T row dv = lr, tokens r0 + 4 lg + e
      float x[4];
#pragma unroll
      for (int e = 0; e < 4; ++e)
        x[e] = bf16_to_f32(lds.v[b][(r0 + 4 * lg + e) * DVT + lr]) - (kh[e] + kl[e]);
      uint32_t h0, h1, l0, l1;
      split2(x[0], x[1], h0, l0);
      split2(x[2], x[3], h1, l1);
      *reinterpret_cast<uint2*>(lds.xt[0] + epos<8>(lr, r0 + 4 * lg)) = make_uint2(h0, h1);
      *reinterpret_cast<uint2*>(lds.xt[1] + epos<8>(lr, r0 + 4 * lg)) = make_uint2(l0, l1);
    }
    // A of chunk n: loads issued after it are (if any) q/k/v of chunk n + 1.
    // The O stores between them are not counted: stores may complete ahead
    // of older loads, so the wait is exact only over loads (which complete in
    // order) and merely longer otherwise.
    if (more) {
      if (w < 2) wait_vmcnt<2 * NQ + 1>();
      else wait_vmcnt<2 * NQ>();
    } else {
      wait_vmcnt<0>();
    }
    lds_barrier();

    // phase 2: U = A X for this wave's tokens
    bf16x8 ah[2], al[2], xh[2], xl[2];
    TC_SB();
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      ah[ks] = ldc<8>(lds.a[b][0], r0 + lr, 4 * ks + lg);
      al[ks] = ldc<8>(lds.a[b][1], r0 + lr, 4 * ks + lg);
      xh[ks] = ldc<8>(lds.xt[0], lr, 4 * ks + lg);
      xl[ks] = ldc<8>(lds.xt[1], lr, 4 * ks + lg);
    }
    TC_SB();
    if (more) issue_a(n + 1, b ^ 1);
    TC_SB();
    floatx4 u = zero4(), u2 = zero4();
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      u = mma(ah[ks], xh[ks], u);
      u2 = mma(ah[ks], xl[ks], u2);
      u = mma(al[ks], xh[ks], u);
    }
    u += u2;
    {
      uint32_t h0, h1, l0, l1;
      split2(u[0], u[1], h0, l0);
      split2(u[2], u[3], h1, l1);
      *reinterpret_cast<uint2*>(lds.ut[0] + epos<8>(lr, r0 + 4 * lg)) = make_uint2(h0, h1);
      *reinterpret_cast<uint2*>(lds.ut[1] + epos<8>(lr, r0 + 4 * lg)) = make_uint2(l0, l1);
    }
    lds_barrier();  // U of every wave

    // phase 3: O = Q S0^T + tril_0(Q K^T) U;  S^T += K^T U.  U as the B
    // operand (row dv0 + lr, keys in the k order of qkm) and the K^T pieces
    // by transpose reads.
    bf16x8 uh[2], ul[2], kt[NT][2];
    TC_SB();
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      const int c0 = 32 * ks + 4 * lg;
      {
        const uint2 h0 = *reinterpret_cast<const uint2*>(lds.ut[0] + epos<8>(lr, c0));
        const uint2 h1 = *reinterpret_cast<const uint2*>(lds.ut[0] + epos<8>(lr, c0 + 16));
        const uint2 l0 = *reinterpret_cast<const uint2*>(lds.ut[1] + epos<8>(lr, c0));
        const uint2 l1 = *reinterpret_cast<const uint2*>(lds.ut[1] + epos<8>(lr, c0 + 16));
        uh[ks] = as_bf16x8(h0.x, h0.y, h1.x, h1.y);
        ul[ks] = as_bf16x8(l0.x, l0.y, l1.x, l1.y);
      }
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        const int col = (D / 4) * w + 16 * t + tr_col;
        const uint2 p0 = lds_tr8(lds.k[b], epos<NCH>(c0 + tr_row, col));
        const uint2 p1 = lds_tr8(lds.k[b], epos<NCH>(c0 + 16 + tr_row, col));
        kt[t][ks] = as_bf16x8(p0.x, p0.y, p1.x, p1.y);
      }
    }
    TC_SB();
    // the state first (the next chunk waits for it), then O
#pragma unroll
    for (int t = 0; t < NT; ++t) {
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        hs[t] = mma(kt[t][ks], uh[ks], hs[t]);
        hs[t] = mma(kt[t][ks], ul[ks], hs[t]);
      }
    }
    // tril_0 as the A operand of O += tril(Q K^T) U: k-step ks takes keys
    // 32 ks + 4 lg .. +3 and 32 ks + 16 + 4 lg .. +3 (tiles 2 ks, 2 ks + 1)
    bf16x8 qkm[2];
    {
      const int rq = r0 + lr;
      uint32_t pw[4][2];
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) {
        const int c0 = 16 * mt + 4 * lg;
        pw[mt][0] = cvt_pk(c0 <= rq ? qkt[mt][0] : 0.f, c0 + 1 <= rq ? qkt[mt][1] : 0.f);
        pw[mt][1] = cvt_pk(c0 + 2 <= rq ? qkt[mt][2] : 0.f, c0 + 3 <= rq ? qkt[mt][3] : 0.f);
      }
      qkm[0] = as_bf16x8(pw[0][0], pw[0][1], pw[1][0], pw[1][1]);
      qkm[1] = as_bf16x8(pw[2][0], pw[2][1], pw[3][0], pw[3][1]);
    }
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) qh = mma(qkm[ks], uh[ks], qh);
    o_prev = qh;
    t_prev = t0;
    publish_state();  // read next after the barrier at the top of the loop
  }
  if (t_prev >= 0) {
#pragma unroll
    for (int e = 0; e < 4; ++e)
      __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(o_prev[e]), ro,
                                            ((t_prev + r0 + 4 * lg + e) * D + dv0 + lr) * 4, 0, 0);
  }
  if (S_final != nullptr) {
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
      for (int e = 0; e < 4; ++e)
        S_final[((long)bh * D + dv0 + lr) * D + (D / 4) * w + 16 * t + 4 * lg + e] = hs[t][e];
  }
}

template <int D>
hipError_t run_delta_bf16(const uint16_t* q, const uint16_t* k, const uint16_t* v, const float* beta,
                          int BH, int T, const float* S0, float* o, float* S_final, void* ws,
                          hipStream_t s) {
  const int n_chunks = (T + CH - 1) / CH;
  uint16_t* a_ws = static_cast<uint16_t*>(ws);
  if (n_chunks > 0)
    hipLaunchKernelGGL(delta_prep_kernel<D>, dim3(n_chunks, BH), dim3(256), 0, s, k, beta, T, n_chunks, a_ws);
  const int n_items = BH * (D / DVT);
  const int grid = (n_items + NXCD - 1) / NXCD * NXCD;
  profile_mark_before(s);
  hipLaunchKernelGGL(delta_main_kernel<D>, dim3(grid), dim3(256), 0, s, q, k, v, a_ws, T, n_chunks, n_items, S0,
                     o, S_final);
  profile_mark_after(s);
  return hipGetLastError();
}

}  // namespace

bool delta_bf16_supported(bool bf16, int d) { return bf16 && (d == 64 || d == 128); }

size_t delta_bf16_ws_bytes(int B, int H, int T, int d) {
  const size_t n_chunks = (T + CH - 1) / CH;
  return (size_t)B * H * n_chunks * 2 * CH * CH * sizeof(uint16_t);
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

// delta_bwd.hip — backward of the chunked delta-rule scan (gfx950), fp32
// inputs, d_k = d_v = D in {16, 32, 64}.
//
// "DeltaNet-family linear attention variants", DeltaNet section: the write
// S_t = S_{t-1} + beta_t (v_t - S_{t-1} k_t) k_t^T with the learned write
// strength beta_t, and the read o_t = S_t q_t.  Gradients of
// L = sum_t <do_t, o_t> + <dS_final, S_T>.
//
// Chunk form (64 tokens, entering state S0, exit state S1):
//   M = I + diag(beta) tril_-1(K K^T),  W = M^-1,
//   X = V - K S0^T,  U = W diag(beta) X,
//   O = Q S0^T + tril_0(Q K^T) U,  S1 = S0 + U^T K.
// Reverse mode through those lines, with dS1 the adjoint of the exit state:
//   dU  = K dS1^T + tril_0(Q K^T)^T dO,   dY = W^T dU,   dX = diag(beta) dY,
//   dS0 = dS1 + dO^T Q - dX^T K                        (the adjoint recurrence),
//   dV  = dX,
//   P1  = tril_0(dO U^T),  P2 = tril_-1(dY U^T),  dLk = -diag(beta) P2,
//   dQ  = dO S0 + P1 K,
//   dK  = -dX S0 + U dS1 + P1^T Q + (dLk + dLk^T) K,
//   dbeta_r = <dY_r, X_r> - sum_{c<r} P2[r][c] <k_r, k_c>.
// Four launches:
//   1. delta_bwd_prep   (chunks in parallel): W of every chunk;
//   2. delta_bwd_fwd    (per b, h and 16-row slice of S, chunks in order):
//      the entering state S0 of every chunk;
//   3. delta_bwd_rev    (per b, h and 16-row slice of dS, chunks in reverse):
//      the exit adjoint dS1 of every chunk, and dS0 of the sequence;
//   4. delta_bwd_grads  (chunks in parallel): dq, dk, dv, dbeta.
// The rows of S (and of dS) are independent in 2 and 3: row j of S only sees
// column j of V and U, row j of dS only column j of dO and dU.
// Products use fp32 MFMA (v_mfma_f32_16x16x4_f32) on LDS tiles.
#include "tc_common.hpp"
#include "tc_kernels.hpp"

namespace tc {

namespace {

constexpr int CH = 64;         // tokens per chunk
constexpr int SL = 16;         // rows of S per workgroup in the state walks
constexpr int SW = CH + 4;     // row stride of [64][64] arrays
template <int D>
struct DB {
  static constexpr int S = D + 4;    // row stride of [.][D] arrays
  static constexpr int SV = SL + 4;  // row stride of [64][16] slice arrays
};

// C += A diag(s) B over K (A[m][k] at pa + m am + k ak, s[k], B[k][n] at pb + k bk + n bn)
template <int K>
__device__ __forceinline__ floatx4 wave_mma_f32_scaled(const float* pa, int am, int ak, const float* s,
                                                       const float* pb, int bk, int bn, floatx4 c) {
  const int l = lane_id();
  const int r = l & 15, kk = l >> 4;
  const float* a = pa + r * am + kk * ak;
  const float* b = pb + kk * bk + r * bn;
  const float* sk = s + kk;
#pragma unroll 8
  for (int k0 = 0; k0 < K; k0 += 4) c = mfma4(a[k0 * ak] * sk[k0], b[k0 * bk], c);
  return c;
}

// rows [0, 64) x [0, NC) of a row-major source (row stride ld, first column
// col0) into LDS (stride dst_ld); rows >= nvalid become zero.
template <int NC>
__device__ __forceinline__ void stage(float* dst, int dst_ld, const float* src, long ld, int col0, int nvalid) {
  constexpr int V4 = NC / 4;
  for (int idx = threadIdx.x; idx < CH * V4; idx += blockDim.x) {
    const int r = idx / V4, c = (idx % V4) * 4;
    float4 x = make_float4(0.f, 0.f, 0.f, 0.f);
    if (r < nvalid) x = *reinterpret_cast<const float4*>(src + (long)r * ld + col0 + c);
    *reinterpret_cast<float4*>(dst + r * dst_ld + c) = x;
  }
}

// one [R][D] block (row stride D in global) <-> LDS (stride S)
template <int R, int D>
__device__ __forceinline__ void load_block(float* dst, const float* src) {
  for (int idx = threadIdx.x; idx < R * D / 4; idx += blockDim.x) {
    const int r = idx / (D / 4), c = (idx % (D / 4)) * 4;
    *reinterpret_cast<float4*>(dst + r * DB<D>::S + c) = *reinterpret_cast<const float4*>(src + (long)r * D + c);
  }
}
template <int R, int D>
__device__ __forceinline__ void store_block(float* dst, const float* src) {
  for (int idx = threadIdx.x; idx < R * D / 4; idx += blockDim.x) {
    const int r = idx / (D / 4), c = (idx % (D / 4)) * 4;
    *reinterpret_cast<float4*>(dst + (long)r * D + c) = *reinterpret_cast<const float4*>(src + r * DB<D>::S + c);
  }
}

// 1. W = (I + diag(beta) tril_-1(K K^T))^-1 of one chunk: one wave; lane c
//    solves column c by forward substitution.  Rows past the sequence end
//    have beta = 0, so their rows and columns of W are those of I.
template <int D>
__global__ __launch_bounds__(64) void delta_bwd_prep(const float* __restrict__ k, const float* __restrict__ beta,
                                                     int T, int n_chunks, float* __restrict__ Wout) {
  constexpr int S = DB<D>::S;
  __shared__ __attribute__((aligned(16))) float sK[CH * S];
  __shared__ __attribute__((aligned(16))) float sM[CH * SW];
  __shared__ float sB[CH];
  const int c = blockIdx.x, bh = blockIdx.y, l = threadIdx.x;
  const int t0 = c * CH, L = min(CH, T - t0);
  stage<D>(sK, S, k + ((long)bh * T + t0) * D, D, 0, L);
  sB[l] = l < L ? beta[(long)bh * T + t0 + l] : 0.f;
  __syncthreads();
  const int col = l & 15, rq = (l >> 4) * 4;
#pragma unroll
  for (int rt = 0; rt < 4; ++rt)
#pragma unroll
    for (int ct = 0; ct < 4; ++ct) {
      floatx4 kk = wave_mma_f32<D>(sK + 16 * rt * S, S, 1, sK + 16 * ct * S, 1, S, zero4());
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = 16 * rt + rq + i, cc = 16 * ct + col;
        sM[r * SW + cc] = cc < r ? sB[r] * kk[i] : 0.f;
      }
    }
  __syncthreads();
  float w[CH];
#pragma unroll
  for (int r = 0; r < CH; ++r) {
    float acc = r == l ? 1.f : 0.f;
#pragma unroll
    for (int i = 0; i < r; ++i) acc -= sM[r * SW + i] * w[i];
    w[r] = acc;
  }
  float* dst = Wout + ((long)bh * n_chunks + c) * CH * CH + l;
#pragma unroll
  for (int r = 0; r < CH; ++r) dst[r * CH] = w[r];
}

// 2. Entering state of every chunk, per (16-row slice of S, b, h).
template <int D>
__global__ __launch_bounds__(256) void delta_bwd_fwd(const float* __restrict__ k, const float* __restrict__ v,
                                                     const float* __restrict__ beta, int T, int n_chunks,
                                                     const float* __restrict__ S0, const float* __restrict__ Wm,
                                                     float* __restrict__ Sc) {
  constexpr int S = DB<D>::S, SV = DB<D>::SV;
  __shared__ __attribute__((aligned(16))) float sS[SL * S];
  __shared__ __attribute__((aligned(16))) float sK[CH * S];
  __shared__ __attribute__((aligned(16))) float sX[CH * SV];
  __shared__ __attribute__((aligned(16))) float sU[CH * SV];
  __shared__ __attribute__((aligned(16))) float sW[CH * SW];
  __shared__ float sB[CH];
  const int j0 = blockIdx.x * SL, bh = blockIdx.y;
  const int w = wave_id(), l = lane_id(), col = l & 15, rq = (l >> 4) * 4;
  for (int i = threadIdx.x; i < SL * D; i += blockDim.x) {
    const int r = i / D, cc = i % D;
    sS[r * S + cc] = S0 != nullptr ? S0[((long)bh * D + j0 + r) * D + cc] : 0.f;
  }
  for (int c = 0; c < n_chunks; ++c) {
    const int t0 = c * CH, L = min(CH, T - t0);
    __syncthreads();  // the previous chunk's update of sS is complete
    store_block<SL, D>(Sc + (((long)bh * n_chunks + c) * D + j0) * D, sS);
    stage<D>(sK, S, k + ((long)bh * T + t0) * D, D, 0, L);
    stage<SL>(sX, SV, v + ((long)bh * T + t0) * D, D, j0, L);
    for (int i = threadIdx.x; i < CH * CH / 4; i += blockDim.x) {
      const int r = i / (CH / 4), cc = (i % (CH / 4)) * 4;
      *reinterpret_cast<float4*>(sW + r * SW + cc) =
          *reinterpret_cast<const float4*>(Wm + ((long)bh * n_chunks + c) * CH * CH + r * CH + cc);
    }
    if (threadIdx.x < CH) sB[threadIdx.x] = (int)threadIdx.x < L ? beta[(long)bh * T + t0 + threadIdx.x] : 0.f;
    __syncthreads();
    {  // X = V - K S^T, rows 16w..
      floatx4 ks = wave_mma_f32<D>(sK + 16 * w * S, S, 1, sS, 1, S, zero4());
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        float* x = sX + (16 * w + rq + i) * SV + col;
        *x -= ks[i];
      }
    }
    __syncthreads();
    {  // U = W diag(beta) X
      floatx4 u = wave_mma_f32_scaled<CH>(sW + 16 * w * SW, SW, 1, sB, sX, SV, 1, zero4());
#pragma unroll
      for (int i = 0; i < 4; ++i) sU[(16 * w + rq + i) * SV + col] = u[i];
    }
    __syncthreads();
    if (w < D / 16) {  // S += U^T K, tile (rows j0.., columns 16w..)
      float* base = sS + rq * S + 16 * w + col;
      floatx4 acc;
#pragma unroll
      for (int i = 0; i < 4; ++i) acc[i] = base[i * S];
      acc = wave_mma_f32<CH>(sU, 1, SV, sK + 16 * w, S, 1, acc);
#pragma unroll
      for (int i = 0; i < 4; ++i) base[i * S] = acc[i];
    }
  }
}

// 3. Exit adjoint dS1 of every chunk, per (16-row slice of dS, b, h), chunks
//    in reverse; dS0 of the sequence at the end.
template <int D>
__global__ __launch_bounds__(256) void delta_bwd_rev(const float* __restrict__ q, const float* __restrict__ k,
                                                     const float* __restrict__ dO, const float* __restrict__ beta,
                                                     int T, int n_chunks, const float* __restrict__ dSf,
                                                     const float* __restrict__ Wm, float* __restrict__ dSc,
                                                     float* __restrict__ dS0) {
  constexpr int S = DB<D>::S, SV = DB<D>::SV;
  __shared__ __attribute__((aligned(16))) float sD[SL * S];   // dS slice
  __shared__ __attribute__((aligned(16))) float sQ[CH * S];
  __shared__ __attribute__((aligned(16))) float sK[CH * S];
  __shared__ __attribute__((aligned(16))) float sO[CH * SV];  // dO slice
  __shared__ __attribute__((aligned(16))) float sA[CH * SW];  // tril_0(Q K^T)
  __shared__ __attribute__((aligned(16))) float sW[CH * SW];
  __shared__ __attribute__((aligned(16))) float sU[CH * SV];  // dU
  __shared__ __attribute__((aligned(16))) float sX[CH * SV];  // dX
  __shared__ float sB[CH];
  const int j0 = blockIdx.x * SL, bh = blockIdx.y;
  const int w = wave_id(), l = lane_id(), col = l & 15, rq = (l >> 4) * 4;
  for (int i = threadIdx.x; i < SL * D; i += blockDim.x) {
    const int r = i / D, cc = i % D;
    sD[r * S + cc] = dSf != nullptr ? dSf[((long)bh * D + j0 + r) * D + cc] : 0.f;
  }
  for (int c = n_chunks - 1; c >= 0; --c) {
    const int t0 = c * CH, L = min(CH, T - t0);
    __syncthreads();  // the previous chunk's update of sD is complete
    store_block<SL, D>(dSc + (((long)bh * n_chunks + c) * D + j0) * D, sD);
    stage<D>(sQ, S, q + ((long)bh * T + t0) * D, D, 0, L);
    stage<D>(sK, S, k + ((long)bh * T + t0) * D, D, 0, L);
    stage<SL>(sO, SV, dO + ((long)bh * T + t0) * D, D, j0, L);
    for (int i = threadIdx.x; i < CH * CH / 4; i += blockDim.x) {
      const int r = i / (CH / 4), cc = (i % (CH / 4)) * 4;
      *reinterpret_cast<float4*>(sW + r * SW + cc) =
          *reinterpret_cast<const float4*>(Wm + ((long)bh * n_chunks + c) * CH * CH + r * CH + cc);
    }
    if (threadIdx.x < CH) sB[threadIdx.x] = (int)threadIdx.x < L ? beta[(long)bh * T + t0 + threadIdx.x] : 0.f;
    __syncthreads();
#pragma unroll
    for (int ct = 0; ct < 4; ++ct) {  // tril_0(Q K^T), rows 16w..
      floatx4 qk = wave_mma_f32<D>(sQ + 16 * w * S, S, 1, sK + 16 * ct * S, 1, S, zero4());
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = 16 * w + rq + i, cc = 16 * ct + col;
        sA[r * SW + cc] = cc <= r ? qk[i] : 0.f;
      }
    }
    __syncthreads();
    {  // dU = K dS^T + A^T dO, rows 16w..
      floatx4 u = wave_mma_f32<D>(sK + 16 * w * S, S, 1, sD, 1, S, zero4());
      u = wave_mma_f32<CH>(sA + 16 * w, 1, SW, sO, SV, 1, u);
#pragma unroll
      for (int i = 0; i < 4; ++i) sU[(16 * w + rq + i) * SV + col] = u[i];
    }
    __syncthreads();
    {  // dX = diag(beta) W^T dU
      floatx4 x = wave_mma_f32<CH>(sW + 16 * w, 1, SW, sU, SV, 1, zero4());
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = 16 * w + rq + i;
        sX[r * SV + col] = sB[r] * x[i];
      }
    }
    __syncthreads();
    if (w < D / 16) {  // dS += dO^T Q - dX^T K, tile (rows j0.., columns 16w..)
      float* base = sD + rq * S + 16 * w + col;
      floatx4 acc, neg = zero4();
#pragma unroll
      for (int i = 0; i < 4; ++i) acc[i] = base[i * S];
      acc = wave_mma_f32<CH>(sO, 1, SV, sQ + 16 * w, S, 1, acc);
      neg = wave_mma_f32<CH>(sX, 1, SV, sK + 16 * w, S, 1, neg);
#pragma unroll
      for (int i = 0; i < 4; ++i) base[i * S] = acc[i] - neg[i];
    }
  }
  if (dS0 != nullptr) {
    __syncthreads();
    for (int i = threadIdx.x; i < SL * D; i += blockDim.x) {
      const int r = i / D, cc = i % D;
      dS0[((long)bh * D + j0 + r) * D + cc] = sD[r * S + cc];
    }
  }
}

// 4. Gradients of one chunk from its S0, dS1 and W.  Wave w owns rows
//    16w..16w+15 of every [64][.] result.
template <int D>
__global__ __launch_bounds__(256) void delta_bwd_grads(
    const float* __restrict__ q, const float* __restrict__ k, const float* __restrict__ v,
    const float* __restrict__ dO, const float* __restrict__ beta, int T, int n_chunks,
    const float* __restrict__ Wm, const float* __restrict__ Sc, const float* __restrict__ dSc,
    float* __restrict__ dq, float* __restrict__ dk, float* __restrict__ dv, float* __restrict__ dbeta) {
  constexpr int S = DB<D>::S;
  constexpr int NT = D / 16;
  __shared__ __attribute__((aligned(16))) float bS[D * S];    // S0, then dS1, then S0
  __shared__ __attribute__((aligned(16))) float bQ[CH * S];
  __shared__ __attribute__((aligned(16))) float bK[CH * S];
  __shared__ __attribute__((aligned(16))) float bX[CH * S];   // V, then X
  __shared__ __attribute__((aligned(16))) float bU[CH * S];
  __shared__ __attribute__((aligned(16))) float bO[CH * S];   // dO
  __shared__ __attribute__((aligned(16))) float bY[CH * SW];  // dU, then P1
  __shared__ __attribute__((aligned(16))) float bW[CH * SW];  // W, then dLk
  __shared__ __attribute__((aligned(16))) float bP[CH * SW];  // tril_0(Q K^T), then dY
  __shared__ float sB[CH], sDb[CH];
  const int c = blockIdx.x, bh = blockIdx.y;
  const int t0 = c * CH, L = min(CH, T - t0);
  const int w = wave_id(), l = lane_id(), col = l & 15, rq = (l >> 4) * 4;
  const long cs = ((long)bh * n_chunks + c) * D * D;  // this chunk's state block
  const long row0 = (long)bh * T + t0;

  load_block<D, D>(bS, Sc + cs);
  stage<D>(bQ, S, q + row0 * D, D, 0, L);
  stage<D>(bK, S, k + row0 * D, D, 0, L);
  stage<D>(bX, S, v + row0 * D, D, 0, L);
  stage<D>(bO, S, dO + row0 * D, D, 0, L);
  for (int i = threadIdx.x; i < CH * CH / 4; i += blockDim.x) {
    const int r = i / (CH / 4), cc = (i % (CH / 4)) * 4;
    *reinterpret_cast<float4*>(bW + r * SW + cc) =
        *reinterpret_cast<const float4*>(Wm + ((long)bh * n_chunks + c) * CH * CH + r * CH + cc);
  }
  if (threadIdx.x < CH) sB[threadIdx.x] = (int)threadIdx.x < L ? beta[row0 + threadIdx.x] : 0.f;
  __syncthreads();

  // X = V - K S0^T; A = tril_0(Q K^T); dQ = dO S0 (first part)
  floatx4 aq[NT], ak[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    floatx4 ks = wave_mma_f32<D>(bK + 16 * w * S, S, 1, bS + 16 * t * S, 1, S, zero4());
#pragma unroll
    for (int i = 0; i < 4; ++i) bX[(16 * w + rq + i) * S + 16 * t + col] -= ks[i];
    aq[t] = wave_mma_f32<D>(bO + 16 * w * S, S, 1, bS + 16 * t, S, 1, zero4());
    ak[t] = zero4();
  }
#pragma unroll
  for (int ct = 0; ct < 4; ++ct) {
    floatx4 qk = wave_mma_f32<D>(bQ + 16 * w * S, S, 1, bK + 16 * ct * S, 1, S, zero4());
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = 16 * w + rq + i, cc = 16 * ct + col;
      bP[r * SW + cc] = cc <= r ? qk[i] : 0.f;
    }
  }
  __syncthreads();
  // U = W diag(beta) X; bring dS1 in
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    floatx4 u = wave_mma_f32_scaled<CH>(bW + 16 * w * SW, SW, 1, sB, bX + 16 * t, S, 1, zero4());
#pragma unroll
    for (int i = 0; i < 4; ++i) bU[(16 * w + rq + i) * S + 16 * t + col] = u[i];
  }
  load_block<D, D>(bS, dSc + cs);
  __syncthreads();
  // dU = K dS1^T + A^T dO; dK = U dS1 (first part)
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    floatx4 u = wave_mma_f32<D>(bK + 16 * w * S, S, 1, bS + 16 * t * S, 1, S, zero4());
    u = wave_mma_f32<CH>(bP + 16 * w, 1, SW, bO + 16 * t, S, 1, u);
#pragma unroll
    for (int i = 0; i < 4; ++i) bY[(16 * w + rq + i) * SW + 16 * t + col] = u[i];
    ak[t] = wave_mma_f32<D>(bU + 16 * w * S, S, 1, bS + 16 * t, S, 1, ak[t]);
  }
  __syncthreads();
  // dY = W^T dU into bP; S0 back in
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    floatx4 y = wave_mma_f32<CH>(bW + 16 * w, 1, SW, bY + 16 * t, SW, 1, zero4());
#pragma unroll
    for (int i = 0; i < 4; ++i) bP[(16 * w + rq + i) * SW + 16 * t + col] = y[i];
  }
  load_block<D, D>(bS, Sc + cs);
  __syncthreads();
  // dV = diag(beta) dY; dbeta first part <dY_r, X_r>; P1 = tril_0(dO U^T) into
  // bY; P2 = tril_-1(dY U^T) gives dLk into bW and the second part of dbeta
#pragma unroll
  for (int t = 0; t < NT; ++t)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = 16 * w + rq + i;
      if (r < L) dv[(row0 + r) * D + 16 * t + col] = sB[r] * bP[r * SW + 16 * t + col];
    }
  {
    const int r = 16 * w + (l >> 2), part = l & 3;
    float s = 0.f;
    for (int j = part; j < D; j += 4) s += bP[r * SW + j] * bX[r * S + j];
    s += __shfl_xor(s, 1);
    s += __shfl_xor(s, 2);
    if (part == 0) sDb[r] = s;
  }
  float db2[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int ct = 0; ct < 4; ++ct) {
    floatx4 p1 = wave_mma_f32<D>(bO + 16 * w * S, S, 1, bU + 16 * ct * S, 1, S, zero4());
    floatx4 p2 = wave_mma_f32<D>(bP + 16 * w * SW, SW, 1, bU + 16 * ct * S, 1, S, zero4());
    floatx4 kk = wave_mma_f32<D>(bK + 16 * w * S, S, 1, bK + 16 * ct * S, 1, S, zero4());
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = 16 * w + rq + i, cc = 16 * ct + col;
      bY[r * SW + cc] = cc <= r ? p1[i] : 0.f;
      const float p = cc < r ? p2[i] : 0.f;
      bW[r * SW + cc] = -sB[r] * p;
      db2[i] += p * kk[i];
    }
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
#pragma unroll
    for (int off = 1; off < 16; off <<= 1) db2[i] += __shfl_xor(db2[i], off);
  }
  __syncthreads();
  if (col == 0) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = 16 * w + rq + i;
      if (r < L) dbeta[row0 + r] = sDb[r] - db2[i];
    }
  }
  // dQ = dO S0 + P1 K;  dK = U dS1 - diag(beta) dY S0 + P1^T Q + dLk K + dLk^T K
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    aq[t] = wave_mma_f32<CH>(bY + 16 * w * SW, SW, 1, bK + 16 * t, S, 1, aq[t]);
    floatx4 ys = wave_mma_f32<D>(bP + 16 * w * SW, SW, 1, bS + 16 * t, S, 1, zero4());
#pragma unroll
    for (int i = 0; i < 4; ++i) ak[t][i] -= sB[16 * w + rq + i] * ys[i];
    ak[t] = wave_mma_f32<CH>(bY + 16 * w, 1, SW, bQ + 16 * t, S, 1, ak[t]);
    ak[t] = wave_mma_f32<CH>(bW + 16 * w * SW, SW, 1, bK + 16 * t, S, 1, ak[t]);
    ak[t] = wave_mma_f32<CH>(bW + 16 * w, 1, SW, bK + 16 * t, S, 1, ak[t]);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = 16 * w + rq + i;
      if (r < L) {
        dq[(row0 + r) * D + 16 * t + col] = aq[t][i];
        dk[(row0 + r) * D + 16 * t + col] = ak[t][i];
      }
    }
  }
}

template <int D>
hipError_t run_delta_backward(const float* q, const float* k, const float* v, const float* beta, int B, int H,
                              int T, const float* S0, const float* dO, const float* dSf, float* dq, float* dk,
                              float* dv, float* dbeta, float* dS0, char* ws, hipStream_t s) {
  const int BH = B * H, nC = (T + CH - 1) / CH;
  float* Wm = reinterpret_cast<float*>(ws);
  float* Sc = Wm + (long)BH * nC * CH * CH;
  float* dSc = Sc + (long)BH * nC * D * D;
  hipLaunchKernelGGL((delta_bwd_prep<D>), dim3(nC, BH), dim3(64), 0, s, k, beta, T, nC, Wm);
  hipLaunchKernelGGL((delta_bwd_fwd<D>), dim3(D / SL, BH), dim3(256), 0, s, k, v, beta, T, nC, S0, Wm, Sc);
  hipLaunchKernelGGL((delta_bwd_rev<D>), dim3(D / SL, BH), dim3(256), 0, s, q, k, dO, beta, T, nC, dSf, Wm, dSc,
                     dS0);
  profile_mark_before(s);
  hipLaunchKernelGGL((delta_bwd_grads<D>), dim3(nC, BH), dim3(256), 0, s, q, k, v, dO, beta, T, nC, Wm, Sc, dSc,
                     dq, dk, dv, dbeta);
  profile_mark_after(s);
  return hipGetLastError();
}

// T = 0: nothing is read or written but dS0 = dS_final (or 0)
__global__ void delta_bwd_empty(const float* __restrict__ dSf, float* __restrict__ dS0, long n) {
  const long i = (long)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) dS0[i] = dSf != nullptr ? dSf[i] : 0.f;
}

}  // namespace

size_t delta_bwd_ws_bytes(int B, int H, int T, int d) {
  const long nC = (T + CH - 1) / CH;
  return (size_t)B * H * nC * ((size_t)CH * CH + 2 * (size_t)d * d) * sizeof(float);
}

hipError_t launch_delta_backward(const float* q, const float* k, const float* v, const float* beta, int B, int H,
                                 int T, int d, const float* S0, const float* dO, const float* dSf, float* dq,
                                 float* dk, float* dv, float* dbeta, float* dS0, void* ws, hipStream_t s) {
  if (T == 0) {
    if (dS0 != nullptr) {
      const long n = (long)B * H * d * d;
      hipLaunchKernelGGL(delta_bwd_empty, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, dSf, dS0, n);
    }
    return hipGetLastError();
  }
  char* w = static_cast<char*>(ws);
  switch (d) {
    case 16: return run_delta_backward<16>(q, k, v, beta, B, H, T, S0, dO, dSf, dq, dk, dv, dbeta, dS0, w, s);
    case 32: return run_delta_backward<32>(q, k, v, beta, B, H, T, S0, dO, dSf, dq, dk, dv, dbeta, dS0, w, s);
    case 64: return run_delta_backward<64>(q, k, v, beta, B, H, T, S0, dO, dSf, dq, dk, dv, dbeta, dS0, w, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace tc

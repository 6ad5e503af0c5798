// delta_bwd.hip — backward of the chunked delta-rule scan (gfx950), fp32
// inputs, d_k = d_v = D in {16, 32, 64, 128}.
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
// Three launches:
//   1. delta_bwd_prep   (chunks in parallel): W of every chunk and the
//      state-independent products the walks use (below);
//   2. delta_bwd_fwd    (per b, h and 16-row slice of S, chunks in order):
//      the entering state S0 of every chunk;
//   3. delta_bwd_rev    (per b, h and 16-row slice of dS, chunks in reverse):
//      the exit adjoint dS1 of every chunk, and dS0 of the sequence
//      (2 and 3 are one launch, delta_bwd_walks);
//   4. delta_bwd_grads  (chunks in parallel): dq, dk, dv, dbeta.
// The rows of S (and of dS) are independent in 2 and 3: row j of S only sees
// column j of V and U, row j of dS only column j of dO and dU.  For the same
// reason every term of 4 is a sum over the rows of S (the d_v index) of
// products that involve one row each (dO S0, U dS1, dX S0, dO U^T, dY U^T,
// <dY_r, X_r>), so at D = 128 the gradient kernel walks the d_v rows in
// pieces of 16 and adds the pieces' terms, which keeps its LDS within a CU.
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

// rows [0, 64) x [0, NC) of a row-major source (row stride ld, first column
// col0) into LDS (stride dst_ld); rows >= nvalid become zero.
// C += A B over K (a multiple of 16), A[m][k] at pa + m am + k ak, B[k][n] at
// pb + k bk + n bn: MFMA 4J + s takes k = 16J + 4g + s from lane (row, g), so
// an operand that is contiguous in k (ak or bk = 1; every such operand here
// starts 16-byte aligned with a row stride that is a multiple of 4) comes in
// one 16-byte read per four MFMAs; the permutation of k is shared by A and B.
template <int K>
__device__ __forceinline__ floatx4 wmma_k4(const float* pa, int am, int ak, const float* pb, int bk, int bn,
                                           floatx4 c) {
  const int l = lane_id(), r = l & 15, g = l >> 4;
  const float* a = pa + r * am + 4 * g * ak;
  const float* b = pb + r * bn + 4 * g * bk;
#pragma unroll
  for (int J = 0; J < K / 16; ++J) {
    float4 x, y;
    if (ak == 1) {
      x = *reinterpret_cast<const float4*>(a + 16 * J);
    } else {
      x = make_float4(a[(16 * J) * ak], a[(16 * J + 1) * ak], a[(16 * J + 2) * ak], a[(16 * J + 3) * ak]);
    }
    if (bk == 1) {
      y = *reinterpret_cast<const float4*>(b + 16 * J);
    } else {
      y = make_float4(b[(16 * J) * bk], b[(16 * J + 1) * bk], b[(16 * J + 2) * bk], b[(16 * J + 3) * bk]);
    }
    c = mfma4(x.x, y.x, c);
    c = mfma4(x.y, y.y, c);
    c = mfma4(x.z, y.z, c);
    c = mfma4(x.w, y.w, c);
  }
  return c;
}

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

// The same rows held in registers (float4 pieces i * 256 + thread), so that
// the next chunk's loads are in flight while the current one is computed.
template <int NC>
struct Rows {
  static constexpr int N = (CH * NC / 4 + 255) / 256;
  float4 x[N];
  __device__ __forceinline__ void load(const float* src, long ld, int col0, int nvalid) {
#pragma unroll
    for (int i = 0; i < N; ++i) {
      const int idx = i * 256 + threadIdx.x, r = idx / (NC / 4), c = (idx % (NC / 4)) * 4;
      x[i] = r < nvalid ? *reinterpret_cast<const float4*>(src + (long)r * ld + col0 + c)
                        : make_float4(0.f, 0.f, 0.f, 0.f);
    }
  }
  __device__ __forceinline__ void put(float* dst, int dst_ld) const {
#pragma unroll
    for (int i = 0; i < N; ++i) {
      const int idx = i * 256 + threadIdx.x, r = idx / (NC / 4), c = (idx % (NC / 4)) * 4;
      *reinterpret_cast<float4*>(dst + r * dst_ld + c) = x[i];
    }
  }
};

// One [D][D] state block (row stride D in global) in registers, for LDS
// (stride D + 4); 256 threads.
template <int D>
struct Blk {
  static constexpr int N = (D * D / 4 + 255) / 256;
  float4 x[N];
  __device__ __forceinline__ void load(const float* src) {
#pragma unroll
    for (int i = 0; i < N; ++i) {
      const int idx = i * 256 + threadIdx.x;
      x[i] = idx < D * D / 4 ? *reinterpret_cast<const float4*>(src + 4 * idx) : make_float4(0.f, 0.f, 0.f, 0.f);
    }
  }
  __device__ __forceinline__ void put(float* dst) const {
#pragma unroll
    for (int i = 0; i < N; ++i) {
      const int idx = i * 256 + threadIdx.x, r = idx / (D / 4), c = 4 * (idx % (D / 4));
      if (idx < D * D / 4) *reinterpret_cast<float4*>(dst + r * DB<D>::S + c) = x[i];
    }
  }
};

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

// Per chunk, the prep kernel leaves [Tm | E2 | G2 | E1] (floats):
//   Tm = W diag(beta) [64][64],  E2 = W^T tril_0(Q K^T)^T [64][64],
//   G2 = Tm K [64][D],           E1 = W^T K [64][D],
// so that the state walks need two products per chunk:
//   U  = Tm V - G2 S0^T                       (forward walk, then S1 = S0 + U^T K),
//   dY = E1 dS1^T + E2 dO,  dX = diag(beta) dY  (reverse walk, then dS0).
template <int D>
struct Pre {
  static constexpr long TM = 0, E2 = CH * CH, G2 = 2 * CH * CH, E1 = 2 * CH * CH + CH * D;
  static constexpr long SIZE = 2 * CH * CH + 2 * CH * D;
};

// 1. Per chunk (in parallel): W = (I + diag(beta) tril_-1(K K^T))^-1 (blocked:
//    diagonal 16-blocks by substitution, the rest by 16x16 products), then
//    Tm, E2, G2, E1.  Rows past the sequence end have beta = 0, so their rows
//    and columns of W are those of I and their rows of Tm, G2 are zero.  The
//    forward (FWD) keeps tril_0(Q K^T) in the E2 slot and Tm V = W diag(beta) V
//    in the E1 slot (v is read only then), and writes no Tm.
template <int D, bool FWD>
__global__ __launch_bounds__(256) void delta_bwd_prep(const float* __restrict__ q, const float* __restrict__ k,
                                                      const float* __restrict__ v, const float* __restrict__ beta,
                                                      int T, int n_chunks, float* __restrict__ pre) {
  constexpr int S = DB<D>::S, NT = D / 16;
  using P = Pre<D>;
  __shared__ __attribute__((aligned(16))) float sQ[CH * S];
  __shared__ __attribute__((aligned(16))) float sK[CH * S];
  __shared__ __attribute__((aligned(16))) float sM[CH * SW];  // beta_r <k_r, k_c> (c < r)
  __shared__ __attribute__((aligned(16))) float sA[CH * SW];  // tril_0(Q K^T)
  __shared__ __attribute__((aligned(16))) float sWx[D == 64 ? 1 : CH * SW];
  __shared__ __attribute__((aligned(16))) float sTmp[3 * 16 * 17];
  __shared__ float sB[CH];
  float* const sWm = D == 64 ? sQ : sWx;  // W; at d = 64 it takes the place of Q, read before it is written
  float* const sVv = D == 64 ? sM : sQ;   // FWD: the V rows, once M (or Q) is no longer read
  const int c = blockIdx.x, bh = blockIdx.y;
  const int t0 = c * CH, L = min(CH, T - t0);
  const int w = wave_id(), l = lane_id(), col = l & 15, rq = (l >> 4) * 4;
  Rows<D> xv;  // FWD: the V rows, loaded now and staged after the inversion
  if constexpr (FWD) xv.load(v + ((long)bh * T + t0) * D, D, 0, L);
  {
    Rows<D> xq, xk;
    xq.load(q + ((long)bh * T + t0) * D, D, 0, L);
    xk.load(k + ((long)bh * T + t0) * D, D, 0, L);
    const float bb = (int)threadIdx.x < L ? beta[(long)bh * T + t0 + threadIdx.x] : 0.f;
    xq.put(sQ, S);
    xk.put(sK, S);
    if (threadIdx.x < CH) sB[threadIdx.x] = bb;
  }
  __syncthreads();
#pragma unroll
  for (int ct = 0; ct < 4; ++ct) {
    floatx4 kk = wmma_k4<D>(sK + 16 * w * S, S, 1, sK + 16 * ct * S, 1, S, zero4());
    floatx4 qk = wmma_k4<D>(sQ + 16 * w * S, S, 1, sK + 16 * ct * S, 1, S, zero4());
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = 16 * w + rq + i, cc = 16 * ct + col;
      sM[r * SW + cc] = cc < r ? sB[r] * kk[i] : 0.f;
      sA[r * SW + cc] = cc <= r ? qk[i] : 0.f;
    }
  }
  __syncthreads();
  // W = M^-1 in 16-row blocks: the four diagonal blocks by substitution
  // (wave 0, one lane per column of every block), then the off-diagonal
  // blocks one block diagonal at a time, W_ab = -W_aa sum_{c=b}^{a-1} M_ac W_cb
  // (a wave per block, 16x16 MFMA products through a small LDS tile).
  for (int i = threadIdx.x; i < CH * CH; i += blockDim.x) {
    const int r = i / CH, cc = i % CH;
    if (cc / 16 > r / 16) sWm[r * SW + cc] = 0.f;
  }
  if (w == 0) {
    const int blk = l >> 4, cc = l & 15, o = 16 * blk;
    float x[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      float acc = r == cc ? 1.f : 0.f;
#pragma unroll
      for (int i = 0; i < r; ++i) acc -= sM[(o + r) * SW + o + i] * x[i];
      x[r] = acc;
    }
#pragma unroll
    for (int r = 0; r < 16; ++r) sWm[(o + r) * SW + o + cc] = x[r];
  }
  __syncthreads();
#pragma unroll
  for (int dist = 1; dist < 4; ++dist) {
    if (w < 4 - dist) {
      const int bb = w, aa = w + dist;
      floatx4 t = zero4();
      for (int cb = bb; cb < aa; ++cb)
        t = wmma_k4<16>(sM + 16 * aa * SW + 16 * cb, SW, 1, sWm + 16 * cb * SW + 16 * bb, SW, 1, t);
      float* tw = sTmp + w * 16 * 17;
#pragma unroll
      for (int i = 0; i < 4; ++i) tw[(rq + i) * 17 + col] = t[i];
      // the tile is read back by this wave only
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront", "local");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront", "local");
      const floatx4 wab = wmma_k4<16>(sWm + 16 * aa * SW + 16 * aa, SW, 1, tw, 17, 1, zero4());
#pragma unroll
      for (int i = 0; i < 4; ++i) sWm[(16 * aa + rq + i) * SW + 16 * bb + col] = -wab[i];
    }
    __syncthreads();
  }
  if constexpr (FWD) {
    xv.put(sVv, S);
    // the forward needs Tm = W diag(beta) only: scaled in place
    for (int i = threadIdx.x; i < CH * CH; i += blockDim.x) {
      const int r = i / CH, cc = i % CH;
      sWm[r * SW + cc] *= sB[cc];
    }
    __syncthreads();
  }
  float* out = pre + ((long)bh * n_chunks + c) * P::SIZE;
  float* const sWt = sM;  // backward: W^T ([64][SW]), once M is no longer read
  if constexpr (!FWD) {  // the forward reads Tm V only
    for (int i = threadIdx.x; i < CH * CH; i += blockDim.x) {
      const int r = i / CH, cc = i % CH;
      const float x = sWm[r * SW + cc];
      out[P::TM + i] = x * sB[cc];
      sWt[cc * SW + r] = x;
    }
    __syncthreads();
  }
  if constexpr (FWD) {  // the forward keeps tril_0(Q K^T) itself in the E2 slot
    for (int i = threadIdx.x; i < CH * CH; i += blockDim.x) out[P::E2 + i] = sA[(i / CH) * SW + i % CH];
  } else {
#pragma unroll
    for (int ct = 0; ct < 4; ++ct) {  // E2 = W^T A^T, W^T rows read 16 bytes at a time
      floatx4 e = wmma_k4<CH>(sWt + 16 * w * SW, SW, 1, sA + 16 * ct * SW, 1, SW, zero4());
#pragma unroll
      for (int i = 0; i < 4; ++i) out[P::E2 + (16 * w + rq + i) * CH + 16 * ct + col] = e[i];
    }
  }
  if constexpr (!FWD) {
#pragma unroll
    for (int t = 0; t < NT; ++t) {  // E1 = W^T K
      floatx4 e = wmma_k4<CH>(sWt + 16 * w * SW, SW, 1, sK + 16 * t, S, 1, zero4());
#pragma unroll
      for (int i = 0; i < 4; ++i) out[P::E1 + (16 * w + rq + i) * D + 16 * t + col] = e[i];
    }
    __syncthreads();  // every wave is done with K itself
    for (int i = threadIdx.x; i < CH * D; i += blockDim.x) sK[(i / D) * S + i % D] *= sB[i / D];
    __syncthreads();
  }
#pragma unroll
  for (int t = 0; t < NT; ++t) {  // G2 = W diag(beta) K (and the forward's Tm V)
    if constexpr (!FWD) {  // sK holds diag(beta) K
      floatx4 g = wmma_k4<CH>(sWm + 16 * w * SW, SW, 1, sK + 16 * t, S, 1, zero4());
#pragma unroll
      for (int i = 0; i < 4; ++i) out[P::G2 + (16 * w + rq + i) * D + 16 * t + col] = g[i];
    } else {  // sWm holds Tm: G2 = Tm K and Tm V, with Tm rows read 16 bytes at a time
      floatx4 g = wmma_k4<CH>(sWm + 16 * w * SW, SW, 1, sK + 16 * t, S, 1, zero4());
      floatx4 u = wmma_k4<CH>(sWm + 16 * w * SW, SW, 1, sVv + 16 * t, S, 1, zero4());
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        out[P::G2 + (16 * w + rq + i) * D + 16 * t + col] = g[i];
        out[P::E1 + (16 * w + rq + i) * D + 16 * t + col] = u[i];
      }
    }
  }
}

// 2. Entering state of every chunk, per (16-row slice of S, b, h).
template <int D>
__device__ __forceinline__ void delta_bwd_fwd(const float* __restrict__ k, const float* __restrict__ v,
                                                     int T, int n_chunks, const float* __restrict__ S0,
                                                     const float* __restrict__ pre, float* __restrict__ Sc) {
  constexpr int S = DB<D>::S, SV = DB<D>::SV;
  using P = Pre<D>;
  __shared__ __attribute__((aligned(16))) float sS[SL * S];
  __shared__ __attribute__((aligned(16))) float sK[CH * S];
  __shared__ __attribute__((aligned(16))) float sG[CH * S];   // G2
  __shared__ __attribute__((aligned(16))) float sV[CH * SV];
  __shared__ __attribute__((aligned(16))) float sU[CH * SV];
  __shared__ __attribute__((aligned(16))) float sT[CH * SW];  // Tm
  const int j0 = blockIdx.x * SL, bh = blockIdx.y;
  const int w = wave_id(), l = lane_id(), col = l & 15, rq = (l >> 4) * 4;
  for (int i = threadIdx.x; i < SL * D; i += blockDim.x) {
    const int r = i / D, cc = i % D;
    sS[r * S + cc] = S0 != nullptr ? S0[((long)bh * D + j0 + r) * D + cc] : 0.f;
  }
  Rows<D> pk, pg;
  Rows<SL> pv;
  Rows<CH> pt;
  auto fetch = [&](int c) {
    const int t0 = c * CH, L = min(CH, T - t0);
    const float* pc = pre + ((long)bh * n_chunks + c) * P::SIZE;
    pk.load(k + ((long)bh * T + t0) * D, D, 0, L);
    pv.load(v + ((long)bh * T + t0) * D, D, j0, L);
    pt.load(pc + P::TM, CH, 0, CH);
    pg.load(pc + P::G2, D, 0, CH);
  };
  fetch(0);
  for (int c = 0; c < n_chunks; ++c) {
    __syncthreads();  // the previous chunk's update of sS is complete
    store_block<SL, D>(Sc + (((long)bh * n_chunks + c) * D + j0) * D, sS);
    pk.put(sK, S);
    pg.put(sG, S);
    pv.put(sV, SV);
    pt.put(sT, SW);
    __syncthreads();
    if (c + 1 < n_chunks) fetch(c + 1);
    {  // U = Tm V - G2 S^T, rows 16w..
      floatx4 u = wmma_k4<CH>(sT + 16 * w * SW, SW, 1, sV, SV, 1, zero4());
      floatx4 g = wmma_k4<D>(sG + 16 * w * S, S, 1, sS, 1, S, zero4());
#pragma unroll
      for (int i = 0; i < 4; ++i) sU[(16 * w + rq + i) * SV + col] = u[i] - g[i];
    }
    __syncthreads();
    for (int t = w; t < D / 16; t += 4) {  // S += U^T K, tile (rows j0.., columns 16t..)
      float* base = sS + rq * S + 16 * t + col;
      floatx4 acc;
#pragma unroll
      for (int i = 0; i < 4; ++i) acc[i] = base[i * S];
      acc = wmma_k4<CH>(sU, 1, SV, sK + 16 * t, S, 1, acc);
#pragma unroll
      for (int i = 0; i < 4; ++i) base[i * S] = acc[i];
    }
  }
}

// 3. Exit adjoint dS1 of every chunk, per (16-row slice of dS, b, h), chunks
//    in reverse; dS0 of the sequence at the end.
template <int D>
__device__ __forceinline__ void delta_bwd_rev(const float* __restrict__ q, const float* __restrict__ k,
                                                     const float* __restrict__ dO, const float* __restrict__ beta,
                                                     int T, int n_chunks, const float* __restrict__ dSf,
                                                     const float* __restrict__ pre, float* __restrict__ dSc,
                                                     float* __restrict__ dS0) {
  constexpr int S = DB<D>::S, SV = DB<D>::SV;
  using P = Pre<D>;
  __shared__ __attribute__((aligned(16))) float sD[SL * S];    // dS slice
  __shared__ __attribute__((aligned(16))) float sQ[CH * S];
  __shared__ __attribute__((aligned(16))) float sK[CH * S];
  __shared__ __attribute__((aligned(16))) float sE1[CH * S];
  __shared__ __attribute__((aligned(16))) float sO[CH * SV];   // dO slice
  __shared__ __attribute__((aligned(16))) float sX[CH * SV];   // dX
  __shared__ __attribute__((aligned(16))) float sE2[CH * SW];
  __shared__ float sB[CH];
  const int j0 = blockIdx.x * SL, bh = blockIdx.y;
  const int w = wave_id(), l = lane_id(), col = l & 15, rq = (l >> 4) * 4;
  for (int i = threadIdx.x; i < SL * D; i += blockDim.x) {
    const int r = i / D, cc = i % D;
    sD[r * S + cc] = dSf != nullptr ? dSf[((long)bh * D + j0 + r) * D + cc] : 0.f;
  }
  Rows<D> pq, pk, pe1;
  Rows<SL> po;
  Rows<CH> pe2;
  float pb = 0.f;
  auto fetch = [&](int c) {
    const int t0 = c * CH, L = min(CH, T - t0);
    const float* pc = pre + ((long)bh * n_chunks + c) * P::SIZE;
    pq.load(q + ((long)bh * T + t0) * D, D, 0, L);
    pk.load(k + ((long)bh * T + t0) * D, D, 0, L);
    po.load(dO + ((long)bh * T + t0) * D, D, j0, L);
    pe1.load(pc + P::E1, D, 0, CH);
    pe2.load(pc + P::E2, CH, 0, CH);
    if (threadIdx.x < CH) pb = (int)threadIdx.x < L ? beta[(long)bh * T + t0 + threadIdx.x] : 0.f;
  };
  fetch(n_chunks - 1);
  for (int c = n_chunks - 1; c >= 0; --c) {
    __syncthreads();  // the previous chunk's update of sD is complete
    store_block<SL, D>(dSc + (((long)bh * n_chunks + c) * D + j0) * D, sD);
    pq.put(sQ, S);
    pk.put(sK, S);
    pe1.put(sE1, S);
    po.put(sO, SV);
    pe2.put(sE2, SW);
    if (threadIdx.x < CH) sB[threadIdx.x] = pb;
    __syncthreads();
    if (c > 0) fetch(c - 1);
    {  // dX = diag(beta) (E1 dS^T + E2 dO), rows 16w..
      floatx4 y = wmma_k4<D>(sE1 + 16 * w * S, S, 1, sD, 1, S, zero4());
      y = wmma_k4<CH>(sE2 + 16 * w * SW, SW, 1, sO, SV, 1, y);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = 16 * w + rq + i;
        sX[r * SV + col] = sB[r] * y[i];
      }
    }
    __syncthreads();
    for (int t = w; t < D / 16; t += 4) {  // dS += dO^T Q - dX^T K, tile (rows j0.., columns 16t..)
      float* base = sD + rq * S + 16 * t + col;
      floatx4 acc, neg = zero4();
#pragma unroll
      for (int i = 0; i < 4; ++i) acc[i] = base[i * S];
      acc = wmma_k4<CH>(sO, 1, SV, sQ + 16 * t, S, 1, acc);
      neg = wmma_k4<CH>(sX, 1, SV, sK + 16 * t, S, 1, neg);
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

// 2 and 3 in one launch: they are independent, and each alone fills only
// D/16 x B x H workgroups.
template <int D>
__global__ __launch_bounds__(256) void delta_bwd_walks(const float* __restrict__ q, const float* __restrict__ k,
                                                       const float* __restrict__ v, const float* __restrict__ dO,
                                                       const float* __restrict__ beta, int T, int n_chunks,
                                                       const float* __restrict__ S0, const float* __restrict__ dSf,
                                                       const float* __restrict__ pre, float* __restrict__ Sc,
                                                       float* __restrict__ dSc, float* __restrict__ dS0) {
  if (blockIdx.z == 0)
    delta_bwd_fwd<D>(k, v, T, n_chunks, S0, pre, Sc);
  else
    delta_bwd_rev<D>(q, k, dO, beta, T, n_chunks, dSf, pre, dSc, dS0);
}

// ... as two launches where their LDS together would not fit a CU (D = 128)
template <int D>
__global__ __launch_bounds__(256) void delta_bwd_fwd_walk(const float* __restrict__ k, const float* __restrict__ v,
                                                          int T, int n_chunks, const float* __restrict__ S0,
                                                          const float* __restrict__ pre, float* __restrict__ Sc) {
  delta_bwd_fwd<D>(k, v, T, n_chunks, S0, pre, Sc);
}
template <int D>
__global__ __launch_bounds__(256) void delta_bwd_rev_walk(const float* __restrict__ q, const float* __restrict__ k,
                                                          const float* __restrict__ dO, const float* __restrict__ beta,
                                                          int T, int n_chunks, const float* __restrict__ dSf,
                                                          const float* __restrict__ pre, float* __restrict__ dSc,
                                                          float* __restrict__ dS0) {
  delta_bwd_rev<D>(q, k, dO, beta, T, n_chunks, dSf, pre, dSc, dS0);
}

// 4. Gradients of one chunk from its S0, dS1 and prep block.  Wave w owns
//    rows 16w..16w+15 of every [64][.] result.
template <int D>
__global__ __launch_bounds__(256) void delta_bwd_grads(
    const float* __restrict__ q, const float* __restrict__ k, const float* __restrict__ v,
    const float* __restrict__ dO, const float* __restrict__ beta, int T, int n_chunks,
    const float* __restrict__ pre, const float* __restrict__ Sc, const float* __restrict__ dSc,
    float* __restrict__ dq, float* __restrict__ dk, float* __restrict__ dv, float* __restrict__ dbeta) {
  constexpr int S = DB<D>::S;
  constexpr int NT = D / 16;
  using P = Pre<D>;
  __shared__ __attribute__((aligned(16))) float bS[D * S];    // S0, then dS1, then S0
  __shared__ __attribute__((aligned(16))) float bQ[CH * S];
  __shared__ __attribute__((aligned(16))) float bK[CH * S];
  __shared__ __attribute__((aligned(16))) float bX[CH * S];   // V, then X
  __shared__ __attribute__((aligned(16))) float bU[CH * S];
  __shared__ __attribute__((aligned(16))) float bO[CH * S];   // dO
  __shared__ __attribute__((aligned(16))) float bT[CH * SW];  // Tm, then dLk
  __shared__ __attribute__((aligned(16))) float bE[CH * SW];  // E2, then dY
  __shared__ __attribute__((aligned(16))) float bF[CH * SW];  // E1, then P1
  __shared__ float sB[CH], sDb[CH];
  const int c = blockIdx.x, bh = blockIdx.y;
  const int t0 = c * CH, L = min(CH, T - t0);
  const int w = wave_id(), l = lane_id(), col = l & 15, rq = (l >> 4) * 4;
  const long cs = ((long)bh * n_chunks + c) * D * D;  // this chunk's state block
  const long row0 = (long)bh * T + t0;
  const float* pc = pre + ((long)bh * n_chunks + c) * P::SIZE;

  // every load of the chunk is issued before the first LDS store; S0 and
  // dS1 stay in registers for the later phases that reload them
  Blk<D> s0, s1;
  s0.load(Sc + cs);
  s1.load(dSc + cs);
  {
    Rows<D> xq, xk, xv, xo, xf;
    Rows<CH> xt, xe;
    xq.load(q + row0 * D, D, 0, L);
    xk.load(k + row0 * D, D, 0, L);
    xv.load(v + row0 * D, D, 0, L);
    xo.load(dO + row0 * D, D, 0, L);
    xt.load(pc + P::TM, CH, 0, CH);
    xe.load(pc + P::E2, CH, 0, CH);
    xf.load(pc + P::E1, D, 0, CH);
    const float bb = (int)threadIdx.x < L ? beta[row0 + threadIdx.x] : 0.f;
    s0.put(bS);
    xq.put(bQ, S);
    xk.put(bK, S);
    xv.put(bX, S);
    xo.put(bO, S);
    xt.put(bT, SW);
    xe.put(bE, SW);
    xf.put(bF, SW);
    if (threadIdx.x < CH) sB[threadIdx.x] = bb;
  }
  __syncthreads();

  // X = V - K S0^T; dQ = dO S0 (first part)
  floatx4 aq[NT], ak[NT], y[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    floatx4 ks = wmma_k4<D>(bK + 16 * w * S, S, 1, bS + 16 * t * S, 1, S, zero4());
#pragma unroll
    for (int i = 0; i < 4; ++i) bX[(16 * w + rq + i) * S + 16 * t + col] -= ks[i];
    aq[t] = wmma_k4<D>(bO + 16 * w * S, S, 1, bS + 16 * t, S, 1, zero4());
  }
  __syncthreads();
  // U = Tm X; bring dS1 in
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    floatx4 u = wmma_k4<CH>(bT + 16 * w * SW, SW, 1, bX + 16 * t, S, 1, zero4());
#pragma unroll
    for (int i = 0; i < 4; ++i) bU[(16 * w + rq + i) * S + 16 * t + col] = u[i];
  }
  s1.put(bS);
  __syncthreads();
  // dY = E1 dS1^T + E2 dO (registers); dK = U dS1 (first part)
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    y[t] = wmma_k4<D>(bF + 16 * w * SW, SW, 1, bS + 16 * t * S, 1, S, zero4());
    y[t] = wmma_k4<CH>(bE + 16 * w * SW, SW, 1, bO + 16 * t, S, 1, y[t]);
    ak[t] = wmma_k4<D>(bU + 16 * w * S, S, 1, bS + 16 * t, S, 1, zero4());
  }
  __syncthreads();
  // dY into bE; S0 back in
#pragma unroll
  for (int t = 0; t < NT; ++t)
#pragma unroll
    for (int i = 0; i < 4; ++i) bE[(16 * w + rq + i) * SW + 16 * t + col] = y[t][i];
  s0.put(bS);
  __syncthreads();
  // dV = diag(beta) dY; dbeta first part <dY_r, X_r>; P1 = tril_0(dO U^T) into
  // bF; P2 = tril_-1(dY U^T) gives dLk into bT and the second part of dbeta
#pragma unroll
  for (int t = 0; t < NT; ++t)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = 16 * w + rq + i;
      if (r < L) dv[(row0 + r) * D + 16 * t + col] = sB[r] * y[t][i];
    }
  {
    const int r = 16 * w + (l >> 2), part = l & 3;
    float s = 0.f;
    for (int j = part; j < D; j += 4) s += bE[r * SW + j] * bX[r * S + j];
    s += __shfl_xor(s, 1);
    s += __shfl_xor(s, 2);
    if (part == 0) sDb[r] = s;
  }
  float db2[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int ct = 0; ct < 4; ++ct) {
    floatx4 p1 = wmma_k4<D>(bO + 16 * w * S, S, 1, bU + 16 * ct * S, 1, S, zero4());
    floatx4 p2 = wmma_k4<D>(bE + 16 * w * SW, SW, 1, bU + 16 * ct * S, 1, S, zero4());
    floatx4 kk = wmma_k4<D>(bK + 16 * w * S, S, 1, bK + 16 * ct * S, 1, S, zero4());
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = 16 * w + rq + i, cc = 16 * ct + col;
      bF[r * SW + cc] = cc <= r ? p1[i] : 0.f;
      const float p = cc < r ? p2[i] : 0.f;
      bT[r * SW + cc] = -sB[r] * p;
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
    aq[t] = wmma_k4<CH>(bF + 16 * w * SW, SW, 1, bK + 16 * t, S, 1, aq[t]);
    floatx4 ys = wmma_k4<D>(bE + 16 * w * SW, SW, 1, bS + 16 * t, S, 1, zero4());
#pragma unroll
    for (int i = 0; i < 4; ++i) ak[t][i] -= sB[16 * w + rq + i] * ys[i];
    ak[t] = wmma_k4<CH>(bF + 16 * w, 1, SW, bQ + 16 * t, S, 1, ak[t]);
    ak[t] = wmma_k4<CH>(bT + 16 * w * SW, SW, 1, bK + 16 * t, S, 1, ak[t]);
    ak[t] = wmma_k4<CH>(bT + 16 * w, 1, SW, bK + 16 * t, S, 1, ak[t]);
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

// 4 at D = 128: the gradients of one chunk with the d_v rows taken in pieces
// of 16 (piece p: rows 16p.. of S0 and dS1, columns 16p.. of V, dO, dV).
// Per piece, with wave w owning the chunk's tokens 16w..16w+15:
//   X_p = V_p - K S0_p^T,  dY_p = E1 dS1_p^T + E2 dO_p,  dV_p = diag(beta) dY_p,
//   U_p = Tm X_p,
// and the sums over the pieces, kept in registers:
//   P1 += dO_p U_p^T,  P2 += dY_p U_p^T,  <dY_r, X_r>,
//   dQ += dO_p S0_p,   dK += U_p dS1_p - diag(beta) dY_p S0_p.
// Then, as in delta_bwd_grads, P1 = tril_0(P1), P2 = tril_-1(P2), dLk =
// -diag(beta) P2, dQ += P1 K, dK += P1^T Q + dLk K + dLk^T K and
// dbeta_r = <dY_r, X_r> - sum_{c<r} P2[r][c] <k_r, k_c>.
__global__ __launch_bounds__(256) void delta_bwd_grads_pieces(
    const float* __restrict__ q, const float* __restrict__ k, const float* __restrict__ v,
    const float* __restrict__ dO, const float* __restrict__ beta, int T, int n_chunks,
    const float* __restrict__ pre, const float* __restrict__ Sc, const float* __restrict__ dSc,
    float* __restrict__ dq, float* __restrict__ dk, float* __restrict__ dv, float* __restrict__ dbeta) {
  constexpr int D = 128, PV = 16;          // d, rows of a piece
  constexpr int S = DB<D>::S, SV = PV + 4;
  constexpr int NT = D / 16;
  using P = Pre<D>;
  __shared__ __attribute__((aligned(16))) float bK[CH * S];
  __shared__ __attribute__((aligned(16))) float bE1[CH * S];  // E1, then Q
  __shared__ __attribute__((aligned(16))) float bT[CH * SW];  // Tm, then P1
  __shared__ __attribute__((aligned(16))) float bE[CH * SW];  // E2, then dLk
  __shared__ __attribute__((aligned(16))) float bS0[PV * S];  // S0 rows of the piece
  __shared__ __attribute__((aligned(16))) float bS1[PV * S];  // dS1 rows of the piece
  __shared__ __attribute__((aligned(16))) float bX[CH * SV];  // V, then X
  __shared__ __attribute__((aligned(16))) float bO[CH * SV];  // dO
  __shared__ __attribute__((aligned(16))) float bU[CH * SV];
  __shared__ __attribute__((aligned(16))) float bY[CH * SV];  // dY
  __shared__ float sB[CH];
  const int c = blockIdx.x, bh = blockIdx.y;
  const int t0 = c * CH, L = min(CH, T - t0);
  const int w = wave_id(), l = lane_id(), col = l & 15, rq = (l >> 4) * 4;
  const long cs = ((long)bh * n_chunks + c) * D * D;  // this chunk's state block
  const long row0 = (long)bh * T + t0;
  const float* pc = pre + ((long)bh * n_chunks + c) * P::SIZE;

  stage<D>(bK, S, k + row0 * D, D, 0, L);
  stage<D>(bE1, S, pc + P::E1, D, 0, CH);
  stage<CH>(bT, SW, pc + P::TM, CH, 0, CH);
  stage<CH>(bE, SW, pc + P::E2, CH, 0, CH);
  if (threadIdx.x < CH) sB[threadIdx.x] = (int)threadIdx.x < L ? beta[row0 + threadIdx.x] : 0.f;

  floatx4 aq[NT], ak[NT], p1[4], p2[4];
#pragma unroll
  for (int t = 0; t < NT; ++t) aq[t] = ak[t] = zero4();
#pragma unroll
  for (int ct = 0; ct < 4; ++ct) p1[ct] = p2[ct] = zero4();
  float db1[4] = {0.f, 0.f, 0.f, 0.f};

#pragma unroll 1
  for (int pp = 0; pp < D / PV; ++pp) {
    const int j0 = PV * pp;
    // the previous piece's reads of bS0, bS1, bX, bO, bU, bY are complete
    __syncthreads();
    for (int i = threadIdx.x; i < PV * D / 4; i += blockDim.x) {
      const int r = i / (D / 4), cc = 4 * (i % (D / 4));
      *reinterpret_cast<float4*>(bS0 + r * S + cc) =
          *reinterpret_cast<const float4*>(Sc + cs + (long)(j0 + r) * D + cc);
      *reinterpret_cast<float4*>(bS1 + r * S + cc) =
          *reinterpret_cast<const float4*>(dSc + cs + (long)(j0 + r) * D + cc);
    }
    stage<PV>(bX, SV, v + row0 * D, D, j0, L);
    stage<PV>(bO, SV, dO + row0 * D, D, j0, L);
    __syncthreads();
    // X_p = V_p - K S0_p^T and dY_p = E1 dS1_p^T + E2 dO_p, rows 16w..
    {
      const floatx4 ks = wmma_k4<D>(bK + 16 * w * S, S, 1, bS0, 1, S, zero4());
      floatx4 y = wmma_k4<D>(bE1 + 16 * w * S, S, 1, bS1, 1, S, zero4());
      y = wmma_k4<CH>(bE + 16 * w * SW, SW, 1, bO, SV, 1, y);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = 16 * w + rq + i;
        const float x = bX[r * SV + col] - ks[i];
        bX[r * SV + col] = x;
        bY[r * SV + col] = y[i];
        db1[i] += x * y[i];
        if (r < L) dv[(row0 + r) * D + j0 + col] = sB[r] * y[i];
      }
    }
    __syncthreads();
    {  // U_p = Tm X_p, rows 16w..
      const floatx4 u = wmma_k4<CH>(bT + 16 * w * SW, SW, 1, bX, SV, 1, zero4());
#pragma unroll
      for (int i = 0; i < 4; ++i) bU[(16 * w + rq + i) * SV + col] = u[i];
    }
    __syncthreads();
    // sums over the pieces: P1, P2 (columns 16ct..), dQ, dK (columns 16t..)
#pragma unroll
    for (int ct = 0; ct < 4; ++ct) {
      p1[ct] = wmma_k4<PV>(bO + 16 * w * SV, SV, 1, bU + 16 * ct * SV, 1, SV, p1[ct]);
      p2[ct] = wmma_k4<PV>(bY + 16 * w * SV, SV, 1, bU + 16 * ct * SV, 1, SV, p2[ct]);
    }
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      aq[t] = wmma_k4<PV>(bO + 16 * w * SV, SV, 1, bS0 + 16 * t, S, 1, aq[t]);
      ak[t] = wmma_k4<PV>(bU + 16 * w * SV, SV, 1, bS1 + 16 * t, S, 1, ak[t]);
      const floatx4 ys = wmma_k4<PV>(bY + 16 * w * SV, SV, 1, bS0 + 16 * t, S, 1, zero4());
#pragma unroll
      for (int i = 0; i < 4; ++i) ak[t][i] -= sB[16 * w + rq + i] * ys[i];
    }
  }
  __syncthreads();  // every wave is done with Tm, E2 and E1
  // P1 = tril_0 into bT, dLk = -diag(beta) tril_-1(P2) into bE, Q into bE1;
  // the second part of dbeta
  stage<D>(bE1, S, q + row0 * D, D, 0, L);
  float db2[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int ct = 0; ct < 4; ++ct) {
    const floatx4 kk = wmma_k4<D>(bK + 16 * w * S, S, 1, bK + 16 * ct * S, 1, S, zero4());
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = 16 * w + rq + i, cc = 16 * ct + col;
      bT[r * SW + cc] = cc <= r ? p1[ct][i] : 0.f;
      const float p = cc < r ? p2[ct][i] : 0.f;
      bE[r * SW + cc] = -sB[r] * p;
      db2[i] += p * kk[i];
    }
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    float d1 = db1[i], d2 = db2[i];
#pragma unroll
    for (int off = 1; off < 16; off <<= 1) {
      d1 += __shfl_xor(d1, off);
      d2 += __shfl_xor(d2, off);
    }
    const int r = 16 * w + rq + i;
    if (col == 0 && r < L) dbeta[row0 + r] = d1 - d2;
  }
  __syncthreads();
  // dQ += P1 K;  dK += P1^T Q + dLk K + dLk^T K
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    aq[t] = wmma_k4<CH>(bT + 16 * w * SW, SW, 1, bK + 16 * t, S, 1, aq[t]);
    ak[t] = wmma_k4<CH>(bT + 16 * w, 1, SW, bE1 + 16 * t, S, 1, ak[t]);
    ak[t] = wmma_k4<CH>(bE + 16 * w * SW, SW, 1, bK + 16 * t, S, 1, ak[t]);
    ak[t] = wmma_k4<CH>(bE + 16 * w, 1, SW, bK + 16 * t, S, 1, ak[t]);
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
  float* pre = reinterpret_cast<float*>(ws);
  float* Sc = pre + (long)BH * nC * Pre<D>::SIZE;
  float* dSc = Sc + (long)BH * nC * D * D;
  hipLaunchKernelGGL((delta_bwd_prep<D, false>), dim3(nC, BH), dim3(256), 0, s, q, k, nullptr, beta, T, nC, pre);
  if constexpr (D == 128) {
    hipLaunchKernelGGL((delta_bwd_fwd_walk<D>), dim3(D / SL, BH), dim3(256), 0, s, k, v, T, nC, S0, pre, Sc);
    hipLaunchKernelGGL((delta_bwd_rev_walk<D>), dim3(D / SL, BH), dim3(256), 0, s, q, k, dO, beta, T, nC, dSf, pre,
                       dSc, dS0);
    profile_mark_before(s);
    hipLaunchKernelGGL(delta_bwd_grads_pieces, dim3(nC, BH), dim3(256), 0, s, q, k, v, dO, beta, T, nC, pre, Sc,
                       dSc, dq, dk, dv, dbeta);
    profile_mark_after(s);
  } else {
    hipLaunchKernelGGL((delta_bwd_walks<D>), dim3(D / SL, BH, 2), dim3(256), 0, s, q, k, v, dO, beta, T, nC, S0,
                       dSf, pre, Sc, dSc, dS0);
    profile_mark_before(s);
    hipLaunchKernelGGL((delta_bwd_grads<D>), dim3(nC, BH), dim3(256), 0, s, q, k, v, dO, beta, T, nC, pre, Sc, dSc,
                       dq, dk, dv, dbeta);
    profile_mark_after(s);
  }
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// The forward itself (fp32, d <= 128) on the same prep: per chunk, with A =
// tril_0(Q K^T) kept by the prep in place of E2 and Tm V in place of E1,
//   U = Tm V - G2 S0^T,   O = Q S0^T + A U,   S1 = S0 + U^T K,
// per (16-row slice of S, b, h), chunks in order, the next chunk prefetched
// into registers.  O's columns j0.. come from the slice (row j of S only
// sees column j of V, U and O).  The products are formed transposed, so that
// every MFMA operand is an LDS row contiguous in k (mma_rows: one 16-byte
// read feeds four MFMAs): wave w takes the chunk's tokens 16w..16w+15 in
//   U^T = (Tm V)^T - S G2^T,   O^T = S Q^T + U^T A^T,
// and the state tile (slice rows, d_k columns 16w..) in S += U^T K.
template <int D>
__global__ __launch_bounds__(256) void delta_fwd_walk(const float* __restrict__ q, const float* __restrict__ k,
                                                      int T, int n_chunks, const float* __restrict__ S0,
                                                      const float* __restrict__ pre, float* __restrict__ o,
                                                      float* __restrict__ S_final) {
  constexpr int S = DB<D>::S;
  using P = Pre<D>;
  __shared__ __attribute__((aligned(16))) float sS[SL * S];        // the slice [16][D]
  __shared__ __attribute__((aligned(16))) float sGQ[2][CH * S];    // G2, Q rows [64][D]
  __shared__ __attribute__((aligned(16))) float sKt[D * SW];       // K^T [D][64]
  __shared__ __attribute__((aligned(16))) float sUt[SL * SW];      // U^T [16][64]
  __shared__ __attribute__((aligned(16))) float sA[CH * SW];       // tril_0(Q K^T)
  const int j0 = blockIdx.x * SL, bh = blockIdx.y;
  const int w = wave_id(), l = lane_id(), r = l & 15, g = l >> 4;
  for (int i = threadIdx.x; i < SL * D; i += blockDim.x) {
    const int rr = i / D, cc = i % D;
    sS[rr * S + cc] = S0 != nullptr ? S0[((long)bh * D + j0 + rr) * D + cc] : 0.f;
  }
  Rows<D> pq, pk, pg;
  Rows<CH> pa;
  float4 tv;  // (Tm V)[token 16 w + r][j0 + 4 g ..] of the chunk
  auto fetch = [&](int c) {
    const int t0 = c * CH, L = min(CH, T - t0);
    const float* pc = pre + ((long)bh * n_chunks + c) * P::SIZE;
    pq.load(q + ((long)bh * T + t0) * D, D, 0, L);
    pk.load(k + ((long)bh * T + t0) * D, D, 0, L);
    pa.load(pc + P::E2, CH, 0, CH);
    pg.load(pc + P::G2, D, 0, CH);
    tv = *reinterpret_cast<const float4*>(pc + P::E1 + (16 * w + r) * D + j0 + 4 * g);
  };
  // a [64][NC] row block into LDS transposed ([NC][64], row stride SW)
  auto put_t = [](float* dst, const float4* x, int n4, int nc) __attribute__((always_inline)) {
    for (int i = 0; i < n4; ++i) {
      const int idx = i * 256 + (int)threadIdx.x, row = idx / (nc / 4), c = (idx % (nc / 4)) * 4;
      if (row < CH) {
        dst[(c + 0) * SW + row] = x[i].x;
        dst[(c + 1) * SW + row] = x[i].y;
        dst[(c + 2) * SW + row] = x[i].z;
        dst[(c + 3) * SW + row] = x[i].w;
      }
    }
  };
  fetch(0);
  for (int c = 0; c < n_chunks; ++c) {
    const int t0 = c * CH, L = min(CH, T - t0);
    __syncthreads();  // the previous chunk's update of sS and reads of U^T are complete
    pg.put(sGQ[0], S);
    pq.put(sGQ[1], S);
    put_t(sKt, pk.x, Rows<D>::N, D);
    pa.put(sA, SW);
    const float ut[4] = {tv.x, tv.y, tv.z, tv.w};  // (Tm V)^T: slice rows 4g + i, token 16w + r
    __syncthreads();
    if (c + 1 < n_chunks) fetch(c + 1);
    floatx4 gq[2] = {zero4(), zero4()};
    mma_rows<D, 2>(sS, S, sGQ[0] + 16 * w * S, CH * S, S, gq);  // S G2^T, S Q^T (tokens 16w..)
    // element i of lane (r, g): slice row 4g + i, token 16w + r
#pragma unroll
    for (int i = 0; i < 4; ++i) sUt[(4 * g + i) * SW + 16 * w + r] = ut[i] - gq[0][i];
    __syncthreads();
    floatx4 ot = gq[1];
    mma_rows<CH, 1>(sUt, SW, sA + 16 * w * SW, 0, SW, &ot);  // O^T += U^T A^T
    if (16 * w + r < L)
      *reinterpret_cast<float4*>(o + ((long)bh * T + t0 + 16 * w + r) * D + j0 + 4 * g) =
          make_float4(ot[0], ot[1], ot[2], ot[3]);
    for (int t = w; t < D / 16; t += 4) {  // S += U^T K, tile (slice rows, columns 16t..)
      float* base = sS + 4 * g * S + 16 * t + r;
      floatx4 acc;
#pragma unroll
      for (int i = 0; i < 4; ++i) acc[i] = base[i * S];
      mma_rows<CH, 1>(sUt, SW, sKt + 16 * t * SW, 0, SW, &acc);
#pragma unroll
      for (int i = 0; i < 4; ++i) base[i * S] = acc[i];
    }
  }
  if (S_final != nullptr) {
    __syncthreads();
    for (int i = threadIdx.x; i < SL * D; i += blockDim.x) {
      const int rr = i / D, cc = i % D;
      S_final[((long)bh * D + j0 + rr) * D + cc] = sS[rr * S + cc];
    }
  }
}

template <int D>
hipError_t run_delta_forward(const float* q, const float* k, const float* v, const float* beta, int B, int H, int T,
                             const float* S0, float* o, float* S_final, char* ws, hipStream_t s) {
  const int BH = B * H, nC = (T + CH - 1) / CH;
  float* pre = reinterpret_cast<float*>(ws);
  hipLaunchKernelGGL((delta_bwd_prep<D, true>), dim3(nC, BH), dim3(256), 0, s, q, k, v, beta, T, nC, pre);
  profile_mark_before(s);
  hipLaunchKernelGGL((delta_fwd_walk<D>), dim3(D / SL, BH), dim3(256), 0, s, q, k, T, nC, S0, pre, o, S_final);
  profile_mark_after(s);
  return hipGetLastError();
}

// T = 0: nothing is read or written but dS0 = dS_final (or 0)
__global__ void delta_bwd_empty(const float* __restrict__ dSf, float* __restrict__ dS0, long n) {
  const long i = (long)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) dS0[i] = dSf != nullptr ? dSf[i] : 0.f;
}

}  // namespace

bool delta_f32_fast(bool bf16, int d) { return !bf16 && (d == 16 || d == 32 || d == 64 || d == 128); }

size_t delta_f32_ws_bytes(int B, int H, int T, int d) {
  const long nC = (T + CH - 1) / CH;
  return (size_t)B * H * nC * (2 * (size_t)CH * CH + 2 * (size_t)CH * d) * sizeof(float);
}

hipError_t launch_delta_f32(const float* q, const float* k, const float* v, const float* beta, int B, int H, int T,
                            int d, const float* S0, float* o, float* S_final, void* ws, hipStream_t s) {
  char* w = static_cast<char*>(ws);
  switch (d) {
    case 16: return run_delta_forward<16>(q, k, v, beta, B, H, T, S0, o, S_final, w, s);
    case 32: return run_delta_forward<32>(q, k, v, beta, B, H, T, S0, o, S_final, w, s);
    case 64: return run_delta_forward<64>(q, k, v, beta, B, H, T, S0, o, S_final, w, s);
    case 128: return run_delta_forward<128>(q, k, v, beta, B, H, T, S0, o, S_final, w, s);
    default: return hipErrorInvalidValue;
  }
}

size_t delta_bwd_ws_bytes(int B, int H, int T, int d) {
  const long nC = (T + CH - 1) / CH;
  return (size_t)B * H * nC * (2 * (size_t)CH * CH + 2 * (size_t)CH * d + 2 * (size_t)d * d) * sizeof(float);
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
    case 128: return run_delta_backward<128>(q, k, v, beta, B, H, T, S0, dO, dSf, dq, dk, dv, dbeta, dS0, w, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace tc

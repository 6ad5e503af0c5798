// delta_scan.hip — chunked delta-rule scan (gfx950).
//
// "DeltaNet-family linear attention variants", DeltaNet section: the write
// is the prediction error, e_t = beta_t (v_t - S_{t-1} k_t), S_t = S_{t-1} + e_t k_t^T,
// and the read after the write is o_t = S_t q_t (S is d_v x d_k).
//
// Chunked form (derived from that rule; the page gives only the per-token
// form).  In a chunk entered with state S0, u_r = beta_r (v_r - S_{r-1} k_r) and
// S_{r-1} k_r = S0 k_r + sum_{i<r} <k_r, k_i> u_i, hence
//   u_r = beta_r (v_r - S0 k_r) - beta_r sum_{i<r} <k_r, k_i> u_i   (forward substitution)
//   O   = Q S0^T + (Q K^T masked to i <= r) U
//   S   = S0 + U^T K.
// The rows of S are independent (row j only sees column j of V and U), so
// one workgroup owns a d_v tile of S for one (b, h) and walks the chunks in
// order.  GEMM-shaped steps use fp32 MFMA (v_mfma_f32_16x16x4_f32) on LDS
// tiles; bf16 inputs are widened to fp32 when staged.
#include "tc_common.hpp"
#include "tc_kernels.hpp"

namespace tc {

namespace {

constexpr int CH = 64;

template <typename TIn, int D>
__device__ __forceinline__ void stage_rows(float* dst, int dst_ld, const TIn* src, long ld,
                                           int col0, int nvalid) {
  constexpr int V4 = D / 4;
  for (int idx = threadIdx.x; idx < CH * V4; idx += blockDim.x) {
    const int r = idx / V4;
    const int c = (idx % V4) * 4;
    float x0 = 0.f, x1 = 0.f, x2 = 0.f, x3 = 0.f;
    if (r < nvalid) {
      const TIn* p = src + r * ld + col0 + c;
      x0 = InT<TIn>::ld(p, 0);
      x1 = InT<TIn>::ld(p, 1);
      x2 = InT<TIn>::ld(p, 2);
      x3 = InT<TIn>::ld(p, 3);
    }
    float* d = dst + r * dst_ld + c;
    d[0] = x0;
    d[1] = x1;
    d[2] = x2;
    d[3] = x3;
  }
}

template <int DK, int DVT, typename TIn>
__global__ __launch_bounds__(256) void delta_kernel(
    const TIn* __restrict__ q, const TIn* __restrict__ k, const TIn* __restrict__ v,
    const float* __restrict__ beta, int T, int dv, const float* __restrict__ S0,
    float* __restrict__ o, float* __restrict__ S_final) {
  constexpr int SQ = DK + 2;    // q, k rows
  constexpr int SU = DVT + 16;  // v / u rows
  constexpr int SP = CH + 2;    // k k^T, q k^T rows
  constexpr int SS = DK + 2;    // state rows (one row per d_v index)
  constexpr int NP = 256 / DVT; // lanes that share one column in the substitution
  __shared__ float sQ[CH * SQ];
  __shared__ float sK[CH * SQ];
  __shared__ float sU[CH * SU];
  __shared__ float sKK[CH * SP];
  __shared__ float sQK[CH * SP];
  __shared__ float sS[DVT * SS];
  __shared__ float sB[CH];

  const int dv0 = blockIdx.x * DVT, bh = blockIdx.y;
  const int l = lane_id(), w = wave_id();
  const int col = l & 15, rq = (l >> 4) * 4;

  for (int i = threadIdx.x; i < DVT * DK; i += blockDim.x) {
    const int r = i / DK, c = i % DK;
    sS[r * SS + c] = S0 ? S0[((long)bh * dv + dv0 + r) * DK + c] : 0.f;
  }

  const TIn* qb = q + (long)bh * T * DK;
  const TIn* kb = k + (long)bh * T * DK;
  const TIn* vb = v + (long)bh * T * dv;
  const float* bb = beta + (long)bh * T;
  float* ob = o + (long)bh * T * dv;

  for (int t0 = 0; t0 < T; t0 += CH) {
    const int L = min(CH, T - t0);
    __syncthreads();
    stage_rows<TIn, DK>(sQ, SQ, qb + (long)t0 * DK, DK, 0, L);
    stage_rows<TIn, DK>(sK, SQ, kb + (long)t0 * DK, DK, 0, L);
    stage_rows<TIn, DVT>(sU, SU, vb + (long)t0 * dv, dv, dv0, L);
    if (threadIdx.x < CH) sB[threadIdx.x] = threadIdx.x < L ? bb[t0 + threadIdx.x] : 0.f;
    __syncthreads();

    // K K^T and masked Q K^T (wave w: rows 16w..16w+15)
#pragma unroll
    for (int ct = 0; ct < 4; ++ct) {
      floatx4 kk = wave_mma_f32<DK>(sK + 16 * w * SQ, SQ, 1, sK + 16 * ct * SQ, 1, SQ, zero4());
      floatx4 qk = wave_mma_f32<DK>(sQ + 16 * w * SQ, SQ, 1, sK + 16 * ct * SQ, 1, SQ, zero4());
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = 16 * w + rq + i, c = 16 * ct + col;
        sKK[r * SP + c] = kk[i];
        sQK[r * SP + c] = (c <= r) ? qk[i] : 0.f;
      }
    }
    // right-hand side beta (V - K S0^T), in place over V
#pragma unroll
    for (int ct = 0; ct < DVT / 16; ++ct) {
      floatx4 ks = wave_mma_f32<DK>(sK + 16 * w * SQ, SQ, 1, sS + 16 * ct * SS, 1, SS, zero4());
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = 16 * w + rq + i;
        float* u = sU + r * SU + 16 * ct + col;
        *u = sB[r] * (*u - ks[i]);
      }
    }
    __syncthreads();

    // forward substitution u_r -= beta_r sum_{i<r} kk[r][i] u_i, one row at a time
    {
      const int c = threadIdx.x / NP, part = threadIdx.x % NP;
      for (int r = 1; r < L; ++r) {
        float acc = 0.f;
        for (int i = part; i < r; i += NP) acc += sKK[r * SP + i] * sU[i * SU + c];
#pragma unroll
        for (int off = 1; off < NP; off <<= 1) acc += __shfl_xor(acc, off);
        if (part == 0) sU[r * SU + c] -= sB[r] * acc;
        __syncthreads();
      }
    }

    // O = Q S0^T + (Q K^T masked) U
#pragma unroll
    for (int ct = 0; ct < DVT / 16; ++ct) {
      floatx4 acc = wave_mma_f32<DK>(sQ + 16 * w * SQ, SQ, 1, sS + 16 * ct * SS, 1, SS, zero4());
      acc = wave_mma_f32<CH>(sQK + 16 * w * SP, SP, 1, sU + 16 * ct, SU, 1, acc);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = 16 * w + rq + i;
        if (r < L) ob[(long)(t0 + r) * dv + dv0 + 16 * ct + col] = acc[i];
      }
    }
    __syncthreads();

    // S += U^T K  (tiles of the DVT x DK state slice)
    constexpr int NDT = DK / 16;
    constexpr int NT = (DVT / 16) * NDT;
    for (int tile = w; tile < NT; tile += 4) {
      const int vt = tile / NDT, dt = tile % NDT;
      float* base = sS + (16 * vt + rq) * SS + 16 * dt + col;
      floatx4 acc;
#pragma unroll
      for (int i = 0; i < 4; ++i) acc[i] = base[i * SS];
      acc = wave_mma_f32<CH>(sU + 16 * vt, 1, SU, sK + 16 * dt, SQ, 1, acc);
#pragma unroll
      for (int i = 0; i < 4; ++i) base[i * SS] = acc[i];
    }
  }
  if (S_final) {
    __syncthreads();
    for (int i = threadIdx.x; i < DVT * DK; i += blockDim.x) {
      const int r = i / DK, c = i % DK;
      S_final[((long)bh * dv + dv0 + r) * DK + c] = sS[r * SS + c];
    }
  }
}

template <typename TIn>
hipError_t dispatch_delta(const void* q, const void* k, const void* v, const float* beta, int B,
                          int H, int T, int d, const float* S0, float* o, float* S_final,
                          hipStream_t s) {
  const TIn* Q = static_cast<const TIn*>(q);
  const TIn* K = static_cast<const TIn*>(k);
  const TIn* V = static_cast<const TIn*>(v);
  const int BH = B * H;
#define TC_DELTA_CASE(DK, DVT)                                                               \
  case DK:                                                                                   \
    profile_mark_before(s);                                                                  \
    hipLaunchKernelGGL((delta_kernel<DK, DVT, TIn>), dim3(DK / DVT, BH), dim3(256), 0, s, Q, K, \
                       V, beta, T, d, S0, o, S_final);                                        \
    profile_mark_after(s);                                                                   \
    break;
  switch (d) {
    TC_DELTA_CASE(16, 16)
    TC_DELTA_CASE(32, 32)
    TC_DELTA_CASE(64, 64)
    TC_DELTA_CASE(128, 64)
    default: return hipErrorInvalidValue;
  }
#undef TC_DELTA_CASE
  return hipGetLastError();
}

}  // namespace

size_t delta_ws_bytes(int B, int H, int T, int dk, int dv, bool bf16) {
  (void)dv;
  if (delta_bf16_supported(bf16, dk)) return delta_bf16_ws_bytes(B, H, T, dk);
  if (delta_f32_fast(bf16, dk) && T > 0) return delta_f32_ws_bytes(B, H, T, dk);
  return 0;
}

hipError_t launch_delta_scan(const void* q, const void* k, const void* v, bool bf16,
                             const float* beta, int B, int H, int T, int dk, int dv,
                             const float* S0, float* o, float* S_final, void* ws, hipStream_t s) {
  (void)dv;
  if (delta_bf16_supported(bf16, dk))
    return launch_delta_bf16(q, k, v, beta, B, H, T, dk, S0, o, S_final, ws, s);
  if (delta_f32_fast(bf16, dk) && T > 0)
    return launch_delta_f32(static_cast<const float*>(q), static_cast<const float*>(k), static_cast<const float*>(v),
                            beta, B, H, T, dk, S0, o, S_final, ws, s);
  if (bf16) return dispatch_delta<uint16_t>(q, k, v, beta, B, H, T, dk, S0, o, S_final, s);
  return dispatch_delta<float>(q, k, v, beta, B, H, T, dk, S0, o, S_final, s);
}

}  // namespace tc

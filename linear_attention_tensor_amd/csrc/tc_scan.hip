// tc_scan.hip — chunked prefill scan of the Tensor Cache L2 memory (gfx950).
//
// Tensor Cache, Methodology 1 (write A <- lam A + eta k v^T when the ring
// overwrites a slot, read m_t = q_t A) and Methodology 2 (a parallel
// weighted-sum scan that equals the sequential writes).
//
// With s = t - W the read is m_{s+W} = eta sum_{j<=s} lam^(s-j) <q_{s+W}, k_j> v_j,
// scalar-decay linear attention whose query stream is shifted by W.  Chunks
// of 64 positions: for chunk n with entering state S_n (all writes j < 64n),
//   o_r     = lam^(r+1) q'_r S_n + eta sum_{c<=r} lam^(r-c) <q'_r, k_c> v_c
//   S_{n+1} = lam^L S_n + eta sum_c lam^(L-1-c) k_c v_c^T        (L = chunk length)
// Three launches:
//   1. scan_state:  per segment of `seg_chunks` chunks, the segment's own
//      contribution to the state (from zero), fully parallel;
//   2. scan_prefix: entering state of every segment, sequential over the
//      segments but parallel over the d_k x d_v elements;
//   3. scan_output: per segment, carry the state through its chunks and
//      write m.  Rows t < W are zero.
// Arithmetic: fp32 MFMA (v_mfma_f32_16x16x4_f32) on LDS tiles; bf16 inputs
// are widened to fp32 when staged, and the state is fp32 throughout.
#include "tc_common.hpp"
#include "tc_kernels.hpp"

#include <algorithm>

namespace tc {

namespace {

constexpr int CH = 64;  // positions per chunk

template <int DK, int DVT>
struct ScanLds {
  static constexpr int SQ = DK + 2;   // row stride of q', k: A-operand pattern
  static constexpr int SV = DVT + 16; // row stride of v, S: B-operand pattern
  static constexpr int SP = CH + 2;
};

// Copy rows [0, 64) x [0, D) of a row-major source (row stride `ld`, first
// column `col0`) into LDS as fp32; rows >= nvalid become zero.
template <typename TIn, int D>
__device__ __forceinline__ void stage(float* dst, int dst_ld, const TIn* src, long ld, int col0,
                                      int nvalid) {
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

// S (DK x DVT, LDS) <- lam^L S + K^T diag(w) V, with w already folded into V.
template <int DK, int DVT>
__device__ __forceinline__ void state_update(float* sS, const float* sK, const float* sV,
                                             float lamL) {
  using Ly = ScanLds<DK, DVT>;
  constexpr int NVT = DVT / 16;
  constexpr int NT = (DK / 16) * NVT;
  const int l = lane_id();
  const int col = l & 15, rq = (l >> 4) * 4;
  for (int tile = wave_id(); tile < NT; tile += 4) {
    const int dt = tile / NVT, vt = tile % NVT;
    float* base = sS + (16 * dt + rq) * Ly::SV + 16 * vt + col;
    floatx4 acc;
#pragma unroll
    for (int i = 0; i < 4; ++i) acc[i] = lamL * base[i * Ly::SV];
    // A(m = d, k = key) = K[key][16dt + m];  B(k = key, n) = V[key][16vt + n]
    acc = wave_mma_f32<CH>(sK + 16 * dt, 1, Ly::SQ, sV + 16 * vt, Ly::SV, 1, acc);
#pragma unroll
    for (int i = 0; i < 4; ++i) base[i * Ly::SV] = acc[i];
  }
}

template <int DK, int DVT, typename TIn>
__global__ __launch_bounds__(256) void scan_state_kernel(const TIn* __restrict__ k,
                                                         const TIn* __restrict__ v,
                                                         const float* __restrict__ lam,
                                                         const float* __restrict__ eta, int H,
                                                         int T, int dv, int n_act,
                                                         int seg_chunks, int n_seg,
                                                         float* __restrict__ ws) {
  using Ly = ScanLds<DK, DVT>;
  __shared__ float sK[CH * Ly::SQ];
  __shared__ float sV[CH * Ly::SV];
  __shared__ float sS[DK * Ly::SV];
  __shared__ float sW[CH];

  const int seg = blockIdx.x, dv0 = blockIdx.y * DVT, bh = blockIdx.z;
  const int h = bh % H;
  const float lm = lam[h], et = eta[h];
  for (int i = threadIdx.x; i < DK * Ly::SV; i += blockDim.x) sS[i] = 0.f;

  const int c_begin = seg * seg_chunks;
  const int c_end = min(c_begin + seg_chunks, (n_act + CH - 1) / CH);
  const TIn* kb = k + (long)bh * T * DK;
  const TIn* vb = v + (long)bh * T * dv;
  for (int c = c_begin; c < c_end; ++c) {
    const int s0 = c * CH;
    const int L = min(CH, n_act - s0);
    __syncthreads();
    stage<TIn, DK>(sK, Ly::SQ, kb + (long)s0 * DK, DK, 0, L);
    stage<TIn, DVT>(sV, Ly::SV, vb + (long)s0 * dv, dv, dv0, L);
    if (threadIdx.x < CH) sW[threadIdx.x] = threadIdx.x < L ? et * pow_int(lm, L - 1 - threadIdx.x) : 0.f;
    __syncthreads();
    for (int i = threadIdx.x; i < CH * DVT; i += blockDim.x) {
      const int r = i / DVT, cc = i % DVT;
      sV[r * Ly::SV + cc] *= sW[r];
    }
    __syncthreads();
    state_update<DK, DVT>(sS, sK, sV, pow_int(lm, L));
  }
  __syncthreads();
  float* out = ws + ((long)bh * n_seg + seg) * DK * dv;
  for (int i = threadIdx.x; i < DK * DVT; i += blockDim.x) {
    const int r = i / DVT, cc = i % DVT;
    out[r * dv + dv0 + cc] = sS[r * Ly::SV + cc];
  }
}

// Turns per-segment contributions into entering states, in place:
// entering(0) = 0, entering(p+1) = lam^len(p) entering(p) + delta(p).
__global__ void scan_prefix_kernel(const float* __restrict__ lam, int H, int n_per_bh, int n_act,
                                   int seg_len, int n_seg, float* __restrict__ ws) {
  const long idx = (long)blockIdx.x * blockDim.x + threadIdx.x;
  const int bh = blockIdx.y;
  if (idx >= n_per_bh) return;
  const float lm = lam[bh % H];
  const float lam_full = pow_int(lm, seg_len);
  float* p = ws + (long)bh * n_seg * n_per_bh + idx;
  float run = 0.f;
  for (int s = 0; s < n_seg - 1; ++s) {
    const float d = p[(long)s * n_per_bh];
    p[(long)s * n_per_bh] = run;
    run = lam_full * run + d;  // every segment but the last is full length
  }
  p[(long)(n_seg - 1) * n_per_bh] = run;
}

template <int DK, int DVT, typename TIn>
__global__ __launch_bounds__(256) void scan_output_kernel(
    const TIn* __restrict__ q, const TIn* __restrict__ k, const TIn* __restrict__ v,
    const float* __restrict__ lam, const float* __restrict__ eta, int H, int T, int dv, int W,
    int n_act, int seg_chunks, int n_seg, const float* __restrict__ ws, float* __restrict__ m,
    float* __restrict__ A_final) {
  using Ly = ScanLds<DK, DVT>;
  __shared__ float sQ[CH * Ly::SQ];
  __shared__ float sK[CH * Ly::SQ];
  __shared__ float sV[CH * Ly::SV];
  __shared__ float sP[CH * Ly::SP];
  __shared__ float sS[DK * Ly::SV];
  __shared__ float sW[CH];

  const int seg = blockIdx.x, dv0 = blockIdx.y * DVT, bh = blockIdx.z;
  const int h = bh % H;
  const float lm = lam[h], et = eta[h];
  const int l = lane_id(), w = wave_id();
  const int col = l & 15, rq = (l >> 4) * 4;

  if (n_seg > 1 && seg > 0) {
    const float* in = ws + ((long)bh * n_seg + seg) * DK * dv;
    for (int i = threadIdx.x; i < DK * DVT; i += blockDim.x) {
      const int r = i / DVT, cc = i % DVT;
      sS[r * Ly::SV + cc] = in[r * dv + dv0 + cc];
    }
  } else {
    for (int i = threadIdx.x; i < DK * Ly::SV; i += blockDim.x) sS[i] = 0.f;
  }

  const int c_begin = seg * seg_chunks;
  const int c_end = min(c_begin + seg_chunks, (n_act + CH - 1) / CH);
  const TIn* qb = q + (long)bh * T * DK;
  const TIn* kb = k + (long)bh * T * DK;
  const TIn* vb = v + (long)bh * T * dv;
  float* mb = m + (long)bh * T * dv;

  for (int c = c_begin; c < c_end; ++c) {
    const int s0 = c * CH;
    const int L = min(CH, n_act - s0);
    __syncthreads();
    stage<TIn, DK>(sQ, Ly::SQ, qb + (long)(s0 + W) * DK, DK, 0, L);
    stage<TIn, DK>(sK, Ly::SQ, kb + (long)s0 * DK, DK, 0, L);
    stage<TIn, DVT>(sV, Ly::SV, vb + (long)s0 * dv, dv, dv0, L);
    if (threadIdx.x < CH) sW[threadIdx.x] = threadIdx.x < L ? et * pow_int(lm, L - 1 - threadIdx.x) : 0.f;
    __syncthreads();

    // P = (Q' K^T) masked to c <= r and weighted by eta lam^(r-c); wave w owns rows 16w..16w+15.
#pragma unroll
    for (int ct = 0; ct < 4; ++ct) {
      floatx4 acc = wave_mma_f32<DK>(sQ + 16 * w * Ly::SQ, Ly::SQ, 1, sK + 16 * ct * Ly::SQ, 1,
                                     Ly::SQ, zero4());
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = 16 * w + rq + i, cc = 16 * ct + col;
        sP[r * Ly::SP + cc] = (cc <= r) ? acc[i] * et * pow_int(lm, r - cc) : 0.f;
      }
    }
    __syncthreads();

    // O = diag(lam^(r+1)) Q' S + P V  -> m rows W + s0 + r
#pragma unroll
    for (int ct = 0; ct < DVT / 16; ++ct) {
      floatx4 acc = wave_mma_f32<DK>(sQ + 16 * w * Ly::SQ, Ly::SQ, 1, sS + 16 * ct, Ly::SV, 1,
                                     zero4());
#pragma unroll
      for (int i = 0; i < 4; ++i) acc[i] *= pow_int(lm, 16 * w + rq + i + 1);
      acc = wave_mma_f32<CH>(sP + 16 * w * Ly::SP, Ly::SP, 1, sV + 16 * ct, Ly::SV, 1, acc);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = 16 * w + rq + i;
        if (r < L) mb[(long)(W + s0 + r) * dv + dv0 + 16 * ct + col] = acc[i];
      }
    }
    __syncthreads();
    for (int i = threadIdx.x; i < CH * DVT; i += blockDim.x) {
      const int r = i / DVT, cc = i % DVT;
      sV[r * Ly::SV + cc] *= sW[r];
    }
    __syncthreads();
    state_update<DK, DVT>(sS, sK, sV, pow_int(lm, L));
  }

  if (A_final != nullptr && seg == n_seg - 1) {
    __syncthreads();
    float* out = A_final + (long)bh * DK * dv;
    for (int i = threadIdx.x; i < DK * DVT; i += blockDim.x) {
      const int r = i / DVT, cc = i % DVT;
      out[r * dv + dv0 + cc] = sS[r * Ly::SV + cc];
    }
  }
}

// m rows t < min(W, T) are exactly zero; with no active position the final
// state is zero too.
__global__ void zero_rows_kernel(float* __restrict__ m, long rows_per_bh, long T, int dv) {
  const long bh = blockIdx.y;
  const long n = rows_per_bh * dv;
  for (long i = (long)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (long)gridDim.x * blockDim.x)
    m[bh * T * dv + i] = 0.f;
}

template <int DK, int DVT, typename TIn>
hipError_t run_scan(const TIn* q, const TIn* k, const TIn* v, const float* lam, const float* eta,
                    int B, int H, int T, int dv, int W, float* m, float* A_final, float* ws,
                    const ScanPlan& p, hipStream_t s) {
  const int BH = B * H;
  const long zrows = std::min<long>(W, T);
  if (zrows > 0) {
    dim3 g((unsigned)std::min<long>((zrows * dv + 255) / 256, 1024), BH);
    hipLaunchKernelGGL(zero_rows_kernel, g, dim3(256), 0, s, m, zrows, (long)T, dv);
  }
  if (p.n_act <= 0) {
    if (A_final != nullptr) {
      dim3 g((unsigned)std::min<long>(((long)DK * dv + 255) / 256, 1024), BH);
      hipLaunchKernelGGL(zero_rows_kernel, g, dim3(256), 0, s, A_final, (long)DK, (long)DK, dv);
    }
    return hipGetLastError();
  }
  const int nvt = dv / DVT;
  if (p.n_seg > 1) {
    dim3 g1(p.n_seg - 1, nvt, BH);
    hipLaunchKernelGGL((scan_state_kernel<DK, DVT, TIn>), g1, dim3(256), 0, s, k, v, lam, eta, H,
                       T, dv, p.n_act, p.seg_chunks, p.n_seg, ws);
    const int nel = DK * dv;
    dim3 g2((nel + 255) / 256, BH);
    hipLaunchKernelGGL(scan_prefix_kernel, g2, dim3(256), 0, s, lam, H, nel, p.n_act,
                       p.seg_chunks * CH, p.n_seg, ws);
  }
  dim3 g3(p.n_seg, nvt, BH);
  profile_mark_before(s);
  hipLaunchKernelGGL((scan_output_kernel<DK, DVT, TIn>), g3, dim3(256), 0, s, q, k, v, lam, eta,
                     H, T, dv, W, p.n_act, p.seg_chunks, p.n_seg, ws, m, A_final);
  profile_mark_after(s);
  return hipGetLastError();
}

template <typename TIn>
hipError_t dispatch_scan(const void* q, const void* k, const void* v, const float* lam,
                         const float* eta, int B, int H, int T, int d, int W, float* m,
                         float* A_final, float* ws, const ScanPlan& p, hipStream_t s) {
  const TIn* Q = static_cast<const TIn*>(q);
  const TIn* K = static_cast<const TIn*>(k);
  const TIn* V = static_cast<const TIn*>(v);
  switch (d) {
    case 16: return run_scan<16, 16, TIn>(Q, K, V, lam, eta, B, H, T, d, W, m, A_final, ws, p, s);
    case 32: return run_scan<32, 32, TIn>(Q, K, V, lam, eta, B, H, T, d, W, m, A_final, ws, p, s);
    case 64: return run_scan<64, 64, TIn>(Q, K, V, lam, eta, B, H, T, d, W, m, A_final, ws, p, s);
    case 128: return run_scan<128, 64, TIn>(Q, K, V, lam, eta, B, H, T, d, W, m, A_final, ws, p, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

ScanPlan plan_scan(int B, int H, int T, int dk, int dv, int W) {
  ScanPlan p{};
  p.n_act = std::max(T - W, 0);
  p.n_chunks = (p.n_act + CH - 1) / CH;
  p.dvt = dv > 64 ? 64 : dv;
  const long units = (long)B * H * (dv / p.dvt);
  // Aim for about 1024 workgroups in the output launch (4 per CU), and never
  // let a segment be shorter than 2 chunks unless the sequence is.
  long want_seg = units > 0 ? (1024 + units - 1) / units : 1;
  int seg_chunks = p.n_chunks > 0 ? (int)std::max<long>(2, (p.n_chunks + want_seg - 1) / want_seg) : 1;
  seg_chunks = std::min(seg_chunks, std::max(p.n_chunks, 1));
  p.seg_chunks = seg_chunks;
  p.n_seg = p.n_chunks > 0 ? (p.n_chunks + seg_chunks - 1) / seg_chunks : 0;
  (void)dk;
  return p;
}

size_t scan_ws_bytes(const ScanPlan& p, int B, int H, int dk, int dv) {
  if (p.n_seg <= 1) return 0;
  return (size_t)B * H * p.n_seg * dk * dv * sizeof(float);
}

hipError_t launch_tc_scan(const void* q, const void* k, const void* v, bool bf16,
                          const float* lam, const float* eta, int B, int H, int T, int dk, int dv,
                          int W, float* m, float* A_final, void* ws, hipStream_t s) {
  (void)dv;
  const ScanPlan p = plan_scan(B, H, T, dk, dv, W);
  float* w = static_cast<float*>(ws);
  if (bf16)
    return dispatch_scan<uint16_t>(q, k, v, lam, eta, B, H, T, dk, W, m, A_final, w, p, s);
  return dispatch_scan<float>(q, k, v, lam, eta, B, H, T, dk, W, m, A_final, w, p, s);
}

}  // namespace tc

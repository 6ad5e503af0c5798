// tc_window.hip — exact sliding-window softmax attention (the L1 cache of the
// Tensor Cache) in fp32 arithmetic, for the inputs the bf16 MFMA main kernel
// does not take: fp32 q, k, v (any d in {16, 32, 64, 128}) and bf16 with
// d in {16, 32}.
//
// Tensor Cache, Methodology 1: the L1 cache holds the W most recent tokens and
// the query attends to them with exact softmax,
//   y_local,t = sum_{j = max(0, t-W+1)}^{t} softmax_j(scale <q_t, k_j>) v_j;
// the fused layer adds the gated L2 read, y = y_local + sigmoid(g) m, where
// m (the read of tc_scan_forward) is already in y when GATED.
//
// One workgroup (4 waves) per 64 consecutive queries of one (b, h).  The keys
// the tile needs, [t0 - W + 1, t0 + 63], pass through LDS in blocks of 64 (K
// and V rows, fp32).  Thread (query r, column group c) scores its query
// against every key of its window itself (all four column groups of a query
// form the same scores, in the same order, so they agree bit for bit), keeps
// an online softmax (running maximum, normaliser and output) in fp32, and
// accumulates its d/4 output columns.
#include "tc_common.hpp"
#include "tc_kernels.hpp"

#include <math.h>

namespace tc {

namespace {

constexpr int WQ = 64;   // queries per workgroup
constexpr int WKB = 64;  // keys per LDS block

template <typename TIn, int D, bool GATED>
__global__ __launch_bounds__(256) void window_kernel(const TIn* __restrict__ q, const TIn* __restrict__ k,
                                                     const TIn* __restrict__ v, int H, int T, int W,
                                                     float scale, const float* __restrict__ g,
                                                     float* __restrict__ y) {
  constexpr int NG = 4, DG = D / NG;  // column groups per query, columns per group
  __shared__ float sk[WKB][D + 1];    // +1: consecutive rows start one bank apart, so lanes
  __shared__ float sv[WKB][D + 1];    // on different keys of one column do not collide
  const int bh = blockIdx.y, t0 = blockIdx.x * WQ;
  const int t = threadIdx.x, r = t % WQ, grp = t / WQ;
  const int tq = t0 + r;
  const long base = (long)bh * T;
  const bool live = tq < T;

  float qr[D];
#pragma unroll
  for (int c = 0; c < D; ++c) qr[c] = live ? InT<TIn>::ld(q, (base + tq) * D + c) : 0.f;
  float mx = -INFINITY, l = 0.f;
  float acc[DG];
#pragma unroll
  for (int i = 0; i < DG; ++i) acc[i] = 0.f;

  const int j_lo = max(0, t0 - W + 1), j_hi = min(T - 1, t0 + WQ - 1);
  for (int jb = j_lo; jb <= j_hi; jb += WKB) {
    __syncthreads();  // the previous block has been read by every thread
    for (int e = t; e < WKB * D; e += 256) {
      const int kr = e / D, c = e % D, j = jb + kr;
      const bool in = j <= j_hi;
      sk[kr][c] = in ? InT<TIn>::ld(k, (base + j) * D + c) : 0.f;
      sv[kr][c] = in ? InT<TIn>::ld(v, (base + j) * D + c) : 0.f;
    }
    __syncthreads();
    if (live) {
      const int lo = max(tq - W + 1, jb), hi = min(tq, jb + WKB - 1);
      for (int j = lo; j <= hi; ++j) {
        const float* kr = sk[j - jb];
        float s = 0.f;
#pragma unroll
        for (int c = 0; c < D; ++c) s = fmaf(qr[c], kr[c], s);
        s *= scale;
        if (s > mx) {  // move the reference maximum; O and l are rescaled with it
          const float a = expf(mx - s);
          l *= a;
#pragma unroll
          for (int i = 0; i < DG; ++i) acc[i] *= a;
          mx = s;
        }
        const float p = expf(s - mx);
        l += p;
        const float* vr = sv[j - jb] + grp * DG;
#pragma unroll
        for (int i = 0; i < DG; ++i) acc[i] = fmaf(p, vr[i], acc[i]);
      }
    }
  }
  if (live) {
    const float inv = 1.f / l;  // l >= 1: the key of the maximum contributes exp(0)
    float* yo = y + (base + tq) * D + grp * DG;
    const float gate = GATED ? 1.f / (1.f + expf(-g[bh % H])) : 0.f;
#pragma unroll
    for (int i = 0; i < DG; ++i) yo[i] = GATED ? fmaf(gate, yo[i], acc[i] * inv) : acc[i] * inv;
  }
}

template <typename TIn, bool GATED>
hipError_t run_window(const TIn* q, const TIn* k, const TIn* v, int B, int H, int T, int d, int W, float scale,
                      const float* g, float* y, hipStream_t s) {
  const dim3 grid((T + WQ - 1) / WQ, B * H), block(256);
  switch (d) {
    case 16: hipLaunchKernelGGL((window_kernel<TIn, 16, GATED>), grid, block, 0, s, q, k, v, H, T, W, scale, g, y); break;
    case 32: hipLaunchKernelGGL((window_kernel<TIn, 32, GATED>), grid, block, 0, s, q, k, v, H, T, W, scale, g, y); break;
    case 64: hipLaunchKernelGGL((window_kernel<TIn, 64, GATED>), grid, block, 0, s, q, k, v, H, T, W, scale, g, y); break;
    case 128: hipLaunchKernelGGL((window_kernel<TIn, 128, GATED>), grid, block, 0, s, q, k, v, H, T, W, scale, g, y); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_window(const void* q, const void* k, const void* v, bool bf16, int B, int H, int T, int d, int W,
                         float scale, const float* g, float* y, hipStream_t s) {
  if (B * H == 0 || T == 0) return hipSuccess;
  if (bf16) {
    const auto* Q = static_cast<const uint16_t*>(q);
    const auto* K = static_cast<const uint16_t*>(k);
    const auto* V = static_cast<const uint16_t*>(v);
    return g ? run_window<uint16_t, true>(Q, K, V, B, H, T, d, W, scale, g, y, s)
             : run_window<uint16_t, false>(Q, K, V, B, H, T, d, W, scale, g, y, s);
  }
  const auto* Q = static_cast<const float*>(q);
  const auto* K = static_cast<const float*>(k);
  const auto* V = static_cast<const float*>(v);
  return g ? run_window<float, true>(Q, K, V, B, H, T, d, W, scale, g, y, s)
           : run_window<float, false>(Q, K, V, B, H, T, d, W, scale, g, y, s);
}

}  // namespace tc

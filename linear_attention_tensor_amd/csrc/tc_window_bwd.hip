// tc_window_bwd.hip — backward of the exact sliding-window softmax (the L1
// cache of the Tensor Cache) in fp32 arithmetic, for fp32 or bf16 inputs.
//
// Tensor Cache, Methodology 1: query t attends to the keys j in
// [max(0, t-W+1), t] with weights p_tj = softmax_j(scale <q_t, k_j>), and
// y_t = sum_j p_tj v_j.  The pages give no backward; reverse mode gives, with
// the cotangent dy and D_t = <dy_t, y_t>,
//   dv_j = sum_t p_tj dy_t,
//   ds_tj = p_tj (<dy_t, v_j> - D_t),
//   dq_t = scale sum_j ds_tj k_j,   dk_j = scale sum_t ds_tj q_t.
// Three launches: (1) per query the log-sum-exp of its scores and D_t
// (recomputing y_t); (2) dq per query over its window; (3) dk, dv per key over
// the W queries that see it, with p_tj = exp(s_tj - lse_t).  (2) and (3) can
// add to what the output buffers hold (the fused layer's backward adds the
// L2 branch this way).
//
// Four consecutive lanes share a row (a query or a key): lane c of the quad
// holds the features 4 i + c, so a quad reads 4 consecutive floats of an LDS
// row and full dot products come from two xor-shuffles.  Partner rows pass
// through LDS in blocks of 64, row stride D + 4 floats, so the 16 quads of a
// wave on 16 different rows hit 16 different 4-bank groups.
#include "tc_common.hpp"
#include "tc_kernels.hpp"

#include <math.h>

namespace tc {

namespace {

constexpr int BR = 64;  // rows (queries or keys) per workgroup
constexpr int BP = 64;  // partner rows per LDS block

__device__ __forceinline__ float quad_sum(float x) {
  x += __shfl_xor(x, 1);
  x += __shfl_xor(x, 2);
  return x;
}

template <typename TIn, int D>
__device__ __forceinline__ void load_row_part(const TIn* p, long row, int c, bool live, float* r) {
#pragma unroll
  for (int i = 0; i < D / 4; ++i) r[i] = live ? InT<TIn>::ld(p, row * D + 4 * i + c) : 0.f;
}

// LDS block of up to BP rows of one or two tensors (fp32, padded stride)
template <int D>
struct RowBlock {
  float a[BP][D + 4];
  float b[BP][D + 4];
};

template <typename TIn, int D, bool TWO>
__device__ __forceinline__ void stage(RowBlock<D>& blk, const TIn* pa, const TIn* pb, long base, int r0, int r_hi) {
  for (int e = threadIdx.x; e < BP * D; e += 256) {
    const int rr = e / D, cc = e % D, row = r0 + rr;
    const bool in = row <= r_hi;
    blk.a[rr][cc] = in ? InT<TIn>::ld(pa, (base + row) * D + cc) : 0.f;
    if (TWO) blk.b[rr][cc] = in ? InT<TIn>::ld(pb, (base + row) * D + cc) : 0.f;
  }
}

// (1) per query: lse_t = max + log(sum exp), D_t = <dy_t, y_t>
template <typename TIn, int D>
__global__ __launch_bounds__(256) void wbwd_stats_kernel(const TIn* __restrict__ q, const TIn* __restrict__ k,
                                                        const TIn* __restrict__ v, const float* __restrict__ dy,
                                                        int T, int W, float scale, float* __restrict__ lse,
                                                        float* __restrict__ dd) {
  __shared__ RowBlock<D> blk;
  const int bh = blockIdx.y, t0 = blockIdx.x * BR;
  const int c = threadIdx.x & 3, tq = t0 + (threadIdx.x >> 2);
  const long base = (long)bh * T;
  const bool live = tq < T;
  float qr[D / 4], acc[D / 4];
  load_row_part<TIn, D>(q, base + tq, c, live, qr);
#pragma unroll
  for (int i = 0; i < D / 4; ++i) acc[i] = 0.f;
  float mx = -INFINITY, l = 0.f;
  const int j_lo = max(0, t0 - W + 1), j_hi = min(T - 1, t0 + BR - 1);
  for (int jb = j_lo; jb <= j_hi; jb += BP) {
    __syncthreads();
    stage<TIn, D, true>(blk, k, v, base, jb, j_hi);
    __syncthreads();
    const int lo = live ? max(tq - W + 1, jb) : 1, hi = live ? min(tq, jb + BP - 1) : 0;
    for (int j = lo; j <= hi; ++j) {
      float s = 0.f;
#pragma unroll
      for (int i = 0; i < D / 4; ++i) s = fmaf(qr[i], blk.a[j - jb][4 * i + c], s);
      s = quad_sum(s) * scale;
      if (s > mx) {
        const float a = expf(mx - s);
        l *= a;
#pragma unroll
        for (int i = 0; i < D / 4; ++i) acc[i] *= a;
        mx = s;
      }
      const float p = expf(s - mx);
      l += p;
#pragma unroll
      for (int i = 0; i < D / 4; ++i) acc[i] = fmaf(p, blk.b[j - jb][4 * i + c], acc[i]);
    }
  }
  float dpart = 0.f;
  if (live) {
    const float inv = 1.f / l;
#pragma unroll
    for (int i = 0; i < D / 4; ++i) dpart = fmaf(dy[(base + tq) * D + 4 * i + c], acc[i] * inv, dpart);
  }
  const float dsum = quad_sum(dpart);
  if (live && c == 0) {
    lse[base + tq] = mx + logf(l);
    dd[base + tq] = dsum;
  }
}

// (2) dq_t = scale sum_j p_tj (<dy_t, v_j> - D_t) k_j
template <typename TIn, int D>
__global__ __launch_bounds__(256) void wbwd_dq_kernel(const TIn* __restrict__ q, const TIn* __restrict__ k,
                                                     const TIn* __restrict__ v, const float* __restrict__ dy,
                                                     int T, int W, float scale, const float* __restrict__ lse,
                                                     const float* __restrict__ dd, bool accumulate,
                                                     float* __restrict__ dq) {
  __shared__ RowBlock<D> blk;
  const int bh = blockIdx.y, t0 = blockIdx.x * BR;
  const int c = threadIdx.x & 3, tq = t0 + (threadIdx.x >> 2);
  const long base = (long)bh * T;
  const bool live = tq < T;
  float qr[D / 4], gr[D / 4], acc[D / 4];
  load_row_part<TIn, D>(q, base + tq, c, live, qr);
  load_row_part<float, D>(dy, base + tq, c, live, gr);
#pragma unroll
  for (int i = 0; i < D / 4; ++i) acc[i] = 0.f;
  const float ls = live ? lse[base + tq] : 0.f, dt = live ? dd[base + tq] : 0.f;
  const int j_lo = max(0, t0 - W + 1), j_hi = min(T - 1, t0 + BR - 1);
  for (int jb = j_lo; jb <= j_hi; jb += BP) {
    __syncthreads();
    stage<TIn, D, true>(blk, k, v, base, jb, j_hi);
    __syncthreads();
    const int lo = live ? max(tq - W + 1, jb) : 1, hi = live ? min(tq, jb + BP - 1) : 0;
    for (int j = lo; j <= hi; ++j) {
      float s = 0.f, dp = 0.f;
#pragma unroll
      for (int i = 0; i < D / 4; ++i) {
        s = fmaf(qr[i], blk.a[j - jb][4 * i + c], s);
        dp = fmaf(gr[i], blk.b[j - jb][4 * i + c], dp);
      }
      s = quad_sum(s) * scale;
      dp = quad_sum(dp);
      const float ds = expf(s - ls) * (dp - dt) * scale;
#pragma unroll
      for (int i = 0; i < D / 4; ++i) acc[i] = fmaf(ds, blk.a[j - jb][4 * i + c], acc[i]);
    }
  }
  if (live) {
#pragma unroll
    for (int i = 0; i < D / 4; ++i) {
      float* o = dq + (base + tq) * D + 4 * i + c;
      *o = accumulate ? *o + acc[i] : acc[i];
    }
  }
}

// (3) dv_j = sum_t p_tj dy_t,  dk_j = scale sum_t p_tj (<dy_t, v_j> - D_t) q_t
// over the queries t in [j, min(T - 1, j + W - 1)]
template <typename TIn, int D>
__global__ __launch_bounds__(256) void wbwd_dkv_kernel(const TIn* __restrict__ q, const TIn* __restrict__ k,
                                                      const TIn* __restrict__ v, const float* __restrict__ dy,
                                                      int T, int W, float scale, const float* __restrict__ lse,
                                                      const float* __restrict__ dd, bool accumulate,
                                                      float* __restrict__ dk, float* __restrict__ dv) {
  __shared__ RowBlock<D> blk;
  __shared__ float sl[BP], sd[BP];
  const int bh = blockIdx.y, j0 = blockIdx.x * BR;
  const int c = threadIdx.x & 3, jk = j0 + (threadIdx.x >> 2);
  const long base = (long)bh * T;
  const bool live = jk < T;
  float kr[D / 4], vr[D / 4], ak[D / 4], av[D / 4];
  load_row_part<TIn, D>(k, base + jk, c, live, kr);
  load_row_part<TIn, D>(v, base + jk, c, live, vr);
#pragma unroll
  for (int i = 0; i < D / 4; ++i) ak[i] = av[i] = 0.f;
  const int t_lo = j0, t_hi = min(T - 1, j0 + BR - 1 + W - 1);
  for (int tb = t_lo; tb <= t_hi; tb += BP) {
    __syncthreads();
    stage<float, D, false>(blk, dy, nullptr, base, tb, t_hi);  // dy rows in a
    for (int e = threadIdx.x; e < BP * D; e += 256) {           // q rows in b
      const int rr = e / D, cc = e % D, row = tb + rr;
      blk.b[rr][cc] = row <= t_hi ? InT<TIn>::ld(q, (base + row) * D + cc) : 0.f;
    }
    if (threadIdx.x < BP) {
      const int row = tb + threadIdx.x;
      sl[threadIdx.x] = row <= t_hi ? lse[base + row] : 0.f;
      sd[threadIdx.x] = row <= t_hi ? dd[base + row] : 0.f;
    }
    __syncthreads();
    const int lo = live ? max(jk, tb) : 1, hi = live ? min(min(jk + W - 1, T - 1), tb + BP - 1) : 0;
    for (int t = lo; t <= hi; ++t) {
      const int r = t - tb;
      float s = 0.f, dp = 0.f;
#pragma unroll
      for (int i = 0; i < D / 4; ++i) {
        s = fmaf(kr[i], blk.b[r][4 * i + c], s);
        dp = fmaf(vr[i], blk.a[r][4 * i + c], dp);
      }
      s = quad_sum(s) * scale;
      dp = quad_sum(dp);
      const float p = expf(s - sl[r]);
      const float ds = p * (dp - sd[r]) * scale;
#pragma unroll
      for (int i = 0; i < D / 4; ++i) {
        av[i] = fmaf(p, blk.a[r][4 * i + c], av[i]);
        ak[i] = fmaf(ds, blk.b[r][4 * i + c], ak[i]);
      }
    }
  }
  if (live) {
#pragma unroll
    for (int i = 0; i < D / 4; ++i) {
      float* ok = dk + (base + jk) * D + 4 * i + c;
      float* ov = dv + (base + jk) * D + 4 * i + c;
      *ok = accumulate ? *ok + ak[i] : ak[i];
      *ov = accumulate ? *ov + av[i] : av[i];
    }
  }
}

template <typename TIn, int D>
hipError_t run_wbwd(const TIn* q, const TIn* k, const TIn* v, const float* dy, int BH, int T, int W, float scale,
                    float* lse, float* dd, bool accumulate, float* dq, float* dk, float* dv, hipStream_t s) {
  const dim3 grid((T + BR - 1) / BR, BH), block(256);
  hipLaunchKernelGGL((wbwd_stats_kernel<TIn, D>), grid, block, 0, s, q, k, v, dy, T, W, scale, lse, dd);
  hipLaunchKernelGGL((wbwd_dq_kernel<TIn, D>), grid, block, 0, s, q, k, v, dy, T, W, scale, lse, dd, accumulate, dq);
  profile_mark_before(s);
  hipLaunchKernelGGL((wbwd_dkv_kernel<TIn, D>), grid, block, 0, s, q, k, v, dy, T, W, scale, lse, dd, accumulate,
                     dk, dv);
  profile_mark_after(s);
  return hipGetLastError();
}

template <typename TIn>
hipError_t dispatch_wbwd(const TIn* q, const TIn* k, const TIn* v, const float* dy, int BH, int T, int d, int W,
                         float scale, float* ws, bool accumulate, float* dq, float* dk, float* dv, hipStream_t s) {
  float* lse = ws;
  float* dd = ws + (long)BH * T;
  switch (d) {
    case 16: return run_wbwd<TIn, 16>(q, k, v, dy, BH, T, W, scale, lse, dd, accumulate, dq, dk, dv, s);
    case 32: return run_wbwd<TIn, 32>(q, k, v, dy, BH, T, W, scale, lse, dd, accumulate, dq, dk, dv, s);
    case 64: return run_wbwd<TIn, 64>(q, k, v, dy, BH, T, W, scale, lse, dd, accumulate, dq, dk, dv, s);
    case 128: return run_wbwd<TIn, 128>(q, k, v, dy, BH, T, W, scale, lse, dd, accumulate, dq, dk, dv, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

size_t window_bwd_ws_bytes(int B, int H, int T, int d, bool bf16) {
  if (window_bwd_mfma(bf16, d)) return window_bwd_mfma_ws_bytes(B, H, T, d);
  return (size_t)2 * B * H * T * sizeof(float);
}

hipError_t launch_window_backward(const void* q, const void* k, const void* v, bool bf16, const float* dy, int B,
                                  int H, int T, int d, int W, float scale, void* ws, bool accumulate, float* dq,
                                  float* dk, float* dv, hipStream_t s) {
  if (B * H == 0 || T == 0) return hipSuccess;
  if (window_bwd_mfma(bf16, d))  // bf16 MFMA kernels (tc_window_bwd_mfma.hip)
    return launch_window_backward_mfma(q, k, v, dy, B, H, T, d, W, scale, ws, accumulate, dq, dk, dv, s);
  float* w = static_cast<float*>(ws);
  if (bf16)
    return dispatch_wbwd<uint16_t>(static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k),
                                   static_cast<const uint16_t*>(v), dy, B * H, T, d, W, scale, w, accumulate, dq,
                                   dk, dv, s);
  return dispatch_wbwd<float>(static_cast<const float*>(q), static_cast<const float*>(k),
                              static_cast<const float*>(v), dy, B * H, T, d, W, scale, w, accumulate, dq, dk, dv, s);
}

}  // namespace tc

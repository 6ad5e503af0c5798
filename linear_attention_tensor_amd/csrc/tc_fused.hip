// tc_fused.hip — fused Tensor Cache layer (gfx950, bf16 inputs, fp32 state).
//
// Tensor Cache, Methodology 1: the L1 cache answers with exact softmax
// attention over the W most recent tokens (the current one included), the L2
// matrix with m_t = q_t A_t, and a learned scalar gate fuses the two,
// y_t = y_local,t + sigmoid(g) m_t.
//
// The L2 read m comes from the chunked scan (tc_scan.hip) into the
// workspace; the L1 kernel below is a sliding-window flash-attention pass
// whose epilogue adds sigmoid(g) m.  Layout of the L1 pass:
//   * one workgroup = 4 waves = 64 queries; wave w owns queries t0+16w..+15;
//   * keys stream through LDS in blocks of 64 (K row-major, V transposed);
//   * each wave computes S^T = K Q^T (keys x its 16 queries) with
//     v_mfma_f32_16x16x32_bf16, so every lane holds one query's scores and
//     the probabilities feed O^T = V^T P^T without leaving registers;
//   * online softmax in the log2 domain with exp2, fp32 statistics.
#include "tc_common.hpp"
#include "tc_kernels.hpp"

#include <math.h>

namespace tc {

namespace {

constexpr int KB = 64;  // keys per block
constexpr float kNegBig = -1.0e30f;

__device__ __forceinline__ bf16x8 ld_bf16x8(const uint16_t* p) {
  return *reinterpret_cast<const bf16x8*>(p);
}

// Eight probabilities (two 4-element score fragments) as one bf16x8 MFMA
// operand.  The vector is assembled in 32-bit integer lanes and bit-cast as a
// whole: element-wise insertion into bf16 vectors is avoided.
__device__ __forceinline__ bf16x8 pack_bf16x8(floatx4 lo, floatx4 hi) {
  const u32x4 w{pack_bf16x2(lo[0], lo[1]), pack_bf16x2(lo[2], lo[3]), pack_bf16x2(hi[0], hi[1]),
                pack_bf16x2(hi[2], hi[3])};
  return __builtin_bit_cast(bf16x8, w);
}

template <int D>
__global__ __launch_bounds__(256) void swa_kernel(const uint16_t* __restrict__ q,
                                                  const uint16_t* __restrict__ k,
                                                  const uint16_t* __restrict__ v,
                                                  const float* __restrict__ g,
                                                  const float* __restrict__ mem, int H, int T,
                                                  int W, float scale_log2, float* __restrict__ y) {
  constexpr int SK = D + 8;    // bf16 per K row in LDS
  constexpr int SVT = KB + 8;  // bf16 per V^T row in LDS
  constexpr int NKS = D / 32;  // k-steps of the QK^T product
  constexpr int NDT = D / 16;  // 16-row tiles of O^T
  __shared__ __attribute__((aligned(16))) uint16_t sK[KB * SK];
  __shared__ __attribute__((aligned(16))) uint16_t sVt[D * SVT];

  const int bh = blockIdx.y;
  const int t0 = blockIdx.x * 64;
  const int w = wave_id(), l = lane_id();
  const int qc = l & 15, g4 = l >> 4;
  const int tq = t0 + 16 * w + qc;
  const long base = (long)bh * T;

  bf16x8 qreg[NKS];
#pragma unroll
  for (int ks = 0; ks < NKS; ++ks) {
    if (tq < T) {
      qreg[ks] = ld_bf16x8(q + (base + tq) * D + 32 * ks + 8 * g4);
    } else {
      qreg[ks] = __builtin_bit_cast(bf16x8, u32x4{0u, 0u, 0u, 0u});
    }
  }

  floatx4 o[NDT];
#pragma unroll
  for (int i = 0; i < NDT; ++i) o[i] = zero4();
  float mrun = kNegBig, lsum = 0.f;

  const int kfirst = max(0, t0 - W + 1) & ~(KB - 1);
  const int kend = min(T, t0 + 64);
  for (int kb = kfirst; kb < kend; kb += KB) {
    __syncthreads();
    // stage K rows kb..kb+63 (row-major) and V (transposed), zero past T
    for (int idx = threadIdx.x; idx < KB * (D / 8); idx += 256) {
      const int r = idx / (D / 8), c8 = (idx % (D / 8)) * 8;
      uint4 kx = make_uint4(0u, 0u, 0u, 0u), vx = make_uint4(0u, 0u, 0u, 0u);
      if (kb + r < T) {
        kx = *reinterpret_cast<const uint4*>(k + (base + kb + r) * D + c8);
        vx = *reinterpret_cast<const uint4*>(v + (base + kb + r) * D + c8);
      }
      *reinterpret_cast<uint4*>(sK + r * SK + c8) = kx;
      const uint32_t vw[4] = {vx.x, vx.y, vx.z, vx.w};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        sVt[(c8 + 2 * j) * SVT + r] = static_cast<uint16_t>(vw[j] & 0xFFFFu);
        sVt[(c8 + 2 * j + 1) * SVT + r] = static_cast<uint16_t>(vw[j] >> 16);
      }
    }
    __syncthreads();

    // S^T tile: keys kb + 16kt + 4g4 + i  x  query tq
    floatx4 s[4];
#pragma unroll
    for (int kt = 0; kt < 4; ++kt) {
      s[kt] = zero4();
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) {
        const bf16x8 a = ld_bf16x8(sK + (16 * kt + qc) * SK + 32 * ks + 8 * g4);
        s[kt] = mfma_bf16_16x16x32(a, qreg[ks], s[kt]);
      }
    }
    float bmax = kNegBig;
#pragma unroll
    for (int kt = 0; kt < 4; ++kt) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int j = kb + 16 * kt + 4 * g4 + i;
        const bool ok = (j <= tq) && (j > tq - W) && (j < T);
        const float x = ok ? s[kt][i] * scale_log2 : -INFINITY;
        s[kt][i] = x;
        bmax = fmaxf(bmax, x);
      }
    }
    bmax = fmaxf(bmax, __shfl_xor(bmax, 16));
    bmax = fmaxf(bmax, __shfl_xor(bmax, 32));
    const float mnew = fmaxf(mrun, bmax);
    const float alpha = exp2f(mrun - mnew);
    mrun = mnew;
    float psum = 0.f;
#pragma unroll
    for (int kt = 0; kt < 4; ++kt) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float p = exp2f(s[kt][i] - mnew);
        s[kt][i] = p;
        psum += p;
      }
    }
    lsum = lsum * alpha + psum;
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) o[dt] *= alpha;

    // O^T += V^T P^T over two 32-key k-steps
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const bf16x8 pb = pack_bf16x8(s[2 * u], s[2 * u + 1]);
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt) {
        const uint16_t* vr = sVt + (16 * dt + qc) * SVT + 32 * u + 4 * g4;
        const uint2 lo = *reinterpret_cast<const uint2*>(vr);
        const uint2 hi = *reinterpret_cast<const uint2*>(vr + 16);
        const bf16x8 a = __builtin_bit_cast(bf16x8, u32x4{lo.x, lo.y, hi.x, hi.y});
        o[dt] = mfma_bf16_16x16x32(a, pb, o[dt]);
      }
    }
  }

  lsum += __shfl_xor(lsum, 16);
  lsum += __shfl_xor(lsum, 32);
  if (tq < T) {
    const float inv = 1.f / lsum;
    const float gate = 1.f / (1.f + expf(-g[bh % H]));
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) {
      const long off = (base + tq) * D + 16 * dt + 4 * g4;
      const float4 mm = *reinterpret_cast<const float4*>(mem + off);
      float4 out;
      out.x = o[dt][0] * inv + gate * mm.x;
      out.y = o[dt][1] * inv + gate * mm.y;
      out.z = o[dt][2] * inv + gate * mm.z;
      out.w = o[dt][3] * inv + gate * mm.w;
      *reinterpret_cast<float4*>(y + off) = out;
    }
  }
}

}  // namespace

size_t fused_ws_bytes(int B, int H, int T, int dk, int dv, int W) {
  const ScanPlan p = plan_scan(B, H, T, dk, dv, W);
  return (size_t)B * H * T * dv * sizeof(float) + scan_ws_bytes(p, B, H, dk, dv);
}

hipError_t launch_tc_fused(const void* q, const void* k, const void* v, const float* lam,
                           const float* eta, const float* g, int B, int H, int T, int d, int W,
                           float scale, float* y, float* A_final, void* ws, hipStream_t s) {
  float* mem = static_cast<float*>(ws);
  float* scan_ws = mem + (size_t)B * H * T * d;
  hipError_t e = launch_tc_scan(q, k, v, true, lam, eta, B, H, T, d, d, W, mem, A_final, scan_ws, s);
  if (e != hipSuccess) return e;
  const float scale_log2 = scale * 1.4426950408889634f;
  const dim3 grid((T + 63) / 64, B * H);
  const uint16_t* Q = static_cast<const uint16_t*>(q);
  const uint16_t* K = static_cast<const uint16_t*>(k);
  const uint16_t* V = static_cast<const uint16_t*>(v);
  if (d == 128)
    hipLaunchKernelGGL(swa_kernel<128>, grid, dim3(256), 0, s, Q, K, V, g, mem, H, T, W, scale_log2, y);
  else if (d == 64)
    hipLaunchKernelGGL(swa_kernel<64>, grid, dim3(256), 0, s, Q, K, V, g, mem, H, T, W, scale_log2, y);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace tc

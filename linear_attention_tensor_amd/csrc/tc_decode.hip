// tc_decode.hip — one streaming step of the Tensor Cache (gfx950).
//
// Tensor Cache, Methodology 1: the L1 cache is a W-slot KV ring; when a new
// token overwrites an occupied slot, the displaced pair is written into the
// L2 matrix, A <- lam A + eta k_e v_e^T, and the query reads m = q A.
//
// The step is bound by HBM traffic on A (d_k x d_v fp32 read and written
// once per head and step), so one workgroup streams one head's A with
// 16-byte coalesced accesses: thread t owns a float4 column group and a set of
// rows, updates them in registers, writes them back and accumulates q_i a_i;
// the per-row-group partial sums are reduced through LDS.
#include "tc_common.hpp"
#include "tc_kernels.hpp"

namespace tc {

namespace {

template <typename TIn>
__global__ __launch_bounds__(256) void decode_kernel(
    const TIn* __restrict__ q, const TIn* __restrict__ k, const TIn* __restrict__ v,
    TIn* __restrict__ ring_k, TIn* __restrict__ ring_v, float* __restrict__ A,
    const float* __restrict__ lam, const float* __restrict__ eta, const int64_t* __restrict__ pos,
    int H, int dk, int dv, int W, float* __restrict__ m) {
  __shared__ float sq[128];
  __shared__ float ske[128];
  __shared__ float sve[128];
  __shared__ float4 part[256];

  const int bh = blockIdx.x;
  const int b = bh / H, h = bh % H;
  const long p = pos[b];
  const long slot = p % W;
  const bool evict = p >= W;
  const int t = threadIdx.x;

  TIn* rk = ring_k + ((long)bh * W + slot) * dk;
  TIn* rv = ring_v + ((long)bh * W + slot) * dv;
  if (t < dk) {
    sq[t] = InT<TIn>::ld(q + (long)bh * dk, t);
    ske[t] = evict ? InT<TIn>::ld(rk, t) : 0.f;
  }
  if (t < dv) sve[t] = evict ? InT<TIn>::ld(rv, t) : 0.f;
  __syncthreads();  // the evicted pair is in LDS before the slot is overwritten
  if (t < dk) rk[t] = k[(long)bh * dk + t];
  if (t < dv) rv[t] = v[(long)bh * dv + t];

  const float lm = lam[h], et = eta[h];
  const int ncg = dv / 4;       // float4 column groups per row
  const int rpp = 256 / ncg;    // rows handled in one pass of the block
  const int cg = t % ncg, r0 = t / ncg;
  float4* Ab = reinterpret_cast<float4*>(A + (long)bh * dk * dv);
  const float4 ve = make_float4(et * sve[4 * cg], et * sve[4 * cg + 1], et * sve[4 * cg + 2],
                                et * sve[4 * cg + 3]);
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  if (evict) {
    for (int r = r0; r < dk; r += rpp) {
      float4 a = Ab[r * ncg + cg];
      const float kr = ske[r];
      a.x = lm * a.x + kr * ve.x;
      a.y = lm * a.y + kr * ve.y;
      a.z = lm * a.z + kr * ve.z;
      a.w = lm * a.w + kr * ve.w;
      Ab[r * ncg + cg] = a;
      const float qr = sq[r];
      acc.x += qr * a.x;
      acc.y += qr * a.y;
      acc.z += qr * a.z;
      acc.w += qr * a.w;
    }
  } else {
    for (int r = r0; r < dk; r += rpp) {
      const float4 a = Ab[r * ncg + cg];
      const float qr = sq[r];
      acc.x += qr * a.x;
      acc.y += qr * a.y;
      acc.z += qr * a.z;
      acc.w += qr * a.w;
    }
  }
  part[t] = acc;
  __syncthreads();
  if (t < ncg) {
    float4 s = part[t];
    for (int j = 1; j < rpp && j * ncg + t < 256; ++j) {
      const float4 o = part[j * ncg + t];
      s.x += o.x;
      s.y += o.y;
      s.z += o.z;
      s.w += o.w;
    }
    reinterpret_cast<float4*>(m + (long)bh * dv)[t] = s;
  }
}

}  // namespace

hipError_t launch_tc_decode(const void* q, const void* k, const void* v, bool bf16, void* ring_k,
                            void* ring_v, float* A, const float* lam, const float* eta,
                            const int64_t* pos, int B, int H, int dk, int dv, int W, float* m,
                            hipStream_t s) {
  const dim3 grid(B * H), block(256);
  profile_mark_before(s);
  if (bf16) {
    hipLaunchKernelGGL(decode_kernel<uint16_t>, grid, block, 0, s,
                       static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k),
                       static_cast<const uint16_t*>(v), static_cast<uint16_t*>(ring_k),
                       static_cast<uint16_t*>(ring_v), A, lam, eta, pos, H, dk, dv, W, m);
  } else {
    hipLaunchKernelGGL(decode_kernel<float>, grid, block, 0, s, static_cast<const float*>(q),
                       static_cast<const float*>(k), static_cast<const float*>(v),
                       static_cast<float*>(ring_k), static_cast<float*>(ring_v), A, lam, eta, pos,
                       H, dk, dv, W, m);
  }
  profile_mark_after(s);
  return hipGetLastError();
}

}  // namespace tc

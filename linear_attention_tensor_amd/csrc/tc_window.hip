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
// Both products are dense fp32 contractions and run on the fp32 matrix cores
// (v_mfma_f32_32x32x2_f32: 32x32 output, two k per instruction, one float of
// each operand per lane):
//   S^T = K Q^T   (32 keys x 32 queries per wave and block; lane n + 32 hh
//                  holds query n and keys 8 (r / 4) + 4 hh + r % 4, r < 16)
//   O^T += V^T P^T (d_v x 32 queries; P^T is the score registers themselves)
// One workgroup (4 waves, 32 queries each) per 128 consecutive queries of one
// (b, h); the keys the tile needs, [t0 - W + 1, t0 + 127], pass through LDS
// in blocks of 32 rows (K and V, fp32, double-buffered, the next block in
// registers while the current one is used).  A wave skips the blocks none of
// its queries sees and masks only the blocks on the edges of its window.  The
// online softmax keeps a reference maximum per query in log2 units (scores
// are formed from q scale log2(e)); O and the normaliser are rescaled only
// when a block's maximum passes the reference by more than 8, so every
// probability stays <= 2^8 and O / l is unchanged.
#include "tc_common.hpp"
#include "tc_kernels.hpp"

#include <math.h>

namespace tc {

namespace {

constexpr int WQ = 128;  // queries per workgroup (4 waves x 32)
constexpr int WKB = 32;  // keys per LDS block
constexpr int NXCD = 8;  // MI355X: 8 accelerator complex dies, workgroups dispatched round-robin
constexpr float kNegBig = -1.0e30f;

__device__ __forceinline__ floatx16 mfma_f32(float a, float b, floatx16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
}

// four consecutive inputs as fp32
__device__ __forceinline__ float4 ld4(const float* p) { return *reinterpret_cast<const float4*>(p); }
__device__ __forceinline__ float4 ld4(const uint16_t* p) {
  const uint2 u = *reinterpret_cast<const uint2*>(p);
  return make_float4(__uint_as_float(u.x << 16), __uint_as_float(u.x & 0xFFFF0000u),
                     __uint_as_float(u.y << 16), __uint_as_float(u.y & 0xFFFF0000u));
}

template <typename TIn, int D, bool GATED>
__global__ __launch_bounds__(256, 2) void window_kernel(const TIn* __restrict__ q, const TIn* __restrict__ k,
                                                        const TIn* __restrict__ v, int H, int T, int W,
                                                        int n_tiles, int n_items, float sl2,
                                                        const float* __restrict__ g, float* __restrict__ y) {
  constexpr int S = D + 4;                   // LDS row stride (floats): 16-byte operand reads by rows hit distinct banks
  constexpr int HALF = D / 2;                // k of the QK^T product per lane half
  constexpr int NDT = (D + 31) / 32;         // 32-row tiles of O^T (d = 16: one, rows 16..31 unused)
  constexpr int NP = 8 * D;                  // float4 pieces of one K (or V) block
  constexpr int NLD = (NP + 255) / 256;      // ... per thread
  __shared__ __attribute__((aligned(16))) float sk[2][WKB * S];
  __shared__ __attribute__((aligned(16))) float sv[2][WKB * S];

  // XCD-aware order: the workgroups dispatched to one XCD take a contiguous
  // run of (head, tile) items, so the tiles that share key blocks share an L2.
  const int L = blockIdx.x;
  const int per_xcd = (n_items + NXCD - 1) / NXCD;
  const int item = (L % NXCD) * per_xcd + L / NXCD;
  if (item >= n_items) return;  // whole workgroup, before any barrier
  const int bh = item / n_tiles, t0 = (item % n_tiles) * WQ;
  const int tid = threadIdx.x, w = tid >> 6, c = tid & 31, hh = (tid >> 5) & 1;
  const long base = (long)bh * T;
  const int q0 = t0 + 32 * w;  // first query of this wave
  const int tq = q0 + c;       // this lane's query
  const int j_lo = max(0, t0 - W + 1), j_hi = min(T - 1, t0 + WQ - 1);
  const int nblk = (j_hi - j_lo + WKB) / WKB;

  // q scale log2(e): lane (hh, n) holds q[tq][HALF hh + j], j < HALF (the k
  // order of the QK^T product, shared with the K operand)
  float qr[HALF];
#pragma unroll
  for (int j4 = 0; j4 < HALF / 4; ++j4) {
    const float4 x = tq < T ? ld4(q + (base + tq) * D + HALF * hh + 4 * j4) : make_float4(0.f, 0.f, 0.f, 0.f);
    qr[4 * j4] = x.x * sl2;
    qr[4 * j4 + 1] = x.y * sl2;
    qr[4 * j4 + 2] = x.z * sl2;
    qr[4 * j4 + 3] = x.w * sl2;
  }
  floatx16 o[NDT];
#pragma unroll
  for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
    for (int r = 0; r < 16; ++r) o[dt][r] = 0.f;
  float m = kNegBig, lsum = 0.f;

  // K and V rows jb .. jb + 31 (zero past T) to registers, then to LDS stage st
  float4 rk[NLD], rv[NLD];
  auto load_block = [&](int jb) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < NLD; ++i) {
      const int f = tid + 256 * i, row = f / (D / 4), c4 = f % (D / 4);
      const bool in = (NP % 256 == 0 || f < NP) && jb + row < T;
      const long off = (base + jb + row) * D + 4 * c4;
      rk[i] = in ? ld4(k + off) : make_float4(0.f, 0.f, 0.f, 0.f);
      rv[i] = in ? ld4(v + off) : make_float4(0.f, 0.f, 0.f, 0.f);
    }
  };
  auto store_block = [&](int st) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < NLD; ++i) {
      const int f = tid + 256 * i, row = f / (D / 4), c4 = f % (D / 4);
      if (NP % 256 == 0 || f < NP) {
        *reinterpret_cast<float4*>(&sk[st][row * S + 4 * c4]) = rk[i];
        *reinterpret_cast<float4*>(&sv[st][row * S + 4 * c4]) = rv[i];
      }
    }
  };

  load_block(j_lo);
  store_block(0);
  __syncthreads();
#pragma unroll 1
  for (int i = 0; i < nblk; ++i) {
    const int jb = j_lo + WKB * i, cur = i & 1;
    if (i + 1 < nblk) load_block(jb + WKB);
    // some key of the block is in the window of some query of the wave (wave-uniform)
    const bool active = q0 < T && jb <= min(q0 + 31, T - 1) && jb + WKB - 1 >= q0 - W + 1;
    if (active) {
      floatx16 sa;
#pragma unroll
      for (int r = 0; r < 16; ++r) sa[r] = 0.f;
      const float* kr = &sk[cur][c * S + HALF * hh];
#pragma unroll
      for (int j4 = 0; j4 < HALF / 4; ++j4) {
        const float4 kk = *reinterpret_cast<const float4*>(kr + 4 * j4);
        sa = mfma_f32(kk.x, qr[4 * j4], sa);
        sa = mfma_f32(kk.y, qr[4 * j4 + 1], sa);
        sa = mfma_f32(kk.z, qr[4 * j4 + 2], sa);
        sa = mfma_f32(kk.w, qr[4 * j4 + 3], sa);
      }
      float s[16];
#pragma unroll
      for (int r = 0; r < 16; ++r) s[r] = sa[r];
      // every key of the block in the window of every query of the wave?
      const bool full = jb + WKB - 1 <= q0 && jb >= q0 + 32 - W;
      if (!full) {
        // keys jb + kk valid for query tq: tq - W < jb + kk <= tq
        const int lo = tq - W + 1 - jb, hi = tq - jb;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int kk = 8 * (r >> 2) + 4 * hh + (r & 3);
          s[r] = (kk >= lo && kk <= hi) ? s[r] : -INFINITY;
        }
      }
      // block maximum of the query (its keys sit in lanes n and n + 32)
      float bm = s[0];
#pragma unroll
      for (int r = 1; r < 16; ++r) bm = fmaxf(bm, s[r]);
      bm = fmaxf(bm, __shfl_xor(bm, 32));
      if (__ballot(bm - m > 8.f) != 0) {
        const float mnew = fmaxf(m, bm);
        const float alpha = __builtin_amdgcn_exp2f(m - mnew);
        lsum *= alpha;
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) o[dt] *= alpha;
        m = mnew;
      }
      float ps = 0.f;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        s[r] = __builtin_amdgcn_exp2f(s[r] - m);
        ps += s[r];
      }
      lsum += ps;
      // O^T += V^T P^T: k-step r takes keys 8 (r / 4) + 4 hh + r % 4, the keys
      // whose probabilities this lane holds in s[r]
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float* vr = &sv[cur][(8 * (r >> 2) + 4 * hh + (r & 3)) * S + c];
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) {
          const float vv = (D >= 32 || c < D) ? vr[32 * dt] : 0.f;
          o[dt] = mfma_f32(vv, s[r], o[dt]);
        }
      }
    }
    if (i + 1 < nblk) store_block(cur ^ 1);  // stage cur ^ 1 was last read in step i - 1
    __syncthreads();
  }

  const float ltot = lsum + __shfl_xor(lsum, 32);
  const float inv = ltot > 0.f ? 1.f / ltot : 0.f;
  if (tq < T) {
    const float gate = GATED ? 1.f / (1.f + expf(-g[bh % H])) : 0.f;
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const int dv = 32 * dt + 8 * g4 + 4 * hh;
        if (dv < D) {
          float4* yo = reinterpret_cast<float4*>(y + (base + tq) * D + dv);
          float4 out = make_float4(o[dt][4 * g4] * inv, o[dt][4 * g4 + 1] * inv, o[dt][4 * g4 + 2] * inv,
                                   o[dt][4 * g4 + 3] * inv);
          if (GATED) {
            const float4 mm = *yo;
            out = make_float4(fmaf(gate, mm.x, out.x), fmaf(gate, mm.y, out.y), fmaf(gate, mm.z, out.z),
                              fmaf(gate, mm.w, out.w));
          }
          *yo = out;
        }
      }
  }
}

template <typename TIn, bool GATED>
hipError_t run_window(const TIn* q, const TIn* k, const TIn* v, int B, int H, int T, int d, int W, float scale,
                      const float* g, float* y, hipStream_t s) {
  const int n_tiles = (T + WQ - 1) / WQ, n_items = B * H * n_tiles;
  const int grid = (n_items + NXCD - 1) / NXCD * NXCD;
  const float sl2 = scale * 1.4426950408889634f;
  const dim3 block(256);
  switch (d) {
    case 16: hipLaunchKernelGGL((window_kernel<TIn, 16, GATED>), dim3(grid), block, 0, s, q, k, v, H, T, W, n_tiles, n_items, sl2, g, y); break;
    case 32: hipLaunchKernelGGL((window_kernel<TIn, 32, GATED>), dim3(grid), block, 0, s, q, k, v, H, T, W, n_tiles, n_items, sl2, g, y); break;
    case 64: hipLaunchKernelGGL((window_kernel<TIn, 64, GATED>), dim3(grid), block, 0, s, q, k, v, H, T, W, n_tiles, n_items, sl2, g, y); break;
    case 128: hipLaunchKernelGGL((window_kernel<TIn, 128, GATED>), dim3(grid), block, 0, s, q, k, v, H, T, W, n_tiles, n_items, sl2, g, y); break;
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

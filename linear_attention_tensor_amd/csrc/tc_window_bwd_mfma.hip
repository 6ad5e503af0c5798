// tc_window_bwd_mfma.hip — backward of the exact sliding-window softmax (the
// L1 cache of the Tensor Cache) on bf16 MFMA, for bf16 inputs with d in
// {64, 128} (gfx950, v_mfma_f32_32x32x16_bf16).
//
// Tensor Cache, Methodology 1: query t attends to the keys j in
// [max(0, t-W+1), t] with p_tj = softmax_j(scale <q_t, k_j>), y_t = sum_j
// p_tj v_j.  The pages give no backward; reverse mode gives, with the
// cotangent dy and D_t = <dy_t, y_t>,
//   dv_j = sum_t p_tj dy_t,   ds_tj = p_tj (<dy_t, v_j> - D_t),
//   dq_t = scale sum_j ds_tj k_j,   dk_j = scale sum_t ds_tj q_t.
// Four launches:
//   (1) the window softmax forward (the fused layer's main kernel without
//       its L2 part) recomputes y_t and writes lse2_t = log2 sum_j
//       exp2(sl2 s_tj) (sl2 = scale log2 e), so that p_tj = exp2(sl2 s_tj -
//       lse2_t);
//   (2) per row dy_t rounded to bf16 (an MFMA operand) and D_t from it;
//   (3) dq per 256-query tile (eight waves of 32 queries) over 64-key blocks:
//       S^T = K Q^T and dP^T = V dY^T (K, V rows from LDS, q and dy of the
//       lane's query in registers), dS in registers, dQ^T += K^T dS^T;
//   (4) dk, dv per 128-key tile (four waves of 32 keys) over 64-query
//       blocks: S = Q K^T and dP = dY V^T (Q, dY rows from LDS, k and v of
//       the lane's key in registers), dV^T += dY^T P, dK^T += Q^T dS.
// The blocks go global -> LDS by buffer_load ... lds in the row layout of
// tc_tr.hpp (RR variant: conflict-free both for whole-piece row reads and
// for transpose reads); the row-read operands take block row perm16(m) in
// lane m, so that the eight probabilities a lane holds for one k-step belong
// to eight consecutive keys (or queries) and feed the next MFMA from
// registers.  P and dS are rounded to bf16 as MFMA operands; everything is
// accumulated in fp32.  (3) and (4) can add to what the output buffers hold.
#include "tc_common.hpp"
#include "tc_kernels.hpp"
#include "tc_dma.hpp"
#include "tc_mfma.hpp"
#include "tc_tr.hpp"

#include <math.h>

namespace tc {

namespace {

using namespace mf;
using dma::dma16;
using dma::i32x4;
using dma::raw_desc;

constexpr int NST = 3;        // LDS stages (blocks in flight)
constexpr int QW = 8;         // waves of the dq kernel: 256 queries per workgroup
constexpr int KW = 4;         // waves of the dk/dv kernel: 128 keys per workgroup

// wait until at most n blocks (C copies each) are still in flight
template <int C>
__device__ __forceinline__ void wait_blocks(int n) {
  switch (n) {
    case 0: wait_vmcnt<0>(); break;
    case 1: wait_vmcnt<C>(); break;
    default: wait_vmcnt<2 * C>(); break;
  }
}

// lanes' row-read offsets of a 32-row half kt: row 32 kt + perm16(col), and its swizzle
template <int D>
struct RowLane {
  uint32_t base[2];
  int sw[2];
  __device__ __forceinline__ RowLane() {
    const int col = lane_id() & 31;
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) {
      const int r = 32 * kt + perm16(col);
      base[kt] = (uint32_t)(r * 2 * D);
      sw[kt] = tr::swz<D, true>(r);
    }
  }
  // operand of k-step ks (features 16 ks + 8 hh ..) of half kt
  __device__ __forceinline__ bf16x8 ld(const char* blk, int kt, int ks, int hh) const {
    return lds16(blk, base[kt] + 16u * (uint32_t)((2 * ks + hh) ^ sw[kt]));
  }
};

// (2) D_t = <dy_t, y_t> into ld[2 t + 1]; dy_t as bf16.  16 lanes per row.
__global__ __launch_bounds__(256) void wbm_prep_kernel(const float* __restrict__ dy, const float* __restrict__ y,
                                                       int d, long rows, uint16_t* __restrict__ dyb,
                                                       float* __restrict__ ld) {
  const long row = ((long)blockIdx.x * blockDim.x + threadIdx.x) >> 4;
  const int sub = threadIdx.x & 15, per = d >> 4;  // 4 or 8 features per lane
  float acc = 0.f;
  if (row < rows) {
    const long o = row * d + (long)sub * per;
    for (int i = 0; i < per; i += 4) {
      const float4 a = *reinterpret_cast<const float4*>(dy + o + i);
      const float4 b = *reinterpret_cast<const float4*>(y + o + i);
      // D from the rounded dy that dP = dY V^T uses, so that dP - D cancels
      // exactly where it should (a window of one key: ds = 0)
      const uint32_t r0 = cvt_pk(a.x, a.y), r1 = cvt_pk(a.z, a.w);
      acc = fmaf(lo_f(r0), b.x, fmaf(hi_f(r0), b.y, fmaf(lo_f(r1), b.z, fmaf(hi_f(r1), b.w, acc))));
      *reinterpret_cast<uint2*>(dyb + o + i) = make_uint2(r0, r1);
    }
  }
#pragma unroll
  for (int m = 8; m >= 1; m >>= 1) acc += __shfl_xor(acc, m);
  if (row < rows && sub == 0) ld[2 * row + 1] = acc;
}

// An empty asm that reads x: the compiler must have x loaded here.  The
// kernels use it on their register loads before the first global -> LDS
// copy, so that no wait of the compiler's for them falls inside the block
// loop (where it would also wait for every copy in flight); the asm is
// volatile, like the copies, so the two keep their order.
template <typename X>
__device__ __forceinline__ void landed(const X& x) {
  asm volatile("" ::"v"(x));
}

// dS (or P) of one S-like tile pair as the bf16 operands of k-steps 0..3:
// element e of half kt belongs to row 16 (2 kt + e / 8) + 8 hh + e % 8.
__device__ __forceinline__ bf16x8 pack8(const float* x) {
  return as_bf16x8(cvt_pk(x[0], x[1]), cvt_pk(x[2], x[3]), cvt_pk(x[4], x[5]), cvt_pk(x[6], x[7]));
}

// (3) dq.  Keys of the tile: [t0 - W + 1, t0 + 255] clipped to [0, T).
template <int D>
__global__ __launch_bounds__(QW * 64) void wbm_dq_kernel(const uint16_t* __restrict__ q,
                                                         const uint16_t* __restrict__ k,
                                                         const uint16_t* __restrict__ v,
                                                         const uint16_t* __restrict__ dyb,
                                                         const float* __restrict__ ld, int T, int W, float sl2,
                                                         float scale, bool accumulate, float* __restrict__ dq) {
  constexpr int NKS = D / 16, NDT = D / 32;
  constexpr int NC = KB * D / 8 / (QW * 64);  // 16-byte copies per thread, block and tensor
  __shared__ __attribute__((aligned(16))) uint16_t sk[NST][KB * D];
  __shared__ __attribute__((aligned(16))) uint16_t sv[NST][KB * D];
  const int bh = blockIdx.y, t0 = blockIdx.x * (QW * 32);
  const int w = wave_id(), l = lane_id(), col = l & 31, hh = l >> 5;
  const long base = (long)bh * T;
  const int tw = t0 + 32 * w, tq = tw + col;
  const bool live = tq < T;

  const __amdgpu_buffer_rsrc_t rq = make_rsrc(q + base * D, (uint32_t)T * D * 2);
  const __amdgpu_buffer_rsrc_t rdy = make_rsrc(dyb + base * D, (uint32_t)T * D * 2);
  bf16x8 qreg[NKS], dyreg[NKS];
#pragma unroll
  for (int ks = 0; ks < NKS; ++ks) {
    qreg[ks] = as_bf16x8(buf_load16(rq, (tq * D + 16 * ks + 8 * hh) * 2));
    dyreg[ks] = as_bf16x8(buf_load16(rdy, (tq * D + 16 * ks + 8 * hh) * 2));
  }
  const float lse2 = live ? ld[2 * (base + tq)] : 0.f;
  const float dd = live ? ld[2 * (base + tq) + 1] : 0.f;
#pragma unroll
  for (int ks = 0; ks < NKS; ++ks) {
    landed(qreg[ks]);
    landed(dyreg[ks]);
  }
  landed(lse2);
  landed(dd);
  floatx16 acc[NDT];
#pragma unroll
  for (int dt = 0; dt < NDT; ++dt) acc[dt] = zero16();

  const int j_lo = max(0, t0 - W + 1), j_hi = min(T - 1, t0 + QW * 32 - 1);
  const int nb = (j_hi - j_lo + KB) / KB;
  const i32x4 rk = raw_desc(k + base * D, (uint32_t)T * D * 2);
  const i32x4 rv = raw_desc(v + base * D, (uint32_t)T * D * 2);
  int src[NC];
#pragma unroll
  for (int i = 0; i < NC; ++i) src[i] = tr::slot_src<D, true>((i * QW + w) * 64 + l);
  auto copy = [&](int b) __attribute__((always_inline)) {
    const int off = (j_lo + KB * b) * D * 2;
#pragma unroll
    for (int i = 0; i < NC; ++i) dma16(rk, sk[b % NST] + (i * QW + w) * 512, src[i] + off);
#pragma unroll
    for (int i = 0; i < NC; ++i) dma16(rv, sv[b % NST] + (i * QW + w) * 512, src[i] + off);
  };
  const RowLane<D> rl;
  uint32_t kl0[NDT], kl1[NDT];
#pragma unroll
  for (int dt = 0; dt < NDT; ++dt) {
    kl0[dt] = tr::lane_offset<D, true>(dt);
    kl1[dt] = tr::lane_offset<D, true>(dt, 4);
  }

#pragma unroll 1
  for (int b = 0; b < nb && b < NST; ++b) copy(b);
#pragma unroll 1
  for (int b = 0; b < nb; ++b) {
    // block b has landed (the blocks issued after it may still be in flight) and is visible to every wave
    wait_blocks<2 * NC>(min(nb - 1, b + NST - 1) - b);
    lds_barrier();
    const char* K = reinterpret_cast<const char*>(sk[b % NST]);
    const char* V = reinterpret_cast<const char*>(sv[b % NST]);
    const int jb = j_lo + KB * b;
    // some key of the block is in the window of some query of the wave (wave-uniform)
    if (tw < T && jb + KB - 1 >= tw - W + 1 && jb <= tw + 31) {
      floatx16 s[2], dp[2];
#pragma unroll
      for (int kt = 0; kt < 2; ++kt) {
        s[kt] = zero16();
        dp[kt] = zero16();
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) {
          s[kt] = mfma32(rl.ld(K, kt, ks, hh), qreg[ks], s[kt]);
          dp[kt] = mfma32(rl.ld(V, kt, ks, hh), dyreg[ks], dp[kt]);
        }
      }
      bf16x8 dsb[4];
#pragma unroll
      for (int kt = 0; kt < 2; ++kt) {
#pragma unroll
        for (int h8 = 0; h8 < 2; ++h8) {
          float x[8];
#pragma unroll
          for (int i = 0; i < 8; ++i) {
            const int e = 8 * h8 + i, j = jb + key_of(kt, e, hh);
            const bool in = live && j >= tq - W + 1 && j <= tq && j < T;
            const float p = in ? __builtin_amdgcn_exp2f(fmaf(s[kt][e], sl2, -lse2)) : 0.f;
            x[i] = p * (dp[kt][e] - dd);
          }
          dsb[2 * kt + h8] = pack8(x);
        }
      }
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt) {
        acc[dt] = mfma32(tr::ld1<D, 0>(K, kl0[dt], kl1[dt]), dsb[0], acc[dt]);
        acc[dt] = mfma32(tr::ld1<D, 1>(K, kl0[dt], kl1[dt]), dsb[1], acc[dt]);
        acc[dt] = mfma32(tr::ld1<D, 2>(K, kl0[dt], kl1[dt]), dsb[2], acc[dt]);
        acc[dt] = mfma32(tr::ld1<D, 3>(K, kl0[dt], kl1[dt]), dsb[3], acc[dt]);
      }
    }
    if (b + NST < nb) {
      lds_barrier();  // every wave is done with this stage before it is refilled
      copy(b + NST);
    }
  }

  if (live) {
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) {
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        float4* o = reinterpret_cast<float4*>(dq + (base + tq) * D + 32 * dt + 8 * g4 + 4 * hh);
        float4 r = make_float4(scale * acc[dt][4 * g4], scale * acc[dt][4 * g4 + 1], scale * acc[dt][4 * g4 + 2],
                               scale * acc[dt][4 * g4 + 3]);
        if (accumulate) {
          const float4 a = *o;
          r.x += a.x;
          r.y += a.y;
          r.z += a.z;
          r.w += a.w;
        }
        *o = r;
      }
    }
  }
}

// (4) dk, dv.  Queries that see the tile's keys: [k0, k0 + 127 + W - 1]
// clipped to [0, T).  Each wave keeps its own copy of the block's (lse2, D)
// pairs, so that nothing but the Q and dY rows is shared between waves.
template <int D>
__global__ __launch_bounds__(KW * 64) __attribute__((amdgpu_waves_per_eu(1, 1))) void wbm_dkv_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
    const uint16_t* __restrict__ dyb, const float* __restrict__ ld, int T, int W, float sl2, float scale,
    bool accumulate, float* __restrict__ dk, float* __restrict__ dv) {
  constexpr int NKS = D / 16, NDT = D / 32;
  constexpr int NC = KB * D / 8 / (KW * 64);  // 16-byte copies per thread, block and tensor
  __shared__ __attribute__((aligned(16))) uint16_t sq[NST][KB * D];
  __shared__ __attribute__((aligned(16))) uint16_t sdy[NST][KB * D];
  __shared__ __attribute__((aligned(16))) float sld[NST][KW][256];  // 64 (lse2, D) pairs, padded to one copy
  const int bh = blockIdx.y, k0 = blockIdx.x * (KW * 32);
  const int w = wave_id(), l = lane_id(), col = l & 31, hh = l >> 5;
  const long base = (long)bh * T;
  const int jw = k0 + 32 * w, jk = jw + col;
  const bool live = jk < T;

  const __amdgpu_buffer_rsrc_t rk = make_rsrc(k + base * D, (uint32_t)T * D * 2);
  const __amdgpu_buffer_rsrc_t rv = make_rsrc(v + base * D, (uint32_t)T * D * 2);
  bf16x8 kreg[NKS], vreg[NKS];
#pragma unroll
  for (int ks = 0; ks < NKS; ++ks) {
    kreg[ks] = as_bf16x8(buf_load16(rk, (jk * D + 16 * ks + 8 * hh) * 2));
    vreg[ks] = as_bf16x8(buf_load16(rv, (jk * D + 16 * ks + 8 * hh) * 2));
  }
#pragma unroll
  for (int ks = 0; ks < NKS; ++ks) {
    landed(kreg[ks]);
    landed(vreg[ks]);
  }
  floatx16 ak[NDT], av[NDT];
#pragma unroll
  for (int dt = 0; dt < NDT; ++dt) ak[dt] = av[dt] = zero16();

  const int t_lo = k0, t_hi = min(T - 1, k0 + KW * 32 - 1 + W - 1);
  const int nb = (t_hi - t_lo + KB) / KB;
  const i32x4 rq = raw_desc(q + base * D, (uint32_t)T * D * 2);
  const i32x4 rdy = raw_desc(dyb + base * D, (uint32_t)T * D * 2);
  const i32x4 rld = raw_desc(ld + 2 * base, (uint32_t)T * 2 * 4);
  int src[NC];
#pragma unroll
  for (int i = 0; i < NC; ++i) src[i] = tr::slot_src<D, true>((i * KW + w) * 64 + l);
  auto copy = [&](int b) __attribute__((always_inline)) {
    const int off = (t_lo + KB * b) * D * 2;
#pragma unroll
    for (int i = 0; i < NC; ++i) dma16(rq, sq[b % NST] + (i * KW + w) * 512, src[i] + off);
#pragma unroll
    for (int i = 0; i < NC; ++i) dma16(rdy, sdy[b % NST] + (i * KW + w) * 512, src[i] + off);
    // the block's 64 (lse2, D) pairs (512 bytes) into this wave's copy; the
    // upper 32 lanes fill the padding
    dma16(rld, sld[b % NST][w], (t_lo + KB * b) * 8 + 16 * l);
  };
  const RowLane<D> rl;
  uint32_t tl0[NDT], tl1[NDT];
#pragma unroll
  for (int dt = 0; dt < NDT; ++dt) {
    tl0[dt] = tr::lane_offset<D, true>(dt);
    tl1[dt] = tr::lane_offset<D, true>(dt, 4);
  }

#pragma unroll 1
  for (int b = 0; b < nb && b < NST; ++b) copy(b);
#pragma unroll 1
  for (int b = 0; b < nb; ++b) {
    wait_blocks<2 * NC + 1>(min(nb - 1, b + NST - 1) - b);
    lds_barrier();
    const char* Qb = reinterpret_cast<const char*>(sq[b % NST]);
    const char* DYb = reinterpret_cast<const char*>(sdy[b % NST]);
    const float* LD = sld[b % NST][w];
    const int tb = t_lo + KB * b;
    // some query of the block sees some key of the wave (wave-uniform)
    if (jw < T && tb + KB - 1 >= jw && tb <= jw + 31 + W - 1) {
      floatx16 s[2], dp[2];
#pragma unroll
      for (int qt = 0; qt < 2; ++qt) {
        s[qt] = zero16();
        dp[qt] = zero16();
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) {
          s[qt] = mfma32(rl.ld(Qb, qt, ks, hh), kreg[ks], s[qt]);
          dp[qt] = mfma32(rl.ld(DYb, qt, ks, hh), vreg[ks], dp[qt]);
        }
      }
      bf16x8 pb[4], dsb[4];
#pragma unroll
      for (int qt = 0; qt < 2; ++qt) {
#pragma unroll
        for (int h8 = 0; h8 < 2; ++h8) {
          // the eight queries of this k-step: rows r0 .. r0 + 7 of the block
          const int r0 = 16 * (2 * qt + h8) + 8 * hh;
          const float4* lp = reinterpret_cast<const float4*>(LD + 2 * r0);
          float pl[8], dl[8];
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const float4 u = lp[i];
            pl[2 * i] = u.x;
            dl[2 * i] = u.y;
            pl[2 * i + 1] = u.z;
            dl[2 * i + 1] = u.w;
          }
          float xp[8], xs[8];
#pragma unroll
          for (int i = 0; i < 8; ++i) {
            const int e = 8 * h8 + i, t = tb + r0 + i;
            const bool in = live && t >= jk && t <= jk + W - 1 && t < T;
            const float p = in ? __builtin_amdgcn_exp2f(fmaf(s[qt][e], sl2, -pl[i])) : 0.f;
            xp[i] = p;
            xs[i] = p * (dp[qt][e] - dl[i]);
          }
          pb[2 * qt + h8] = pack8(xp);
          dsb[2 * qt + h8] = pack8(xs);
        }
      }
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt) {
        av[dt] = mfma32(tr::ld1<D, 0>(DYb, tl0[dt], tl1[dt]), pb[0], av[dt]);
        ak[dt] = mfma32(tr::ld1<D, 0>(Qb, tl0[dt], tl1[dt]), dsb[0], ak[dt]);
        av[dt] = mfma32(tr::ld1<D, 1>(DYb, tl0[dt], tl1[dt]), pb[1], av[dt]);
        ak[dt] = mfma32(tr::ld1<D, 1>(Qb, tl0[dt], tl1[dt]), dsb[1], ak[dt]);
        av[dt] = mfma32(tr::ld1<D, 2>(DYb, tl0[dt], tl1[dt]), pb[2], av[dt]);
        ak[dt] = mfma32(tr::ld1<D, 2>(Qb, tl0[dt], tl1[dt]), dsb[2], ak[dt]);
        av[dt] = mfma32(tr::ld1<D, 3>(DYb, tl0[dt], tl1[dt]), pb[3], av[dt]);
        ak[dt] = mfma32(tr::ld1<D, 3>(Qb, tl0[dt], tl1[dt]), dsb[3], ak[dt]);
      }
    }
    if (b + NST < nb) {
      lds_barrier();
      copy(b + NST);
    }
  }

  if (live) {
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) {
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const long o = (base + jk) * D + 32 * dt + 8 * g4 + 4 * hh;
        float4 rkv = make_float4(scale * ak[dt][4 * g4], scale * ak[dt][4 * g4 + 1], scale * ak[dt][4 * g4 + 2],
                                 scale * ak[dt][4 * g4 + 3]);
        float4 rvv = make_float4(av[dt][4 * g4], av[dt][4 * g4 + 1], av[dt][4 * g4 + 2], av[dt][4 * g4 + 3]);
        float4* pk = reinterpret_cast<float4*>(dk + o);
        float4* pv = reinterpret_cast<float4*>(dv + o);
        if (accumulate) {
          const float4 a = *pk, c = *pv;
          rkv.x += a.x;
          rkv.y += a.y;
          rkv.z += a.z;
          rkv.w += a.w;
          rvv.x += c.x;
          rvv.y += c.y;
          rvv.z += c.z;
          rvv.w += c.w;
        }
        *pk = rkv;
        *pv = rvv;
      }
    }
  }
}

size_t r256(size_t n) { return (n + 255) & ~(size_t)255; }

template <int D>
hipError_t run_wbm(const uint16_t* q, const uint16_t* k, const uint16_t* v, const float* dy, int B, int H, int T,
                   int W, float scale, char* ws, bool accumulate, float* dq, float* dk, float* dv, hipStream_t s) {
  const long rows = (long)B * H * T;
  float* y = reinterpret_cast<float*>(ws);
  uint16_t* dyb = reinterpret_cast<uint16_t*>(ws + r256(rows * D * 4));
  float* ld = reinterpret_cast<float*>(ws + r256(rows * D * 4) + r256(rows * D * 2));
  const float sl2 = scale * 1.4426950408889634f;
  hipError_t e = launch_swa(q, k, v, nullptr, nullptr, nullptr, nullptr, B, H, T, D, W, scale, y, ld, s);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(wbm_prep_kernel, dim3((unsigned)((rows * 16 + 255) / 256)), dim3(256), 0, s, dy, y, D, rows,
                     dyb, ld);
  hipLaunchKernelGGL(wbm_dq_kernel<D>, dim3((T + QW * 32 - 1) / (QW * 32), B * H), dim3(QW * 64), 0, s, q, k, v,
                     dyb, ld, T, W, sl2, scale, accumulate, dq);
  profile_mark_before(s);
  hipLaunchKernelGGL(wbm_dkv_kernel<D>, dim3((T + KW * 32 - 1) / (KW * 32), B * H), dim3(KW * 64), 0, s, q, k, v,
                     dyb, ld, T, W, sl2, scale, accumulate, dk, dv);
  profile_mark_after(s);
  return hipGetLastError();
}

}  // namespace

bool window_bwd_mfma(bool bf16, int d) { return bf16 && (d == 64 || d == 128); }

size_t window_bwd_mfma_ws_bytes(int B, int H, int T, int d) {
  const size_t rows = (size_t)B * H * T;
  return r256(rows * d * 4) + r256(rows * d * 2) + r256(rows * 2 * 4);
}

hipError_t launch_window_backward_mfma(const void* q, const void* k, const void* v, const float* dy, int B, int H,
                                       int T, int d, int W, float scale, void* ws, bool accumulate, float* dq,
                                       float* dk, float* dv, hipStream_t s) {
  if (B * H == 0 || T == 0) return hipSuccess;
  const auto* Q = static_cast<const uint16_t*>(q);
  const auto* K = static_cast<const uint16_t*>(k);
  const auto* V = static_cast<const uint16_t*>(v);
  char* w = static_cast<char*>(ws);
  if (d == 128) return run_wbm<128>(Q, K, V, dy, B, H, T, W, scale, w, accumulate, dq, dk, dv, s);
  if (d == 64) return run_wbm<64>(Q, K, V, dy, B, H, T, W, scale, w, accumulate, dq, dk, dv, s);
  return hipErrorInvalidValue;
}

}  // namespace tc

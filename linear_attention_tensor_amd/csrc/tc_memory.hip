// tc_memory.hip — outer-product fact memories and their recall (gfx950, fp32).
//
// "Hebbian-memory MLP stores facts in a Transformer without training",
// simple MLP construction: with Gaussian A, G in R^{m x d} the gated feature
// map is phi(x) = (A x) * (G x), the output matrix B = (1/F) sum_i
// v_f(i) phi(k_i)^T and the MLP B phi(x); a fact is stored when the output
// for k_i has its largest inner product with v_f(i).
// "Tensor Cache", Methodology 1: the read of the L2 matrix, m = q A.
//
// Kernels (fp32 MFMA v_mfma_f32_16x16x4_f32, every operand k-contiguous in
// LDS so that one 16-byte read feeds four MFMAs):
//   hebbian_write_kernel: per (64-feature tile, segment of facts), phi of a
//     64-fact chunk (two 64x64xd products and their elementwise product) is
//     formed in registers, written transposed to LDS and accumulated into the
//     tile of B^T; the segments' partial tiles are summed by a second kernel.
//     phi(K) [F x m] is never stored.
//   hebbian_read_kernel: per 64 queries, phi of a 64-feature chunk and its
//     product with that chunk of B, accumulated over the m features.
//   memory_read_kernel: per 64 queries of one (b, h), q A.
//   recall_argmax_kernel: per 64 queries of one group, scores against 64
//     candidates at a time and a running (max, index) per query.
#include "tc_common.hpp"
#include "tc_kernels.hpp"

#include <algorithm>

namespace tc {

namespace {

constexpr int CH = 64;

template <int D>
struct MT {
  static constexpr int S = D + 4;    // row stride of [64][D] arrays
  static constexpr int ST = CH + 4;  // row stride of [D][64] and [64][64] arrays
  static constexpr int NV = CH * D / 4 / 256;  // float4 pieces per thread of a [64][D] block
  static constexpr int NT = D / 16;
};

// 64 rows x D of a row-major array in registers (pieces i * 256 + thread);
// row r at src + r ld, rows >= nvalid are zero.
template <int D>
struct Rows {
  float4 x[MT<D>::NV];
  __device__ __forceinline__ void load(const float* src, long ld, int nvalid) {
#pragma unroll
    for (int i = 0; i < MT<D>::NV; ++i) {
      const int e4 = i * 256 + threadIdx.x, r = e4 / (D / 4), c = 4 * (e4 % (D / 4));
      x[i] = r < nvalid ? *reinterpret_cast<const float4*>(src + (long)r * ld + c)
                        : make_float4(0.f, 0.f, 0.f, 0.f);
    }
  }
  // rows base[idx[r]] (a gather through an index array); an index outside
  // [0, n_rows) reads as a zero row
  __device__ __forceinline__ void gather(const float* base, const int* idx, int n_rows, int nvalid) {
#pragma unroll
    for (int i = 0; i < MT<D>::NV; ++i) {
      const int e4 = i * 256 + threadIdx.x, r = e4 / (D / 4), c = 4 * (e4 % (D / 4));
      const int j = r < nvalid ? idx[r] : -1;
      x[i] = j >= 0 && j < n_rows ? *reinterpret_cast<const float4*>(base + (long)j * D + c)
                                  : make_float4(0.f, 0.f, 0.f, 0.f);
    }
  }
  __device__ __forceinline__ void put_rows(float* dst) const {
#pragma unroll
    for (int i = 0; i < MT<D>::NV; ++i) {
      const int e4 = i * 256 + threadIdx.x, r = e4 / (D / 4), c = 4 * (e4 % (D / 4));
      *reinterpret_cast<float4*>(dst + r * MT<D>::S + c) = x[i];
    }
  }
  __device__ __forceinline__ void put_cols(float* dst) const {  // dst[col][row], stride ST
#pragma unroll
    for (int i = 0; i < MT<D>::NV; ++i) {
      const int e4 = i * 256 + threadIdx.x, r = e4 / (D / 4), c = 4 * (e4 % (D / 4));
      dst[(c + 0) * MT<D>::ST + r] = x[i].x;
      dst[(c + 1) * MT<D>::ST + r] = x[i].y;
      dst[(c + 2) * MT<D>::ST + r] = x[i].z;
      dst[(c + 3) * MT<D>::ST + r] = x[i].w;
    }
  }
};

// phi of this wave's 16 rows (of sX) against the 64 feature rows of sA, sG:
// element (row 16w + 4g + e, feature 16ct + r) in p[ct][e].
template <int D>
__device__ __forceinline__ void phi_tile(const float* sX, const float* sA, const float* sG, floatx4* p) {
  constexpr int S = MT<D>::S;
  const int w = wave_id();
  floatx4 pa[4] = {zero4(), zero4(), zero4(), zero4()};
  floatx4 pg[4] = {zero4(), zero4(), zero4(), zero4()};
  mma_rows<D, 4>(sX + 16 * w * S, S, sA, 16 * S, S, pa);
  mma_rows<D, 4>(sX + 16 * w * S, S, sG, 16 * S, S, pg);
#pragma unroll
  for (int ct = 0; ct < 4; ++ct) p[ct] = pa[ct] * pg[ct];
}

// B^T partial tile [64 features][D] of one segment of facts.
template <int D>
__global__ __launch_bounds__(256) void hebbian_write_kernel(const float* __restrict__ K, const float* __restrict__ V,
                                                            const int* __restrict__ f, int F, int n_values,
                                                            const float* __restrict__ A,
                                                            const float* __restrict__ G, int m, int seg_len,
                                                            float* __restrict__ part) {
  using M = MT<D>;
  __shared__ __attribute__((aligned(16))) float sA[CH * M::S];
  __shared__ __attribute__((aligned(16))) float sG[CH * M::S];
  __shared__ __attribute__((aligned(16))) float sK[CH * M::S];
  __shared__ __attribute__((aligned(16))) float sPt[CH * M::ST];  // phi^T [feature][fact]
  __shared__ __attribute__((aligned(16))) float sVt[D * M::ST];   // V_f^T [dv][fact]
  const int c0 = blockIdx.x * CH, seg = blockIdx.y;
  const int w = wave_id(), l = lane_id(), r = l & 15, g = l >> 4;
  const int i_begin = seg * seg_len, i_end = min(F, i_begin + seg_len);
  {
    Rows<D> ra, rg;
    ra.load(A + (long)c0 * D, D, CH);
    rg.load(G + (long)c0 * D, D, CH);
    ra.put_rows(sA);
    rg.put_rows(sG);
  }
  floatx4 acc[M::NT];
#pragma unroll
  for (int t = 0; t < M::NT; ++t) acc[t] = zero4();
  Rows<D> xk, xv;
  if (i_begin < i_end) {
    xk.load(K + (long)i_begin * D, D, min(CH, i_end - i_begin));
    xv.gather(V, f + i_begin, n_values, min(CH, i_end - i_begin));
  }
  for (int i0 = i_begin; i0 < i_end; i0 += CH) {
    lds_barrier();  // every wave is done with the previous chunk
    xk.put_rows(sK);
    xv.put_cols(sVt);
    lds_barrier();
    if (i0 + CH < i_end) {
      const int n = min(CH, i_end - i0 - CH);
      xk.load(K + (long)(i0 + CH) * D, D, n);
      xv.gather(V, f + i0 + CH, n_values, n);
    }
    floatx4 p[4];
    phi_tile<D>(sK, sA, sG, p);
#pragma unroll
    for (int ct = 0; ct < 4; ++ct)
#pragma unroll
      for (int e = 0; e < 4; ++e) sPt[(16 * ct + r) * M::ST + 16 * w + 4 * g + e] = p[ct][e];
    lds_barrier();
    mma_rows<CH, M::NT>(sPt + 16 * w * M::ST, M::ST, sVt, 16 * M::ST, M::ST, acc);
  }
  float* out = part + ((long)seg * m + c0) * D;
#pragma unroll
  for (int t = 0; t < M::NT; ++t)
#pragma unroll
    for (int e = 0; e < 4; ++e) out[(long)(16 * w + 4 * g + e) * D + 16 * t + r] = acc[t][e];
}

// B^T = (1/F) sum over segments, in segment order.
__global__ void hebbian_reduce_kernel(const float* __restrict__ part, int n_seg, long n, float inv_f,
                                      float* __restrict__ Bt) {
  const long i = (long)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n) return;
  float s = 0.f;
  for (int k = 0; k < n_seg; ++k) s += part[(long)k * n + i];
  Bt[i] = s * inv_f;
}

// out [n][D] = phi(Q) B, B given as B^T [m][D].
template <int D>
__global__ __launch_bounds__(256) void hebbian_read_kernel(const float* __restrict__ Q, int n,
                                                           const float* __restrict__ A, const float* __restrict__ G,
                                                           const float* __restrict__ Bt, int m,
                                                           float* __restrict__ out) {
  using M = MT<D>;
  __shared__ __attribute__((aligned(16))) float sQ[CH * M::S];
  __shared__ __attribute__((aligned(16))) float sA[CH * M::S];
  __shared__ __attribute__((aligned(16))) float sG[CH * M::S];
  __shared__ __attribute__((aligned(16))) float sBt[D * M::ST];   // B chunk [dv][feature]
  __shared__ __attribute__((aligned(16))) float sP[CH * M::ST];   // phi [query][feature]
  const int q0 = blockIdx.x * CH, nq = min(CH, n - q0);
  const int w = wave_id(), l = lane_id(), r = l & 15, g = l >> 4;
  {
    Rows<D> rq;
    rq.load(Q + (long)q0 * D, D, nq);
    rq.put_rows(sQ);
  }
  floatx4 acc[M::NT];
#pragma unroll
  for (int t = 0; t < M::NT; ++t) acc[t] = zero4();
  Rows<D> xa, xg, xb;
  xa.load(A, D, CH);
  xg.load(G, D, CH);
  xb.load(Bt, D, CH);
  for (int c0 = 0; c0 < m; c0 += CH) {
    lds_barrier();  // every wave is done with the previous chunk
    xa.put_rows(sA);
    xg.put_rows(sG);
    xb.put_cols(sBt);
    lds_barrier();
    if (c0 + CH < m) {
      xa.load(A + (long)(c0 + CH) * D, D, CH);
      xg.load(G + (long)(c0 + CH) * D, D, CH);
      xb.load(Bt + (long)(c0 + CH) * D, D, CH);
    }
    floatx4 p[4];
    phi_tile<D>(sQ, sA, sG, p);
    // this wave's rows of phi, read back by the same wave only
#pragma unroll
    for (int ct = 0; ct < 4; ++ct)
#pragma unroll
      for (int e = 0; e < 4; ++e) sP[(16 * w + 4 * g + e) * M::ST + 16 * ct + r] = p[ct][e];
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront", "local");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront", "local");
    mma_rows<CH, M::NT>(sP + 16 * w * M::ST, M::ST, sBt, 16 * M::ST, M::ST, acc);
  }
#pragma unroll
  for (int t = 0; t < M::NT; ++t)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int row = 16 * w + 4 * g + e;
      if (row < nq) out[(long)(q0 + row) * D + 16 * t + r] = acc[t][e];
    }
}

// out[gr] [n][D] = Q[gr] [n][D] A[gr] [D][D] for every group gr (a (b, h)).
template <int D>
__global__ __launch_bounds__(256) void memory_read_kernel(const float* __restrict__ Q, const float* __restrict__ A,
                                                          int n, float* __restrict__ out) {
  using M = MT<D>;
  __shared__ __attribute__((aligned(16))) float sQ[CH * M::S];
  __shared__ __attribute__((aligned(16))) float sAt[D * M::S];  // A^T [dv][dk]
  const int q0 = blockIdx.x * CH, gr = blockIdx.y, nq = min(CH, n - q0);
  const int w = wave_id(), l = lane_id(), r = l & 15, g = l >> 4;
  const float* qg = Q + ((long)gr * n + q0) * D;
  {
    Rows<D> rq;
    rq.load(qg, D, nq);
    rq.put_rows(sQ);
  }
  const float* ag = A + (long)gr * D * D;
  for (int i = threadIdx.x; i < D * D; i += blockDim.x) {
    const int k = i / D, v = i % D;
    sAt[v * M::S + k] = ag[i];
  }
  __syncthreads();
  floatx4 acc[M::NT];
#pragma unroll
  for (int t = 0; t < M::NT; ++t) acc[t] = zero4();
  mma_rows<D, M::NT>(sQ + 16 * w * M::S, M::S, sAt, 16 * M::S, M::S, acc);
  float* og = out + ((long)gr * n + q0) * D;
#pragma unroll
  for (int t = 0; t < M::NT; ++t)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int row = 16 * w + 4 * g + e;
      if (row < nq) og[(long)row * D + 16 * t + r] = acc[t][e];
    }
}

// Per query of group gr: index and value of the largest <R_q, V_j> over the
// group's candidates j (the smallest index on a tie).
template <int D>
__global__ __launch_bounds__(256) void recall_argmax_kernel(const float* __restrict__ R, const float* __restrict__ V,
                                                            int nq, int nc, int* __restrict__ arg,
                                                            float* __restrict__ best) {
  using M = MT<D>;
  __shared__ __attribute__((aligned(16))) float sR[CH * M::S];
  __shared__ __attribute__((aligned(16))) float sV[CH * M::S];
  const int q0 = blockIdx.x * CH, gr = blockIdx.y, n = min(CH, nq - q0);
  const int w = wave_id(), l = lane_id(), r = l & 15, g = l >> 4;
  {
    Rows<D> rr;
    rr.load(R + ((long)gr * nq + q0) * D, D, n);
    rr.put_rows(sR);
  }
  const float* vg = V + (long)gr * nc * D;
  float bv[4];
  int bi[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    bv[e] = -__builtin_inff();
    bi[e] = 0;
  }
  Rows<D> xv;
  xv.load(vg, D, min(CH, nc));
  for (int j0 = 0; j0 < nc; j0 += CH) {
    lds_barrier();  // every wave is done with the previous chunk
    xv.put_rows(sV);
    lds_barrier();
    if (j0 + CH < nc) xv.load(vg + (long)(j0 + CH) * D, D, min(CH, nc - j0 - CH));
    floatx4 s[4] = {zero4(), zero4(), zero4(), zero4()};
    mma_rows<D, 4>(sR + 16 * w * M::S, M::S, sV, 16 * M::S, M::S, s);
    // this lane's running best over its own columns 16 ct + r: they come in
    // increasing order, so a strict > keeps the smallest index of a tie
#pragma unroll
    for (int e = 0; e < 4; ++e) {
#pragma unroll
      for (int ct = 0; ct < 4; ++ct) {
        const int jj = j0 + 16 * ct + r;
        if (jj < nc && s[ct][e] > bv[e]) {
          bv[e] = s[ct][e];
          bi[e] = jj;
        }
      }
    }
  }
  // the 16 lanes of a row: largest value, smallest index among equal ones
#pragma unroll
  for (int e = 0; e < 4; ++e) {
#pragma unroll
    for (int off = 1; off < 16; off <<= 1) {
      const float ov = __shfl_xor(bv[e], off);
      const int oj = __shfl_xor(bi[e], off);
      if (ov > bv[e] || (ov == bv[e] && oj < bi[e])) {
        bv[e] = ov;
        bi[e] = oj;
      }
    }
  }
  if (r == 0) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int row = 16 * w + 4 * g + e;
      if (row < n) {
        arg[(long)gr * nq + q0 + row] = bi[e];
        if (best != nullptr) best[(long)gr * nq + q0 + row] = bv[e];
      }
    }
  }
}

int hebbian_segments(int F, int m) {
  const int tiles = m / CH;
  const int chunks = (F + CH - 1) / CH;
  return std::max(1, std::min(chunks, (512 + tiles - 1) / tiles));
}

template <int D>
hipError_t run_hebbian_write(const float* K, const float* V, const int* f, int F, int n_values, const float* A,
                             const float* G, int m, float* Bt, float* part, hipStream_t s) {
  const int n_seg = hebbian_segments(F, m);
  const int seg_len = ((F + n_seg - 1) / n_seg + CH - 1) / CH * CH;
  profile_mark_before(s);
  hipLaunchKernelGGL((hebbian_write_kernel<D>), dim3(m / CH, n_seg), dim3(256), 0, s, K, V, f, F, n_values, A, G, m,
                     seg_len, part);
  profile_mark_after(s);
  const long n = (long)m * D;
  hipLaunchKernelGGL(hebbian_reduce_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, part, n_seg, n,
                     1.f / (float)F, Bt);
  return hipGetLastError();
}

}  // namespace

size_t hebbian_ws_bytes(int F, int m, int d) {
  return (size_t)hebbian_segments(F, m) * m * d * sizeof(float);
}

hipError_t launch_hebbian_write(const float* K, const float* V, const int* f, int F, int n_values, const float* A,
                                const float* G, int m, int d, float* Bt, void* ws, hipStream_t s) {
  float* part = static_cast<float*>(ws);
  switch (d) {
    case 32: return run_hebbian_write<32>(K, V, f, F, n_values, A, G, m, Bt, part, s);
    case 64: return run_hebbian_write<64>(K, V, f, F, n_values, A, G, m, Bt, part, s);
    case 128: return run_hebbian_write<128>(K, V, f, F, n_values, A, G, m, Bt, part, s);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_hebbian_read(const float* Q, int n, const float* A, const float* G, const float* Bt, int m, int d,
                               float* out, hipStream_t s) {
  const dim3 grid((n + CH - 1) / CH);
  switch (d) {
    case 32: hipLaunchKernelGGL((hebbian_read_kernel<32>), grid, dim3(256), 0, s, Q, n, A, G, Bt, m, out); break;
    case 64: hipLaunchKernelGGL((hebbian_read_kernel<64>), grid, dim3(256), 0, s, Q, n, A, G, Bt, m, out); break;
    case 128: hipLaunchKernelGGL((hebbian_read_kernel<128>), grid, dim3(256), 0, s, Q, n, A, G, Bt, m, out); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_memory_read(const float* Q, const float* A, int groups, int n, int d, float* out, hipStream_t s) {
  const dim3 grid((n + CH - 1) / CH, groups);
  switch (d) {
    case 32: hipLaunchKernelGGL((memory_read_kernel<32>), grid, dim3(256), 0, s, Q, A, n, out); break;
    case 64: hipLaunchKernelGGL((memory_read_kernel<64>), grid, dim3(256), 0, s, Q, A, n, out); break;
    case 128: hipLaunchKernelGGL((memory_read_kernel<128>), grid, dim3(256), 0, s, Q, A, n, out); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_recall_argmax(const float* R, const float* V, int groups, int nq, int nc, int d, int* arg,
                                float* best, hipStream_t s) {
  const dim3 grid((nq + CH - 1) / CH, groups);
  switch (d) {
    case 32: hipLaunchKernelGGL((recall_argmax_kernel<32>), grid, dim3(256), 0, s, R, V, nq, nc, arg, best); break;
    case 64: hipLaunchKernelGGL((recall_argmax_kernel<64>), grid, dim3(256), 0, s, R, V, nq, nc, arg, best); break;
    case 128: hipLaunchKernelGGL((recall_argmax_kernel<128>), grid, dim3(256), 0, s, R, V, nq, nc, arg, best); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace tc

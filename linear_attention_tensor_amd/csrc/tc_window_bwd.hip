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
//
// Every product is a dense fp32 contraction and runs on the fp32 matrix cores
// (v_mfma_f32_16x16x4_f32: A(m, k) from lane m + 16 k, B(k, n) from lane
// n + 16 k, D(m, n) in lane n + 16 (m / 4), element m % 4).  A wave owns 16
// rows (queries, or keys); its partner rows pass through LDS in blocks of 32
// (fp32, row stride D + 4 floats, double-buffered, the next block in
// registers meanwhile).  The k order of the D-long dot products is permuted
// so that lane group g takes the features g D/4 .. g D/4 + D/4 - 1 (one
// 16-byte LDS read feeds four MFMAs).  A score tile leaves lane (g, n) with
// row n and partner rows 4 g + e (e < 4), which are exactly the k rows lane
// (g, n) supplies to a product over the partner rows at k-step e: the
// probabilities and ds feed the next products from their registers.
//   (1) per 128 queries (8 waves x 16): pass 1 over the key blocks forms the
//       softmax of the scores (scaled by scale log2 e) and y, and writes
//       lse2_t (log2 of the normaliser, in those units) and D_t = <dy_t, y_t>;
//       pass 2 forms p = 2^(s - lse2), dp = <dy_t, v_j>, ds = p (dp - D_t) and
//       dq^T += K^T ds^T.
//   (2) per 128 keys (8 waves x 16): over the query blocks that see them,
//       s and dp as above (transposed), dv^T += dY^T p, dk^T += Q^T ds.
// (1) and (2) can add to what the output buffers hold (the fused layer's
// backward adds the L2 branch this way).
#include "tc_common.hpp"
#include "tc_kernels.hpp"

#include <math.h>

namespace tc {

namespace {

constexpr int NW = 8;               // waves per workgroup
constexpr int NT = 64 * NW;         // threads per workgroup
constexpr int RB = 16 * NW;         // rows (queries or keys) per workgroup
constexpr int PB = 32;              // partner rows per LDS block
constexpr int NXCD = 8;             // MI355X: 8 accelerator complex dies, workgroups dispatched round-robin
constexpr float kNegBig = -1.0e30f;

__device__ __forceinline__ floatx4 mfma4(float a, float b, floatx4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ float4 ld4(const float* p) { return *reinterpret_cast<const float4*>(p); }
__device__ __forceinline__ float4 ld4(const uint16_t* p) {
  const uint2 u = *reinterpret_cast<const uint2*>(p);
  return make_float4(__uint_as_float(u.x << 16), __uint_as_float(u.x & 0xFFFF0000u),
                     __uint_as_float(u.y << 16), __uint_as_float(u.y & 0xFFFF0000u));
}
// max / sum over the four lane groups (lanes n, n + 16, n + 32, n + 48)
__device__ __forceinline__ float max_groups(float x) {
  x = fmaxf(x, __shfl_xor(x, 16));
  return fmaxf(x, __shfl_xor(x, 32));
}
__device__ __forceinline__ float sum_groups(float x) {
  x += __shfl_xor(x, 16);
  return x + __shfl_xor(x, 32);
}

// Rows r0 .. r0 + 31 of two [T][D] arrays (zero past T) through registers into
// an LDS stage (row stride D + 4).
template <typename TA, typename TB, int D>
struct Block2 {
  static constexpr int S = D + 4;
  static constexpr int NP = 8 * D;             // float4 pieces per array and block
  static constexpr int NLD = (NP + NT - 1) / NT;
  float4 ra[NLD], rb[NLD];
  __device__ __forceinline__ void load(const TA* a, const TB* b, long base, int r0, int T) {
#pragma unroll
    for (int i = 0; i < NLD; ++i) {
      const int f = threadIdx.x + NT * i, row = f / (D / 4), c4 = f % (D / 4);
      const bool in = (NP % NT == 0 || f < NP) && r0 + row < T;
      const long off = (base + r0 + row) * D + 4 * c4;
      ra[i] = in ? ld4(a + off) : make_float4(0.f, 0.f, 0.f, 0.f);
      rb[i] = in ? ld4(b + off) : make_float4(0.f, 0.f, 0.f, 0.f);
    }
  }
  __device__ __forceinline__ void store(float* sa, float* sb) const {
#pragma unroll
    for (int i = 0; i < NLD; ++i) {
      const int f = threadIdx.x + NT * i, row = f / (D / 4), c4 = f % (D / 4);
      if (NP % NT == 0 || f < NP) {
        *reinterpret_cast<float4*>(sa + row * S + 4 * c4) = ra[i];
        *reinterpret_cast<float4*>(sb + row * S + 4 * c4) = rb[i];
      }
    }
  }
};

// 16 x 32 score-like tile of a wave: acc[t] (t = 0, 1) += sum over the
// features of A rows (16 t + m of the LDS stage, m < 16) times the lane's own
// row held in registers (xr[j] = feature D/4 g + j).
template <int D>
__device__ __forceinline__ void tile_dot(const float* stage, const float* xr, floatx4* acc) {
  constexpr int S = D + 4, Q = D / 4;
  const int l = threadIdx.x & 63, m = l & 15, g = l >> 4;
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    const float* ar = stage + (16 * t + m) * S + Q * g;
#pragma unroll
    for (int j4 = 0; j4 < Q / 4; ++j4) {
      const float4 a = *reinterpret_cast<const float4*>(ar + 4 * j4);
      acc[t] = mfma4(a.x, xr[4 * j4], acc[t]);
      acc[t] = mfma4(a.y, xr[4 * j4 + 1], acc[t]);
      acc[t] = mfma4(a.z, xr[4 * j4 + 2], acc[t]);
      acc[t] = mfma4(a.w, xr[4 * j4 + 3], acc[t]);
    }
  }
}

// out^T[f][row n] (f = 16 dt + 4 g + e in acc[dt][e]) += sum over the 32
// partner rows r of stage[r][f] w[r], where lane (g, n) holds w of partner
// rows 16 t + 4 g + e in wt[t][e].
template <int D>
__device__ __forceinline__ void accum_rows(const float* stage, const floatx4* wt, floatx4* acc) {
  constexpr int S = D + 4;
  const int l = threadIdx.x & 63, m = l & 15, g = l >> 4;
#pragma unroll
  for (int t = 0; t < 2; ++t)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float* row = stage + (16 * t + 4 * g + e) * S + m;
#pragma unroll
      for (int dt = 0; dt < D / 16; ++dt) acc[dt] = mfma4(row[16 * dt], wt[t][e], acc[dt]);
    }
}

__device__ __forceinline__ int xcd_item(int n_items) {
  const int per_xcd = (n_items + NXCD - 1) / NXCD;
  return ((int)blockIdx.x % NXCD) * per_xcd + (int)blockIdx.x / NXCD;
}

// (1) statistics and dq, per 128 queries
template <typename TIn, int D>
__global__ __launch_bounds__(NT) void wbwd_q_kernel(const TIn* __restrict__ q, const TIn* __restrict__ k,
                                                   const TIn* __restrict__ v, const float* __restrict__ dy,
                                                   int T, int W, int n_tiles, int n_items, float sl2, float scale,
                                                   float* __restrict__ lse2, float* __restrict__ dd,
                                                   bool accumulate, float* __restrict__ dq) {
  constexpr int S = D + 4, Q = D / 4, ND = D / 16;
  __shared__ __attribute__((aligned(16))) float sk[2][PB * S];
  __shared__ __attribute__((aligned(16))) float sv[2][PB * S];
  const int item = xcd_item(n_items);
  if (item >= n_items) return;  // whole workgroup, before any barrier
  const int bh = item / n_tiles, t0 = (item % n_tiles) * RB;
  const int w = threadIdx.x >> 6, l = threadIdx.x & 63, n = l & 15, g = l >> 4;
  const long base = (long)bh * T;
  const int q0 = t0 + 16 * w, tq = q0 + n;
  const int j_lo = max(0, t0 - W + 1), j_hi = min(T - 1, t0 + RB - 1);
  const int nblk = (j_hi - j_lo + PB) / PB;
  // the wave's key range: some key of the block in the window of one of its queries
  auto active_at = [&](int jb) { return q0 < T && jb <= min(q0 + 15, T - 1) && jb + PB - 1 >= q0 - W + 1; };
  auto full_at = [&](int jb) { return jb + PB - 1 <= q0 && jb >= q0 + 16 - W; };
  // scores of keys jb + 16 t + 4 g + e (valid: tq - W < j <= tq, j < T) into s
  auto mask = [&](int jb, floatx4* s) __attribute__((always_inline)) {
    const int lo = tq - W + 1 - jb, hi = min(tq, T - 1) - jb;
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int kk = 16 * t + 4 * g + e;
        s[t][e] = (kk >= lo && kk <= hi) ? s[t][e] : -INFINITY;
      }
  };

  float xr[Q];  // q scale log2(e), features Q g ..
#pragma unroll
  for (int j4 = 0; j4 < Q / 4; ++j4) {
    const float4 x = tq < T ? ld4(q + (base + tq) * D + Q * g + 4 * j4) : make_float4(0.f, 0.f, 0.f, 0.f);
    xr[4 * j4] = x.x * sl2;
    xr[4 * j4 + 1] = x.y * sl2;
    xr[4 * j4 + 2] = x.z * sl2;
    xr[4 * j4 + 3] = x.w * sl2;
  }
  floatx4 acc[ND];
#pragma unroll
  for (int dt = 0; dt < ND; ++dt) acc[dt] = floatx4{0.f, 0.f, 0.f, 0.f};
  Block2<TIn, TIn, D> blk;

  // ---- pass 1: softmax statistics and y
  float m = kNegBig, lsum = 0.f;
  blk.load(k, v, base, j_lo, T);
  blk.store(sk[0], sv[0]);
  __syncthreads();
#pragma unroll 1
  for (int i = 0; i < nblk; ++i) {
    const int jb = j_lo + PB * i, cur = i & 1;
    if (i + 1 < nblk) blk.load(k, v, base, jb + PB, T);
    if (active_at(jb)) {
      floatx4 s[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
      tile_dot<D>(sk[cur], xr, s);
      if (!full_at(jb)) mask(jb, s);
      float bm = s[0][0];
#pragma unroll
      for (int e = 1; e < 4; ++e) bm = fmaxf(bm, s[0][e]);
#pragma unroll
      for (int e = 0; e < 4; ++e) bm = fmaxf(bm, s[1][e]);
      bm = max_groups(bm);
      if (__ballot(bm - m > 8.f) != 0) {  // lazy rescale: every probability stays <= 2^8
        const float mnew = fmaxf(m, bm);
        const float alpha = __builtin_amdgcn_exp2f(m - mnew);
        lsum *= alpha;
#pragma unroll
        for (int dt = 0; dt < ND; ++dt) acc[dt] *= alpha;
        m = mnew;
      }
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          s[t][e] = __builtin_amdgcn_exp2f(s[t][e] - m);
          lsum += s[t][e];
        }
      accum_rows<D>(sv[cur], s, acc);  // y^T += V^T p^T
    }
    if (i + 1 < nblk) blk.store(sk[cur ^ 1], sv[cur ^ 1]);
    __syncthreads();
  }
  const float ltot = sum_groups(lsum);
  const float ls2 = m + log2f(ltot > 0.f ? ltot : 1.f);  // log2 of the normaliser
  float dpart = 0.f;
  if (tq < T) {
    const float inv = 1.f / ltot;
#pragma unroll
    for (int dt = 0; dt < ND; ++dt) {
      const float4 gy = *reinterpret_cast<const float4*>(dy + (base + tq) * D + 16 * dt + 4 * g);
      dpart += gy.x * acc[dt][0] * inv + gy.y * acc[dt][1] * inv + gy.z * acc[dt][2] * inv + gy.w * acc[dt][3] * inv;
    }
  }
  const float dt_t = sum_groups(dpart);
  if (tq < T && g == 0) {
    lse2[base + tq] = ls2;
    dd[base + tq] = dt_t;
  }

  // ---- pass 2: dq
  float yr[Q];  // dy, features Q g ..
#pragma unroll
  for (int j4 = 0; j4 < Q / 4; ++j4) {
    const float4 x = tq < T ? ld4(dy + (base + tq) * D + Q * g + 4 * j4) : make_float4(0.f, 0.f, 0.f, 0.f);
    yr[4 * j4] = x.x;
    yr[4 * j4 + 1] = x.y;
    yr[4 * j4 + 2] = x.z;
    yr[4 * j4 + 3] = x.w;
  }
#pragma unroll
  for (int dt = 0; dt < ND; ++dt) acc[dt] = floatx4{0.f, 0.f, 0.f, 0.f};
  blk.load(k, v, base, j_lo, T);
  blk.store(sk[0], sv[0]);  // every wave passed the last barrier of pass 1
  __syncthreads();
#pragma unroll 1
  for (int i = 0; i < nblk; ++i) {
    const int jb = j_lo + PB * i, cur = i & 1;
    if (i + 1 < nblk) blk.load(k, v, base, jb + PB, T);
    if (active_at(jb)) {
      floatx4 s[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
      floatx4 dp[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
      tile_dot<D>(sk[cur], xr, s);
      tile_dot<D>(sv[cur], yr, dp);
      if (!full_at(jb)) mask(jb, s);
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int e = 0; e < 4; ++e) s[t][e] = __builtin_amdgcn_exp2f(s[t][e] - ls2) * (dp[t][e] - dt_t);
      accum_rows<D>(sk[cur], s, acc);  // dq^T += K^T ds^T
    }
    if (i + 1 < nblk) blk.store(sk[cur ^ 1], sv[cur ^ 1]);
    __syncthreads();
  }
  if (tq < T) {
#pragma unroll
    for (int dt = 0; dt < ND; ++dt) {
      float4* o = reinterpret_cast<float4*>(dq + (base + tq) * D + 16 * dt + 4 * g);
      float4 r = make_float4(scale * acc[dt][0], scale * acc[dt][1], scale * acc[dt][2], scale * acc[dt][3]);
      if (accumulate) {
        const float4 x = *o;
        r = make_float4(x.x + r.x, x.y + r.y, x.z + r.z, x.w + r.w);
      }
      *o = r;
    }
  }
}

// (2) dk, dv per 128 keys, over the queries t in [j, min(T - 1, j + W - 1)]
template <typename TIn, int D>
__global__ __launch_bounds__(NT) void wbwd_kv_kernel(const TIn* __restrict__ q, const TIn* __restrict__ k,
                                                    const TIn* __restrict__ v, const float* __restrict__ dy,
                                                    int T, int W, int n_tiles, int n_items, float sl2, float scale,
                                                    const float* __restrict__ lse2, const float* __restrict__ dd,
                                                    bool accumulate, float* __restrict__ dk, float* __restrict__ dv) {
  constexpr int S = D + 4, Q = D / 4, ND = D / 16;
  __shared__ __attribute__((aligned(16))) float sq[2][PB * S];
  __shared__ __attribute__((aligned(16))) float sy[2][PB * S];
  __shared__ __attribute__((aligned(16))) float sl[2][PB];
  __shared__ __attribute__((aligned(16))) float sd[2][PB];
  const int item = xcd_item(n_items);
  if (item >= n_items) return;  // whole workgroup, before any barrier
  const int bh = item / n_tiles, j0 = (item % n_tiles) * RB;
  const int w = threadIdx.x >> 6, l = threadIdx.x & 63, n = l & 15, g = l >> 4;
  const long base = (long)bh * T;
  const int kw = j0 + 16 * w, jk = kw + n;  // the wave's first key, this lane's key
  const int t_lo = j0, t_hi = min(T - 1, j0 + RB - 1 + W - 1);
  const int nblk = (t_hi - t_lo + PB) / PB;

  float kr[Q], vr[Q];  // k scale log2(e) and v, features Q g ..
#pragma unroll
  for (int j4 = 0; j4 < Q / 4; ++j4) {
    const bool in = jk < T;
    const float4 x = in ? ld4(k + (base + jk) * D + Q * g + 4 * j4) : make_float4(0.f, 0.f, 0.f, 0.f);
    const float4 y = in ? ld4(v + (base + jk) * D + Q * g + 4 * j4) : make_float4(0.f, 0.f, 0.f, 0.f);
    kr[4 * j4] = x.x * sl2;
    kr[4 * j4 + 1] = x.y * sl2;
    kr[4 * j4 + 2] = x.z * sl2;
    kr[4 * j4 + 3] = x.w * sl2;
    vr[4 * j4] = y.x;
    vr[4 * j4 + 1] = y.y;
    vr[4 * j4 + 2] = y.z;
    vr[4 * j4 + 3] = y.w;
  }
  floatx4 ak[ND], av[ND];
#pragma unroll
  for (int dt = 0; dt < ND; ++dt) ak[dt] = av[dt] = floatx4{0.f, 0.f, 0.f, 0.f};
  Block2<TIn, float, D> blk;
  float rl = 0.f, rd = 0.f;  // lse2, D of query row tb + threadIdx.x (threads < 32)
  auto load_stats = [&](int tb) __attribute__((always_inline)) {
    if (threadIdx.x < PB) {
      const int row = tb + threadIdx.x;
      rl = row < T ? lse2[base + row] : 0.f;
      rd = row < T ? dd[base + row] : 0.f;
    }
  };
  auto store_stats = [&](int st) __attribute__((always_inline)) {
    if (threadIdx.x < PB) {
      sl[st][threadIdx.x] = rl;
      sd[st][threadIdx.x] = rd;
    }
  };
  blk.load(q, dy, base, t_lo, T);
  load_stats(t_lo);
  blk.store(sq[0], sy[0]);
  store_stats(0);
  __syncthreads();
#pragma unroll 1
  for (int i = 0; i < nblk; ++i) {
    const int tb = t_lo + PB * i, cur = i & 1;
    if (i + 1 < nblk) {
      blk.load(q, dy, base, tb + PB, T);
      load_stats(tb + PB);
    }
    // some query of the block sees some key of the wave (wave-uniform)
    const bool active = kw < T && tb <= kw + 15 + W - 1 && tb + PB - 1 >= kw;
    if (active) {
      floatx4 s[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
      floatx4 dp[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
      tile_dot<D>(sq[cur], kr, s);   // s[t][e]: query tb + 16 t + 4 g + e, key jk
      tile_dot<D>(sy[cur], vr, dp);  // <dy_t, v_j>, same layout
      const bool full = tb >= kw + 15 && tb + PB - 1 <= kw + W - 1 && tb + PB - 1 < T;
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        const float4 l4 = *reinterpret_cast<const float4*>(&sl[cur][16 * t + 4 * g]);
        const float4 d4 = *reinterpret_cast<const float4*>(&sd[cur][16 * t + 4 * g]);
        const float lv[4] = {l4.x, l4.y, l4.z, l4.w}, dv4[4] = {d4.x, d4.y, d4.z, d4.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int tt = tb + 16 * t + 4 * g + e;
          const bool ok = full || (tt >= jk && tt <= jk + W - 1 && tt < T);
          const float p = ok ? __builtin_amdgcn_exp2f(s[t][e] - lv[e]) : 0.f;
          s[t][e] = p;
          dp[t][e] = p * (dp[t][e] - dv4[e]);
        }
      }
      accum_rows<D>(sy[cur], s, av);   // dv^T += dY^T p
      accum_rows<D>(sq[cur], dp, ak);  // dk^T += Q^T ds
    }
    if (i + 1 < nblk) {
      blk.store(sq[cur ^ 1], sy[cur ^ 1]);
      store_stats(cur ^ 1);
    }
    __syncthreads();
  }
  if (jk < T) {
#pragma unroll
    for (int dt = 0; dt < ND; ++dt) {
      float4* ok = reinterpret_cast<float4*>(dk + (base + jk) * D + 16 * dt + 4 * g);
      float4* ov = reinterpret_cast<float4*>(dv + (base + jk) * D + 16 * dt + 4 * g);
      float4 rk = make_float4(scale * ak[dt][0], scale * ak[dt][1], scale * ak[dt][2], scale * ak[dt][3]);
      float4 rv = make_float4(av[dt][0], av[dt][1], av[dt][2], av[dt][3]);
      if (accumulate) {
        const float4 xk = *ok, xv = *ov;
        rk = make_float4(xk.x + rk.x, xk.y + rk.y, xk.z + rk.z, xk.w + rk.w);
        rv = make_float4(xv.x + rv.x, xv.y + rv.y, xv.z + rv.z, xv.w + rv.w);
      }
      *ok = rk;
      *ov = rv;
    }
  }
}

template <typename TIn, int D>
hipError_t run_wbwd(const TIn* q, const TIn* k, const TIn* v, const float* dy, int BH, int T, int W, float scale,
                    float* lse2, float* dd, bool accumulate, float* dq, float* dk, float* dv, hipStream_t s) {
  const int n_tiles = (T + RB - 1) / RB, n_items = BH * n_tiles;
  const int grid = (n_items + NXCD - 1) / NXCD * NXCD;
  const float sl2 = scale * 1.4426950408889634f;
  hipLaunchKernelGGL((wbwd_q_kernel<TIn, D>), dim3(grid), dim3(NT), 0, s, q, k, v, dy, T, W, n_tiles, n_items, sl2,
                     scale, lse2, dd, accumulate, dq);
  profile_mark_before(s);
  hipLaunchKernelGGL((wbwd_kv_kernel<TIn, D>), dim3(grid), dim3(NT), 0, s, q, k, v, dy, T, W, n_tiles, n_items, sl2,
                     scale, lse2, dd, accumulate, dk, dv);
  profile_mark_after(s);
  return hipGetLastError();
}

template <typename TIn>
hipError_t dispatch_wbwd(const TIn* q, const TIn* k, const TIn* v, const float* dy, int BH, int T, int d, int W,
                         float scale, float* ws, bool accumulate, float* dq, float* dk, float* dv, hipStream_t s) {
  float* lse2 = ws;
  float* dd = ws + (long)BH * T;
  switch (d) {
    case 16: return run_wbwd<TIn, 16>(q, k, v, dy, BH, T, W, scale, lse2, dd, accumulate, dq, dk, dv, s);
    case 32: return run_wbwd<TIn, 32>(q, k, v, dy, BH, T, W, scale, lse2, dd, accumulate, dq, dk, dv, s);
    case 64: return run_wbwd<TIn, 64>(q, k, v, dy, BH, T, W, scale, lse2, dd, accumulate, dq, dk, dv, s);
    case 128: return run_wbwd<TIn, 128>(q, k, v, dy, BH, T, W, scale, lse2, dd, accumulate, dq, dk, dv, s);
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

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
//
// The full decode step of the layer (decode_layer_kernel) adds, in the same
// workgroup, the L1 part of Methodology 1: exact softmax attention of q over
// the W most recent tokens (the ring after the write, the current token
// included) and the gated sum y = y_local + sigmoid(g) m.  Its bytes are
// dominated by the ring (2 W d elements per head and step), which the four
// waves stream in contiguous slot ranges, 16 bytes per lane.
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

// d = 128: every A load of the thread (16 rows, one float4 each) is issued
// before the evicted pair arrives, so the loads overlap the ring access and
// each other; then the rows are updated, written and read in turn.  When A is
// far larger than the Infinity Cache (STREAM), its stores are non-temporal:
// A then streams from HBM every step anyway, and stores that bypass the cache
// hierarchy free it for the reads (6.5 against 5.1 TB/s at 512 MiB of A,
// measured same box).  When A fits, plain stores keep it cached for the next
// step.
typedef float f32x4v __attribute__((ext_vector_type(4)));

template <typename TIn, bool STREAM>
__global__ __launch_bounds__(256) void decode_kernel_128(
    const TIn* __restrict__ q, const TIn* __restrict__ k, const TIn* __restrict__ v,
    TIn* __restrict__ ring_k, TIn* __restrict__ ring_v, float* __restrict__ A,
    const float* __restrict__ lam, const float* __restrict__ eta, const int64_t* __restrict__ pos,
    int H, int W, float* __restrict__ m) {
  constexpr int D = 128, NCG = D / 4, RPP = 256 / NCG, RPT = D / RPP;  // 32 groups, 8 rows a pass, 16 rows
  __shared__ float sq[D];
  __shared__ float ske[D];
  __shared__ float sve[D];
  __shared__ float4 part[256];

  const int bh = blockIdx.x;
  const int b = bh / H, h = bh % H;
  const int t = threadIdx.x;
  const int cg = t % NCG, r0 = t / NCG;
  f32x4v* Ab = reinterpret_cast<f32x4v*>(A + (long)bh * D * D);
  f32x4v a[RPT];
#pragma unroll
  for (int i = 0; i < RPT; ++i) a[i] = Ab[(r0 + RPP * i) * NCG + cg];

  const long p = pos[b];
  const long slot = p % W;
  const bool evict = p >= W;
  TIn* rk = ring_k + ((long)bh * W + slot) * D;
  TIn* rv = ring_v + ((long)bh * W + slot) * D;
  if (t < D) {
    sq[t] = InT<TIn>::ld(q + (long)bh * D, t);
    ske[t] = evict ? InT<TIn>::ld(rk, t) : 0.f;
  } else {
    sve[t - D] = evict ? InT<TIn>::ld(rv, t - D) : 0.f;
  }
  __syncthreads();  // the evicted pair is in LDS before the slot is overwritten
  if (t < D) rk[t] = k[(long)bh * D + t];
  else rv[t - D] = v[(long)bh * D + t - D];

  const float lm = lam[h], et = eta[h];
  const f32x4v ve = {et * sve[4 * cg], et * sve[4 * cg + 1], et * sve[4 * cg + 2], et * sve[4 * cg + 3]};
  f32x4v acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int i = 0; i < RPT; ++i) {
    const int r = r0 + RPP * i;
    f32x4v x = a[i];
    if (evict) {
      x = lm * x + ske[r] * ve;
      if (STREAM) __builtin_nontemporal_store(x, &Ab[r * NCG + cg]);
      else Ab[r * NCG + cg] = x;
    }
    acc += sq[r] * x;
  }
  part[t] = make_float4(acc[0], acc[1], acc[2], acc[3]);
  __syncthreads();
  if (t < NCG) {
    float4 s = part[t];
#pragma unroll
    for (int j = 1; j < RPP; ++j) {
      const float4 o = part[j * NCG + t];
      s.x += o.x;
      s.y += o.y;
      s.z += o.z;
      s.w += o.w;
    }
    reinterpret_cast<float4*>(m + (long)bh * D)[t] = s;
  }
}

// ---------------------------------------------------------------------------
// L1 part: K and V rows of the ring in 16-byte pieces.  E elements per piece,
// LPR lanes per row, RPI rows per wave instruction.
template <typename TIn>
struct Piece;
template <>
struct Piece<float> {
  static constexpr int E = 4;
  __device__ __forceinline__ static void cvt(u32x4 a, float* x) {
#pragma unroll
    for (int i = 0; i < 4; ++i) x[i] = __uint_as_float(a[i]);
  }
};
template <>
struct Piece<uint16_t> {
  static constexpr int E = 8;
  __device__ __forceinline__ static void cvt(u32x4 a, float* x) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      x[2 * i] = __uint_as_float(a[i] << 16);
      x[2 * i + 1] = __uint_as_float(a[i] & 0xFFFF0000u);
    }
  }
};
// Ring loads are non-temporal: the ring streams through once per step, and
// marking it so keeps A (reused every step) in the caches.
template <typename TIn>
__device__ __forceinline__ u32x4 ld16(const TIn* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
}

// One decode step of the whole layer per (b, h): the L2 step above, then
// y = softmax over the ring after the write (the current token included)
// + sigmoid(g) m.  The four waves take turns over batches of consecutive ring
// slots (so the workgroup reads one K and one V stream); every group of LPR
// lanes keeps its own running maximum, sum and output piece, merged at the end.
template <typename TIn, int D>
__global__ __launch_bounds__(256) void decode_layer_kernel(
    const TIn* __restrict__ q, const TIn* __restrict__ k, const TIn* __restrict__ v,
    TIn* __restrict__ ring_k, TIn* __restrict__ ring_v, float* __restrict__ A,
    const float* __restrict__ lam, const float* __restrict__ eta, const float* __restrict__ g,
    const int64_t* __restrict__ pos, int H, int W, float sl2, float* __restrict__ y) {
  constexpr int E = Piece<TIn>::E, LPR = D / E, RPI = 64 / LPR, U = 2;
  static_assert(D % E == 0 && LPR <= 64, "row pieces");
  __shared__ float sq[D], ske[D], sve[D], skn[D], svn[D], sm[D];
  __shared__ float4 part[256];
  __shared__ float sO[4][D], sMw[4], sLw[4];

  const int bh = blockIdx.x;
  const int b = bh / H, h = bh % H;
  const long p = pos[b];
  const int slot = (int)(p % W);
  const bool evict = p >= W;
  const int t = threadIdx.x;
  TIn* rk = ring_k + ((long)bh * W + slot) * D;
  TIn* rv = ring_v + ((long)bh * W + slot) * D;
  if (t < D) {
    sq[t] = InT<TIn>::ld(q + (long)bh * D, t);
    ske[t] = evict ? InT<TIn>::ld(rk, t) : 0.f;
    sve[t] = evict ? InT<TIn>::ld(rv, t) : 0.f;
    skn[t] = InT<TIn>::ld(k + (long)bh * D, t);
    svn[t] = InT<TIn>::ld(v + (long)bh * D, t);
  }
  __syncthreads();  // the evicted pair is in LDS before the slot is overwritten
  if (t < D) {
    rk[t] = k[(long)bh * D + t];
    rv[t] = v[(long)bh * D + t];
  }

  // L2: A <- lam A + eta k_e v_e^T (if a pair was evicted) and m = q A, one pass
  {
    const float lm = lam[h], et = eta[h];
    constexpr int ncg = D / 4, rpp = 256 / ncg;
    const int cg = t % ncg, r0 = t / ncg;
    float4* Ab = reinterpret_cast<float4*>(A + (long)bh * D * D);
    const float4 ve = make_float4(et * sve[4 * cg], et * sve[4 * cg + 1], et * sve[4 * cg + 2],
                                  et * sve[4 * cg + 3]);
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int r = r0; r < D; r += rpp) {
      float4 a = Ab[r * ncg + cg];
      if (evict) {
        const float kr = ske[r];
        a.x = lm * a.x + kr * ve.x;
        a.y = lm * a.y + kr * ve.y;
        a.z = lm * a.z + kr * ve.z;
        a.w = lm * a.w + kr * ve.w;
        Ab[r * ncg + cg] = a;
      }
      const float qr = sq[r];
      acc.x += qr * a.x;
      acc.y += qr * a.y;
      acc.z += qr * a.z;
      acc.w += qr * a.w;
    }
    part[t] = acc;
  }

  // L1 over the ring slots holding the other tokens of the window: [0, min(p, W))
  // without the slot just overwritten; the current token is added at the end.
  const int w = t >> 6, l = t & 63, c = l % LPR, rs = l / LPR;
  const int n_ring = (int)(p < W ? p : W);
  const int lo = 0, hi = n_ring;
  constexpr int BATCH = RPI * U;  // slots per wave and batch; wave w takes batches w, w + 4, ...
  float qs[E];
#pragma unroll
  for (int e = 0; e < E; ++e) qs[e] = sq[c * E + e] * sl2;
  float mx = -1.0e30f, ls = 0.f, o[E];
#pragma unroll
  for (int e = 0; e < E; ++e) o[e] = 0.f;
  const TIn* kb = ring_k + (long)bh * W * D + c * E;
  const TIn* vb = ring_v + (long)bh * W * D + c * E;
  // The K and V pieces of a batch (U rows per lane group) are loaded one
  // batch ahead; rows past the range reload a valid row whose values are
  // not used.
  u32x4 kr[U], vr[U];
  auto load_batch = [&](int r0) __attribute__((always_inline)) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int row = r0 + u * RPI + rs;
      const int rr = row < hi ? row : lo;
      kr[u] = ld16(kb + (long)rr * D);
      vr[u] = ld16(vb + (long)rr * D);
    }
  };
  if (w * BATCH < hi) load_batch(w * BATCH);
  for (int r0 = w * BATCH; r0 < hi; r0 += 4 * BATCH) {
    float sc[U], vx[U][E];
    {
      float kx[U][E];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        Piece<TIn>::cvt(kr[u], kx[u]);
        Piece<TIn>::cvt(vr[u], vx[u]);
      }
      if (r0 + 4 * BATCH < hi) load_batch(r0 + 4 * BATCH);
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int row = r0 + u * RPI + rs;
        float d = 0.f;
#pragma unroll
        for (int e = 0; e < E; ++e) d = fmaf(qs[e], kx[u][e], d);
#pragma unroll
        for (int off = LPR / 2; off >= 1; off >>= 1) d += __shfl_xor(d, off);
        sc[u] = row < hi && row != slot ? d : -INFINITY;
      }
    }
    float bm = mx;
#pragma unroll
    for (int u = 0; u < U; ++u) bm = fmaxf(bm, sc[u]);
    const float alpha = __builtin_amdgcn_exp2f(mx - bm);
    mx = bm;
    ls *= alpha;
#pragma unroll
    for (int e = 0; e < E; ++e) o[e] *= alpha;
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const float pu = __builtin_amdgcn_exp2f(sc[u] - bm);
      ls += pu;
#pragma unroll
      for (int e = 0; e < E; ++e) o[e] = fmaf(pu, vx[u][e], o[e]);
    }
  }
  // merge the RPI lane groups of the wave (lanes with the same piece c)
#pragma unroll
  for (int off = LPR; off < 64; off <<= 1) {
    const float m2 = __shfl_xor(mx, off), l2 = __shfl_xor(ls, off);
    const float mn = fmaxf(mx, m2);
    const float a1 = __builtin_amdgcn_exp2f(mx - mn), a2 = __builtin_amdgcn_exp2f(m2 - mn);
    ls = ls * a1 + l2 * a2;
#pragma unroll
    for (int e = 0; e < E; ++e) o[e] = o[e] * a1 + __shfl_xor(o[e], off) * a2;
    mx = mn;
  }
  if (rs == 0) {
#pragma unroll
    for (int e = 0; e < E; ++e) sO[w][c * E + e] = o[e];
  }
  if (l == 0) {
    sMw[w] = mx;
    sLw[w] = ls;
  }
  __syncthreads();
  if (t < D) {
    // L2 read: the partial sums of the pass over A
    constexpr int ncg = D / 4, rpp = 256 / ncg;
    const float4* pf = part;
    float mt = 0.f;
    for (int j = 0; j < rpp; ++j) {
      const float4 x = pf[j * ncg + t / 4];
      mt += (t & 3) == 0 ? x.x : (t & 3) == 1 ? x.y : (t & 3) == 2 ? x.z : x.w;
    }
    sm[t] = mt;
  }
  // score of the current token (every thread forms it from LDS)
  float scur = 0.f;
#pragma unroll 8
  for (int e = 0; e < D; ++e) scur = fmaf(sq[e] * sl2, skn[e], scur);
  __syncthreads();
  if (t < D) {
    float mm = scur;
#pragma unroll
    for (int j = 0; j < 4; ++j) mm = fmaxf(mm, sMw[j]);
    const float acur = __builtin_amdgcn_exp2f(scur - mm);
    float num = acur * svn[t], den = acur;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float aj = __builtin_amdgcn_exp2f(sMw[j] - mm);
      num = fmaf(aj, sO[j][t], num);
      den = fmaf(aj, sLw[j], den);
    }
    const float gate = 1.f / (1.f + expf(-g[h]));
    y[(long)bh * D + t] = num / den + gate * sm[t];
  }
}

}  // namespace

hipError_t launch_tc_decode_layer(const void* q, const void* k, const void* v, bool bf16,
                                  void* ring_k, void* ring_v, float* A, const float* lam,
                                  const float* eta, const float* g, const int64_t* pos, int B,
                                  int H, int d, int W, float scale, float* y, hipStream_t s) {
  const dim3 grid(B * H), block(256);
  const float sl2 = scale * 1.4426950408889634f;
#define TC_DL(TI, DD)                                                                          \
  hipLaunchKernelGGL((decode_layer_kernel<TI, DD>), grid, block, 0, s,                          \
                     static_cast<const TI*>(q), static_cast<const TI*>(k),                     \
                     static_cast<const TI*>(v), static_cast<TI*>(ring_k), static_cast<TI*>(ring_v), \
                     A, lam, eta, g, pos, H, W, sl2, y)
  profile_mark_before(s);
  if (bf16) {
    switch (d) {
      case 16: TC_DL(uint16_t, 16); break;
      case 32: TC_DL(uint16_t, 32); break;
      case 64: TC_DL(uint16_t, 64); break;
      case 128: TC_DL(uint16_t, 128); break;
      default: return hipErrorInvalidValue;
    }
  } else {
    switch (d) {
      case 16: TC_DL(float, 16); break;
      case 32: TC_DL(float, 32); break;
      case 64: TC_DL(float, 64); break;
      case 128: TC_DL(float, 128); break;
      default: return hipErrorInvalidValue;
    }
  }
#undef TC_DL
  profile_mark_after(s);
  return hipGetLastError();
}

hipError_t launch_tc_decode(const void* q, const void* k, const void* v, bool bf16, void* ring_k,
                            void* ring_v, float* A, const float* lam, const float* eta,
                            const int64_t* pos, int B, int H, int dk, int dv, int W, float* m,
                            hipStream_t s) {
  const dim3 grid(B * H), block(256);
  profile_mark_before(s);
  if (dk == 128 && dv == 128) {
    // more A than half the 256 MB Infinity Cache: stream it (see decode_kernel_128)
    const bool stream = (size_t)B * H * dk * dv * sizeof(float) > ((size_t)128 << 20);
    if (bf16) {
      const auto* Q = static_cast<const uint16_t*>(q);
      const auto* K = static_cast<const uint16_t*>(k);
      const auto* V = static_cast<const uint16_t*>(v);
      auto* RK = static_cast<uint16_t*>(ring_k);
      auto* RV = static_cast<uint16_t*>(ring_v);
      if (stream)
        hipLaunchKernelGGL((decode_kernel_128<uint16_t, true>), grid, block, 0, s, Q, K, V, RK, RV, A, lam, eta,
                           pos, H, W, m);
      else
        hipLaunchKernelGGL((decode_kernel_128<uint16_t, false>), grid, block, 0, s, Q, K, V, RK, RV, A, lam, eta,
                           pos, H, W, m);
    } else {
      const auto* Q = static_cast<const float*>(q);
      const auto* K = static_cast<const float*>(k);
      const auto* V = static_cast<const float*>(v);
      auto* RK = static_cast<float*>(ring_k);
      auto* RV = static_cast<float*>(ring_v);
      if (stream)
        hipLaunchKernelGGL((decode_kernel_128<float, true>), grid, block, 0, s, Q, K, V, RK, RV, A, lam, eta, pos,
                           H, W, m);
      else
        hipLaunchKernelGGL((decode_kernel_128<float, false>), grid, block, 0, s, Q, K, V, RK, RV, A, lam, eta, pos,
                           H, W, m);
    }
  } else if (bf16) {
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

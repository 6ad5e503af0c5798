// tc_fused.hip — fused Tensor Cache layer (gfx950, bf16 inputs, fp32 state):
// pre-pass, state prefix and launch of the main kernel (tc_swa.hip).
//
// Tensor Cache, Methodology 1: a token leaves the L1 window exactly when it
// is written into the L2 matrix, A <- lam A + eta k v^T; Methodology 2
// evaluates the L2 part in chunk form.  Here the chunks are the 256-query
// tiles of the main kernel: tile p writes the evictions of the keys
// [256 p - W, 256 (p+1) - W) clipped to [0, T - W).
//
// Launches (all on the caller's stream):
//   state_tile    per (tile, b, h): the tile's own contribution to the
//                 state, from zero, delta_p = sum_c eta lam^(L-1-c) v_c k_c^T
//                 (S^T layout, bf16 MFMA with fp32 accumulation, stored as
//                 bf16);
//   fused_prefix  S_0 = 0, S_{p+1} = lam^L_p S_p + delta_p, carried in fp32:
//                 the state entering every tile (bf16) and the final state A
//                 (fp32);
//   swa           per (tile, b, h): window softmax plus the L2 read.
// Workspace: delta (bf16) | entering states (bf16).
#include "tc_common.hpp"
#include "tc_kernels.hpp"
#include "tc_bwd_paths.hpp"
#include "tc_mfma.hpp"
#include "tc_dma.hpp"
#include "tc_tr.hpp"

#include <math.h>

#include <algorithm>

namespace tc {

namespace {

using namespace mf;
using dma::dma16;
using dma::i32x4;
using dma::raw_desc;

constexpr int NWAVE = 8;
constexpr int NTHR = 64 * NWAVE;
constexpr int MQ = 32 * NWAVE;  // queries per tile (must match the main kernel)
constexpr int kComputeUnits = 256;

// Tiles and their evictions: tile p (queries 256 p ..) writes the keys
// [256 p - W, 256 (p + 1) - W) clipped to [0, T - W) into the L2 memory.
struct FusedGeom {
  int T, W, n_tiles;
  __host__ __device__ int key_begin(int p) const {
    const long a = (long)MQ * p - W;
    return (int)(a < 0 ? 0 : a);
  }
  __host__ __device__ int key_end(int p) const {
    long b = (long)MQ * (p + 1) - W;
    const long lim = (long)T - W;
    if (b > lim) b = lim;
    return (int)(b < 0 ? 0 : b);
  }
};

// ---------------------------------------------------------------------------
// Pre-pass.  Workgroup (tile p, b, h), four waves: the tile's own contribution
// to the state, from zero,
//   delta_p^T = sum_{j in [a_p, e_p)} eta lam^(e_p - 1 - j) v_j k_j^T   (D x D, [dv][dk]),
// over its at most 256 evictions in 64-key blocks.  K and V rows travel
// global -> LDS by buffer_load ... lds in the row layout of tc_tr.hpp, and
// both MFMA operands are transpose reads of those rows:
// A = (w V)^T, the weights w_j = eta lam^(e_p - 1 - j) applied in registers
// and rounded to bf16 (keys past e_p weigh 0), and B = K.  Wave w owns the
// 32x32 output tiles w TPW .. w TPW + TPW - 1 (row-major over the D/32 x D/32
// tiles: one row of tiles at d = 128).  delta leaves through LDS as bf16
// rows, 16 bytes per lane.
constexpr int PW = 4;  // waves per pre-pass workgroup
constexpr int PTHR = 64 * PW;
// LDS stages per workgroup.  One (32 KiB at d = 128) lets five workgroups
// share a CU, whose copies and waits overlap; same-box timings at B=1 H=16
// T=32768 d=128 W=1024: 62 us with one stage, 65 us with two (two
// workgroups per CU), 107 us with four (a tile's blocks all in flight, one
// workgroup per CU).
constexpr int PSTG = 1;

template <int D>
struct PrepLds {
  uint16_t k[PSTG][KB * D];
  uint16_t v[PSTG][KB * D];
};

// wait until at most n blocks (2 NS copies each) are still in flight
template <int NS>
__device__ __forceinline__ void wait_blocks(int n) {
  switch (n) {
    case 0: wait_vmcnt<0>(); break;
    case 1: wait_vmcnt<2 * NS>(); break;
    case 2: wait_vmcnt<4 * NS>(); break;
    default: wait_vmcnt<6 * NS>(); break;
  }
}

// One 16-key step of a block: acc[i] += (w V)^T K over keys jb + 16 KK ..
template <int D, int KK, int TPW>
__device__ __forceinline__ void prep_step(const char* sk, const char* sv, uint32_t vl, const uint32_t* kl,
                                          int jb, int e, float et, const Decay& dec, floatx16* acc) {
  const int hh = lane_id() >> 5;
  u32x4 u = __builtin_bit_cast(u32x4, tr::ld1<D, KK>(sv, vl));  // keys j .. j + 7 of one feature
  const int j = jb + 16 * KK + 8 * hh;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int j0 = j + 2 * q, j1 = j0 + 1;
    const float w0 = j0 < e ? et * dec(e - 1 - j0) : 0.f;
    const float w1 = j1 < e ? et * dec(e - 1 - j1) : 0.f;
    u[q] = cvt_pk(lo_f(u[q]) * w0, hi_f(u[q]) * w1);
  }
  const bf16x8 xa = __builtin_bit_cast(bf16x8, u);
#pragma unroll
  for (int i = 0; i < TPW; ++i) acc[i] = mfma32(xa, tr::ld1<D, KK>(sk, kl[i]), acc[i]);
}

template <int D>
__global__ __launch_bounds__(PTHR) void state_tile_kernel(const uint16_t* __restrict__ k,
                                                          const uint16_t* __restrict__ v,
                                                          const float* __restrict__ lam,
                                                          const float* __restrict__ eta, int H, FusedGeom G,
                                                          uint16_t* __restrict__ ws_state) {
  constexpr int NT = D / 32;             // 32-wide tiles per dimension
  constexpr int TPW = NT * NT / PW;      // output tiles per wave: 4 (d = 128), 1 (d = 64)
  constexpr int NS = KB * D / 8 / PTHR;  // 16-byte copies per thread and block, K and V each
  static_assert(sizeof(PrepLds<D>) >= sizeof(uint16_t) * D * D, "delta staging fits in the stages");
  __shared__ __attribute__((aligned(16))) PrepLds<D> lds;
  const int p = blockIdx.x, bh = blockIdx.y;
  const int w = wave_id(), l = lane_id(), col = l & 31, hh = l >> 5;
  const int a = G.key_begin(p), e = G.key_end(p);
  const int t0 = w * TPW, dvt = t0 / NT;  // this wave's tiles share one row of tiles
  floatx16 acc[TPW];
#pragma unroll
  for (int i = 0; i < TPW; ++i) acc[i] = zero16();

  if (e > a) {
    const long base = (long)bh * G.T;
    const i32x4 rk = raw_desc(k + base * D, (uint32_t)G.T * D * 2);
    const i32x4 rv = raw_desc(v + base * D, (uint32_t)G.T * D * 2);
    int src[NS];
#pragma unroll
    for (int i = 0; i < NS; ++i) src[i] = tr::slot_src<D>((i * PW + w) * 64 + l);
    // block b (keys a + 64 b ..; rows past T read as zero) into stage b % PSTG
    auto copy = [&](int b) __attribute__((always_inline)) {
      const int off = (a + KB * b) * D * 2;
#pragma unroll
      for (int i = 0; i < NS; ++i) dma16(rk, lds.k[b % PSTG] + (i * PW + w) * 512, src[i] + off);
#pragma unroll
      for (int i = 0; i < NS; ++i) dma16(rv, lds.v[b % PSTG] + (i * PW + w) * 512, src[i] + off);
    };
    const uint32_t vl = tr::lane_offset<D>(dvt);
    uint32_t kl[TPW];
#pragma unroll
    for (int i = 0; i < TPW; ++i) kl[i] = tr::lane_offset<D>((t0 + i) % NT);
    const Decay dec(lam[bh % H]);
    const float et = eta[bh % H];
    const int nblk = (e - a + KB - 1) / KB;  // 1 .. 4
#pragma unroll 1
    for (int b = 0; b < nblk && b < PSTG; ++b) copy(b);
#pragma unroll 1
    for (int b = 0; b < nblk; ++b) {
      // block b has landed (the blocks issued after it may still be in flight) and is visible to every wave
      wait_blocks<NS>(min(nblk - 1, b + PSTG - 1) - b);
      lds_barrier();
      const char* sk = reinterpret_cast<const char*>(lds.k[b % PSTG]);
      const char* sv = reinterpret_cast<const char*>(lds.v[b % PSTG]);
      const int jb = a + KB * b;
      prep_step<D, 0, TPW>(sk, sv, vl, kl, jb, e, et, dec, acc);
      prep_step<D, 1, TPW>(sk, sv, vl, kl, jb, e, et, dec, acc);
      prep_step<D, 2, TPW>(sk, sv, vl, kl, jb, e, et, dec, acc);
      prep_step<D, 3, TPW>(sk, sv, vl, kl, jb, e, et, dec, acc);
      if (b + PSTG < nblk) {
        lds_barrier();  // every wave is done with this stage before it is refilled
        copy(b + PSTG);
      }
    }
    lds_barrier();  // ... and before the stages hold delta below
  }

  // delta as bf16 [dv][dk] rows through LDS, then 16 bytes per lane
  uint16_t* stage = reinterpret_cast<uint16_t*>(&lds);
#pragma unroll
  for (int i = 0; i < TPW; ++i) {
    const int dk = 32 * ((t0 + i) % NT) + col;
#pragma unroll
    for (int r = 0; r < 16; ++r) stage[(32 * dvt + 8 * (r >> 2) + 4 * hh + (r & 3)) * D + dk] = f32_to_bf16(acc[i][r]);
  }
  lds_barrier();
  uint4* out = reinterpret_cast<uint4*>(ws_state + ((long)bh * G.n_tiles + p) * D * D);
  const uint4* st = reinterpret_cast<const uint4*>(stage);
#pragma unroll
  for (int c = threadIdx.x; c < D * D / 8; c += PTHR) out[c] = st[c];
}

// S_0 = 0, S_{p+1} = lam^len(p) S_p + delta_p, carried in fp32 (delta_p is
// stored as bf16); element idx = dv * D + dk of S^T, four consecutive
// elements per thread.  Entering states go out as bf16 (round to nearest
// even), the final state as fp32 A[dk][dv].
__global__ void fused_prefix_kernel(const float* __restrict__ lam, int H, int D, FusedGeom G,
                                    const uint16_t* __restrict__ delta, uint16_t* __restrict__ sst,
                                    float* __restrict__ A_final) {
  const int n_el = D * D, n4 = n_el / 4;
  const int i4 = blockIdx.x * blockDim.x + threadIdx.x;
  const int bh = blockIdx.y;
  if (i4 >= n4) return;
  const Decay dec(lam[bh % H]);
  const uint2* dp = reinterpret_cast<const uint2*>(delta + (long)bh * G.n_tiles * n_el) + i4;
  uint2* sp = reinterpret_cast<uint2*>(sst + (long)bh * G.n_tiles * n_el) + i4;
  float4 run = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll 16
  for (int p = 0; p < G.n_tiles; ++p) {
    sp[(long)p * n4] = make_uint2(pack_bf16x2(run.x, run.y), pack_bf16x2(run.z, run.w));
    const float d = dec(G.key_end(p) - G.key_begin(p));
    const uint2 x = dp[(long)p * n4];
    run = make_float4(fmaf(d, run.x, lo_f(x.x)), fmaf(d, run.y, hi_f(x.x)), fmaf(d, run.z, lo_f(x.y)),
                      fmaf(d, run.w, hi_f(x.y)));
  }
  if (A_final != nullptr) {
    float* af = A_final + (long)bh * n_el;
    const float r4[4] = {run.x, run.y, run.z, run.w};
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const int idx = 4 * i4 + c;
      af[(idx % D) * D + idx / D] = r4[c];
    }
  }
}

// ---------------------------------------------------------------------------
// The L2 read alone (tc_scan_forward with bf16 inputs, d in {64, 128}), on the
// same pre-pass and prefix: per 256-query tile p with entering state S_n
// (bf16 S^T) and evictions k_c, v_c = keys t0 - W + c,
//   m_r = lam^(r+1) q_r S_n + sum_{c <= r} eta lam^(r-c) <q_r, k_c> v_c.
// A workgroup (8 waves) handles one (tile, b, h) at a time; K (256 rows), V^T
// (256 columns, transposed from the V rows on their way to LDS) and S^T are
// staged whole in LDS (160 KiB at d = 128); the pre-pass writes no V^T copy
// here.  v_mfma_f32_16x16x32_bf16 (A: lane m + 16 (k / 8), B: lane
// n + 16 (k / 8), eight consecutive k per lane; D: lane n + 16 (m / 4),
// element m % 4):
//   O^T  = S^T Q^T                         (then column r scaled by lam^(r+1)),
//   P^T  = K Q^T over 32-key steps, masked to c <= r and weighted eta lam^(r-c),
//   O^T += V^T P^T.
// The two 16-key M tiles of a 32-key step take keys 8 (m / 4) + m % 4 (+ 4),
// so that lane (n, g) ends up with keys 8g .. 8g+7 of the step: P^T feeds the
// next MFMA from registers.  A wave owns 32 queries and visits only the steps
// with c <= its last query; the row groups are paired on the SIMDs
// (waves w and w + 4 take groups w and 7 - w) to balance that triangle.
template <int NCH>
__device__ __forceinline__ int rswz(int r) {  // 16-byte chunk swizzle of a row
  return NCH >= 16 ? ((r & 3) | (((r >> 3) & 3) << 2)) : (((r >> 1) & 1) | (((r >> 3) & 3) << 1));
}
template <int NCH>
__device__ __forceinline__ int rpos(int r, int c) {  // element offset of chunk c of row r
  return (r * NCH + (c ^ rswz<NCH>(r))) * 8;
}

// Global operands of one (tile, b, h) unit that go through LDS, in 16-byte
// pieces (every thread the same count): the K rows, loaded one unit ahead,
// and (ReadLateRegs) the V rows and S^T, loaded at the top of the unit.
template <int D>
struct ReadUnitRegs {
  static constexpr int NCK = D / 8, NCV = MQ / 8, NKS = D / 32;
  static constexpr int NLK = MQ * NCK / NTHR, NLS = D * NCK / NTHR;
  static constexpr int NIV = D / 32;  // V items per thread: two keys x 8 columns
  uint4 xk[NLK];
};

// V item u of a thread: keys 2 kp and 2 kp + 1 (kp = 16 w + l % 16, relative
// to the tile's first eviction) at columns 8 ch .. 8 ch + 7 (ch = 4 u + l / 16).
// Stored transposed (S^T-like [d_v][key] layout, key pairs as 4-byte words),
// the 64 lanes of a store hit 64 different banks: the word's bank is
// 4 ((kp / 4) ^ rswz(d_v)) % 16 + kp % 4, and rswz(d_v) carries ch % 4 in its
// upper two bits.
template <int D>
struct ReadLateRegs {
  uint4 xv[2 * ReadUnitRegs<D>::NIV], xs[ReadUnitRegs<D>::NLS];
};

template <int D>
__device__ __forceinline__ void load_read_late(ReadLateRegs<D>& L, const uint16_t* __restrict__ v,
                                               const uint16_t* __restrict__ sst, const FusedGeom& G, int p,
                                               int bh) {
  using RU = ReadUnitRegs<D>;
  const int T = G.T, j0 = MQ * p - G.W;
  const int w = threadIdx.x >> 6, l = threadIdx.x & 63, kp = 16 * w + (l & 15);
#pragma unroll
  for (int u = 0; u < RU::NIV; ++u) {
    const int ch = 4 * u + (l >> 4);
#pragma unroll
    for (int h = 0; h < 2; ++h) {  // keys outside [0, T) read as zero
      const int j = j0 + 2 * kp + h;
      L.xv[2 * u + h] = make_uint4(0u, 0u, 0u, 0u);
      if (j >= 0 && j < T) L.xv[2 * u + h] = *reinterpret_cast<const uint4*>(v + ((long)bh * T + j) * D + 8 * ch);
    }
  }
  const uint16_t* sp = sst + ((long)bh * G.n_tiles + p) * D * D;
#pragma unroll
  for (int u = 0; u < RU::NLS; ++u) {
    const int i = u * NTHR + threadIdx.x;
    L.xs[u] = *reinterpret_cast<const uint4*>(sp + (i / RU::NCK) * D + 8 * (i % RU::NCK));
  }
}

// Q^T operand: lane (n, g) holds q[query][32 ks + 8 g .. + 7]
template <int D>
__device__ __forceinline__ void load_read_q(bf16x8 (&qb)[2][D / 32], const uint16_t* __restrict__ q,
                                            int T, int t0, int bh, int r0) {
  const int l = threadIdx.x & 63, n = l & 15, g = l >> 4;
#pragma unroll
  for (int nt = 0; nt < 2; ++nt) {
    const int t = t0 + r0 + 16 * nt + n;
#pragma unroll
    for (int ks = 0; ks < D / 32; ++ks) {
      uint4 x = make_uint4(0u, 0u, 0u, 0u);
      if (t < T) x = *reinterpret_cast<const uint4*>(q + ((long)bh * T + t) * D + 32 * ks + 8 * g);
      qb[nt][ks] = as_bf16x8(x);
    }
  }
}

template <int D>
__device__ __forceinline__ void load_read_unit(ReadUnitRegs<D>& R, const uint16_t* __restrict__ k,
                                               const FusedGeom& G, int p, int bh) {
  using RU = ReadUnitRegs<D>;
  const int T = G.T, t0 = MQ * p, j0 = t0 - G.W;
#pragma unroll
  for (int u = 0; u < RU::NLK; ++u) {  // K rows c: key j0 + c
    const int i = u * NTHR + threadIdx.x, c = i / RU::NCK, ch = i % RU::NCK, j = j0 + c;
    R.xk[u] = make_uint4(0u, 0u, 0u, 0u);
    if (j >= 0 && j < T) R.xk[u] = *reinterpret_cast<const uint4*>(k + ((long)bh * T + j) * D + 8 * ch);
  }
}

// Persistent: workgroup i takes the units i, i + gridDim.x, ... (unit =
// tile + n_tiles * bh).  The next unit's K rows are loaded before the
// current unit's MFMAs and wait in registers until the LDS is free; V^T, S^T
// and Q are loaded at the top of their unit.  (Loading more of the next unit
// ahead, or loading V^T and S^T ahead of the current unit's stores, made the
// compiler spill: slower.)
// With REV the read of position t is stored in row T - 1 - t of m (a scan of
// time-reversed inputs handing back rows in the original order).
template <int D, bool REV>
__global__ __launch_bounds__(NTHR) void scan_read_kernel(const uint16_t* __restrict__ q,
                                                         const uint16_t* __restrict__ k,
                                                         const uint16_t* __restrict__ v,
                                                         const uint16_t* __restrict__ sst,
                                                         const float* __restrict__ lam,
                                                         const float* __restrict__ eta, int H,
                                                         FusedGeom G, int n_units, float* __restrict__ m) {
  using RU = ReadUnitRegs<D>;
  constexpr int NCK = RU::NCK, NCV = RU::NCV, NKS = RU::NKS;
  __shared__ __attribute__((aligned(16))) uint16_t sK[MQ * D];
  __shared__ __attribute__((aligned(16))) uint16_t sV[D * MQ];
  __shared__ __attribute__((aligned(16))) uint16_t sS[D * D];
  const int T = G.T;
  const int w = threadIdx.x >> 6, l = threadIdx.x & 63, n = l & 15, g = l >> 4;
  const int grp = w < 4 ? w : 11 - w;  // 32-query row group of this wave
  const int r0 = 32 * grp;
  int unit = blockIdx.x;
  if (unit >= n_units) return;  // uniform over the workgroup
  ReadUnitRegs<D> R;
  load_read_unit<D>(R, k, G, unit % G.n_tiles, unit / G.n_tiles);
  for (; unit < n_units; unit += gridDim.x) {
    const int p = unit % G.n_tiles, bh = unit / G.n_tiles, t0 = MQ * p;
    ReadLateRegs<D> L;
    load_read_late<D>(L, v, sst, G, p, bh);
    bf16x8 qb[2][NKS];
    load_read_q<D>(qb, q, T, t0, bh, r0);
    __syncthreads();  // the previous unit's LDS reads are done
#pragma unroll
    for (int u = 0; u < RU::NLK; ++u) {
      const int i = u * NTHR + threadIdx.x;
      *reinterpret_cast<uint4*>(sK + rpos<NCK>(i / NCK, i % NCK)) = R.xk[u];
    }
    {
      const int kp = 16 * w + (l & 15);
#pragma unroll
      for (int u = 0; u < RU::NIV; ++u) {
        const int ch = 4 * u + (l >> 4);
        const uint4 xa = L.xv[2 * u], xb = L.xv[2 * u + 1];
        const uint32_t a[4] = {xa.x, xa.y, xa.z, xa.w}, b[4] = {xb.x, xb.y, xb.z, xb.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int dv = 8 * ch + 2 * e;
          *reinterpret_cast<uint32_t*>(sV + rpos<NCV>(dv, kp >> 2) + 2 * (kp & 3)) = (a[e] & 0xFFFFu) | (b[e] << 16);
          *reinterpret_cast<uint32_t*>(sV + rpos<NCV>(dv + 1, kp >> 2) + 2 * (kp & 3)) =
              (a[e] >> 16) | (b[e] & 0xFFFF0000u);
        }
      }
    }
#pragma unroll
    for (int u = 0; u < RU::NLS; ++u) {
      const int i = u * NTHR + threadIdx.x;
      *reinterpret_cast<uint4*>(sS + rpos<NCK>(i / NCK, i % NCK)) = L.xs[u];
    }
    __syncthreads();
    const int next = unit + gridDim.x;
    if (next < n_units) load_read_unit<D>(R, k, G, next % G.n_tiles, next / G.n_tiles);

    const Decay dec(lam[bh % H]);
    const float et = eta[bh % H];
    floatx4 o[D / 16][2];
    // state term, then column r scaled by lam^(r+1)
#pragma unroll
    for (int mt = 0; mt < D / 16; ++mt) {
      o[mt][0] = zero4();
      o[mt][1] = zero4();
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) {
        const bf16x8 a = as_bf16x8(*reinterpret_cast<const uint4*>(sS + rpos<NCK>(16 * mt + n, 4 * ks + g)));
        o[mt][0] = mfma_bf16_16x16x32(a, qb[0][ks], o[mt][0]);
        o[mt][1] = mfma_bf16_16x16x32(a, qb[1][ks], o[mt][1]);
      }
    }
    {
      const float f0 = dec(r0 + n + 1), f1 = dec(r0 + 16 + n + 1);
#pragma unroll
      for (int mt = 0; mt < D / 16; ++mt) {
        o[mt][0] *= f0;
        o[mt][1] *= f1;
      }
    }
    // evictions of the tile, 32 keys per step, up to this wave's last query
    for (int st = 0; st <= grp; ++st) {
      floatx4 sc[2][2] = {{zero4(), zero4()}, {zero4(), zero4()}};  // [key half][query tile]
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) {
#pragma unroll
        for (int hf = 0; hf < 2; ++hf) {
          const int row = 32 * st + 8 * (n >> 2) + (n & 3) + 4 * hf;
          const bf16x8 a = as_bf16x8(*reinterpret_cast<const uint4*>(sK + rpos<NCK>(row, 4 * ks + g)));
          sc[hf][0] = mfma_bf16_16x16x32(a, qb[0][ks], sc[hf][0]);
          sc[hf][1] = mfma_bf16_16x16x32(a, qb[1][ks], sc[hf][1]);
        }
      }
      bf16x8 pb[2];
#pragma unroll
      for (int nt = 0; nt < 2; ++nt) {
        const int dr = r0 + 16 * nt + n - (32 * st + 8 * g);  // r - c of element (hf, e) is dr - 4 hf - e
        uint32_t pk[4];
#pragma unroll
        for (int hf = 0; hf < 2; ++hf) {
          const floatx4 x = sc[hf][nt];
          const float w0 = dr - 4 * hf >= 0 ? et * dec(dr - 4 * hf) * x[0] : 0.f;
          const float w1 = dr - 4 * hf - 1 >= 0 ? et * dec(dr - 4 * hf - 1) * x[1] : 0.f;
          const float w2 = dr - 4 * hf - 2 >= 0 ? et * dec(dr - 4 * hf - 2) * x[2] : 0.f;
          const float w3 = dr - 4 * hf - 3 >= 0 ? et * dec(dr - 4 * hf - 3) * x[3] : 0.f;
          pk[2 * hf] = cvt_pk(w0, w1);
          pk[2 * hf + 1] = cvt_pk(w2, w3);
        }
        pb[nt] = as_bf16x8(pk[0], pk[1], pk[2], pk[3]);
      }
#pragma unroll
      for (int mt = 0; mt < D / 16; ++mt) {
        const bf16x8 a = as_bf16x8(*reinterpret_cast<const uint4*>(sV + rpos<NCV>(16 * mt + n, 4 * st + g)));
        o[mt][0] = mfma_bf16_16x16x32(a, pb[0], o[mt][0]);
        o[mt][1] = mfma_bf16_16x16x32(a, pb[1], o[mt][1]);
      }
    }
    // O^T element (dv = 16 mt + 4 g + e, query r0 + 16 nt + n)
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) {
      const int t = t0 + r0 + 16 * nt + n;
      if (t >= T) continue;
      float* out = m + ((long)bh * T + (REV ? T - 1 - t : t)) * D + 4 * g;
#pragma unroll
      for (int mt = 0; mt < D / 16; ++mt)
        *reinterpret_cast<float4*>(out + 16 * mt) = make_float4(o[mt][nt][0], o[mt][nt][1], o[mt][nt][2], o[mt][nt][3]);
    }
  }
}

FusedGeom make_geom(int T, int W) {
  FusedGeom G{};
  G.T = T;
  G.W = W;
  G.n_tiles = (T + MQ - 1) / MQ;
  return G;
}

size_t state_elems(const FusedGeom& G, int B, int H, int d) { return (size_t)B * H * G.n_tiles * d * d; }

template <int D>
hipError_t run_fused(const uint16_t* q, const uint16_t* k, const uint16_t* v, const float* lam,
                     const float* eta, const float* g, int B, int H, const FusedGeom& G, float scale,
                     float* y, float* A_final, void* ws, hipStream_t s) {
  const int BH = B * H;
  const size_t ne = state_elems(G, B, H, D);
  uint16_t* delta = static_cast<uint16_t*>(ws);
  uint16_t* sst = delta + ne;
  hipLaunchKernelGGL(state_tile_kernel<D>, dim3(G.n_tiles, BH), dim3(PTHR), 0, s, k, v, lam, eta, H, G, delta);
  hipLaunchKernelGGL(fused_prefix_kernel, dim3((D * D / 4 + 63) / 64, BH), dim3(64), 0, s, lam, H, D,
                     G, delta, sst, A_final);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  profile_mark_before(s);
  const hipError_t e2 = launch_swa(q, k, v, sst, lam, eta, g, B, H, G.T, D, G.W, scale, y, nullptr, s);
  profile_mark_after(s);
  return e2;
}

}  // namespace

template <int D>
hipError_t run_scan_bf16(const uint16_t* q, const uint16_t* k, const uint16_t* v, const float* lam,
                         const float* eta, int B, int H, const FusedGeom& G, float* m, float* A_final, void* ws,
                         bool rev_out, hipStream_t s) {
  const int BH = B * H;
  const size_t ne = state_elems(G, B, H, D);
  uint16_t* delta = static_cast<uint16_t*>(ws);
  uint16_t* sst = delta + ne;
  hipLaunchKernelGGL(state_tile_kernel<D>, dim3(G.n_tiles, BH), dim3(PTHR), 0, s, k, v, lam, eta, H, G, delta);
  hipLaunchKernelGGL(fused_prefix_kernel, dim3((D * D / 4 + 63) / 64, BH), dim3(64), 0, s, lam, H, D,
                     G, delta, sst, A_final);
  profile_mark_before(s);
  // persistent: as many workgroups as fit at once (LDS: one per CU at d = 128, two at d = 64)
  const int n_units = G.n_tiles * BH;
  const int grid = std::min<int>(n_units, kComputeUnits * (D == 128 ? 1 : 2));
  if (rev_out)
    hipLaunchKernelGGL((scan_read_kernel<D, true>), dim3(grid), dim3(NTHR), 0, s, q, k, v, sst, lam, eta, H, G,
                       n_units, m);
  else
    hipLaunchKernelGGL((scan_read_kernel<D, false>), dim3(grid), dim3(NTHR), 0, s, q, k, v, sst, lam, eta, H, G,
                       n_units, m);
  profile_mark_after(s);
  return hipGetLastError();
}

size_t scan_bf16_ws_bytes(int B, int H, int T, int d, int W) {
  return state_elems(make_geom(T, W), B, H, d) * 2 * sizeof(uint16_t);
}

size_t fused_ws_bytes(int B, int H, int T, int dk, int dv, int W) {
  (void)dv;
  return state_elems(make_geom(T, W), B, H, dk) * 2 * sizeof(uint16_t);
}

bool scan_bf16_fast(bool bf16, int dk, int dv, int T) { return bf16 && dk == dv && (dk == 64 || dk == 128) && T > 0; }

static hipError_t scan_bf16(const void* q, const void* k, const void* v, const float* lam, const float* eta, int B,
                            int H, int T, int d, int W, float* m, float* A_final, void* ws, hipStream_t s,
                            bool rev_out) {
  const FusedGeom G = make_geom(T, W);
  const uint16_t* Q = static_cast<const uint16_t*>(q);
  const uint16_t* K = static_cast<const uint16_t*>(k);
  const uint16_t* V = static_cast<const uint16_t*>(v);
  if (d == 128) return run_scan_bf16<128>(Q, K, V, lam, eta, B, H, G, m, A_final, ws, rev_out, s);
  if (d == 64) return run_scan_bf16<64>(Q, K, V, lam, eta, B, H, G, m, A_final, ws, rev_out, s);
  return hipErrorInvalidValue;
}

hipError_t launch_tc_scan_bf16(const void* q, const void* k, const void* v, const float* lam, const float* eta,
                               int B, int H, int T, int d, int W, float* m, float* A_final, void* ws, hipStream_t s) {
  return scan_bf16(q, k, v, lam, eta, B, H, T, d, W, m, A_final, ws, s, false);
}

hipError_t launch_tc_scan_bf16_rev_out(const void* q, const void* k, const void* v, const float* lam,
                                       const float* eta, int B, int H, int T, int d, int W, float* m, float* A_final,
                                       void* ws, hipStream_t s) {
  return scan_bf16(q, k, v, lam, eta, B, H, T, d, W, m, A_final, ws, s, true);
}

hipError_t launch_tc_fused(const void* q, const void* k, const void* v, const float* lam,
                           const float* eta, const float* g, int B, int H, int T, int d, int W,
                           float scale, float* y, float* A_final, void* ws, hipStream_t s) {
  const FusedGeom G = make_geom(T, W);
  const uint16_t* Q = static_cast<const uint16_t*>(q);
  const uint16_t* K = static_cast<const uint16_t*>(k);
  const uint16_t* V = static_cast<const uint16_t*>(v);
  if (d == 128) return run_fused<128>(Q, K, V, lam, eta, g, B, H, G, scale, y, A_final, ws, s);
  if (d == 64) return run_fused<64>(Q, K, V, lam, eta, g, B, H, G, scale, y, A_final, ws, s);
  return hipErrorInvalidValue;
}

}  // namespace tc

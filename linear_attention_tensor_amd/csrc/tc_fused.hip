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
//   fused_state   per (tile, b, h): the tile's own contribution to the
//                 state, from zero, delta_p = sum_c eta lam^(L-1-c) v_c k_c^T
//                 (S^T layout, bf16 MFMA with fp32 accumulation, stored as
//                 bf16); for the layer it also writes V^T (per head [d][Tp]
//                 bf16) into the workspace, so that the main kernel can copy
//                 V^T blocks straight to LDS;
//   fused_prefix  S_0 = 0, S_{p+1} = lam^L_p S_p + delta_p, carried in fp32:
//                 the state entering every tile (bf16) and the final state A
//                 (fp32);
//   swa           per (tile, b, h): window softmax plus the L2 read.
// Workspace: delta (bf16) | entering states (bf16) | V^T copy (bf16, the
// layer only).
#include "tc_common.hpp"
#include "tc_kernels.hpp"
#include "tc_mfma.hpp"

#include <math.h>

#include <algorithm>

namespace tc {

namespace {

using namespace mf;

constexpr int NWAVE = 8;
constexpr int NTHR = 64 * NWAVE;
constexpr int MQ = 32 * NWAVE;  // queries per tile (must match the main kernel)
constexpr long kPrepassWorkgroups = 256;  // MI355X: 256 CUs
constexpr int kComputeUnits = 256;

// Tiles and their evictions; V^T copy geometry.
struct FusedGeom {
  int T, W, n_tiles;
  // V^T copy: key j sits in column j + voff of rows of length Tp; voff = W mod 8
  // puts every main-kernel block (first key t0 - W) on a 16-byte boundary.
  int voff, Tp;
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
  // copy columns the pre-pass visits for tile p (keys are column - voff): at
  // least one 64-column block; with the copy, the last tile runs to Tp, and
  // together the tiles cover every column of the copy.
  __host__ __device__ int col_begin(int p) const { return (key_begin(p) + voff) & ~(KB - 1); }
  __host__ __device__ int col_end(int p) const {
    const int e = (vt_copy && p == n_tiles - 1) ? Tp : ((key_end(p) + voff + KB - 1) & ~(KB - 1));
    return e > col_begin(p) ? e : col_begin(p) + KB;
  }
  int tiles_per_seg;  // tiles one pre-pass workgroup walks through
  int vt_copy;        // 1: the pre-pass writes the V^T copy
};

// Distribution of the fp32 state S^T (D x D, 32x32 tiles) over the waves.
template <int D>
struct StateTiles {
  static constexpr int NST = (D / 32) * (D / 32);
  static constexpr int TPW = NST >= NWAVE ? NST / NWAVE : 1;
  __device__ static bool owns(int w, int i) { return w * TPW + i < NST; }
  __device__ static int dv0(int w, int i) { return 32 * ((w * TPW + i) / (D / 32)); }
  __device__ static int dk0(int w, int i) { return 32 * ((w * TPW + i) % (D / 32)); }
};

// Pre-pass piece: rows r, r+1 of K and V at 8 consecutive columns.  Lane l of
// wave w takes the row pair l % 16 (+16 for odd waves) and the column group
// 4 (w / 2) + l / 16, so each 4-byte LDS store of the transposed pieces hits
// 64 different banks.
struct PairRegs {
  uint4 k0, k1, v0, v1;
};

template <int D>
__device__ __forceinline__ void pair_piece(int& r, int& c8) {
  const int t = threadIdx.x, l = t & 63, w = t >> 6;
  r = 2 * (l & 15) + 32 * (w & 1);
  c8 = 8 * (4 * (w >> 1) + (l >> 4));
  if (c8 >= D) c8 = 0;  // threads without a piece (D < 128) still address valid memory
}

// rows j + row, j + row + 1 (j may be negative: those rows read as zero)
template <int D>
__device__ __forceinline__ PairRegs load_pair(__amdgpu_buffer_rsrc_t rk, __amdgpu_buffer_rsrc_t rv, int j) {
  int row, c8;
  pair_piece<D>(row, c8);
  PairRegs p;
  p.k0 = buf_load16(rk, ((j + row) * D + c8) * 2);
  p.v0 = buf_load16(rv, ((j + row) * D + c8) * 2);
  p.k1 = buf_load16(rk, ((j + row + 1) * D + c8) * 2);
  p.v1 = buf_load16(rv, ((j + row + 1) * D + c8) * 2);
  return p;
}

// K^T and (w V)^T of one block into LDS (keys contiguous, 34-word rows), and
// the raw V^T into the global copy.  The block holds keys col - voff for the
// copy's columns col = jc .. jc+63 (jc a multiple of 64, so the 4-byte key
// pair stores are aligned); w_j = eta lam^(wend-1-j) on [wbeg, wend).
template <int D, int SKT>
__device__ __forceinline__ void store_pair(const PairRegs& p, uint16_t* skt, uint16_t* svt,
                                           uint16_t* __restrict__ vt_out, int Tp, int jc, int voff,
                                           int wbeg, int wend, float et, const Decay& dec) {
  if (threadIdx.x >= 32 * (D / 8)) return;
  int row, c8;
  pair_piece<D>(row, c8);
  const int cc = jc + row;      // copy column of the first key of the pair
  const int jj = cc - voff;     // that key
  const float w0 = (jj >= wbeg && jj < wend) ? et * dec(wend - 1 - jj) : 0.f;
  const float w1 = (jj + 1 >= wbeg && jj + 1 < wend) ? et * dec(wend - 2 - jj) : 0.f;
  const uint32_t ka[4] = {p.k0.x, p.k0.y, p.k0.z, p.k0.w}, kb[4] = {p.k1.x, p.k1.y, p.k1.z, p.k1.w};
  const uint32_t va[4] = {p.v0.x, p.v0.y, p.v0.z, p.v0.w}, vb[4] = {p.v1.x, p.v1.y, p.v1.z, p.v1.w};
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const uint32_t vlo = (va[e] & 0xFFFFu) | (vb[e] << 16), vhi = (va[e] >> 16) | (vb[e] & 0xFFFF0000u);
    *reinterpret_cast<uint32_t*>(skt + (c8 + 2 * e) * SKT + row) = (ka[e] & 0xFFFFu) | (kb[e] << 16);
    *reinterpret_cast<uint32_t*>(skt + (c8 + 2 * e + 1) * SKT + row) = (ka[e] >> 16) | (kb[e] & 0xFFFF0000u);
    *reinterpret_cast<uint32_t*>(svt + (c8 + 2 * e) * SKT + row) = cvt_pk(lo_f(va[e]) * w0, lo_f(vb[e]) * w1);
    *reinterpret_cast<uint32_t*>(svt + (c8 + 2 * e + 1) * SKT + row) = cvt_pk(hi_f(va[e]) * w0, hi_f(vb[e]) * w1);
    if (vt_out != nullptr && cc < Tp) {  // cc is even and Tp a multiple of 64: the pair is in range
      *reinterpret_cast<uint32_t*>(vt_out + (long)(c8 + 2 * e) * Tp + cc) = vlo;
      *reinterpret_cast<uint32_t*>(vt_out + (long)(c8 + 2 * e + 1) * Tp + cc) = vhi;
    }
  }
}

// acc (this wave's S^T tiles) += (w V)^T K over one 64-key block in LDS
template <int D, int SKT>
__device__ __forceinline__ void state_block_mma(floatx16* acc, const uint16_t* sKt, const uint16_t* sVt) {
  using ST = StateTiles<D>;
  const int w = wave_id(), l = lane_id(), col = l & 31, hh = l >> 5;
#pragma unroll
  for (int i = 0; i < ST::TPW; ++i) {
    if (!ST::owns(w, i)) continue;
    const int dv0 = ST::dv0(w, i), dk0 = ST::dk0(w, i);
#pragma unroll
    for (int ks = 0; ks < KB / 16; ++ks) {
      const int kb = 16 * ks + 8 * hh;
      const uint2 a0 = *reinterpret_cast<const uint2*>(sVt + (dv0 + col) * SKT + kb);
      const uint2 a1 = *reinterpret_cast<const uint2*>(sVt + (dv0 + col) * SKT + kb + 4);
      const uint2 b0 = *reinterpret_cast<const uint2*>(sKt + (dk0 + col) * SKT + kb);
      const uint2 b1 = *reinterpret_cast<const uint2*>(sKt + (dk0 + col) * SKT + kb + 4);
      acc[i] = mfma32(as_bf16x8(a0.x, a0.y, a1.x, a1.y), as_bf16x8(b0.x, b0.y, b1.x, b1.y), acc[i]);
    }
  }
}

// A tile's delta (this wave's S^T tiles) into the workspace as bf16.  At
// d = 128 a wave's two 32x32 tiles cover the same rows and adjacent column
// blocks (dk0, dk0 + 32): the two halves of the wave trade values (lane
// c <-> c + 32), so that each store writes 64 consecutive columns (128 bytes)
// of one row instead of 32.
template <int D>
__device__ __forceinline__ void store_delta(uint16_t* __restrict__ out, const floatx16* acc) {
  using ST = StateTiles<D>;
  const int w = wave_id(), l = lane_id(), col = l & 31, hh = l >> 5;
  if constexpr (ST::TPW == 2) {
    const int dv0 = ST::dv0(w, 0), dk0 = ST::dk0(w, 0);  // tile 1: same rows, columns dk0 + 32 ..
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const float a0 = acc[0][e], a1 = acc[1][e];
      const float s0 = __shfl_xor(a0, 32), s1 = __shfl_xor(a1, 32);
      const int ra = dv0 + 8 * (e >> 2) + (e & 3);  // row of element e in the lower half
      uint16_t* p = out + ra * D + dk0 + 32 * hh + col;
      p[0] = f32_to_bf16(hh ? s1 : a0);      // row ra
      p[4 * D] = f32_to_bf16(hh ? a1 : s0);  // row ra + 4
    }
  } else {
#pragma unroll
    for (int i = 0; i < ST::TPW; ++i) {
      if (!ST::owns(w, i)) continue;
      const int dv0 = ST::dv0(w, i), dk0 = ST::dk0(w, i);
#pragma unroll
      for (int e = 0; e < 16; ++e) out[(dv0 + 8 * (e >> 2) + 4 * hh + (e & 3)) * D + dk0 + col] = f32_to_bf16(acc[i][e]);
    }
  }
}

// Next (tile, column block) of a pre-pass walk: every tile has >= 1 block.
__device__ __forceinline__ void next_block(const FusedGeom& G, int& p, int& j) {
  j += KB;
  if (j >= G.col_end(p)) {
    ++p;
    j = G.col_begin(p);
  }
}

// Workgroup (segment, b, h) walks tiles_per_seg consecutive tiles.  For each
// tile p: the contribution of its evictions to the state, from zero,
// delta_p = sum_j eta lam^(b_p - 1 - j) v_j k_j^T over [a_p, b_p), and the
// V^T copy of its column blocks (keys outside [0, T) written as zero).  The
// blocks of all the segment's tiles form one stream with three blocks in
// flight in registers.
template <int D>
__global__ __launch_bounds__(NTHR) void fused_state_kernel(const uint16_t* __restrict__ k,
                                                           const uint16_t* __restrict__ v,
                                                           const float* __restrict__ lam,
                                                           const float* __restrict__ eta, int H,
                                                           FusedGeom G, uint16_t* __restrict__ ws_state,
                                                           uint16_t* __restrict__ ws_vt) {
  constexpr int SKT = KB + 4;  // K^T and V^T rows: keys contiguous, 34-word stride
  __shared__ __attribute__((aligned(16))) uint16_t sKt[D * SKT];
  __shared__ __attribute__((aligned(16))) uint16_t sVt[D * SKT];
  using ST = StateTiles<D>;
  const int bh = blockIdx.y;
  const int p_begin = blockIdx.x * G.tiles_per_seg;
  const int p_end = min(p_begin + G.tiles_per_seg, G.n_tiles);
  const Decay dec(lam[bh % H]);
  const float et = eta[bh % H];
  const long base = (long)bh * G.T;
  const int voff = G.voff;
  uint16_t* vt_out = G.vt_copy ? ws_vt + (long)bh * D * G.Tp : nullptr;
  const __amdgpu_buffer_rsrc_t rk = make_rsrc(k + base * D, (uint32_t)G.T * D * 2);
  const __amdgpu_buffer_rsrc_t rv = make_rsrc(v + base * D, (uint32_t)G.T * D * 2);

  floatx16 acc[ST::TPW];
#pragma unroll
  for (int i = 0; i < ST::TPW; ++i) acc[i] = zero16();

  // compute cursor (pc, jc) and load cursor (pl, jl), three blocks apart.
  // r0, r1, r2 keep fixed roles (a register that is the target of a load in
  // flight is never copied) and the loads are issued on every path, so their
  // count is the same everywhere; loads past the segment read zeros or data
  // that is not used.
  int pc = p_begin, jc = G.col_begin(pc);
  int pl = pc, jl = jc;
  PairRegs r0 = load_pair<D>(rk, rv, jl - voff);
  next_block(G, pl, jl);
  PairRegs r1 = load_pair<D>(rk, rv, jl - voff);
  next_block(G, pl, jl);
  PairRegs r2 = load_pair<D>(rk, rv, jl - voff);
  next_block(G, pl, jl);
#define TC_STATE_STEP(R)                                                              \
  if (pc < p_end) {                                                                   \
    lds_barrier();                                                                    \
    store_pair<D, SKT>(R, sKt, sVt, vt_out, G.Tp, jc, voff, G.key_begin(pc),          \
                       G.key_end(pc), et, dec);                                       \
    lds_barrier();                                                                    \
  }                                                                                   \
  R = load_pair<D>(rk, rv, jl - voff);                                                \
  next_block(G, pl, jl);                                                              \
  if (pc < p_end) {                                                                   \
    state_block_mma<D, SKT>(acc, sKt, sVt);                                           \
    if (jc + KB >= G.col_end(pc)) {                                                   \
      store_delta<D>(ws_state + ((long)bh * G.n_tiles + pc) * D * D, acc);            \
      _Pragma("unroll") for (int i = 0; i < ST::TPW; ++i) acc[i] = zero16();          \
    }                                                                                 \
    next_block(G, pc, jc);                                                            \
  }
  while (pc < p_end) {
    TC_STATE_STEP(r0)
    TC_STATE_STEP(r1)
    TC_STATE_STEP(r2)
  }
#undef TC_STATE_STEP
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
template <int D>
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
      float* out = m + ((long)bh * T + t) * D + 4 * g;
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
  G.voff = W & 7;
  G.Tp = (T + G.voff + KB - 1) / KB * KB;
  G.n_tiles = (T + MQ - 1) / MQ;
  G.tiles_per_seg = 1;
  G.vt_copy = 1;
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
  uint16_t* vt = sst + ne;
  // about one pre-pass workgroup per CU, each streaming several tiles
  FusedGeom Gs = G;
  const long units = (long)G.n_tiles * BH;
  Gs.tiles_per_seg = (int)std::max<long>(1, (units + kPrepassWorkgroups - 1) / kPrepassWorkgroups);
  const int n_seg = (G.n_tiles + Gs.tiles_per_seg - 1) / Gs.tiles_per_seg;
  hipLaunchKernelGGL(fused_state_kernel<D>, dim3(n_seg, BH), dim3(NTHR), 0, s, k, v, lam, eta, H, Gs,
                     delta, vt);
  hipLaunchKernelGGL(fused_prefix_kernel, dim3((D * D / 4 + 63) / 64, BH), dim3(64), 0, s, lam, H, D,
                     G, delta, sst, A_final);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  profile_mark_before(s);
  const hipError_t e2 = launch_swa(q, k, vt, sst, lam, eta, g, B, H, G.T, D, G.W, G.Tp, G.voff, scale, y, s);
  profile_mark_after(s);
  return e2;
}

}  // namespace

template <int D>
hipError_t run_scan_bf16(const uint16_t* q, const uint16_t* k, const uint16_t* v, const float* lam,
                         const float* eta, int B, int H, const FusedGeom& G, float* m, float* A_final, void* ws,
                         hipStream_t s) {
  const int BH = B * H;
  const size_t ne = state_elems(G, B, H, D);
  uint16_t* delta = static_cast<uint16_t*>(ws);
  uint16_t* sst = delta + ne;
  // the read kernel transposes V itself: no V^T copy
  FusedGeom Gs = G;
  Gs.vt_copy = 0;
  const long units = (long)G.n_tiles * BH;
  Gs.tiles_per_seg = (int)std::max<long>(1, (units + kPrepassWorkgroups - 1) / kPrepassWorkgroups);
  const int n_seg = (G.n_tiles + Gs.tiles_per_seg - 1) / Gs.tiles_per_seg;
  hipLaunchKernelGGL(fused_state_kernel<D>, dim3(n_seg, BH), dim3(NTHR), 0, s, k, v, lam, eta, H, Gs,
                     delta, static_cast<uint16_t*>(nullptr));
  hipLaunchKernelGGL(fused_prefix_kernel, dim3((D * D / 4 + 63) / 64, BH), dim3(64), 0, s, lam, H, D,
                     G, delta, sst, A_final);
  profile_mark_before(s);
  // persistent: as many workgroups as fit at once (LDS: one per CU at d = 128, two at d = 64)
  const int n_units = G.n_tiles * BH;
  const int grid = std::min<int>(n_units, kComputeUnits * (D == 128 ? 1 : 2));
  hipLaunchKernelGGL(scan_read_kernel<D>, dim3(grid), dim3(NTHR), 0, s, q, k, v, sst, lam, eta, H, G, n_units, m);
  profile_mark_after(s);
  return hipGetLastError();
}

size_t scan_bf16_ws_bytes(int B, int H, int T, int d, int W) {
  return state_elems(make_geom(T, W), B, H, d) * 2 * sizeof(uint16_t);
}

size_t fused_ws_bytes(int B, int H, int T, int dk, int dv, int W) {
  (void)dv;
  const FusedGeom G = make_geom(T, W);
  return state_elems(G, B, H, dk) * 2 * sizeof(uint16_t) +
         (size_t)B * H * dk * G.Tp * sizeof(uint16_t);
}

bool scan_bf16_fast(bool bf16, int dk, int dv, int T) { return bf16 && dk == dv && (dk == 64 || dk == 128) && T > 0; }

hipError_t launch_tc_scan_bf16(const void* q, const void* k, const void* v, const float* lam, const float* eta,
                               int B, int H, int T, int d, int W, float* m, float* A_final, void* ws, hipStream_t s) {
  const FusedGeom G = make_geom(T, W);
  const uint16_t* Q = static_cast<const uint16_t*>(q);
  const uint16_t* K = static_cast<const uint16_t*>(k);
  const uint16_t* V = static_cast<const uint16_t*>(v);
  if (d == 128) return run_scan_bf16<128>(Q, K, V, lam, eta, B, H, G, m, A_final, ws, s);
  if (d == 64) return run_scan_bf16<64>(Q, K, V, lam, eta, B, H, G, m, A_final, ws, s);
  return hipErrorInvalidValue;
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

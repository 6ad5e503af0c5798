// tc_fused.hip — fused Tensor Cache layer (gfx950, bf16 inputs, fp32 state).
//
// Tensor Cache, Methodology 1: the L1 cache answers with exact softmax
// attention over the W most recent tokens (the current one included); a
// token leaves the window exactly when it is written into the L2 matrix,
// A <- lam A + eta k v^T; the L2 read is m_t = q_t A_t; a learned scalar gate
// fuses the two, y_t = y_local,t + sigmoid(g) m_t.  Methodology 2: the L2
// part is evaluated as a chunked weighted-sum scan equal to the sequential
// writes.
//
// Launches (all on the caller's stream):
//   fused_state   per (segment, b, h): the segment's own contribution to the
//                 state, from zero (bf16 MFMA, fp32 accumulation);
//   fused_prefix  entering state of every segment;
//   fused_main    per (segment, b, h): walks the segment's 256-query tiles in
//                 order, carrying the fp32 state S^T = A^T in registers.
// Per tile (t0 = 256 i) the keys are taken in 64-key blocks aligned to
// j0 = t0 - W, so blocks 0-3 hold exactly the tokens evicted while the tile's
// queries are read: with c = j - j0 and r = t - t0, key j is in the query's
// window iff r < c <= r + W, and it has already been evicted iff c <= r.  One
// S^T = K Q^T block product therefore serves both the softmax (c > r) and
// the decayed linear read (c <= r).  Each wave owns 32 queries; S^T tiles come
// from v_mfma_f32_32x32x16_bf16 so that every lane holds one query's scores,
// and the probabilities feed O^T += V^T P^T straight from registers.
//
// Tile epilogue, per L2 chunk of 128 evictions with entering state S_n:
//   O += sigmoid(g) [ sum_{c<=r} eta lam^(r-c) <q_r,k_c> v_c + lam^(r+1) q_r S_n ]
//   S_{n+1} = lam^L S_n + sum_c eta lam^(L-1-c) k_c v_c^T     (L valid evictions)
#include "tc_common.hpp"
#include "tc_kernels.hpp"

#include <math.h>

#include <algorithm>

namespace tc {

namespace {

constexpr int NWAVE = 8;
constexpr int NTHR = 64 * NWAVE;
constexpr int MQ = 32 * NWAVE;  // queries per tile
constexpr int KB = 64;          // keys per block
constexpr int CHK = 128;        // evictions per L2 chunk
constexpr float kNegBig = -1.0e30f;

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ floatx16 mfma32(bf16x8 a, bf16x8 b, floatx16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// two floats -> packed bf16 pair (hardware round-to-nearest-even)
__device__ __forceinline__ uint32_t cvt_pk(float lo, float hi) {
  const f32x2 f = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f, bf16x2));
}

__device__ __forceinline__ bf16x8 as_bf16x8(uint32_t a, uint32_t b, uint32_t c, uint32_t d) {
  return __builtin_bit_cast(bf16x8, u32x4{a, b, c, d});
}

__device__ __forceinline__ float lo_f(uint32_t u) { return __uint_as_float(u << 16); }
__device__ __forceinline__ float hi_f(uint32_t u) { return __uint_as_float(u & 0xFFFF0000u); }

__device__ __forceinline__ floatx16 zero16() {
  floatx16 z;
#pragma unroll
  for (int i = 0; i < 16; ++i) z[i] = 0.f;
  return z;
}

// lam^e for an integer e >= 0 (0^0 = 1, 1^e = 1).
struct Decay {
  float lam, log2lam;
  __device__ __forceinline__ explicit Decay(float l) : lam(l), log2lam(l > 0.f ? log2f(l) : 0.f) {}
  __device__ __forceinline__ float operator()(int e) const {
    if (e == 0) return 1.f;
    if (lam == 0.f) return 0.f;
    return __builtin_amdgcn_exp2f(static_cast<float>(e) * log2lam);
  }
};

template <int D>
struct Lds {
  static constexpr int SK = D + 8;    // bf16 per K row: 16-byte reads, 16 lanes per bank cycle
  static constexpr int SVT = KB + 4;  // bf16 per V^T row: 8-byte reads, 32 lanes per bank cycle
  static constexpr int SSF = D + 4;   // floats per state row
  uint16_t k[2][KB * SK];
  uint16_t vt[2][D * SVT];
  float s[D * SSF];                   // fp32 state S^T = A^T, [dv][dk]
  float w[CHK];
};

// One 64-key block (K and V rows j..j+63) held in registers between its
// global load and its LDS store.  K is copied row-major in 16-byte pieces.
// V is stored transposed: a thread holds rows r, r+1 of 8 consecutive d_v
// columns and writes 4-byte (key pair) words.  Lane l of a wave takes the row
// pair l % 16 and the column group l / 16, so one store instruction touches
// 64 different LDS banks (row stride of V^T: 34 words, 16 column groups of 8
// rows apart = 16 banks).
template <int D>
struct BlockRegs {
  static constexpr int NK = KB * D / 8 / NTHR;  // 16-byte K pieces per thread
  static constexpr int NV = 32 * (D / 8);       // threads that own a V piece pair
  uint4 k[NK], v0, v1;
};

template <int D>
__device__ __forceinline__ void v_piece(int& r, int& c8) {
  const int t = threadIdx.x, l = t & 63, w = t >> 6;
  r = 2 * (l & 15) + 32 * (w & 1);
  c8 = 8 * (4 * (w >> 1) + (l >> 4));
  if (c8 >= D) c8 = 0;  // threads without a piece (D < 128) still address valid memory
}

// rk, rv: buffer resources over this head's K and V rows [0, T)
template <int D>
__device__ __forceinline__ BlockRegs<D> load_block(__amdgpu_buffer_rsrc_t rk, __amdgpu_buffer_rsrc_t rv,
                                                   int j) {
  BlockRegs<D> r;
#pragma unroll
  for (int i = 0; i < BlockRegs<D>::NK; ++i) {
    const int idx = threadIdx.x + i * NTHR;
    const int row = idx / (D / 8), c8 = (idx % (D / 8)) * 8;
    r.k[i] = buf_load16(rk, ((j + row) * D + c8) * 2);
  }
  int row, c8;
  v_piece<D>(row, c8);
  r.v0 = buf_load16(rv, ((j + row) * D + c8) * 2);
  r.v1 = buf_load16(rv, ((j + row + 1) * D + c8) * 2);
  return r;
}

template <int D>
__device__ __forceinline__ void store_block(const BlockRegs<D>& r, uint16_t* sk, uint16_t* svt) {
  using L = Lds<D>;
#pragma unroll
  for (int i = 0; i < BlockRegs<D>::NK; ++i) {
    const int idx = threadIdx.x + i * NTHR;
    const int row = idx / (D / 8), c8 = (idx % (D / 8)) * 8;
    *reinterpret_cast<uint4*>(sk + row * L::SK + c8) = r.k[i];
  }
  if (threadIdx.x < BlockRegs<D>::NV) {
    int row, c8;
    v_piece<D>(row, c8);
    const uint32_t a[4] = {r.v0.x, r.v0.y, r.v0.z, r.v0.w};
    const uint32_t b[4] = {r.v1.x, r.v1.y, r.v1.z, r.v1.w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      // column c8+2e: (row, row+1) low halves; column c8+2e+1: high halves
      *reinterpret_cast<uint32_t*>(svt + (c8 + 2 * e) * L::SVT + row) = (a[e] & 0xFFFFu) | (b[e] << 16);
      *reinterpret_cast<uint32_t*>(svt + (c8 + 2 * e + 1) * L::SVT + row) = (a[e] >> 16) | (b[e] & 0xFFFF0000u);
    }
  }
}

// key offset (within a 64-key block) of element e of S^T tile kt for this lane
__device__ __forceinline__ int key_of(int kt, int e, int hh) {
  return 32 * kt + 8 * (e >> 2) + 4 * hh + (e & 3);
}

// S^T (keys 32kt..32kt+31 of the block x this wave's 32 queries), kt = 0, 1.
template <int D>
__device__ __forceinline__ void block_scores(const uint16_t* sk, const bf16x8* qreg, floatx16* s) {
  using L = Lds<D>;
  const int l = lane_id(), col = l & 31, hh = l >> 5;
#pragma unroll
  for (int kt = 0; kt < 2; ++kt) {
    floatx16 acc = zero16();
    const uint16_t* row = sk + (32 * kt + col) * L::SK + 8 * hh;
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks) {
      const bf16x8 a = *reinterpret_cast<const bf16x8*>(row + 16 * ks);
      acc = mfma32(a, qreg[ks], acc);
    }
    s[kt] = acc;
  }
}

// O^T += V^T P^T for one 64-key block; p holds weights in S^T layout.  The
// B operand of k-step kk takes elements 8(kk%2)..+7 of tile kk/2, i.e. keys
// k0..k0+3 and k0+8..k0+11 with k0 = 32(kk/2) + 16(kk%2) + 4hh; the V^T
// operand reads the same keys.
template <int D>
__device__ __forceinline__ void block_pv(const uint16_t* svt, const floatx16* p, floatx16* o) {
  using L = Lds<D>;
  const int l = lane_id(), col = l & 31, hh = l >> 5;
#pragma unroll
  for (int kk = 0; kk < 4; ++kk) {
    const int kt = kk >> 1, e0 = (kk & 1) * 8;
    const bf16x8 pb = as_bf16x8(cvt_pk(p[kt][e0 + 0], p[kt][e0 + 1]), cvt_pk(p[kt][e0 + 2], p[kt][e0 + 3]),
                                cvt_pk(p[kt][e0 + 4], p[kt][e0 + 5]), cvt_pk(p[kt][e0 + 6], p[kt][e0 + 7]));
    const int k0 = 32 * kt + 2 * e0 + 4 * hh;
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt) {
      const uint16_t* vr = svt + (32 * dt + col) * L::SVT + k0;
      const uint2 a0 = *reinterpret_cast<const uint2*>(vr);
      const uint2 a1 = *reinterpret_cast<const uint2*>(vr + 8);
      o[dt] = mfma32(as_bf16x8(a0.x, a0.y, a1.x, a1.y), pb, o[dt]);
    }
  }
}

// Distribution of the fp32 state S^T (D x D, 32x32 tiles) over the waves.
template <int D>
struct StateTiles {
  static constexpr int NST = (D / 32) * (D / 32);
  static constexpr int TPW = NST >= NWAVE ? NST / NWAVE : 1;
  __device__ static bool owns(int w, int i) { return w * TPW + i < NST; }
  __device__ static int dv0(int w, int i) { return 32 * ((w * TPW + i) / (D / 32)); }
  __device__ static int dk0(int w, int i) { return 32 * ((w * TPW + i) % (D / 32)); }
};

// S^T <- decay S^T + (V^T scaled) K over the 128 keys of two resident blocks.
// The fp32 state lives in LDS; each wave updates its own 32x32 tiles.  V^T
// has already been multiplied by the per-key write weights.
template <int D>
__device__ __forceinline__ void state_update(float* ss, float decay, const uint16_t* sk0,
                                             const uint16_t* svt0, const uint16_t* sk1,
                                             const uint16_t* svt1) {
  using L = Lds<D>;
  using ST = StateTiles<D>;
  const int w = wave_id(), l = lane_id(), col = l & 31, hh = l >> 5;
#pragma unroll
  for (int i = 0; i < ST::TPW; ++i) {
    if (!ST::owns(w, i)) continue;
    const int dv0 = ST::dv0(w, i), dk0 = ST::dk0(w, i);
    float* base = ss + (dv0 + 4 * hh) * L::SSF + dk0 + col;
    floatx16 acc;
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[e] = decay * base[(8 * (e >> 2) + (e & 3)) * L::SSF];
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
      const uint16_t* sk = ks < 4 ? sk0 : sk1;
      const uint16_t* svt = ks < 4 ? svt0 : svt1;
      const int kb = 16 * (ks & 3) + 8 * hh;  // this lane's keys kb..kb+7
      const uint16_t* vr = svt + (dv0 + col) * L::SVT + kb;
      const uint2 a0 = *reinterpret_cast<const uint2*>(vr);
      const uint2 a1 = *reinterpret_cast<const uint2*>(vr + 4);
      const uint16_t* kc = sk + kb * L::SK + dk0 + col;
      uint32_t b[4];
#pragma unroll
      for (int j = 0; j < 4; ++j)
        b[j] = static_cast<uint32_t>(kc[(2 * j) * L::SK]) |
               (static_cast<uint32_t>(kc[(2 * j + 1) * L::SK]) << 16);
      acc = mfma32(as_bf16x8(a0.x, a0.y, a1.x, a1.y), as_bf16x8(b[0], b[1], b[2], b[3]), acc);
    }
#pragma unroll
    for (int e = 0; e < 16; ++e) base[(8 * (e >> 2) + (e & 3)) * L::SSF] = acc[e];
  }
}

// Multiply the V^T columns of two resident blocks by the write weights w[c]
// (c = key index within the 128-key chunk).
template <int D>
__device__ __forceinline__ void scale_vt(uint16_t* svt0, uint16_t* svt1, const float* w) {
  using L = Lds<D>;
  constexpr int PER_BLK = D * (KB / 2);
  for (int idx = threadIdx.x; idx < 2 * PER_BLK; idx += NTHR) {
    const int blk = idx / PER_BLK, rem = idx % PER_BLK;
    const int row = rem / (KB / 2), kp = (rem % (KB / 2)) * 2;
    uint16_t* p = (blk == 0 ? svt0 : svt1) + row * L::SVT + kp;
    const uint32_t u = *reinterpret_cast<uint32_t*>(p);
    *reinterpret_cast<uint32_t*>(p) = cvt_pk(lo_f(u) * w[KB * blk + kp], hi_f(u) * w[KB * blk + kp + 1]);
  }
}

// ---------------------------------------------------------------------------
// Segments: tiles_per_seg consecutive 256-query tiles per workgroup.  Segment p
// owns the evictions [key_begin(p), key_end(p)) its tiles write into A.
struct FusedGeom {
  int T, W, n_tiles, tiles_per_seg, n_seg;
  __host__ __device__ int key_begin(int p) const {
    const long a = (long)MQ * tiles_per_seg * p - W;
    return (int)(a < 0 ? 0 : a);
  }
  __host__ __device__ int key_end(int p) const {
    long b = (long)MQ * tiles_per_seg * (p + 1) - W;
    const long lim = (long)T - W;
    if (b > lim) b = lim;
    return (int)(b < 0 ? 0 : b);
  }
};

// Registers of one 64-key block for the state pass: rows r, r+1 of K and V
// at 8 consecutive columns (the transposed-store piece of v_piece).
struct PairRegs {
  uint4 k0, k1, v0, v1;
};

// rk, rv: buffer resources over this head's K and V rows [0, end)
template <int D>
__device__ __forceinline__ PairRegs load_pair(__amdgpu_buffer_rsrc_t rk, __amdgpu_buffer_rsrc_t rv, int j) {
  int row, c8;
  v_piece<D>(row, c8);
  PairRegs p;
  p.k0 = buf_load16(rk, ((j + row) * D + c8) * 2);
  p.v0 = buf_load16(rv, ((j + row) * D + c8) * 2);
  p.k1 = buf_load16(rk, ((j + row + 1) * D + c8) * 2);
  p.v1 = buf_load16(rv, ((j + row + 1) * D + c8) * 2);
  return p;
}

// K^T and (w V)^T into LDS, keys contiguous; w_j = eta lam^(end-1-j).
template <int D, int SKT>
__device__ __forceinline__ void store_pair(const PairRegs& p, uint16_t* skt, uint16_t* svt, int j,
                                           int end, float et, const Decay& dec) {
  if (threadIdx.x >= 32 * (D / 8)) return;
  int row, c8;
  v_piece<D>(row, c8);
  const int jj = j + row;
  const float w0 = jj < end ? et * dec(end - 1 - jj) : 0.f;
  const float w1 = jj + 1 < end ? et * dec(end - 2 - jj) : 0.f;
  const uint32_t ka[4] = {p.k0.x, p.k0.y, p.k0.z, p.k0.w}, kb[4] = {p.k1.x, p.k1.y, p.k1.z, p.k1.w};
  const uint32_t va[4] = {p.v0.x, p.v0.y, p.v0.z, p.v0.w}, vb[4] = {p.v1.x, p.v1.y, p.v1.z, p.v1.w};
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    *reinterpret_cast<uint32_t*>(skt + (c8 + 2 * e) * SKT + row) = (ka[e] & 0xFFFFu) | (kb[e] << 16);
    *reinterpret_cast<uint32_t*>(skt + (c8 + 2 * e + 1) * SKT + row) = (ka[e] >> 16) | (kb[e] & 0xFFFF0000u);
    *reinterpret_cast<uint32_t*>(svt + (c8 + 2 * e) * SKT + row) = cvt_pk(lo_f(va[e]) * w0, lo_f(vb[e]) * w1);
    *reinterpret_cast<uint32_t*>(svt + (c8 + 2 * e + 1) * SKT + row) = cvt_pk(hi_f(va[e]) * w0, hi_f(vb[e]) * w1);
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

template <int D>
__global__ __launch_bounds__(NTHR) void fused_state_kernel(const uint16_t* __restrict__ k,
                                                           const uint16_t* __restrict__ v,
                                                           const float* __restrict__ lam,
                                                           const float* __restrict__ eta, int H,
                                                           FusedGeom G, float* __restrict__ ws) {
  constexpr int SKT = KB + 4;  // K^T and V^T rows: keys contiguous, 34-word stride
  __shared__ __attribute__((aligned(16))) uint16_t sKt[D * SKT];
  __shared__ __attribute__((aligned(16))) uint16_t sVt[D * SKT];
  using ST = StateTiles<D>;
  const int p = blockIdx.x, bh = blockIdx.y;
  const int w = wave_id(), l = lane_id(), col = l & 31, hh = l >> 5;
  const Decay dec(lam[bh % H]);
  const float et = eta[bh % H];
  const long base = (long)bh * G.T;
  const int a = G.key_begin(p), b = G.key_end(p);

  floatx16 acc[ST::TPW];
#pragma unroll
  for (int i = 0; i < ST::TPW; ++i) acc[i] = zero16();

  // three blocks in flight in registers; one LDS buffer
  const __amdgpu_buffer_rsrc_t rk = make_rsrc(k + base * D, (uint32_t)b * D * 2);
  const __amdgpu_buffer_rsrc_t rv = make_rsrc(v + base * D, (uint32_t)b * D * 2);
  PairRegs r0 = load_pair<D>(rk, rv, a);
  PairRegs r1 = load_pair<D>(rk, rv, a + KB);
  PairRegs r2 = load_pair<D>(rk, rv, a + 2 * KB);
  // r0, r1, r2 keep fixed roles (a register that is the target of a load in
  // flight is never copied), so up to three blocks stay in flight.
  // Loads are issued unconditionally (past the end they read clamped rows as
  // zero) so the count of loads in flight is the same on every path.
#define TC_STATE_STEP(R, J)                                    \
  if ((J) < b) {                                               \
    lds_barrier();                                             \
    store_pair<D, SKT>(R, sKt, sVt, (J), b, et, dec);          \
    lds_barrier();                                             \
  }                                                            \
  R = load_pair<D>(rk, rv, (J) + 3 * KB);                      \
  if ((J) < b) state_block_mma<D, SKT>(acc, sKt, sVt);
  for (int j = a; j < b; j += 3 * KB) {
    TC_STATE_STEP(r0, j)
    TC_STATE_STEP(r1, j + KB)
    TC_STATE_STEP(r2, j + 2 * KB)
  }
#undef TC_STATE_STEP
  float* out = ws + ((long)bh * G.n_seg + p) * D * D;
#pragma unroll
  for (int i = 0; i < ST::TPW; ++i) {
    if (!ST::owns(w, i)) continue;
    const int dv0 = ST::dv0(w, i), dk0 = ST::dk0(w, i);
#pragma unroll
    for (int e = 0; e < 16; ++e)
      out[(dv0 + 8 * (e >> 2) + 4 * hh + (e & 3)) * D + dk0 + col] = acc[i][e];
  }
}

// entering(0) = 0, entering(p+1) = lam^len(p) entering(p) + delta(p), in place
__global__ void fused_prefix_kernel(const float* __restrict__ lam, int H, int n_el, FusedGeom G,
                                    float* __restrict__ ws) {
  const int idx = blockIdx.x * blockDim.x + threadIdx.x;
  const int bh = blockIdx.y;
  if (idx >= n_el) return;
  const Decay dec(lam[bh % H]);
  float* p = ws + (long)bh * G.n_seg * n_el + idx;
  float run = 0.f;
  for (int s = 0; s < G.n_seg - 1; ++s) {
    const float d = p[(long)s * n_el];
    p[(long)s * n_el] = run;
    run = dec(G.key_end(s) - G.key_begin(s)) * run + d;
  }
  p[(long)(G.n_seg - 1) * n_el] = run;
}

template <int D>
__global__ __launch_bounds__(NTHR) void fused_main_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
    const float* __restrict__ lam, const float* __restrict__ eta, const float* __restrict__ g, int H,
    FusedGeom G, float scale_log2, const float* __restrict__ ws, float* __restrict__ y,
    float* __restrict__ A_final) {
  using L = Lds<D>;
  using ST = StateTiles<D>;
  constexpr int NKS = D / 16;  // k-steps over the head dimension
  constexpr int NDT = D / 32;  // 32-row tiles of O^T
  __shared__ __attribute__((aligned(16))) L lds;

  const int seg = blockIdx.x, bh = blockIdx.y, h = bh % H;
  const int w = wave_id(), l = lane_id(), col = l & 31, hh = l >> 5;
  const int T = G.T, W = G.W;
  const Decay dec(lam[h]);
  const float et = eta[h];
  const float sg = 1.f / (1.f + expf(-g[h]));
  const long base = (long)bh * T;
  const __amdgpu_buffer_rsrc_t rq = make_rsrc(q + base * D, (uint32_t)T * D * 2);
  const __amdgpu_buffer_rsrc_t rk = make_rsrc(k + base * D, (uint32_t)T * D * 2);
  const __amdgpu_buffer_rsrc_t rv = make_rsrc(v + base * D, (uint32_t)T * D * 2);

  // entering state of the segment, fp32 in LDS
  {
    const float* in = (seg > 0 && ws != nullptr) ? ws + ((long)bh * G.n_seg + seg) * D * D : nullptr;
    for (int i = threadIdx.x; i < D * D; i += NTHR)
      lds.s[(i / D) * L::SSF + (i % D)] = in ? in[i] : 0.f;
  }
  lds_barrier();

  const int nb = (W + MQ + KB - 1) / KB;  // key blocks per tile (>= 5)
  const int tile_begin = seg * G.tiles_per_seg;
  const int tile_end = min(tile_begin + G.tiles_per_seg, G.n_tiles);

  for (int tile = tile_begin; tile < tile_end; ++tile) {
    const int t0 = tile * MQ;
    const int j0 = t0 - W;
    const int tw = t0 + 32 * w;  // first query of this wave
    const int tq = tw + col;     // this lane's query
    const bool wave_live = tw < T;

    bf16x8 qreg[NKS];
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
      const uint4 x = buf_load16(rq, (tq * D + 16 * ks + 8 * hh) * 2);
      qreg[ks] = as_bf16x8(x.x, x.y, x.z, x.w);
    }
    floatx16 o[NDT];
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) o[dt] = zero16();
    float mrun = kNegBig, lsum = 0.f;

    // ---- L1 softmax over the window; blocks in the order 4..nb-1, 2, 3, 0, 1 ----
    auto block_at = [nb](int idx) {
      return idx < nb - 4 ? idx + 4 : (idx < nb - 2 ? idx - (nb - 4) + 2 : idx - (nb - 2));
    };
    BlockRegs<D> pre = load_block<D>(rk, rv, j0 + KB * block_at(0));
    store_block<D>(pre, lds.k[0], lds.vt[0]);
    lds_barrier();
#pragma unroll 1
    for (int idx = 0; idx < nb; ++idx) {
      const int b = block_at(idx);
      const int buf = idx & 1;
      pre = load_block<D>(rk, rv, j0 + KB * block_at(min(idx + 1, nb - 1)));
      const int c_lo = KB * b, c_hi = KB * b + KB - 1;
      const int r_lo = 32 * w, r_hi = 32 * w + 31;
      const int jb = j0 + c_lo;
      const bool active = wave_live && c_hi > r_lo && c_lo <= r_hi + W && jb + KB - 1 >= 0 && jb < T;
      if (active) {
        const bool full = c_lo > r_hi && c_hi <= r_lo + W && jb >= 0 && jb + KB - 1 < T;
        floatx16 s[2];
        block_scores<D>(lds.k[buf], qreg, s);
        const int r = 32 * w + col;
        float bmax = kNegBig;
        if (full) {
#pragma unroll
          for (int kt = 0; kt < 2; ++kt)
#pragma unroll
            for (int e = 0; e < 16; ++e) bmax = fmaxf(bmax, s[kt][e]);
        } else {
          // valid key offsets within the block: lo <= key_of(..) <= hi
          const int lo = max(r + 1 - c_lo, -jb);
          const int hi = min(r + W - c_lo, T - 1 - jb);
          const unsigned span = static_cast<unsigned>(hi - lo);
#pragma unroll
          for (int kt = 0; kt < 2; ++kt) {
#pragma unroll
            for (int e = 0; e < 16; ++e) {
              const bool ok = hi >= lo && static_cast<unsigned>(key_of(kt, e, hh) - lo) <= span;
              s[kt][e] = ok ? s[kt][e] : -INFINITY;
              bmax = fmaxf(bmax, s[kt][e]);
            }
          }
        }
        bmax = fmaxf(bmax, __shfl_xor(bmax, 32));
        // Lazy rescaling: the reference maximum moves only when some score of
        // the wave exceeds it by more than 8 (log2 units), so p <= 2^8 and the
        // accumulators stay far from overflow; O and lsum share the reference,
        // so the final O / lsum is unchanged.
        if (__ballot((bmax - mrun) * scale_log2 > 8.f) != 0) {
          const float mnew = fmaxf(mrun, bmax);
          const float alpha = __builtin_amdgcn_exp2f((mrun - mnew) * scale_log2);
          lsum *= alpha;
#pragma unroll
          for (int dt = 0; dt < NDT; ++dt) o[dt] *= alpha;
          mrun = mnew;
        }
        const float nms = -mrun * scale_log2;
        float psum = 0.f;
#pragma unroll
        for (int kt = 0; kt < 2; ++kt) {
#pragma unroll
          for (int e = 0; e < 16; ++e) {
            const float p = __builtin_amdgcn_exp2f(fmaf(s[kt][e], scale_log2, nms));
            s[kt][e] = p;
            psum += p;
          }
        }
        lsum += psum;
        block_pv<D>(lds.vt[buf], s, o);
      }
      if (idx + 1 < nb) store_block<D>(pre, lds.k[buf ^ 1], lds.vt[buf ^ 1]);
      lds_barrier();
    }
    {
      const float tot = lsum + __shfl_xor(lsum, 32);
      const float inv = tot > 0.f ? 1.f / tot : 0.f;
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt) o[dt] *= inv;
    }
    // the buffers now hold block 0 (buffer (nb-2)&1) and block 1 (buffer (nb-1)&1)

    // ---- L2: two chunks of 128 evictions; waves 0-3 read chunk 0, waves 4-7 chunk 1 ----
#pragma unroll 1
    for (int ch = 0; ch < 2; ++ch) {
      const int jc = j0 + CHK * ch;           // first eviction index of the chunk
      const int jend = min(jc + CHK, T - W);  // one past its last valid eviction
      const bool chunk_live = jc + CHK - 1 >= 0 && jc < T - W;
      if (ch == 1) {
        const BlockRegs<D> r2 = load_block<D>(rk, rv, j0 + 2 * KB);
        const BlockRegs<D> r3 = load_block<D>(rk, rv, j0 + 3 * KB);
        store_block<D>(r2, lds.k[0], lds.vt[0]);
        store_block<D>(r3, lds.k[1], lds.vt[1]);
        lds_barrier();
      }
      const uint16_t* sk0 = ch == 0 ? lds.k[(nb - 2) & 1] : lds.k[0];
      const uint16_t* sk1 = ch == 0 ? lds.k[(nb - 1) & 1] : lds.k[1];
      uint16_t* svt0 = ch == 0 ? lds.vt[(nb - 2) & 1] : lds.vt[0];
      uint16_t* svt1 = ch == 0 ? lds.vt[(nb - 1) & 1] : lds.vt[1];
      if (chunk_live && (w >> 2) == ch && wave_live) {
        const int r = 32 * (w & 3) + col;  // query offset within the chunk
        // decayed linear read of the chunk's own evictions (c <= r)
#pragma unroll 1
        for (int hb = 0; hb < 2; ++hb) {
          if (hb == 1 && (w & 3) < 2) continue;  // queries r < 64 see no key of the second block
          floatx16 s[2];
          block_scores<D>(hb == 0 ? sk0 : sk1, qreg, s);
#pragma unroll
          for (int kt = 0; kt < 2; ++kt) {
#pragma unroll
            for (int e = 0; e < 16; ++e) {
              const int c = KB * hb + key_of(kt, e, hh);
              const bool ok = c <= r && jc + c >= 0;
              s[kt][e] = ok ? s[kt][e] * (sg * et) * dec(r - c) : 0.f;
            }
          }
          block_pv<D>(hb == 0 ? svt0 : svt1, s, o);
        }
        // read of the entering state: O^T += S_n^T (sigmoid(g) lam^(r+1) q_r)^T
        const float gam = sg * dec(r + 1);
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) {
          const u32x4 u = __builtin_bit_cast(u32x4, qreg[ks]);
          const bf16x8 qs = as_bf16x8(cvt_pk(lo_f(u[0]) * gam, hi_f(u[0]) * gam),
                                      cvt_pk(lo_f(u[1]) * gam, hi_f(u[1]) * gam),
                                      cvt_pk(lo_f(u[2]) * gam, hi_f(u[2]) * gam),
                                      cvt_pk(lo_f(u[3]) * gam, hi_f(u[3]) * gam));
#pragma unroll
          for (int dt = 0; dt < NDT; ++dt) {
            const float* row = lds.s + (32 * dt + col) * L::SSF + 16 * ks + 8 * hh;
            const float4 x0 = *reinterpret_cast<const float4*>(row);
            const float4 x1 = *reinterpret_cast<const float4*>(row + 4);
            const bf16x8 a = as_bf16x8(cvt_pk(x0.x, x0.y), cvt_pk(x0.z, x0.w), cvt_pk(x1.x, x1.y),
                                       cvt_pk(x1.z, x1.w));
            o[dt] = mfma32(a, qs, o[dt]);
          }
        }
      }
      if (ch == 1 && tq < T) {
        // every contribution to this lane's query is in: y = O^T column
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) {
#pragma unroll
          for (int g4 = 0; g4 < 4; ++g4) {
            const float4 out = make_float4(o[dt][4 * g4], o[dt][4 * g4 + 1], o[dt][4 * g4 + 2], o[dt][4 * g4 + 3]);
            *reinterpret_cast<float4*>(y + (base + tq) * D + 32 * dt + 8 * g4 + 4 * hh) = out;
          }
        }
      }
      // state step over the chunk's evictions [max(jc, 0), jend)
      const bool writes = jend > max(jc, 0);
      lds_barrier();  // all reads of unscaled V^T and of the state copy are done
      if (writes) {
        if (threadIdx.x < CHK) {
          const int j = jc + threadIdx.x;
          lds.w[threadIdx.x] = (j >= 0 && j < jend) ? et * dec(jend - 1 - j) : 0.f;
        }
        lds_barrier();
        scale_vt<D>(svt0, svt1, lds.w);
        lds_barrier();
        state_update<D>(lds.s, dec(jend - jc), sk0, svt0, sk1, svt1);
      }
      // chunk 0 leaves S_{n+1} for chunk 1's readers, chunk 1 the next tile's state
      lds_barrier();
    }
  }

  if (A_final != nullptr && seg == G.n_seg - 1) {
    float* out = A_final + (long)bh * D * D;  // A[dk][dv] = S^T[dv][dk]
    for (int i = threadIdx.x; i < D * D; i += NTHR) {
      const int dk = i / D, dv = i % D;
      out[i] = lds.s[dv * L::SSF + dk];
    }
  }
}

FusedGeom make_geom(int B, int H, int T, int W) {
  FusedGeom G{};
  G.T = T;
  G.W = W;
  G.n_tiles = (T + MQ - 1) / MQ;
  const long units = (long)B * H;
  // one workgroup per CU: aim for about 256 (segment, head) workgroups
  const long want = std::max<long>(1, (256 + units - 1) / units);
  G.tiles_per_seg = (int)std::max<long>(1, (G.n_tiles + want - 1) / want);
  G.n_seg = G.n_tiles > 0 ? (G.n_tiles + G.tiles_per_seg - 1) / G.tiles_per_seg : 0;
  return G;
}

template <int D>
hipError_t run_fused(const uint16_t* q, const uint16_t* k, const uint16_t* v, const float* lam,
                     const float* eta, const float* g, int B, int H, const FusedGeom& G, float scale,
                     float* y, float* A_final, float* ws, hipStream_t s) {
  const int BH = B * H;
  if (G.n_seg > 1) {
    hipLaunchKernelGGL(fused_state_kernel<D>, dim3(G.n_seg - 1, BH), dim3(NTHR), 0, s, k, v, lam,
                       eta, H, G, ws);
    hipLaunchKernelGGL(fused_prefix_kernel, dim3((D * D + 255) / 256, BH), dim3(256), 0, s, lam, H,
                       D * D, G, ws);
  }
  hipLaunchKernelGGL(fused_main_kernel<D>, dim3(G.n_seg, BH), dim3(NTHR), 0, s, q, k, v, lam, eta,
                     g, H, G, scale * 1.4426950408889634f, G.n_seg > 1 ? ws : nullptr, y, A_final);
  return hipGetLastError();
}

}  // namespace

size_t fused_ws_bytes(int B, int H, int T, int dk, int dv, int W) {
  (void)dv;
  const FusedGeom G = make_geom(B, H, T, W);
  if (G.n_seg <= 1) return 0;
  return (size_t)B * H * G.n_seg * dk * dk * sizeof(float);
}

hipError_t launch_tc_fused(const void* q, const void* k, const void* v, const float* lam,
                           const float* eta, const float* g, int B, int H, int T, int d, int W,
                           float scale, float* y, float* A_final, void* ws, hipStream_t s) {
  const FusedGeom G = make_geom(B, H, T, W);
  const uint16_t* Q = static_cast<const uint16_t*>(q);
  const uint16_t* K = static_cast<const uint16_t*>(k);
  const uint16_t* V = static_cast<const uint16_t*>(v);
  float* wsf = static_cast<float*>(ws);
  if (d == 128) return run_fused<128>(Q, K, V, lam, eta, g, B, H, G, scale, y, A_final, wsf, s);
  if (d == 64) return run_fused<64>(Q, K, V, lam, eta, g, B, H, G, scale, y, A_final, wsf, s);
  return hipErrorInvalidValue;
}

}  // namespace tc

// tc_swa.hip — main kernel of the fused Tensor Cache layer (gfx950, bf16
// inputs): exact softmax attention over the W most recent tokens (L1) plus
// the gated read of the L2 memory, y = y_local + sigmoid(g) m.
//
// Tensor Cache, Methodology 1: the L1 cache is a KV ring of the W most recent
// tokens with exact softmax attention over it; a token leaves it exactly when
// it is written into the L2 matrix, A <- lam A + eta k v^T; the read is
// m_t = q_t A_t, and y_t = y_local,t + sigmoid(g) m_t.  Methodology 2: the L2
// part is evaluated in chunk form, here one chunk per 256-query tile:
//   m_r = lam^(r+1) q_r S_n + sum_{c <= r} eta lam^(r-c) <q_r, k_c> v_c,
// with S_n the state entering the tile (computed by the pre-pass and prefix).
//
// One workgroup = 8 waves = 256 queries (one tile); wave w owns 32 queries.
// Keys are taken in 64-key blocks from j0 = t0 - W (c = j - j0, r = t - t0;
// key j is in the window of query t iff r < c <= r + W, and has been written
// into the L2 memory iff c <= r).  Blocks travel global -> LDS by
// buffer_load ... lds (K and V rows as they are in memory, 16-byte pieces
// permuted within each row), four blocks resident.  S^T = K Q^T puts one
// query's scores in every lane (v_mfma_f32_32x32x16_bf16), and P feeds
// O^T += V^T P^T from registers; the V^T operand comes from the V rows by
// LDS transpose reads (ds_read_b64_tr_b16), so V needs no transposed copy.  The loop is software-pipelined: the QK^T MFMAs of block i+1
// are interleaved with the softmax of block i and its PV MFMAs, so the matrix
// cores and the vector ALUs work at the same time.  Blocks 4.. come first (in an
// order rotated per tile, so that neighbouring tiles read the same keys at the
// same time) and blocks 0-3 last, so the latter (the tile's evictions) are
// still resident for the L2 epilogue.  The grid is persistent (as many workgroups as fit at
// once, each walking several tiles), and tiles are mapped so that the
// workgroups that share an XCD at the same time work on neighbouring tiles of
// one head and share K/V through its L2 cache.
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

constexpr int NWAVE = 8;
constexpr int NTHR = 64 * NWAVE;
constexpr int MQ = 32 * NWAVE;  // queries per tile
constexpr int NSTAGE = 4;       // blocks resident in LDS
constexpr int NXCD = 8;         // MI355X: 8 accelerator complex dies, dispatched round-robin
constexpr int kComputeUnits = 256;
constexpr float kNegBig = -1.0e30f;

template <int D>
struct SwaLds {
  uint16_t k[NSTAGE][KB * D];
  uint16_t v[NSTAGE][KB * D];  // V rows in the row layout of tc_tr.hpp (16-byte pieces permuted per row)
  uint16_t st[D * D];  // entering L2 state S^T (rows dv), as D/64 K-layout blocks
};

template <int D>
struct Dma {
  static constexpr int NK = KB * D / 8 / NTHR;  // 16-byte K slots per thread
  static constexpr int NV = KB * D / 8 / NTHR;  // 16-byte V slots per thread
  static constexpr int N = NK + NV;
};

// Lane parts of the DMA source offsets (bytes, block start excluded).
template <int D>
struct DmaOff {
  int k[Dma<D>::NK];
  int v[Dma<D>::NV];
  int w512;  // this wave's first 1 KiB piece of a stage (in elements)
};

template <int D>
__device__ __forceinline__ DmaOff<D> dma_offsets() {
  DmaOff<D> o;
  const int w = wave_id(), l = lane_id();
  o.w512 = w * 512;
#pragma unroll
  for (int i = 0; i < Dma<D>::NK; ++i) {
    int m, c;
    k_slot_inv<D>((i * NWAVE + w) * 64 + l, m, c);
    o.k[i] = (perm16(m) * D + 8 * c) * 2;
  }
#pragma unroll
  for (int i = 0; i < Dma<D>::NV; ++i) {
    const int sl = (i * NWAVE + w) * 64 + l;
    o.v[i] = tr::slot_src<D>(sl);
  }
  return o;
}

// DMA of the 64-key block starting at key j (any sign) into one stage.  dk,
// dv: this head's K and V rows [0, T).  Reads outside the descriptors return
// zero.  Instruction i of wave w fills the 1 KiB piece i * 8 + w of the stage.
template <int D>
__device__ __forceinline__ void dma_block(i32x4 dk, i32x4 dv, const DmaOff<D>& off, int j,
                                          uint16_t* sk, uint16_t* sv) {
#pragma unroll
  for (int i = 0; i < Dma<D>::NK; ++i) dma16(dk, sk + i * NWAVE * 512 + off.w512, off.k[i] + j * D * 2);
#pragma unroll
  for (int i = 0; i < Dma<D>::NV; ++i) dma16(dv, sv + i * NWAVE * 512 + off.w512, off.v[i] + j * D * 2);
}

// DMA of the tile's entering state (bf16, [dv][dk] row-major in global) into
// the K-block layout, rows in natural order (row m of block h holds dv =
// 64 h + m), so that S^T Q^T comes out in the layout of O^T.
template <int D>
__device__ __forceinline__ void dma_state(i32x4 dst_desc, uint16_t* sst) {
  constexpr int NI = D * D / 8 / NTHR;  // 16-byte slots per thread
  const int w = wave_id(), l = lane_id();
#pragma unroll
  for (int i = 0; i < NI; ++i) {
    const int slot = (i * NWAVE + w) * 64 + l;
    int m, c;
    k_slot_inv<D>(slot & (8 * D - 1), m, c);
    const int dv = 64 * (slot / (8 * D)) + m;
    dma16(dst_desc, sst + (i * NWAVE + w) * 512, (dv * D + 8 * c) * 2);
  }
}

// One block's DMA, issued one instruction at a time across a step so that
// the workgroup's 32 copy instructions do not all queue at the same moment.
template <int D>
struct DmaJob {
  i32x4 dk, dv;
  int off;            // block start in bytes: j * D * 2 (K and V rows)
  uint16_t *sk, *sv;
  bool on;            // a block is left to fetch
};
template <int D, int I>
__device__ __forceinline__ void dma_part(const DmaJob<D>& job, const DmaOff<D>& off) {
  if (!job.on) return;
  if constexpr (I < Dma<D>::NK)
    dma16(job.dk, job.sk + I * NWAVE * 512 + off.w512, off.k[I] + job.off);
  else
    dma16(job.dv, job.sv + (I - Dma<D>::NK) * NWAVE * 512 + off.w512, off.v[I - Dma<D>::NK] + job.off);
}

// floor(a / b) and ceil(a / b) for b > 0 and any sign of a
__device__ __forceinline__ int floordiv(int a, int b) { return a >= 0 ? a / b : -((-a + b - 1) / b); }
__device__ __forceinline__ int ceildiv(int a, int b) { return a >= 0 ? (a + b - 1) / b : -((-a) / b); }

// max / sum over the two 32-lane halves (the two halves of a query's keys)
__device__ __forceinline__ float max_halves(float x) {
  const auto s = __builtin_amdgcn_permlane32_swap(__float_as_int(x), __float_as_int(x), false, false);
  return fmaxf(__int_as_float(s[0]), __int_as_float(s[1]));
}
__device__ __forceinline__ float sum_halves(float x) {
  const auto s = __builtin_amdgcn_permlane32_swap(__float_as_int(x), __float_as_int(x), false, false);
  return __int_as_float(s[0]) + __int_as_float(s[1]);
}

// ---------------------------------------------------------------------------
// Operand batches.  Every LDS operand read is issued one batch (four MFMAs,
// >= 128 cycles) before the MFMA that uses it, and sched_barrier fences keep
// the compiler from sinking the reads next to their uses (which would expose
// the LDS latency on every MFMA).

// K operands of k-steps KS, KS+1: rows 0-31 and 32-63 of the block
template <int KS>
__device__ __forceinline__ void ld_k2(const char* sk, const uint32_t* ls, bf16x8* x) {
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const uint32_t off = ls[(KS + i) & 3] + 8192u * ((KS + i) >> 2);
    x[2 * i] = lds16(sk, off);
    x[2 * i + 1] = lds16(sk, off + 4096u);
  }
}
template <int KS>
__device__ __forceinline__ void mm_k2(const bf16x8* x, const bf16x8* qreg, floatx16& a0, floatx16& a1) {
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    a0 = mfma32(x[2 * i], qreg[KS + i], a0);
    a1 = mfma32(x[2 * i + 1], qreg[KS + i], a1);
  }
}
template <int D>
__device__ __forceinline__ void mm_v(const bf16x8* x, bf16x8 pb, floatx16* o) {
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt) o[dt] = mfma32(x[dt], pb, o[dt]);
}

#define TC_SB() __builtin_amdgcn_sched_barrier(0)
// reads first, then MFMAs each followed by NV VALU instructions
#define TC_GROUPS(NR, NM, NV)                                     \
  do {                                                            \
    __builtin_amdgcn_sched_group_barrier(0x100, (NR), 0);         \
    _Pragma("unroll") for (int i_ = 0; i_ < (NM); ++i_) {         \
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);          \
      __builtin_amdgcn_sched_group_barrier(0x002, (NV), 0);       \
    }                                                             \
  } while (0)

// S^T of a whole block (keys 0-31 -> a0, 32-63 -> a1), batched
template <int D>
__device__ __forceinline__ void qk_block(const char* sk, const uint32_t* ls, const bf16x8* qreg,
                                         floatx16& a0, floatx16& a1) {
  bf16x8 x0[4], x1[4];
  a0 = zero16();
  a1 = zero16();
  ld_k2<0>(sk, ls, x0);
  ld_k2<2>(sk, ls, x1);
  TC_SB();
  mm_k2<0>(x0, qreg, a0, a1);
  if constexpr (D == 128) {
    ld_k2<4>(sk, ls, x0);
    TC_SB();
    mm_k2<2>(x1, qreg, a0, a1);
    ld_k2<6>(sk, ls, x1);
    TC_SB();
    mm_k2<4>(x0, qreg, a0, a1);
    TC_SB();
    mm_k2<6>(x1, qreg, a0, a1);
  } else {
    TC_SB();
    mm_k2<2>(x1, qreg, a0, a1);
  }
}

struct Softmax {
  float m;  // reference maximum (raw score units), shared by the wave
  float l;  // sum of this lane's probabilities
};

// Valid keys of this lane's query in a block: lo <= key <= lo + span (as
// unsigned), with lo already lowered by 8 hh (key_of without the 8 hh term).
struct KeyRange {
  int lo;
  unsigned span;
};

// Probabilities of PV k-step KK: p = 2^(s sl2 - m sl2) as bf16, and their
// sum (of the same bf16 values that multiply V) into psum.
template <int KK>
__device__ __forceinline__ bf16x8 probs(const floatx16* sc, float sl2, float nms, float& psum) {
  constexpr int kt = KK >> 1, e0 = (KK & 1) * 8;
  const bf16x2 one2 = __builtin_bit_cast(bf16x2, 0x3F803F80u);
  uint32_t pw[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const float p0 = __builtin_amdgcn_exp2f(fmaf(sc[kt][e0 + 2 * e], sl2, nms));
    const float p1 = __builtin_amdgcn_exp2f(fmaf(sc[kt][e0 + 2 * e + 1], sl2, nms));
    pw[e] = cvt_pk(p0, p1);
    psum = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, pw[e]), one2, psum, false);
  }
  return as_bf16x8(pw[0], pw[1], pw[2], pw[3]);
}

// One pipelined step: QK^T of the next block (into sn) interleaved with the
// softmax of the current block (sc) and its PV product.
template <int D>
__device__ __forceinline__ void swa_step(const char* sk_nxt, const char* sv_cur, const uint32_t* ls,
                                         const uint32_t* vls, const bf16x8* qreg, floatx16* sc, floatx16* sn, floatx16* o,
                                         Softmax& sm, float sl2, bool active, bool masked, KeyRange kr,
                                         const DmaJob<D>& job, const DmaOff<D>& doff) {
  constexpr int NDT = D / 32;
  constexpr int NVR = 2 * NDT;  // LDS reads of one V operand batch (two transpose reads per tile)
  constexpr int ND = Dma<D>::N;  // 4 for D = 128, 2 for D = 64
  if (!active) {
    dma_part<D, 0>(job, doff);
    dma_part<D, 1>(job, doff);
    if constexpr (ND > 2) {
      dma_part<D, 2>(job, doff);
      dma_part<D, 3>(job, doff);
    }
    qk_block<D>(sk_nxt, ls, qreg, sn[0], sn[1]);
    return;
  }
  if (masked) {
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const unsigned d = static_cast<unsigned>(key_of(kt, e, 0) - kr.lo);
        sc[kt][e] = d <= kr.span ? sc[kt][e] : -INFINITY;
      }
  }
  floatx16 a0 = zero16(), a1 = zero16();
  bf16x8 ka[4], kb[4];
  float m0 = kNegBig, m1 = kNegBig;
  // region A: QK^T k-steps 0..NKS/2-1 of the next block; block maximum
  TC_SB();
  ld_k2<0>(sk_nxt, ls, ka);
  TC_SB();
  dma_part<D, 0>(job, doff);
  TC_SB();
  ld_k2<2>(sk_nxt, ls, kb);
  mm_k2<0>(ka, qreg, a0, a1);
#pragma unroll
  for (int e = 0; e < 16; ++e) m0 = fmaxf(m0, sc[0][e]);
  if constexpr (D == 64) {
#pragma unroll
    for (int e = 0; e < 16; ++e) m1 = fmaxf(m1, sc[1][e]);
  }
  TC_GROUPS(4, 4, D == 128 ? 2 : 4);
  TC_SB();
  if constexpr (D == 128) {
    dma_part<D, 1>(job, doff);
    TC_SB();
    ld_k2<4>(sk_nxt, ls, ka);
    mm_k2<2>(kb, qreg, a0, a1);
#pragma unroll
    for (int e = 0; e < 16; ++e) m1 = fmaxf(m1, sc[1][e]);
    TC_GROUPS(4, 4, 2);
    TC_SB();
  }
  const float bmax = max_halves(fmaxf(m0, m1));
  // Lazy rescaling: the reference maximum moves only when a score of the
  // wave exceeds it by more than 2^8 in probability; O and l share the
  // reference, so O / l is unchanged and p stays <= 2^8.
  if (__ballot((bmax - sm.m) * sl2 > 8.f) != 0) {
    const float mnew = fmaxf(sm.m, bmax);
    const float alpha = __builtin_amdgcn_exp2f((sm.m - mnew) * sl2);
    sm.l *= alpha;
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) o[dt] *= alpha;
    sm.m = mnew;
  }
  TC_SB();
  // region B: remaining QK^T k-steps, exponentials, PV
  const float nms = -sm.m * sl2;
  float psum = 0.f;
  bf16x8 va[NDT], vb[NDT];
  bf16x8 p0, p1, p2, p3;
  if constexpr (D == 128) {
    dma_part<D, 2>(job, doff);
    TC_SB();
    ld_k2<6>(sk_nxt, ls, kb);
    mm_k2<4>(ka, qreg, a0, a1);
    p0 = probs<0>(sc, sl2, nms, psum);
    TC_GROUPS(4, 4, 6);
    TC_SB();
    tr::ld<D, 0>(sv_cur, vls, va);
    mm_k2<6>(kb, qreg, a0, a1);
  } else {
    dma_part<D, 1>(job, doff);
    TC_SB();
    tr::ld<D, 0>(sv_cur, vls, va);
    mm_k2<2>(kb, qreg, a0, a1);
    p0 = probs<0>(sc, sl2, nms, psum);
    TC_GROUPS(NVR, 4, 6);
    TC_SB();
  }
  p1 = probs<1>(sc, sl2, nms, psum);
  if constexpr (D == 128) {
    TC_GROUPS(NVR, 4, 6);
    TC_SB();
  }
  if constexpr (D == 128) {
    dma_part<D, 3>(job, doff);
    TC_SB();
  }
  tr::ld<D, 1>(sv_cur, vls, vb);
  mm_v<D>(va, p0, o);
  p2 = probs<2>(sc, sl2, nms, psum);
  TC_GROUPS(NVR, NDT, 24 / NDT);
  TC_SB();
  tr::ld<D, 2>(sv_cur, vls, va);
  mm_v<D>(vb, p1, o);
  p3 = probs<3>(sc, sl2, nms, psum);
  TC_GROUPS(NVR, NDT, 24 / NDT);
  TC_SB();
  tr::ld<D, 3>(sv_cur, vls, vb);
  mm_v<D>(va, p2, o);
  TC_SB();
  mm_v<D>(vb, p3, o);
  sm.l += psum;
  TC_SB();
  sn[0] = a0;
  sn[1] = a1;
}

// Per-head parameters of the L2 read (nullptr sst: no L2 term).
struct L2Args {
  const uint16_t* sst;  // entering states, [B*H][n_tiles][D][D] bf16 (S^T: row dv)
  const float* lam;
  const float* eta;
  const float* g;
  int H;
};

// L2 weights of PV k-step KK: p = fe lam^(r-c) <q_r, k_c> for valid keys.
template <int KK>
__device__ __forceinline__ bf16x8 l2probs(const floatx16* s, int lo, unsigned span, float xl,
                                          float log2lam, float fe) {
  constexpr int kt = KK >> 1, e0 = (KK & 1) * 8;
  uint32_t pw[4];
#pragma unroll
  for (int e = 0; e < 8; e += 2) {
    const int k0 = key_of(kt, e0 + e, 0), k1 = key_of(kt, e0 + e + 1, 0);
    const float w0 = __builtin_amdgcn_exp2f(fmaf(static_cast<float>(-k0), log2lam, xl));
    const float w1 = __builtin_amdgcn_exp2f(fmaf(static_cast<float>(-k1), log2lam, xl));
    const float q0 = static_cast<unsigned>(k0 - lo) <= span ? s[kt][e0 + e] * fe * w0 : 0.f;
    const float q1 = static_cast<unsigned>(k1 - lo) <= span ? s[kt][e0 + e + 1] * fe * w1 : 0.f;
    pw[e >> 1] = cvt_pk(q0, q1);
  }
  return as_bf16x8(pw[0], pw[1], pw[2], pw[3]);
}

// L2 term of one resident block b (0..3) of the tile's evictions:
// o += V^T P^T with P[c][r] = fe lam^(r-c) <q_r, k_c> for c <= r, 0 <= j.
template <int D>
__device__ __forceinline__ void l2_block(const char* sk, const char* sv, const uint32_t* ls,
                                         const uint32_t* vls, const bf16x8* qreg, floatx16* o, int b, int jb, int r,
                                         float log2lam, float fe) {
  constexpr int NDT = D / 32;
  const int hh = lane_id() >> 5;
  floatx16 s[2];
  qk_block<D>(sk, ls, qreg, s[0], s[1]);
  // valid keys: max(0, -jb) <= key <= r - 64 b  (key = key_of(kt, e, 0) + 8 hh)
  int lo = max(0, -jb);
  const int hi = r - KB * b;
  unsigned span = static_cast<unsigned>(hi - lo);
  if (hi < lo) {
    lo = 1 << 20;
    span = 0;
  }
  lo -= 8 * hh;
  // lam^(r - c) = 2^((n - key0) log2 lam), n = r - 64 b - 8 hh
  const float xl = static_cast<float>(hi - 8 * hh) * log2lam;
  bf16x8 va[NDT], vb[NDT];
  TC_SB();
  tr::ld<D, 0>(sv, vls, va);
  const bf16x8 p0 = l2probs<0>(s, lo, span, xl, log2lam, fe);
  TC_SB();
  tr::ld<D, 1>(sv, vls, vb);
  mm_v<D>(va, p0, o);
  const bf16x8 p1 = l2probs<1>(s, lo, span, xl, log2lam, fe);
  TC_SB();
  tr::ld<D, 2>(sv, vls, va);
  mm_v<D>(vb, p1, o);
  const bf16x8 p2 = l2probs<2>(s, lo, span, xl, log2lam, fe);
  TC_SB();
  tr::ld<D, 3>(sv, vls, vb);
  mm_v<D>(va, p2, o);
  const bf16x8 p3 = l2probs<3>(s, lo, span, xl, log2lam, fe);
  TC_SB();
  mm_v<D>(vb, p3, o);
  TC_SB();
}

// bf16x8 * f, rounded to bf16
__device__ __forceinline__ bf16x8 scale_bf16x8(bf16x8 x, float f) {
  const u32x4 u = __builtin_bit_cast(u32x4, x);
  return as_bf16x8(cvt_pk(lo_f(u[0]) * f, hi_f(u[0]) * f), cvt_pk(lo_f(u[1]) * f, hi_f(u[1]) * f),
                   cvt_pk(lo_f(u[2]) * f, hi_f(u[2]) * f), cvt_pk(lo_f(u[3]) * f, hi_f(u[3]) * f));
}

template <int D>
__global__ __launch_bounds__(NTHR) void swa_kernel(const uint16_t* __restrict__ q,
                                                   const uint16_t* __restrict__ k,
                                                   const uint16_t* __restrict__ v, L2Args l2,
                                                   int T, int W, int n_tiles, int n_items, float sl2,
                                                   float* __restrict__ y, float* __restrict__ lse2) {
  constexpr int NKS = D / 16;
  constexpr int NDT = D / 32;
  __shared__ __attribute__((aligned(16))) SwaLds<D> lds;

  // Persistent, XCD-aware: the workgroups dispatched to one XCD share a
  // contiguous run of (head, tile) items and walk it with the stride of their
  // number, so the tiles in flight on an XCD are neighbours of one head that
  // share K/V through its L2.  A workgroup's next tile starts while the
  // previous tile's output stores drain.
  const int per_xcd = (n_items + NXCD - 1) / NXCD;
  const int xcd = blockIdx.x % NXCD, n_slots = gridDim.x / NXCD;
  const int w = wave_id(), l = lane_id(), col = l & 31, hh = l >> 5;
  const DmaOff<D> doff = dma_offsets<D>();
  uint32_t ls[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) ls[j] = lane_slot(j);
  uint32_t vls[NDT];
  tr::lane_offsets<D>(vls);

#pragma unroll 1
  for (int local = blockIdx.x / NXCD; local < per_xcd; local += n_slots) {
    const int item = xcd * per_xcd + local;
    if (item >= n_items) break;
    const int bh = item / n_tiles, tile = item % n_tiles;
    // every wave is done with the LDS stages and the state of the previous tile
    lds_barrier();
    const long base = (long)bh * T;
    const __amdgpu_buffer_rsrc_t rq = make_rsrc(q + base * D, (uint32_t)T * D * 2);
    const i32x4 rk = raw_desc(k + base * D, (uint32_t)T * D * 2);
    const i32x4 rv = raw_desc(v + base * D, (uint32_t)T * D * 2);

    const int t0 = tile * MQ;
    const int j0 = t0 - W;
    // Query slice of this wave.  Waves w and w + 4 share a SIMD and slice s
    // needs floor(s / 2) + 1 blocks in the L2 epilogue, so the slices 0..3
    // pair with 7..4 to give every SIMD the same epilogue work.
    const int slice = w < 4 ? w : 11 - w;
    const int r_lo = 32 * slice, r_hi = r_lo + 31;
    const int tw = t0 + r_lo;    // first query of this wave
    const int tq = tw + col;     // this lane's query
    const int nb = (W + MQ + KB - 1) / KB;  // >= 5
    // the tile writes evictions into the L2 memory iff some key j0 .. j0 + 255 is >= 0
    const bool has_l2 = l2.sst != nullptr && j0 + MQ > 0;
    // Blocks 4 .. nb-1 first, then 0 .. 3 (left resident for the L2 epilogue).
    // The first part is rotated by 4 blocks per tile: block b of tile p + 1 is
    // block b + 4 of tile p, so neighbouring tiles (which run at the same time
    // on one XCD) read the same keys at the same step, out of its L2.
    const int nw = nb - 4, rot = (MQ / KB * tile) % nw;
    auto block_at = [nw, rot](int idx) {
      if (idx >= nw) return idx - nw;
      const int x = idx + nw - rot;  // in [1, 2 nw): (idx - rot) mod nw without a division
      return 4 + (x >= nw ? x - nw : x);
    };

    bf16x8 qreg[NKS];
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) qreg[ks] = as_bf16x8(buf_load16(rq, (tq * D + 16 * ks + 8 * hh) * 2));
    floatx16 o[NDT];
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) o[dt] = zero16();
    Softmax sm{kNegBig, 0.f};

    // Copies complete in issue order: blocks 0..2, then the state (used only in
    // the epilogue).  The state is issued after the first scores: the compiler
    // waits for the q loads with counts that also cover every copy issued
    // before them, so the first scores wait for blocks 0..2 but not for it.
    constexpr int NS = D * D / 8 / NTHR;  // state copy instructions per thread
#pragma unroll
    for (int i = 0; i < NSTAGE - 1; ++i)
      dma_block<D>(rk, rv, doff, j0 + KB * block_at(i), lds.k[i], lds.v[i]);
    wait_vmcnt<2 * Dma<D>::N>();
    lds_barrier();
    floatx16 s0[2], s1[2];
    qk_block<D>(reinterpret_cast<const char*>(lds.k[0]), ls, qreg, s0[0], s0[1]);
    if (has_l2) dma_state<D>(raw_desc(l2.sst + ((long)bh * n_tiles + tile) * D * D, D * D * 2), lds.st);

    // The blocks b (keys j0 + 64 b ..) that some query of this wave sees
    // (active) and the ones that every query of the wave sees whole (full,
    // no masking) are two ranges of b:
    //   active: 64 b + 63 > r_lo, 64 b <= r_hi + W, j0 + 64 b + 63 >= 0, j0 + 64 b < T;
    //   full:   64 b > r_hi, 64 b + 63 <= r_lo + W, j0 + 64 b >= 0, j0 + 64 b + 63 < T.
    int a_lo = max(max(0, ceildiv(r_lo - KB + 2, KB)), ceildiv(-j0 - KB + 1, KB));
    int a_hi = min(min(nb - 1, floordiv(r_hi + W, KB)), floordiv(T - j0 - 1, KB));
    if (tw >= T) a_lo = nb;
    int f_lo = max(max(0, floordiv(r_hi, KB) + 1), ceildiv(-j0, KB));
    const int f_hi = min(min(nb - 1, floordiv(r_lo + W - KB + 1, KB)), floordiv(T - KB - j0, KB));
    if (tw + 31 >= T) f_lo = nb;

    // One step per block position; the scores alternate between s0 and s1.
    auto step = [&](int idx, floatx16* sc, floatx16* sn) __attribute__((always_inline)) {
      // block idx + 1 must have landed: its scores are formed in this step.
      // Outstanding copies allowed: block idx + 2, and for idx < 2 the state,
      // which was issued between blocks 2 and 3 (at idx = 0 block 1 has landed
      // already).
      if (idx < 2 && has_l2) wait_vmcnt<Dma<D>::N + NS>();
      else if (idx + 2 < nb) wait_vmcnt<Dma<D>::N>();
      else wait_vmcnt<0>();
      lds_barrier();  // also: every wave is done with step idx - 1, whose stage the next DMA reuses
      DmaJob<D> job;
      {
        const int st = (idx + NSTAGE - 1) & (NSTAGE - 1);
        const int jn = j0 + KB * block_at(idx + NSTAGE - 1);
        job = DmaJob<D>{rk, rv, jn * D * 2, lds.k[st], lds.v[st], idx + NSTAGE - 1 < nb};
      }
      const int b = block_at(idx);
      // (bitwise &: the flags are formed without branches)
      const bool active = (idx < nb) & (b >= a_lo) & (b <= a_hi);
      const bool full = (b >= f_lo) & (b <= f_hi);
      KeyRange kr{0, 0u};
      if (!full) {
        // keys c_lo + key valid for query r: r < c <= r + W and 0 <= j < T
        const int c_lo = KB * b, jb = j0 + c_lo, r = r_lo + col;
        int lo = max(r + 1 - c_lo, -jb);
        const int hi = min(r + W - c_lo, T - 1 - jb);
        kr.span = static_cast<unsigned>(hi - lo);
        if (hi < lo) {
          lo = 1 << 20;  // no key matches
          kr.span = 0;
        }
        kr.lo = lo - 8 * hh;
      }
      swa_step<D>(reinterpret_cast<const char*>(lds.k[(idx + 1) & (NSTAGE - 1)]),
                  reinterpret_cast<const char*>(lds.v[idx & (NSTAGE - 1)]), ls, vls, qreg, sc, sn, o, sm,
                  sl2, active, !full, kr, job, doff);
    };
#pragma unroll 1
    for (int idx = 0; idx < nb; idx += 2) {
      step(idx, s0, s1);
      step(idx + 1, s1, s0);  // past the last block: an inactive step
    }

    const float tot = sum_halves(sm.l);
    const float inv = tot > 0.f ? 1.f / tot : 0.f;
    // log2 of the softmax denominator in the exp2(sl2 s) units of the scores
    // (for the backward), every other float of lse2
    if (lse2 != nullptr && tq < T && hh == 0) lse2[2 * (base + tq)] = sm.m * sl2 + log2f(tot);
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) o[dt] *= inv;

    if (has_l2 && tw < T) {
      // Every DMA has completed (the last step waited for all of them) and the
      // barrier of that step made them visible to the whole workgroup.
      const int h = bh % l2.H;
      const float lam = l2.lam[h];
      const float log2lam = lam > 0.f ? log2f(lam) : -1.0e4f;  // 0^0 = 1, 0^n = 0
      const float gate = 1.f / (1.f + expf(-l2.g[h]));
      const int r = r_lo + col;
      // state term: o^T += S_n^T (fs Q)^T, fs = gate lam^(r+1) per query
      const float fs = gate * __builtin_amdgcn_exp2f(static_cast<float>(r + 1) * log2lam);
      const char* sst = reinterpret_cast<const char*>(lds.st);
      bf16x8 sbuf[2][NDT];
      TC_SB();
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt)
        sbuf[0][dt] = lds16(sst + (dt >> 1) * (KB * D * 2), ls[0] + 4096u * (dt & 1));
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) {
        TC_SB();
        if (ks + 1 < NKS) {
#pragma unroll
          for (int dt = 0; dt < NDT; ++dt)
            sbuf[(ks + 1) & 1][dt] = lds16(sst + (dt >> 1) * (KB * D * 2),
                                           ls[(ks + 1) & 3] + 8192u * ((ks + 1) >> 2) + 4096u * (dt & 1));
        }
        const bf16x8 qs = scale_bf16x8(qreg[ks], fs);
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) o[dt] = mfma32(sbuf[ks & 1][dt], qs, o[dt]);
      }
      TC_SB();
      // evictions of the tile: blocks 0..3, resident in stages (nb - 4 + b) % 4
      const float fe = gate * l2.eta[h];
#pragma unroll 1
      for (int b = 0; b < 4; ++b) {
        const int jb = j0 + KB * b;
        if (KB * b > r_hi || jb + KB - 1 < 0) continue;  // wave-uniform
        const int st = (nb - 4 + b) & (NSTAGE - 1);
        l2_block<D>(reinterpret_cast<const char*>(lds.k[st]), reinterpret_cast<const char*>(lds.v[st]),
                    ls, vls, qreg, o, b, jb, r, log2lam, fe);
      }
    }

    if (tq < T) {
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt) {
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
          const int dv = 32 * dt + 8 * g4 + 4 * hh;
          const float4 out = make_float4(o[dt][4 * g4], o[dt][4 * g4 + 1], o[dt][4 * g4 + 2], o[dt][4 * g4 + 3]);
          *reinterpret_cast<float4*>(y + (base + tq) * D + dv) = out;
        }
      }
    }
  }  // tiles
}

}  // namespace

hipError_t launch_swa(const uint16_t* q, const uint16_t* k, const uint16_t* v, const uint16_t* sst,
                      const float* lam, const float* eta, const float* g, int B, int H, int T, int d,
                      int W, float scale, float* y, float* lse2, hipStream_t s) {
  const int n_tiles = (T + MQ - 1) / MQ;
  const int n_items = B * H * n_tiles;
  // as many workgroups as fit at once (LDS: one per CU at d = 128, two at d = 64), a multiple of NXCD
  const int per_xcd = (n_items + NXCD - 1) / NXCD;
  const int grid = NXCD * std::min(per_xcd, kComputeUnits / NXCD * (d == 128 ? 1 : 2));
  const float sl2 = scale * 1.4426950408889634f;
  const L2Args l2{sst, lam, eta, g, H};
  if (d == 128)
    hipLaunchKernelGGL(swa_kernel<128>, dim3(grid), dim3(NTHR), 0, s, q, k, v, l2, T, W, n_tiles, n_items,
                       sl2, y, lse2);
  else if (d == 64)
    hipLaunchKernelGGL(swa_kernel<64>, dim3(grid), dim3(NTHR), 0, s, q, k, v, l2, T, W, n_tiles, n_items,
                       sl2, y, lse2);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace tc

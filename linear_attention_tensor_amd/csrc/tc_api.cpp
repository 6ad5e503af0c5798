// tc_api.cpp — C ABI of libtc.so: argument checks, workspace sizing,
// dispatch to the gfx950 kernels, thread-local error messages.
//
// Every check runs before the first HIP call, so a rejected call launches
// nothing and needs no device.  Nothing throws across the ABI.
#include <hip/hip_runtime.h>

#include "../../include/tc.h"
#include "tc_kernels.hpp"
#include "tc_bwd_paths.hpp"

#include <stdarg.h>
#include <stdint.h>
#include <stdio.h>

#include <exception>
#include <mutex>

namespace {

thread_local char g_err[512] = "";
thread_local hipEvent_t g_prof_before = nullptr, g_prof_after = nullptr;

tc_status fail(tc_status st, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return st;
}

tc_status ok() {
  g_err[0] = '\0';
  return TC_OK;
}

tc_status from_hip(hipError_t e, const char* where) {
  if (e == hipSuccess) return ok();
  return fail(TC_ERR_HIP, "%s: %s", where, hipGetErrorString(e));
}

bool supported_d(int d) { return d == 16 || d == 32 || d == 64 || d == 128; }

// Checks shared by the sequence entry points.  Returns TC_OK when the shapes
// are valid and supported.
tc_status check_seq(const char* fn, int B, int H, int T, int dk, int dv, int chunk, tc_dtype dt) {
  if (B < 0 || H < 0 || T < 0) return fail(TC_ERR_INVALID_ARG, "%s: B, H, T must be >= 0 (got %d, %d, %d)", fn, B, H, T);
  if (dk <= 0 || dv <= 0) return fail(TC_ERR_INVALID_ARG, "%s: dk, dv must be > 0 (got %d, %d)", fn, dk, dv);
  if (dt != TC_F32 && dt != TC_BF16) return fail(TC_ERR_INVALID_ARG, "%s: unknown dtype %d", fn, (int)dt);
  if (chunk != 64) return fail(TC_ERR_UNSUPPORTED, "%s: chunk must be 64 (got %d)", fn, chunk);
  if (dk != dv || !supported_d(dk))
    return fail(TC_ERR_UNSUPPORTED, "%s: need dk == dv in {16, 32, 64, 128} (got %d, %d)", fn, dk, dv);
  // one (b, h) block of rows is addressed with 32-bit byte offsets
  if ((long long)T * dk >= (1LL << 29)) return fail(TC_ERR_UNSUPPORTED, "%s: T * d must be < 2^29", fn);
  if ((long long)B * H >= 65536) return fail(TC_ERR_UNSUPPORTED, "%s: B * H must be < 65536", fn);
  return TC_OK;
}

template <typename F>
tc_status guarded(const char* fn, F&& f) {
  try {
    const tc_status st = f();
    if (st == TC_OK || st == TC_ERR_HIP) g_prof_before = g_prof_after = nullptr;  // hook consumed
    return st;
  } catch (const std::exception& e) {
    return fail(TC_ERR_INTERNAL, "%s: %s", fn, e.what());
  } catch (...) {
    return fail(TC_ERR_INTERNAL, "%s: unknown exception", fn);
  }
}

}  // namespace

namespace tc {
void profile_mark_before(hipStream_t s) {
  if (g_prof_before != nullptr) (void)hipEventRecord(g_prof_before, s);
}
void profile_mark_after(hipStream_t s) {
  if (g_prof_after != nullptr) (void)hipEventRecord(g_prof_after, s);
}
}  // namespace tc

// The backward passes run on fp32 kernels; with bf16 inputs, q, k and v are
// widened to fp32 copies placed after the fp32 workspace (256-byte aligned).
static size_t round_up_256(size_t n) { return (n + 255) & ~(size_t)255; }
static size_t widened_bytes(int B, int H, int T, int d) { return round_up_256((size_t)B * H * T * d * sizeof(float)); }

// The fused layer and the window attention run on the bf16 MFMA kernels for
// bf16 inputs with d in {64, 128}, and on the fp32-arithmetic window kernel
// (plus, for the layer, the prefill scan) otherwise.
static bool fused_mfma_path(tc_dtype dt, int d) { return dt == TC_BF16 && (d == 64 || d == 128); }

// ---------------------------------------------------------------------------
// Scratch memory of tc_scan_forward_noalloc: a file-scope device array that
// each GPU the library runs on holds from module load to process end.  In
// host code `scratch` names a host-side stand-in, not device memory: the
// device address comes from hipGetSymbolAddress, once per device with that
// device current, and only that address is ever handed to a kernel.
constexpr size_t kScratchBytes = (size_t)32 << 20;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of the current device's copy of `scratch`.
tc_status current_scratch(const char* fn, void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(TC_ERR_HIP, "%s: hipGetDevice: %s", fn, hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices) return fail(TC_ERR_UNSUPPORTED, "%s: device %d out of range", fn, dev);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || p == nullptr)
      return fail(TC_ERR_HIP, "%s: hipGetSymbolAddress(scratch) on device %d: %s", fn, dev,
                  hipGetErrorString(e));
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return TC_OK;
}

}  // namespace

extern "C" {

tc_status tc_profile_next_call(hipEvent_t before, hipEvent_t after) {
  if ((before == nullptr) != (after == nullptr))
    return fail(TC_ERR_INVALID_ARG, "tc_profile_next_call: pass two events or none");
  g_prof_before = before;
  g_prof_after = after;
  return ok();
}

const char* tc_last_error(void) { return g_err; }

const char* tc_version(void) { return "libtc 0.1.0 (gfx950)"; }

size_t tc_scan_workspace_bytes(int B, int H, int T, int dk, int dv, int W, int chunk, tc_dtype dt) {
  if (check_seq("tc_scan_workspace_bytes", B, H, T, dk, dv, chunk, dt) != TC_OK) return SIZE_MAX;
  if (W < 1) {
    fail(TC_ERR_INVALID_ARG, "tc_scan_workspace_bytes: W must be >= 1 (got %d)", W);
    return SIZE_MAX;
  }
  ok();
  if (tc::scan_bf16_fast(dt == TC_BF16, dk, dv, T)) return tc::scan_bf16_ws_bytes(B, H, T, dk, W);
  return tc::scan_ws_bytes(tc::plan_scan(B, H, T, dk, dv, W), B, H, dk, dv);
}

tc_status tc_scan_forward(const void* q, const void* k, const void* v, tc_dtype dt,
                          const float* lam, const float* eta, int B, int H, int T, int dk, int dv,
                          int W, int chunk, float* m, float* A_final, void* ws, size_t ws_bytes,
                          hipStream_t s) {
  return guarded("tc_scan_forward", [&]() -> tc_status {
    const char* fn = "tc_scan_forward";
    tc_status st = check_seq(fn, B, H, T, dk, dv, chunk, dt);
    if (st != TC_OK) return st;
    if (W < 1) return fail(TC_ERR_INVALID_ARG, "%s: W must be >= 1 (got %d)", fn, W);
    if (B == 0 || H == 0) return ok();
    if (!lam || !eta) return fail(TC_ERR_INVALID_ARG, "%s: lam and eta must not be NULL", fn);
    if (T > 0 && (!q || !k || !v || !m))
      return fail(TC_ERR_INVALID_ARG, "%s: q, k, v, m must not be NULL", fn);
    const bool fast16 = tc::scan_bf16_fast(dt == TC_BF16, dk, dv, T);
    const size_t need = fast16 ? tc::scan_bf16_ws_bytes(B, H, T, dk, W)
                               : tc::scan_ws_bytes(tc::plan_scan(B, H, T, dk, dv, W), B, H, dk, dv);
    if (ws_bytes < need)
      return fail(TC_ERR_WORKSPACE, "%s: workspace %zu bytes < %zu needed", fn, ws_bytes, need);
    if (need > 0 && !ws) return fail(TC_ERR_INVALID_ARG, "%s: ws must not be NULL", fn);
    if (T == 0 && !A_final) return ok();
    if (fast16)
      return from_hip(tc::launch_tc_scan_bf16(q, k, v, lam, eta, B, H, T, dk, W, m, A_final, ws, s), fn);
    return from_hip(tc::launch_tc_scan(q, k, v, dt == TC_BF16, lam, eta, B, H, T, dk, dv, W, m,
                                       A_final, ws, s),
                    fn);
  });
}

tc_status tc_scan_forward_noalloc(const void* q, const void* k, const void* v, tc_dtype dt,
                                  const float* lam, const float* eta, int B, int H, int T, int dk,
                                  int dv, int W, int chunk, float* m, float* A_final, hipStream_t s) {
  return guarded("tc_scan_forward_noalloc", [&]() -> tc_status {
    const char* fn = "tc_scan_forward_noalloc";
    tc_status st = check_seq(fn, B, H, T, dk, dv, chunk, dt);
    if (st != TC_OK) return st;
    if (W < 1) return fail(TC_ERR_INVALID_ARG, "%s: W must be >= 1 (got %d)", fn, W);
    if (B == 0 || H == 0) return ok();
    if (!lam || !eta) return fail(TC_ERR_INVALID_ARG, "%s: lam and eta must not be NULL", fn);
    if (T > 0 && (!q || !k || !v || !m))
      return fail(TC_ERR_INVALID_ARG, "%s: q, k, v, m must not be NULL", fn);
    const bool fast16 = tc::scan_bf16_fast(dt == TC_BF16, dk, dv, T);
    const size_t need = fast16 ? tc::scan_bf16_ws_bytes(B, H, T, dk, W)
                               : tc::scan_ws_bytes(tc::plan_scan(B, H, T, dk, dv, W), B, H, dk, dv);
    if (need > kScratchBytes)
      return fail(TC_ERR_WORKSPACE,
                  "%s: this call needs %zu bytes of scratch, more than the %zu the library holds per "
                  "device; call tc_scan_forward with a workspace instead",
                  fn, need, kScratchBytes);
    if (T == 0 && !A_final) return ok();
    void* ws = nullptr;
    if (need > 0) {
      st = current_scratch(fn, &ws);
      if (st != TC_OK) return st;
    }
    // Every kernel below writes the scratch it reads (segment or tile states)
    // earlier in the same call, so the previous call's contents never matter.
    if (fast16)
      return from_hip(tc::launch_tc_scan_bf16(q, k, v, lam, eta, B, H, T, dk, W, m, A_final, ws, s), fn);
    return from_hip(tc::launch_tc_scan(q, k, v, dt == TC_BF16, lam, eta, B, H, T, dk, dv, W, m,
                                       A_final, ws, s),
                    fn);
  });
}

static tc_status check_scan_bwd(const char* fn, int B, int H, int T, int dk, int dv, int W, int chunk,
                                tc_dtype dt) {
  tc_status st = check_seq(fn, B, H, T, dk, dv, chunk, dt);
  if (st != TC_OK) return st;
  if (W < 1) return fail(TC_ERR_INVALID_ARG, "%s: W must be >= 1 (got %d)", fn, W);
  return TC_OK;
}

// d = 128: the read m = q A splits over halves of d_k and d_v into four
// d = 64 reads m^(a,b) (q, k columns 64a.., v, dm columns 64b..), whose
// gradients add: dq[:, a] and dk[:, a] sum over b, dv[:, b] over a, and the
// per-head terms over all four.  The d = 64 kernels read the halves in place
// (rows 128 floats apart) and add into the halves of the outputs, so the
// workspace is the d = 64 backward's (plus the widened copies for bf16).
//
// bf16 inputs with d in {64, 128}: the reverse direction (dk, dv) runs on the
// bf16 forward scan instead of the fp32 kernels.  For t >= i + W the weight of
// the pair (t, i) is eta lam^(t - W - i); with t' = T - 1 - t, i' = T - 1 - i
// that is eta lam^(i' - W - t') over t' <= i' - W, so on the time-reversed
// sequences (primed)
//   dv'_i' = sum_{t' <= i' - W} eta lam^(i' - W - t') <k'_i', q'_t'> dm'_t'  = read(q = k', k = q', v = dm'),
//   dk'_i' = sum_{t' <= i' - W} eta lam^(i' - W - t') <v'_i', dm'_t'> q'_t' = read(q = v', k = dm', v = q'),
// and rows i' < W (i >= T - W) are 0 in both.  The workspace then also holds
// q', k', v', dm' (bf16) and the scan's own workspace.
static bool scan_bwd_rev16(int d, tc_dtype dt, int T) { return dt == TC_BF16 && (d == 64 || d == 128) && T > 0; }
static size_t rev16_bytes(int B, int H, int T, int d) { return round_up_256((size_t)B * H * T * d * sizeof(uint16_t)); }

static size_t scan_bwd_need_fp32(int B, int H, int T, int d, int W, tc_dtype dt) {
  const size_t base = tc::scan_bwd_ws_bytes(B, H, T, d, W);
  if (d == 128) return (dt == TC_BF16 ? 3 * widened_bytes(B, H, T, d) : 0) + round_up_256(base);
  return dt == TC_BF16 ? round_up_256(base) + 3 * widened_bytes(B, H, T, d) : base;
}

static size_t scan_bwd_need(int B, int H, int T, int d, int W, tc_dtype dt) {
  const size_t fp32 = scan_bwd_need_fp32(B, H, T, d, W, dt);
  if (!scan_bwd_rev16(d, dt, T)) return fp32;
  return round_up_256(fp32) + 4 * rev16_bytes(B, H, T, d) + round_up_256(tc::scan_bf16_ws_bytes(B, H, T, d, W));
}

size_t tc_scan_backward_workspace_bytes(int B, int H, int T, int dk, int dv, int W, int chunk,
                                        tc_dtype dt) {
  if (check_scan_bwd("tc_scan_backward_workspace_bytes", B, H, T, dk, dv, W, chunk, dt) != TC_OK)
    return SIZE_MAX;
  ok();
  return scan_bwd_need(B, H, T, dk, W, dt);
}

tc_status tc_scan_backward(const void* q, const void* k, const void* v, tc_dtype dt, const float* lam,
                           const float* eta, const float* g, int B, int H, int T, int dk, int dv, int W,
                           int chunk, const float* dm, float* dq, float* dk_out, float* dv_out, float* dlam,
                           float* deta, float* dg, void* ws, size_t ws_bytes, hipStream_t s) {
  return guarded("tc_scan_backward", [&]() -> tc_status {
    const char* fn = "tc_scan_backward";
    tc_status st = check_scan_bwd(fn, B, H, T, dk, dv, W, chunk, dt);
    if (st != TC_OK) return st;
    if ((g == nullptr) != (dg == nullptr))
      return fail(TC_ERR_INVALID_ARG, "%s: g and dg are given together or not at all", fn);
    if (B == 0 || H == 0) return ok();
    if (!lam || !eta || !dlam || !deta)
      return fail(TC_ERR_INVALID_ARG, "%s: lam, eta, dlam, deta must not be NULL", fn);
    if (T > 0 && (!q || !k || !v || !dm || !dq || !dk_out || !dv_out))
      return fail(TC_ERR_INVALID_ARG, "%s: q, k, v, dm, dq, dk, dv must not be NULL", fn);
    const size_t need = scan_bwd_need(B, H, T, dk, W, dt);
    if (ws_bytes < need)
      return fail(TC_ERR_WORKSPACE, "%s: workspace %zu bytes < %zu needed", fn, ws_bytes, need);
    if (need > 0 && !ws) return fail(TC_ERR_INVALID_ARG, "%s: ws must not be NULL", fn);
    const float *q32 = static_cast<const float*>(q), *k32 = static_cast<const float*>(k),
                *v32 = static_cast<const float*>(v);
    // d = 128: the widened copies come first, then the workspace of the four-piece backward
    const size_t wide_off = dk == 128 ? 0 : round_up_256(tc::scan_bwd_ws_bytes(B, H, T, dk, W));
    if (dt == TC_BF16 && T > 0) {
      char* wide = static_cast<char*>(ws) + wide_off;
      float* tmp[3];
      const void* src[3] = {q, k, v};
      for (int i = 0; i < 3; ++i) {
        tmp[i] = reinterpret_cast<float*>(wide + i * widened_bytes(B, H, T, dk));
        const hipError_t e = tc::launch_widen_bf16(src[i], tmp[i], (long)B * H * T * dk, s);
        if (e != hipSuccess) return from_hip(e, fn);
      }
      q32 = tmp[0];
      k32 = tmp[1];
      v32 = tmp[2];
    }
    const bool rev16 = scan_bwd_rev16(dk, dt, T);
    char* w = static_cast<char*>(ws) + (dk == 128 && dt == TC_BF16 ? 3 * widened_bytes(B, H, T, dk) : 0);
    hipError_t e = rev16 ? tc::launch_tc_scan_backward_fwd_only(q32, k32, v32, lam, eta, g, B, H, T, dk, W, dm, dq,
                                                                 dlam, deta, dg, w, s)
                         : tc::launch_tc_scan_backward(q32, k32, v32, lam, eta, g, B, H, T, dk, W, dm, dq, dk_out,
                                                       dv_out, dlam, deta, dg, w, s);
    if (e != hipSuccess || !rev16) return from_hip(e, fn);
    // reverse direction on the bf16 scan (see scan_bwd_need)
    char* r = static_cast<char*>(ws) + round_up_256(scan_bwd_need_fp32(B, H, T, dk, W, dt));
    const size_t rb = rev16_bytes(B, H, T, dk);
    void *qr = r, *kr = r + rb, *vr = r + 2 * rb, *gr = r + 3 * rb, *sws = r + 4 * rb;
    const void* src[3] = {q, k, v};
    void* dst[3] = {qr, kr, vr};
    for (int i = 0; i < 3 && e == hipSuccess; ++i) e = tc::launch_reverse_rows_bf16(src[i], dst[i], B * H, T, dk, s);
    if (e == hipSuccess) e = tc::launch_reverse_rows_f32(dm, g, H, gr, B * H, T, dk, s);
    if (e == hipSuccess)
      e = tc::launch_tc_scan_bf16_rev_out(kr, qr, gr, lam, eta, B, H, T, dk, W, dv_out, nullptr, sws, s);
    if (e == hipSuccess)
      e = tc::launch_tc_scan_bf16_rev_out(vr, gr, qr, lam, eta, B, H, T, dk, W, dk_out, nullptr, sws, s);
    return from_hip(e, fn);
  });
}

static size_t fused_bwd_need(int B, int H, int T, int d, int W, tc_dtype dt) {
  return round_up_256(scan_bwd_need(B, H, T, d, W, dt)) + tc::window_bwd_ws_bytes(B, H, T, d, dt == TC_BF16);
}

size_t tc_fused_layer_backward_workspace_bytes(int B, int H, int T, int dk, int dv, int W, int chunk, tc_dtype dt) {
  if (check_scan_bwd("tc_fused_layer_backward_workspace_bytes", B, H, T, dk, dv, W, chunk, dt) != TC_OK)
    return SIZE_MAX;
  ok();
  return fused_bwd_need(B, H, T, dk, W, dt);
}

tc_status tc_fused_layer_backward(const void* q, const void* k, const void* v, tc_dtype dt, const float* lam,
                                  const float* eta, const float* g, int B, int H, int T, int dk, int dv, int W,
                                  int chunk, float softmax_scale, const float* dy, float* dq, float* dk_out,
                                  float* dv_out, float* dlam, float* deta, float* dg, void* ws, size_t ws_bytes,
                                  hipStream_t s) {
  return guarded("tc_fused_layer_backward", [&]() -> tc_status {
    const char* fn = "tc_fused_layer_backward";
    tc_status st = check_scan_bwd(fn, B, H, T, dk, dv, W, chunk, dt);
    if (st != TC_OK) return st;
    if (!(softmax_scale > 0.f) || softmax_scale > 1e30f)
      return fail(TC_ERR_INVALID_ARG, "%s: softmax_scale must be finite and > 0", fn);
    if (B == 0 || H == 0) return ok();
    if (!lam || !eta || !g || !dlam || !deta || !dg)
      return fail(TC_ERR_INVALID_ARG, "%s: lam, eta, g, dlam, deta, dg must not be NULL", fn);
    if (T > 0 && (!q || !k || !v || !dy || !dq || !dk_out || !dv_out))
      return fail(TC_ERR_INVALID_ARG, "%s: q, k, v, dy, dq, dk, dv must not be NULL", fn);
    const size_t need = fused_bwd_need(B, H, T, dk, W, dt);
    if (ws_bytes < need) return fail(TC_ERR_WORKSPACE, "%s: workspace %zu bytes < %zu needed", fn, ws_bytes, need);
    if (!ws) return fail(TC_ERR_INVALID_ARG, "%s: ws must not be NULL", fn);
    // the L2 branch (gated read) writes dq, dk, dv, dlam, deta, dg; the window
    // softmax's gradients are then added to dq, dk, dv
    st = tc_scan_backward(q, k, v, dt, lam, eta, g, B, H, T, dk, dv, W, chunk, dy, dq, dk_out, dv_out, dlam, deta,
                          dg, ws, round_up_256(scan_bwd_need(B, H, T, dk, W, dt)), s);
    if (st != TC_OK) return st;
    void* wws = static_cast<char*>(ws) + round_up_256(scan_bwd_need(B, H, T, dk, W, dt));
    return from_hip(tc::launch_window_backward(q, k, v, dt == TC_BF16, dy, B, H, T, dk, W, softmax_scale, wws, true,
                                               dq, dk_out, dv_out, s),
                    fn);
  });
}

tc_status tc_decode_step(const void* q, const void* k, const void* v, tc_dtype dt, void* ring_k,
                         void* ring_v, float* A, const float* lam, const float* eta,
                         const int64_t* pos, int B, int H, int dk, int dv, int W, float* m,
                         hipStream_t s) {
  return guarded("tc_decode_step", [&]() -> tc_status {
    const char* fn = "tc_decode_step";
    tc_status st = check_seq(fn, B, H, 1, dk, dv, 64, dt);
    if (st != TC_OK) return st;
    if (W < 1) return fail(TC_ERR_INVALID_ARG, "%s: W must be >= 1 (got %d)", fn, W);
    if ((long long)W * dk >= (1LL << 31)) return fail(TC_ERR_UNSUPPORTED, "%s: W * d too large", fn);
    if (B == 0 || H == 0) return ok();
    if (!q || !k || !v || !ring_k || !ring_v || !A || !lam || !eta || !pos || !m)
      return fail(TC_ERR_INVALID_ARG, "%s: a required pointer is NULL", fn);
    return from_hip(tc::launch_tc_decode(q, k, v, dt == TC_BF16, ring_k, ring_v, A, lam, eta, pos,
                                         B, H, dk, dv, W, m, s),
                    fn);
  });
}

tc_status tc_decode_layer_step(const void* q, const void* k, const void* v, tc_dtype dt,
                               void* ring_k, void* ring_v, float* A, const float* lam,
                               const float* eta, const float* g, const int64_t* pos, int B, int H,
                               int dk, int dv, int W, float softmax_scale, float* y, hipStream_t s) {
  return guarded("tc_decode_layer_step", [&]() -> tc_status {
    const char* fn = "tc_decode_layer_step";
    tc_status st = check_seq(fn, B, H, 1, dk, dv, 64, dt);
    if (st != TC_OK) return st;
    if (W < 1) return fail(TC_ERR_INVALID_ARG, "%s: W must be >= 1 (got %d)", fn, W);
    if ((long long)W * dk >= (1LL << 31)) return fail(TC_ERR_UNSUPPORTED, "%s: W * d too large", fn);
    if (!(softmax_scale > 0.f) || softmax_scale > 1e30f)
      return fail(TC_ERR_INVALID_ARG, "%s: softmax_scale must be finite and > 0", fn);
    if (B == 0 || H == 0) return ok();
    if (!q || !k || !v || !ring_k || !ring_v || !A || !lam || !eta || !g || !pos || !y)
      return fail(TC_ERR_INVALID_ARG, "%s: a required pointer is NULL", fn);
    return from_hip(tc::launch_tc_decode_layer(q, k, v, dt == TC_BF16, ring_k, ring_v, A, lam, eta, g,
                                               pos, B, H, dk, W, softmax_scale, y, s),
                    fn);
  });
}

size_t tc_fused_workspace_bytes(int B, int H, int T, int dk, int dv, int W, int chunk, tc_dtype dt) {
  const char* fn = "tc_fused_workspace_bytes";
  if (check_seq(fn, B, H, T, dk, dv, chunk, dt) != TC_OK) return SIZE_MAX;
  if (W < 1) {
    fail(TC_ERR_INVALID_ARG, "%s: W must be >= 1 (got %d)", fn, W);
    return SIZE_MAX;
  }
  ok();
  if (fused_mfma_path(dt, dk)) return tc::fused_ws_bytes(B, H, T, dk, dv, W);
  return tc::scan_ws_bytes(tc::plan_scan(B, H, T, dk, dv, W), B, H, dk, dv);
}

tc_status tc_fused_layer(const void* q, const void* k, const void* v, tc_dtype dt,
                         const float* lam, const float* eta, const float* g, int B, int H, int T,
                         int dk, int dv, int W, int chunk, float softmax_scale, float* y,
                         float* A_final, void* ws, size_t ws_bytes, hipStream_t s) {
  return guarded("tc_fused_layer", [&]() -> tc_status {
    const char* fn = "tc_fused_layer";
    tc_status st = check_seq(fn, B, H, T, dk, dv, chunk, dt);
    if (st != TC_OK) return st;
    if (W < 1) return fail(TC_ERR_INVALID_ARG, "%s: W must be >= 1 (got %d)", fn, W);
    if (!(softmax_scale > 0.f) || softmax_scale > 1e30f)
      return fail(TC_ERR_INVALID_ARG, "%s: softmax_scale must be finite and > 0", fn);
    if (B == 0 || H == 0) return ok();
    if (!lam || !eta || !g) return fail(TC_ERR_INVALID_ARG, "%s: lam, eta, g must not be NULL", fn);
    if (T > 0 && (!q || !k || !v || !y))
      return fail(TC_ERR_INVALID_ARG, "%s: q, k, v, y must not be NULL", fn);
    const bool mfma = fused_mfma_path(dt, dk);
    const size_t need = mfma ? tc::fused_ws_bytes(B, H, T, dk, dv, W)
                             : tc::scan_ws_bytes(tc::plan_scan(B, H, T, dk, dv, W), B, H, dk, dv);
    if (ws_bytes < need)
      return fail(TC_ERR_WORKSPACE, "%s: workspace %zu bytes < %zu needed", fn, ws_bytes, need);
    if (need > 0 && !ws) return fail(TC_ERR_INVALID_ARG, "%s: ws must not be NULL", fn);
    if (T == 0) {
      if (!A_final) return ok();
      return from_hip(tc::launch_tc_scan(q, k, v, true, lam, eta, B, H, 0, dk, dv, W, y, A_final,
                                         ws, s),
                      fn);
    }
    if (mfma)
      return from_hip(tc::launch_tc_fused(q, k, v, lam, eta, g, B, H, T, dk, W, softmax_scale, y,
                                          A_final, ws, s),
                      fn);
    // the L2 read into y (rows t < W are 0), then y = window softmax + sigmoid(g) y
    hipError_t e = tc::launch_tc_scan(q, k, v, dt == TC_BF16, lam, eta, B, H, T, dk, dv, W, y, A_final, ws, s);
    if (e != hipSuccess) return from_hip(e, fn);
    tc::profile_mark_before(s);
    e = tc::launch_window(q, k, v, dt == TC_BF16, B, H, T, dk, W, softmax_scale, g, y, s);
    tc::profile_mark_after(s);
    return from_hip(e, fn);
  });
}

tc_status tc_window_attention(const void* q, const void* k, const void* v, tc_dtype dt, int B, int H, int T,
                              int dk, int dv, int W, float softmax_scale, float* y, hipStream_t s) {
  return guarded("tc_window_attention", [&]() -> tc_status {
    const char* fn = "tc_window_attention";
    tc_status st = check_seq(fn, B, H, T, dk, dv, 64, dt);
    if (st != TC_OK) return st;
    if (W < 1) return fail(TC_ERR_INVALID_ARG, "%s: W must be >= 1 (got %d)", fn, W);
    if (!(softmax_scale > 0.f) || softmax_scale > 1e30f)
      return fail(TC_ERR_INVALID_ARG, "%s: softmax_scale must be finite and > 0", fn);
    if (B == 0 || H == 0 || T == 0) return ok();
    if (!q || !k || !v || !y) return fail(TC_ERR_INVALID_ARG, "%s: q, k, v, y must not be NULL", fn);
    if (fused_mfma_path(dt, dk)) {
      tc::profile_mark_before(s);
      const hipError_t e = tc::launch_swa(static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k),
                                          static_cast<const uint16_t*>(v), nullptr, nullptr, nullptr, nullptr, B,
                                          H, T, dk, W, softmax_scale, y, nullptr, s);
      tc::profile_mark_after(s);
      return from_hip(e, fn);
    }
    tc::profile_mark_before(s);
    const hipError_t e = tc::launch_window(q, k, v, dt == TC_BF16, B, H, T, dk, W, softmax_scale, nullptr, y, s);
    tc::profile_mark_after(s);
    return from_hip(e, fn);
  });
}

size_t tc_window_attention_backward_workspace_bytes(int B, int H, int T, int dk, int dv, int W, tc_dtype dt) {
  const char* fn = "tc_window_attention_backward_workspace_bytes";
  if (check_seq(fn, B, H, T, dk, dv, 64, dt) != TC_OK) return SIZE_MAX;
  if (W < 1) {
    fail(TC_ERR_INVALID_ARG, "%s: W must be >= 1 (got %d)", fn, W);
    return SIZE_MAX;
  }
  ok();
  return tc::window_bwd_ws_bytes(B, H, T, dk, dt == TC_BF16);
}

tc_status tc_window_attention_backward(const void* q, const void* k, const void* v, tc_dtype dt, int B, int H, int T,
                                       int dk, int dv, int W, float softmax_scale, const float* dy, float* dq,
                                       float* dk_out, float* dv_out, void* ws, size_t ws_bytes, hipStream_t s) {
  return guarded("tc_window_attention_backward", [&]() -> tc_status {
    const char* fn = "tc_window_attention_backward";
    tc_status st = check_seq(fn, B, H, T, dk, dv, 64, dt);
    if (st != TC_OK) return st;
    if (W < 1) return fail(TC_ERR_INVALID_ARG, "%s: W must be >= 1 (got %d)", fn, W);
    if (!(softmax_scale > 0.f) || softmax_scale > 1e30f)
      return fail(TC_ERR_INVALID_ARG, "%s: softmax_scale must be finite and > 0", fn);
    if (B == 0 || H == 0 || T == 0) return ok();
    if (!q || !k || !v || !dy || !dq || !dk_out || !dv_out)
      return fail(TC_ERR_INVALID_ARG, "%s: q, k, v, dy, dq, dk, dv must not be NULL", fn);
    const size_t need = tc::window_bwd_ws_bytes(B, H, T, dk, dt == TC_BF16);
    if (ws_bytes < need) return fail(TC_ERR_WORKSPACE, "%s: workspace %zu bytes < %zu needed", fn, ws_bytes, need);
    if (!ws) return fail(TC_ERR_INVALID_ARG, "%s: ws must not be NULL", fn);
    return from_hip(tc::launch_window_backward(q, k, v, dt == TC_BF16, dy, B, H, T, dk, W, softmax_scale, ws, false,
                                               dq, dk_out, dv_out, s),
                    fn);
  });
}

size_t delta_scan_workspace_bytes(int B, int H, int T, int dk, int dv, int chunk, tc_dtype dt) {
  if (check_seq("delta_scan_workspace_bytes", B, H, T, dk, dv, chunk, dt) != TC_OK) return SIZE_MAX;
  ok();
  return tc::delta_ws_bytes(B, H, T, dk, dv, dt == TC_BF16);
}

tc_status delta_scan_forward(const void* q, const void* k, const void* v, tc_dtype dt,
                             const float* beta, int B, int H, int T, int dk, int dv, int chunk,
                             const float* S0, float* o, float* S_final, void* ws, size_t ws_bytes,
                             hipStream_t s) {
  return guarded("delta_scan_forward", [&]() -> tc_status {
    const char* fn = "delta_scan_forward";
    tc_status st = check_seq(fn, B, H, T, dk, dv, chunk, dt);
    if (st != TC_OK) return st;
    if (B == 0 || H == 0) return ok();
    if (T > 0 && (!q || !k || !v || !beta || !o))
      return fail(TC_ERR_INVALID_ARG, "%s: q, k, v, beta, o must not be NULL", fn);
    const size_t need = tc::delta_ws_bytes(B, H, T, dk, dv, dt == TC_BF16);
    if (ws_bytes < need)
      return fail(TC_ERR_WORKSPACE, "%s: workspace %zu bytes < %zu needed", fn, ws_bytes, need);
    if (need > 0 && !ws) return fail(TC_ERR_INVALID_ARG, "%s: ws must not be NULL", fn);
    if (T == 0 && !S_final) return ok();
    return from_hip(tc::launch_delta_scan(q, k, v, dt == TC_BF16, beta, B, H, T, dk, dv, S0, o,
                                          S_final, ws, s),
                    fn);
  });
}

static tc_status check_delta_bwd(const char* fn, int B, int H, int T, int dk, int dv, int chunk, tc_dtype dt) {
  tc_status st = check_seq(fn, B, H, T, dk, dv, chunk, dt);
  if (st != TC_OK) return st;
  if (dk != 16 && dk != 32 && dk != 64 && dk != 128)
    return fail(TC_ERR_UNSUPPORTED, "%s: the backward takes d in {16, 32, 64, 128}", fn);
  return TC_OK;
}

static size_t delta_bwd_need(int B, int H, int T, int d, tc_dtype dt) {
  const size_t base = tc::delta_bwd_ws_bytes(B, H, T, d);
  return dt == TC_BF16 ? round_up_256(base) + 3 * widened_bytes(B, H, T, d) : base;
}

size_t delta_scan_backward_workspace_bytes(int B, int H, int T, int dk, int dv, int chunk, tc_dtype dt) {
  if (check_delta_bwd("delta_scan_backward_workspace_bytes", B, H, T, dk, dv, chunk, dt) != TC_OK)
    return SIZE_MAX;
  ok();
  return delta_bwd_need(B, H, T, dk, dt);
}

tc_status delta_scan_backward(const void* q, const void* k, const void* v, tc_dtype dt, const float* beta,
                              int B, int H, int T, int dk, int dv, int chunk, const float* S0,
                              const float* d_o, const float* dS_final, float* dq, float* dk_out,
                              float* dv_out, float* dbeta, float* dS0, void* ws, size_t ws_bytes,
                              hipStream_t s) {
  return guarded("delta_scan_backward", [&]() -> tc_status {
    const char* fn = "delta_scan_backward";
    tc_status st = check_delta_bwd(fn, B, H, T, dk, dv, chunk, dt);
    if (st != TC_OK) return st;
    if (B == 0 || H == 0) return ok();
    if (T > 0 && (!q || !k || !v || !beta || !d_o || !dq || !dk_out || !dv_out || !dbeta))
      return fail(TC_ERR_INVALID_ARG, "%s: q, k, v, beta, do, dq, dk, dv, dbeta must not be NULL", fn);
    const size_t need = delta_bwd_need(B, H, T, dk, dt);
    if (ws_bytes < need)
      return fail(TC_ERR_WORKSPACE, "%s: workspace %zu bytes < %zu needed", fn, ws_bytes, need);
    if (need > 0 && !ws) return fail(TC_ERR_INVALID_ARG, "%s: ws must not be NULL", fn);
    if (T == 0 && !dS0) return ok();
    const float *q32 = static_cast<const float*>(q), *k32 = static_cast<const float*>(k),
                *v32 = static_cast<const float*>(v);
    if (dt == TC_BF16 && T > 0) {
      char* wide = static_cast<char*>(ws) + round_up_256(tc::delta_bwd_ws_bytes(B, H, T, dk));
      float* tmp[3];
      const void* src[3] = {q, k, v};
      for (int i = 0; i < 3; ++i) {
        tmp[i] = reinterpret_cast<float*>(wide + i * widened_bytes(B, H, T, dk));
        const hipError_t e = tc::launch_widen_bf16(src[i], tmp[i], (long)B * H * T * dk, s);
        if (e != hipSuccess) return from_hip(e, fn);
      }
      q32 = tmp[0];
      k32 = tmp[1];
      v32 = tmp[2];
    }
    return from_hip(tc::launch_delta_backward(q32, k32, v32, beta, B, H, T, dk, S0, d_o, dS_final, dq, dk_out,
                                              dv_out, dbeta, dS0, ws, s),
                    fn);
  });
}

static tc_status check_mem_d(const char* fn, int d) {
  if (d != 32 && d != 64 && d != 128) return fail(TC_ERR_UNSUPPORTED, "%s: d must be 32, 64 or 128 (got %d)", fn, d);
  return TC_OK;
}

static tc_status check_hebbian(const char* fn, int F, int n_values, int m, int d) {
  if (F < 1 || n_values < 1 || m < 1)
    return fail(TC_ERR_INVALID_ARG, "%s: F, n_values and m must be >= 1 (got %d, %d, %d)", fn, F, n_values, m);
  if (m % 64 != 0) return fail(TC_ERR_UNSUPPORTED, "%s: m must be a multiple of 64 (got %d)", fn, m);
  if ((long long)F * d >= (1LL << 31) || (long long)m * d >= (1LL << 31))
    return fail(TC_ERR_UNSUPPORTED, "%s: sizes too large", fn);
  return check_mem_d(fn, d);
}

size_t hebbian_workspace_bytes(int F, int m, int d) {
  if (check_hebbian("hebbian_workspace_bytes", F, 1, m, d) != TC_OK) return SIZE_MAX;
  ok();
  return tc::hebbian_ws_bytes(F, m, d);
}

tc_status hebbian_write(const float* K, const float* V, const int32_t* f, int F, int n_values, const float* A,
                        const float* G, int m, int d, float* Bt, void* ws, size_t ws_bytes, hipStream_t s) {
  return guarded("hebbian_write", [&]() -> tc_status {
    const char* fn = "hebbian_write";
    tc_status st = check_hebbian(fn, F, n_values, m, d);
    if (st != TC_OK) return st;
    if (!K || !V || !f || !A || !G || !Bt || !ws)
      return fail(TC_ERR_INVALID_ARG, "%s: a required pointer is NULL", fn);
    const size_t need = tc::hebbian_ws_bytes(F, m, d);
    if (ws_bytes < need)
      return fail(TC_ERR_WORKSPACE, "%s: workspace %zu bytes < %zu needed", fn, ws_bytes, need);
    return from_hip(tc::launch_hebbian_write(K, V, f, F, n_values, A, G, m, d, Bt, ws, s), fn);
  });
}

tc_status hebbian_read(const float* Q, int n, const float* A, const float* G, const float* Bt, int m, int d,
                       float* out, hipStream_t s) {
  return guarded("hebbian_read", [&]() -> tc_status {
    const char* fn = "hebbian_read";
    tc_status st = check_hebbian(fn, 1, 1, m, d);
    if (st != TC_OK) return st;
    if (n < 0) return fail(TC_ERR_INVALID_ARG, "%s: n must be >= 0 (got %d)", fn, n);
    if ((long long)n * d >= (1LL << 31)) return fail(TC_ERR_UNSUPPORTED, "%s: n * d too large", fn);
    if (n == 0) return ok();
    if (!Q || !A || !G || !Bt || !out) return fail(TC_ERR_INVALID_ARG, "%s: a required pointer is NULL", fn);
    return from_hip(tc::launch_hebbian_read(Q, n, A, G, Bt, m, d, out, s), fn);
  });
}

tc_status tc_memory_read(const float* Q, const float* A, int groups, int n, int d, float* out, hipStream_t s) {
  return guarded("tc_memory_read", [&]() -> tc_status {
    const char* fn = "tc_memory_read";
    tc_status st = check_mem_d(fn, d);
    if (st != TC_OK) return st;
    if (groups < 0 || n < 0) return fail(TC_ERR_INVALID_ARG, "%s: groups and n must be >= 0", fn);
    if (groups > 65535) return fail(TC_ERR_UNSUPPORTED, "%s: at most 65535 groups", fn);
    if ((long long)groups * n * d >= (1LL << 31)) return fail(TC_ERR_UNSUPPORTED, "%s: sizes too large", fn);
    if (groups == 0 || n == 0) return ok();
    if (!Q || !A || !out) return fail(TC_ERR_INVALID_ARG, "%s: a required pointer is NULL", fn);
    return from_hip(tc::launch_memory_read(Q, A, groups, n, d, out, s), fn);
  });
}

tc_status recall_argmax(const float* R, const float* V, int groups, int nq, int nc, int d, int32_t* arg,
                        float* best, hipStream_t s) {
  return guarded("recall_argmax", [&]() -> tc_status {
    const char* fn = "recall_argmax";
    tc_status st = check_mem_d(fn, d);
    if (st != TC_OK) return st;
    if (groups < 0 || nq < 0 || nc < 1)
      return fail(TC_ERR_INVALID_ARG, "%s: groups, nq must be >= 0 and nc >= 1", fn);
    if (groups > 65535) return fail(TC_ERR_UNSUPPORTED, "%s: at most 65535 groups", fn);
    if ((long long)groups * nq * d >= (1LL << 31) || (long long)groups * nc * d >= (1LL << 31))
      return fail(TC_ERR_UNSUPPORTED, "%s: sizes too large", fn);
    if (groups == 0 || nq == 0) return ok();
    if (!R || !V || !arg) return fail(TC_ERR_INVALID_ARG, "%s: R, V, arg must not be NULL", fn);
    return from_hip(tc::launch_recall_argmax(R, V, groups, nq, nc, d, arg, best, s), fn);
  });
}

}  // extern "C"

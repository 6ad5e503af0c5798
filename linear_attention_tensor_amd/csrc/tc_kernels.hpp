// tc_kernels.hpp — host-side launchers implemented in the .hip files.
// Argument checking happens in tc_api.cpp before any of these is called;
// every launcher returns the hipError_t of its last launch.
#pragma once

#include <hip/hip_runtime_api.h>
#include <stddef.h>
#include <stdint.h>

namespace tc {

// Segmenting of the prefill scan: the active positions s = t - W in [0, T-W)
// are split into chunks of 64 and the chunks into segments of `seg_chunks`;
// one workgroup carries the state through one segment.
struct ScanPlan {
  int n_act;       // T - W (>= 0)
  int n_chunks;    // ceil(n_act / 64)
  int seg_chunks;  // chunks per segment
  int n_seg;       // segments per (b, h)
};
ScanPlan plan_scan(int B, int H, int T, int dk, int dv, int W);
size_t scan_ws_bytes(const ScanPlan& p, int B, int H, int dk, int dv);
// Backward of the read (fp32 inputs, d = dk = dv in {16, 32, 64, 128}; d = 128
// runs as four d = 64 pieces over the column halves).
size_t scan_bwd_ws_bytes(int B, int H, int T, int d, int W);
hipError_t launch_tc_scan_backward(const float* q, const float* k, const float* v, const float* lam,
                                   const float* eta, const float* g, int B, int H, int T, int d, int W,
                                   const float* dm, float* dq, float* dk, float* dv, float* dlam,
                                   float* deta, float* dg, void* ws, hipStream_t s);

// bf16 -> fp32 of n elements (tc_convert.hip); any alignment, any n.
hipError_t launch_widen_bf16(const void* in, float* out, long n, hipStream_t s);

hipError_t launch_tc_scan(const void* q, const void* k, const void* v, bool bf16,
                          const float* lam, const float* eta, int B, int H, int T, int dk, int dv,
                          int W, float* m, float* A_final, void* ws, hipStream_t s);

hipError_t launch_tc_decode(const void* q, const void* k, const void* v, bool bf16, void* ring_k,
                            void* ring_v, float* A, const float* lam, const float* eta,
                            const int64_t* pos, int B, int H, int dk, int dv, int W, float* m,
                            hipStream_t s);
// Full decode step of the layer (L1 ring softmax + L2 step + gate); d = dk = dv.
hipError_t launch_tc_decode_layer(const void* q, const void* k, const void* v, bool bf16,
                                  void* ring_k, void* ring_v, float* A, const float* lam,
                                  const float* eta, const float* g, const int64_t* pos, int B,
                                  int H, int d, int W, float scale, float* y, hipStream_t s);

// Benchmark timing hook (armed by tc_profile_next_call, tc_api.cpp): record
// the armed events around an entry point's main kernel, on its stream.
void profile_mark_before(hipStream_t s);
void profile_mark_after(hipStream_t s);

size_t fused_ws_bytes(int B, int H, int T, int dk, int dv, int W);
// tc_scan_forward with bf16 inputs and d in {64, 128} runs on the fused
// layer's pre-pass (without the V^T copy) and prefix plus an L2-read kernel
// (tc_fused.hip); its workspace is scan_bf16_ws_bytes.
size_t scan_bf16_ws_bytes(int B, int H, int T, int d, int W);
bool scan_bf16_fast(bool bf16, int dk, int dv, int T);
hipError_t launch_tc_scan_bf16(const void* q, const void* k, const void* v, const float* lam, const float* eta,
                               int B, int H, int T, int d, int W, float* m, float* A_final, void* ws, hipStream_t s);
hipError_t launch_tc_fused(const void* q, const void* k, const void* v, const float* lam,
                           const float* eta, const float* g, int B, int H, int T, int d, int W,
                           float scale, float* y, float* A_final, void* ws, hipStream_t s);
// Exact window softmax in fp32 arithmetic (tc_window.hip): fp32 inputs or
// bf16 with d in {16, 32}.  With g, y already holds the L2 read m and becomes
// y_local + sigmoid(g[h]) m; without, y = y_local.
hipError_t launch_window(const void* q, const void* k, const void* v, bool bf16, int B, int H, int T, int d, int W,
                         float scale, const float* g, float* y, hipStream_t s);
// Backward of the exact window softmax: dq, dk, dv of sum <dy, y_local>; with
// accumulate they are added to what the buffers hold.  bf16 inputs with d in
// {64, 128} run on bf16 MFMA (tc_window_bwd_mfma.hip: ws holds y_local fp32,
// dy as bf16 and the (log-sum-exp, <dy, y>) pairs), everything else in fp32
// arithmetic (tc_window_bwd.hip: ws holds the log-sum-exp and <dy, y>).
size_t window_bwd_ws_bytes(int B, int H, int T, int d, bool bf16);
bool window_bwd_mfma(bool bf16, int d);
size_t window_bwd_mfma_ws_bytes(int B, int H, int T, int d);
hipError_t launch_window_backward_mfma(const void* q, const void* k, const void* v, const float* dy, int B, int H,
                                       int T, int d, int W, float scale, void* ws, bool accumulate, float* dq,
                                       float* dk, float* dv, hipStream_t s);
hipError_t launch_window_backward(const void* q, const void* k, const void* v, bool bf16, const float* dy, int B,
                                  int H, int T, int d, int W, float scale, void* ws, bool accumulate, float* dq,
                                  float* dk, float* dv, hipStream_t s);
// Main kernel of the fused layer (tc_swa.hip): q, k, v rows [B*H][T][d] bf16,
// sst the entering state of every 256-query tile
// ([B*H][ceil(T/256)][d][d] bf16, S^T) or nullptr for no L2 term; lse2, when
// not nullptr, receives log2 of every query's softmax denominator in the
// units exp2(scale log2(e) s) at lse2[2 row].
hipError_t launch_swa(const uint16_t* q, const uint16_t* k, const uint16_t* v, const uint16_t* sst,
                      const float* lam, const float* eta, const float* g, int B, int H, int T, int d,
                      int W, float scale, float* y, float* lse2, hipStream_t s);

size_t delta_ws_bytes(int B, int H, int T, int dk, int dv, bool bf16);
hipError_t launch_delta_scan(const void* q, const void* k, const void* v, bool bf16,
                             const float* beta, int B, int H, int T, int dk, int dv,
                             const float* S0, float* o, float* S_final, void* ws, hipStream_t s);
// bf16 inputs with d in {64, 128} (delta_bf16.hip): bf16 MFMA with split
// operands; launch_delta_scan dispatches to it.
bool delta_bf16_supported(bool bf16, int d);
// Outer-product fact memories and recall (tc_memory.hip): fp32, d in {32, 64, 128}.
size_t hebbian_ws_bytes(int F, int m, int d);
hipError_t launch_hebbian_write(const float* K, const float* V, const int* f, int F, int n_values, const float* A,
                                const float* G, int m, int d, float* Bt, void* ws, hipStream_t s);
hipError_t launch_hebbian_read(const float* Q, int n, const float* A, const float* G, const float* Bt, int m, int d,
                               float* out, hipStream_t s);
hipError_t launch_memory_read(const float* Q, const float* A, int groups, int n, int d, float* out, hipStream_t s);
hipError_t launch_recall_argmax(const float* R, const float* V, int groups, int nq, int nc, int d, int* arg,
                                float* best, hipStream_t s);
// The delta-rule forward for fp32 inputs with d in {16, 32, 64, 128} on the
// backward's chunk preparation (delta_bwd.hip); launch_delta_scan dispatches to it.
bool delta_f32_fast(bool bf16, int d);
size_t delta_f32_ws_bytes(int B, int H, int T, int d);
hipError_t launch_delta_f32(const float* q, const float* k, const float* v, const float* beta, int B, int H, int T,
                            int d, const float* S0, float* o, float* S_final, void* ws, hipStream_t s);
// Backward of the delta-rule scan (delta_bwd.hip): fp32 inputs, d in {16, 32, 64, 128}.
size_t delta_bwd_ws_bytes(int B, int H, int T, int d);
hipError_t launch_delta_backward(const float* q, const float* k, const float* v, const float* beta, int B, int H,
                                 int T, int d, const float* S0, const float* dO, const float* dSf, float* dq,
                                 float* dk, float* dv, float* dbeta, float* dS0, void* ws, hipStream_t s);
size_t delta_bf16_ws_bytes(int B, int H, int T, int d);
hipError_t launch_delta_bf16(const void* q, const void* k, const void* v, const float* beta, int B,
                             int H, int T, int d, const float* S0, float* o, float* S_final, void* ws,
                             hipStream_t s);

}  // namespace tc

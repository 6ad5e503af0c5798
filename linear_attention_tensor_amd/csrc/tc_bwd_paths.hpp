// tc_bwd_paths.hpp — entry points of the L2-read backward's bf16 path: the
// reverse direction (dk, dv) as forward reads of the time-reversed sequences.
#pragma once

#include "tc_kernels.hpp"

namespace tc {

// Time reversal of BH sequences of T rows of d elements (tc_convert.hip): row
// t goes to row T - 1 - t of out, as bf16; the fp32 form multiplies the rows
// of head bh % H by sigmoid(gate[bh % H]) (gate may be NULL: factor 1) and
// rounds to the nearest even bf16.
hipError_t launch_reverse_rows_bf16(const void* in, void* out, int BH, int T, int d, hipStream_t s);
hipError_t launch_reverse_rows_f32(const float* in, const float* gate, int H, void* out, int BH, int T, int d,
                                   hipStream_t s);

// launch_tc_scan_bf16 with the read of position t stored in row T - 1 - t of m
// (tc_fused.hip); same workspace (scan_bf16_ws_bytes).
hipError_t launch_tc_scan_bf16_rev_out(const void* q, const void* k, const void* v, const float* lam,
                                       const float* eta, int B, int H, int T, int d, int W, float* m, float* A_final,
                                       void* ws, hipStream_t s);

// launch_tc_scan_backward without the reverse direction: dq, dlam, deta (and
// dg) only; dk and dv are not touched (tc_scan.hip).
hipError_t launch_tc_scan_backward_fwd_only(const float* q, const float* k, const float* v, const float* lam,
                                            const float* eta, const float* g, int B, int H, int T, int d, int W,
                                            const float* dm, float* dq, float* dlam, float* deta, float* dg, void* ws,
                                            hipStream_t s);

}  // namespace tc

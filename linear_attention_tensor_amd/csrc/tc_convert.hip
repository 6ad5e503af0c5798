// tc_convert.hip — layout and precision conversions for the backward passes.
//
// Widening: the backward passes run on fp32 kernels; bf16 inputs are widened
// first into the caller's workspace.  Every bf16 value is exact in fp32, so
// the gradients are those of the bf16 values, at fp32 accuracy.
//
// Time reversal: the reverse direction of the read's backward with bf16
// inputs is a forward scan of the time-reversed sequences (row t of every
// (b, h) sequence moved to row T - 1 - t), so q, k, v and the cotangent go
// into the workspace reversed and as bf16; the cotangent (fp32) is scaled by
// a per-head factor on the way (the gate, or 1) and rounded to the nearest
// even bf16.
#include "tc_common.hpp"
#include "tc_kernels.hpp"
#include "tc_bwd_paths.hpp"

#include <algorithm>

namespace tc {

namespace {

// 8 elements per thread and step (16-byte loads, two 16-byte stores); the
// tail of fewer than 8 elements (or everything, when a buffer is not
// 16-byte aligned) is done element by element.
__global__ __launch_bounds__(256) void widen_bf16_kernel(const uint16_t* __restrict__ in, float* __restrict__ out,
                                                         long n, bool vec) {
  const long n8 = vec ? n / 8 : 0;  // 16-byte pieces only when both buffers are 16-byte aligned
  const long stride = (long)gridDim.x * blockDim.x;
  for (long i = (long)blockIdx.x * blockDim.x + threadIdx.x; i < n8; i += stride) {
    const uint4 x = reinterpret_cast<const uint4*>(in)[i];
    float4* o = reinterpret_cast<float4*>(out) + 2 * i;
    o[0] = make_float4(__uint_as_float(x.x << 16), __uint_as_float(x.x & 0xFFFF0000u),
                       __uint_as_float(x.y << 16), __uint_as_float(x.y & 0xFFFF0000u));
    o[1] = make_float4(__uint_as_float(x.z << 16), __uint_as_float(x.z & 0xFFFF0000u),
                       __uint_as_float(x.w << 16), __uint_as_float(x.w & 0xFFFF0000u));
  }
  for (long i = 8 * n8 + (long)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride)
    out[i] = bf16_to_f32(in[i]);
}

// Rows of d elements (d a multiple of 8), 16 bytes per thread and step when
// both buffers are 16-byte aligned, element by element otherwise.
__global__ __launch_bounds__(256) void reverse_rows_bf16_kernel(const uint16_t* __restrict__ in,
                                                                uint16_t* __restrict__ out, int T, int d, long n,
                                                                bool vec) {
  const long stride = (long)gridDim.x * blockDim.x;
  if (vec) {
    const int d8 = d / 8;
    for (long i = (long)blockIdx.x * blockDim.x + threadIdx.x; i < n / 8; i += stride) {
      const long row = i / d8, bh = row / T;
      const int t = (int)(row - bh * T);
      reinterpret_cast<uint4*>(out)[(bh * T + (T - 1 - t)) * d8 + (i - row * d8)] =
          reinterpret_cast<const uint4*>(in)[i];
    }
    return;
  }
  for (long i = (long)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride) {
    const long row = i / d, bh = row / T;
    const int t = (int)(row - bh * T);
    out[(bh * T + (T - 1 - t)) * d + (i - row * d)] = in[i];
  }
}

__global__ __launch_bounds__(256) void reverse_rows_f32_kernel(const float* __restrict__ in,
                                                               const float* __restrict__ gate, int H,
                                                               uint16_t* __restrict__ out, int T, int d, long n,
                                                               bool vec) {
  const long stride = (long)gridDim.x * blockDim.x;
  if (vec) {
    const int d8 = d / 8;
    for (long i = (long)blockIdx.x * blockDim.x + threadIdx.x; i < n / 8; i += stride) {
      const long row = i / d8, bh = row / T;
      const int t = (int)(row - bh * T);
      const float f = gate != nullptr ? 1.f / (1.f + expf(-gate[bh % H])) : 1.f;
      const float4 a = reinterpret_cast<const float4*>(in)[2 * i];
      const float4 b = reinterpret_cast<const float4*>(in)[2 * i + 1];
      reinterpret_cast<uint4*>(out)[(bh * T + (T - 1 - t)) * d8 + (i - row * d8)] =
          make_uint4(pack_bf16x2(a.x * f, a.y * f), pack_bf16x2(a.z * f, a.w * f), pack_bf16x2(b.x * f, b.y * f),
                     pack_bf16x2(b.z * f, b.w * f));
    }
    return;
  }
  for (long i = (long)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride) {
    const long row = i / d, bh = row / T;
    const int t = (int)(row - bh * T);
    const float f = gate != nullptr ? 1.f / (1.f + expf(-gate[bh % H])) : 1.f;
    out[(bh * T + (T - 1 - t)) * d + (i - row * d)] = f32_to_bf16(in[i] * f);
  }
}

bool aligned16(const void* a, const void* b) {
  return ((reinterpret_cast<uintptr_t>(a) | reinterpret_cast<uintptr_t>(b)) & 15) == 0;
}

unsigned grid_for(long n8) { return (unsigned)std::min<long>((n8 + 255) / 256 + 1, 4096); }

}  // namespace

hipError_t launch_reverse_rows_bf16(const void* in, void* out, int BH, int T, int d, hipStream_t s) {
  const long n = (long)BH * T * d;
  if (n <= 0) return hipSuccess;
  const bool vec = d % 8 == 0 && aligned16(in, out);
  hipLaunchKernelGGL(reverse_rows_bf16_kernel, dim3(grid_for(n / 8)), dim3(256), 0, s,
                     static_cast<const uint16_t*>(in), static_cast<uint16_t*>(out), T, d, n, vec);
  return hipGetLastError();
}

hipError_t launch_reverse_rows_f32(const float* in, const float* gate, int H, void* out, int BH, int T, int d,
                                   hipStream_t s) {
  const long n = (long)BH * T * d;
  if (n <= 0) return hipSuccess;
  const bool vec = d % 8 == 0 && aligned16(in, out);
  hipLaunchKernelGGL(reverse_rows_f32_kernel, dim3(grid_for(n / 8)), dim3(256), 0, s, in, gate, H,
                     static_cast<uint16_t*>(out), T, d, n, vec);
  return hipGetLastError();
}

hipError_t launch_widen_bf16(const void* in, float* out, long n, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  const long blocks = std::min<long>((n / 8 + 255) / 256 + 1, 4096);
  const bool vec = ((reinterpret_cast<uintptr_t>(in) | reinterpret_cast<uintptr_t>(out)) & 15) == 0;
  hipLaunchKernelGGL(widen_bf16_kernel, dim3((unsigned)blocks), dim3(256), 0, s, static_cast<const uint16_t*>(in),
                     out, n, vec);
  return hipGetLastError();
}

}  // namespace tc

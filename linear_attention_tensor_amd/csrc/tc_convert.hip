// tc_convert.hip — bf16 -> fp32 widening for the backward passes.
//
// The backward passes run on fp32 kernels; bf16 inputs are widened first
// into the caller's workspace.  Every bf16 value is exact in fp32, so the
// gradients are those of the bf16 values, at fp32 accuracy.
#include "tc_common.hpp"
#include "tc_kernels.hpp"

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

}  // namespace

hipError_t launch_widen_bf16(const void* in, float* out, long n, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  const long blocks = std::min<long>((n / 8 + 255) / 256 + 1, 4096);
  const bool vec = ((reinterpret_cast<uintptr_t>(in) | reinterpret_cast<uintptr_t>(out)) & 15) == 0;
  hipLaunchKernelGGL(widen_bf16_kernel, dim3((unsigned)blocks), dim3(256), 0, s, static_cast<const uint16_t*>(in),
                     out, n, vec);
  return hipGetLastError();
}

}  // namespace tc

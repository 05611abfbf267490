// Sustained rate of the bf16 matrix instruction the kernels are built on, for
// the roofline report: every wave runs four independent accumulation chains of
// v_mfma_f32_32x32x16_bf16 on register operands, with no memory traffic in the
// loop, and the products' flop count over the elapsed time is the rate the
// matrix cores hold under a full load (the published peak assumes the maximum
// clock, which this load does not hold).
#include "device_common.hpp"
#include "launch.hpp"

namespace skl {

constexpr int kProbeThreads = 256;  // four waves

__global__ __launch_bounds__(kProbeThreads) void mfma_rate_kernel(int iters, float *sink) {
  const int lane = threadIdx.x & 63;
  // Operand values that the compiler cannot fold: small integers from the
  // lane and workgroup index, exact in bf16.
  bf16x8 a, b;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    a[i] = (bf16)(float)((lane + i) & 7);
    b[i] = (bf16)(float)(((int)blockIdx.x + i) & 3);
  }
  f32x16 c0 = f32x16{}, c1 = f32x16{}, c2 = f32x16{}, c3 = f32x16{};
  for (int it = 0; it < iters; ++it) {
    c0 = mma16(a, b, c0);
    c1 = mma16(b, a, c1);
    c2 = mma16(a, b, c2);
    c3 = mma16(b, a, c3);
  }
  float s = 0.f;
#pragma unroll
  for (int r = 0; r < 16; ++r) s += c0[r] + c1[r] + c2[r] + c3[r];
  if (lane == 0) sink[blockIdx.x * (kProbeThreads / 64) + (threadIdx.x >> 6)] = s;
}

hipError_t launch_mfma_rate(int iters, int workgroups, float *sink, hipStream_t s) {
  hipLaunchKernelGGL(mfma_rate_kernel, dim3((uint32_t)workgroups), dim3(kProbeThreads), 0, s, iters, sink);
  return hipGetLastError();
}

}  // namespace skl

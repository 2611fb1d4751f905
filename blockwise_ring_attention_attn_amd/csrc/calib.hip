// Calibration kernel for the hardware counters: a register-only loop of a
// known number of bf16 MFMAs (v_mfma_f32_32x32x16_bf16, 32768 FLOPs each)
// with eight independent accumulator chains per wave and eight waves per
// SIMD, so that the matrix pipe never waits for a dependency.  What the MFMA
// counters read for this launch, divided by its known MFMA count, is their
// scale; its rate is the dense bf16 MFMA rate the chip reaches in practice.
#include "ra_device.h"
#include "ra_internal.h"

namespace ra {
namespace {

using namespace dev;

constexpr int kCalibThreads = 256;
constexpr int kCalibChains = 8;

__global__ __launch_bounds__(kCalibThreads) void mfma_loop_kernel(int iters, float* sink) {
  const int t = threadIdx.x;
  bf16x8 a, b;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    a[e] = (__bf16)((float)((t + e) & 15) * (1.f / 64));
    b[e] = (__bf16)((float)((3 * t + e) & 15) * (1.f / 64));
  }
  f32x16 acc[kCalibChains];
#pragma unroll
  for (int c = 0; c < kCalibChains; ++c) acc[c] = f32x16{};
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int c = 0; c < kCalibChains; ++c) acc[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[c], 0, 0, 0);
  }
  float s = 0.f;
#pragma unroll
  for (int c = 0; c < kCalibChains; ++c)
#pragma unroll
    for (int r = 0; r < 16; ++r) s += acc[c][r];
  // The launcher passes no sink: the store never happens, but the compiler
  // cannot know that, so the loop stays.
  if (sink) sink[(int64_t)blockIdx.x * kCalibThreads + t] = s;
}

}  // namespace

hipError_t launch_mfma_loop(int workgroups, int iters, hipStream_t s, double* mfma_count) {
  *mfma_count = (double)workgroups * (kCalibThreads / 64) * (double)iters * kCalibChains;
  hipLaunchKernelGGL(mfma_loop_kernel, dim3(workgroups), dim3(kCalibThreads), 0, s, iters, nullptr);
  return hipGetLastError();
}

}  // namespace ra

// lse_merge and finalize kernels (HBM-bound, one wavefront per row).
//
// Page cited: "RingAttention 심층 아키텍처 ..." (techknowgenie.com), §3:
// the m_new / alpha / beta / l_new / O_new updates combine two partial
// softmax states; written for normalized partials (O, lse = m + ln l) they
// become lse = ln(e^lse_a + e^lse_b), O = e^(lse_a-lse) O_a + e^(lse_b-lse) O_b.
// §3 O_final: O = O / l.
#include "ra_internal.h"

namespace ra {
namespace {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kNegInf = -__builtin_huge_valf();
constexpr int kRowsPerBlock = 4;  // 4 wavefronts of 64 lanes

__global__ __launch_bounds__(256) void lse_merge_kernel(MergeArgs A) {
  const int64_t row = (int64_t)blockIdx.x * kRowsPerBlock + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (row >= A.rows) return;
  const float la = A.lse_a[row];
  const float lb = A.lse_b[row];
  const float M = fmaxf(la, lb);
  float wa = 0.f, wb = 0.f, lse = kNegInf;
  if (M != kNegInf) {
    wa = __builtin_amdgcn_exp2f((la - M) * kLog2e);
    wb = __builtin_amdgcn_exp2f((lb - M) * kLog2e);
    const float tot = wa + wb;
    lse = M + __builtin_amdgcn_logf(tot) * kLn2;
    const float inv = 1.f / tot;
    wa *= inv;
    wb *= inv;
  }
  float* oa = A.o_a + row * A.d;
  const float* ob = A.o_b + row * A.d;
  for (int c = lane; c < A.d; c += 64) oa[c] = wa * oa[c] + wb * ob[c];
  if (lane == 0) A.lse_a[row] = lse;
}

template <bool kBf16>
__global__ __launch_bounds__(256) void finalize_kernel(FinalizeArgs A) {
  const int64_t row = (int64_t)blockIdx.x * kRowsPerBlock + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (row >= A.rows) return;
  const float l = A.l[row];
  const float m = A.m[row];
  const float inv = l > 0.f ? 1.f / l : 0.f;
  const float* o = A.o + row * A.d;
  for (int c = lane; c < A.d; c += 64) {
    const float x = o[c] * inv;
    if constexpr (kBf16) reinterpret_cast<__bf16*>(A.out)[row * A.d + c] = (__bf16)x;
    else reinterpret_cast<float*>(A.out)[row * A.d + c] = x;
  }
  if (lane == 0) A.lse[row] = l > 0.f ? m + __builtin_amdgcn_logf(l) * kLn2 : kNegInf;
}

// Busy-waits for about `us` microseconds of the 100 MHz constant clock
// (s_memrealtime).  The iteration count is bounded (each iteration takes well
// over 1/64 us), so the kernel always ends.
__global__ void spin_kernel(int us, unsigned* sink) {
  const unsigned long long t0 = __builtin_amdgcn_s_memrealtime();
  const unsigned long long ticks = (unsigned long long)us * 100ull;
  const unsigned bound = (unsigned)us * 64u + 1024u;
  unsigned n = 0;
  for (unsigned it = 0; it < bound; ++it) {
    if (__builtin_amdgcn_s_memrealtime() - t0 >= ticks) break;
    ++n;
  }
  if (n == 0xffffffffu) sink[0] = n;  // never true; keeps the loop
}

}  // namespace

hipError_t launch_spin(int microseconds, hipStream_t s) {
  if (microseconds <= 0) return hipSuccess;
  hipLaunchKernelGGL(spin_kernel, dim3(1), dim3(1), 0, s, microseconds, nullptr);
  return hipGetLastError();
}

hipError_t launch_lse_merge(const MergeArgs& a, hipStream_t s) {
  if (a.rows <= 0) return hipSuccess;
  const int64_t g = (a.rows + kRowsPerBlock - 1) / kRowsPerBlock;
  if (g > 0x7fffffffLL) return hipErrorInvalidValue;
  hipLaunchKernelGGL(lse_merge_kernel, dim3((unsigned)g), dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_finalize(const FinalizeArgs& a, int out_bf16, hipStream_t s) {
  if (a.rows <= 0) return hipSuccess;
  const int64_t g = (a.rows + kRowsPerBlock - 1) / kRowsPerBlock;
  if (g > 0x7fffffffLL) return hipErrorInvalidValue;
  if (out_bf16) hipLaunchKernelGGL(finalize_kernel<true>, dim3((unsigned)g), dim3(256), 0, s, a);
  else hipLaunchKernelGGL(finalize_kernel<false>, dim3((unsigned)g), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace ra

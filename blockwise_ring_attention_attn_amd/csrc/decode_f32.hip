// Split-KV decode, fp32 partial pass (gfx950).
//
// Pages cited (by title; section named alone):
//   [TKG] "RingAttention 심층 아키텍처 ..." (techknowgenie.com): §3, the online
//         softmax over key blocks (running max m, row sum l, rescaled
//         output) and the exact merge of partial results through lse.
//   [CML] "Makale Bülteni — RingAttention" (cmlonder.com): the KV cache of
//         long-context decoding.
//
// The fp32 counterpart of decode_partial_kernel: the same grid (one
// workgroup per batch, kv head, sub-group of 16 query heads and split of a
// ring block; four waves, wave w taking the interleaved key tiles w, w + 4,
// ... of the split) and the same
// output, one normalized (O, lse) partial per wave and query head, merged by
// decode_merge_kernel.  Arithmetic is fp32 throughout.  Each wave spreads
// the d dimensions over its 64 lanes and walks its keys one at a time: for
// every query head of the sub-group the score is a butterfly sum,
// and the online-softmax update of [TKG] §3 runs in base 2 per key.  This
// path is for fp32 callers and is not tuned.
#include "ra_device.h"
#include "ra_internal.h"

namespace ra {
namespace {

using namespace dev;

constexpr int kWavesF = 4;     // waves per workgroup (as the bf16 partial kernel)
constexpr int kTileF = 32;     // keys per interleaved tile (as the bf16 partial kernel)
constexpr int kMaxGroup = 16;  // query heads per sub-group (as the bf16 pass's MFMA columns)

__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) x += __shfl_xor(x, o);
  return x;
}

template <int D>
__global__ __launch_bounds__(64 * kWavesF) void decode_partial_f32_kernel(DecodeArgs A) {
  constexpr int NC = D / 64;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int S_blk = A.P * A.chunks_per_block;
  const int split = blockIdx.x % S_blk;
  const int rest = blockIdx.x / S_blk;
  const int sg = rest % A.sub_groups;     // query heads sg * 16 .. + 15 of the group
  const int bh = rest / A.sub_groups;
  const int hkv = bh % A.Hkv;
  const int b = bh / A.Hkv;
  const int p = split / A.chunks_per_block;
  const int cidx = split % A.chunks_per_block;
  const int64_t k_begin = (int64_t)p * A.block + (int64_t)cidx * A.chunk;
  int64_t k_end = k_begin + A.chunk;
  const int64_t blk_end = (int64_t)(p + 1) * A.block;
  if (k_end > blk_end) k_end = blk_end;
  const float* Kp = static_cast<const float*>(A.k) + ((int64_t)b * A.Hkv + hkv) * A.L * D;
  const float* Vp = static_cast<const float*>(A.v) + ((int64_t)b * A.Hkv + hkv) * A.L * D;
  const int group = A.group;
  const int h0 = hkv * group + sg * kMaxGroup;                        // first query head of the sub-group
  const int ng = group - sg * kMaxGroup < kMaxGroup ? group - sg * kMaxGroup : kMaxGroup;   // heads in it

  float qv[kMaxGroup][NC], o[kMaxGroup][NC], m[kMaxGroup], l[kMaxGroup];
#pragma unroll
  for (int g = 0; g < kMaxGroup; ++g) {
    const float* Q = static_cast<const float*>(A.q) + ((int64_t)b * A.H + h0 + (g < ng ? g : 0)) * D;
#pragma unroll
    for (int e = 0; e < NC; ++e) {
      qv[g][e] = g < ng ? Q[lane + 64 * e] : 0.f;
      o[g][e] = 0.f;
    }
    m[g] = kNegInf;
    l[g] = 0.f;
  }
  const float c = A.scale_log2;
  for (int64_t t0 = k_begin + (int64_t)wave * kTileF; t0 < k_end; t0 += (int64_t)kWavesF * kTileF) {
    const int64_t t1 = t0 + kTileF < k_end ? t0 + kTileF : k_end;
    for (int64_t j = t0; j < t1; ++j) {
      float kv[NC], vv[NC];
#pragma unroll
      for (int e = 0; e < NC; ++e) {
        kv[e] = Kp[j * D + lane + 64 * e];
        vv[e] = Vp[j * D + lane + 64 * e];
      }
#pragma unroll
      for (int g = 0; g < kMaxGroup; ++g) {
        if (g >= ng) break;
        float s = 0.f;
#pragma unroll
        for (int e = 0; e < NC; ++e) s += qv[g][e] * kv[e];
        s = wave_sum(s) * c;                      // score in base 2
        const float m_new = fmaxf(m[g], s);
        const float alpha = fast_exp2(m[g] - m_new);   // 0 on the first key (m = -inf)
        const float w = fast_exp2(s - m_new);
        l[g] = l[g] * alpha + w;
#pragma unroll
        for (int e = 0; e < NC; ++e) o[g][e] = o[g][e] * alpha + w * vv[e];
        m[g] = m_new;
      }
    }
  }
  const int sidx = split * kWavesF + wave;
#pragma unroll
  for (int g = 0; g < kMaxGroup; ++g) {
    if (g >= ng) break;
    const int64_t pidx = ((int64_t)b * A.H + h0 + g) * A.S + sidx;
    const float inv = l[g] > 0.f ? 1.f / l[g] : 0.f;
#pragma unroll
    for (int e = 0; e < NC; ++e) A.o_part[pidx * D + lane + 64 * e] = o[g][e] * inv;
    if (lane == 0) A.lse_part[pidx] = l[g] > 0.f ? (m[g] + fast_log2(l[g])) * kLn2 : kNegInf;
  }
}

}  // namespace

hipError_t launch_decode_partial_f32(const DecodeArgs& a, int d, hipStream_t s) {
  const int64_t g = (int64_t)a.B * a.Hkv * a.sub_groups * a.P * a.chunks_per_block;
  if (g <= 0) return hipSuccess;
  if (g > 0x7fffffffLL) return hipErrorInvalidValue;
  if (a.group < 1 || a.sub_groups != (a.group + kMaxGroup - 1) / kMaxGroup) return hipErrorInvalidValue;
  if (d == 128) hipLaunchKernelGGL(decode_partial_f32_kernel<128>, dim3((unsigned)g), dim3(64 * kWavesF), 0, s, a);
  else if (d == 64) hipLaunchKernelGGL(decode_partial_f32_kernel<64>, dim3((unsigned)g), dim3(64 * kWavesF), 0, s, a);
  else return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace ra

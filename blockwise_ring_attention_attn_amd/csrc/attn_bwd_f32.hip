// Backward pass of blockwise ring attention in fp32 (gfx950).
//
// Pages cited (by title; section named alone):
//   [TKG] "RingAttention 심층 아키텍처: 통신-연산 완전 중첩과 블록 단위 온라인
//         소프트맥스로 1,000만 토큰 컨텍스트를 정복한 분산 어텐션 엔지니어링"
//         (techknowgenie.com).  §7 "활성화 체크포인팅과 메모리 재연산": keep the
//         queries and the row statistics of each block, send the key/value
//         blocks around the ring the other way and recompute the attention
//         map.
//
// The same recomputation, ring order and accumulation conventions as the
// bf16 kernels, for fp32 inputs, outputs and arithmetic throughout (no
// rounding of P or dS): per (query host, kv block) pair of a ring step
//   S = scale Q K^T,  P = exp(S - lse),  dP = dO V^T,  dS = P (dP - delta)
//   dV += P^T dO,  dK += scale dS^T Q,  dQ += scale dS K.
// One wavefront per row: the d dimensions are spread over the 64 lanes
// (one or two per lane) and each dot product is a butterfly sum, which
// leaves the identical value in every lane.  This path is for fp32 callers
// and for checking; it is latency-bound and not tuned.
#include "ra_device.h"
#include "ra_internal.h"

namespace ra {
namespace {

using namespace dev;

constexpr int kWaves = 4;   // rows per workgroup

__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) x += __shfl_xor(x, o);
  return x;
}

// Row statistics (lse2_i, delta_i) from fp32 O and dO: one wavefront per
// row, delta_i = sum_c dO_ic O_ic, lse2_i = lse_i log2(e) (+inf for a row
// without visible keys, so that its P is 0).
template <int D>
__global__ __launch_bounds__(64 * kWaves) void bwd_prep_f32_kernel(const float* out, const float* dout,
                                                                   const float* lse, float* rowstat, int64_t rows) {
  constexpr int NC = D / 64;
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * kWaves + (threadIdx.x >> 6);
  if (row >= rows) return;
  float acc = 0.f;
#pragma unroll
  for (int e = 0; e < NC; ++e) acc += out[row * D + lane + 64 * e] * dout[row * D + lane + 64 * e];
  acc = wave_sum(acc);
  if (lane == 0) {
    const float l = lse[row];
    rowstat[2 * row] = l == kNegInf ? __builtin_huge_valf() : l * kLog2e;
    rowstat[2 * row + 1] = acc;
  }
}

// Work of one row: the pair (query host q_rank, kv block kv_rank) and the
// batch / head of the wave with global index gw over rows per
// (host, batch, head).
__device__ __forceinline__ Work pair_work(const StepArgs& A, int64_t rest, int heads) {
  Work w{};
  const int hh = (int)(rest % heads);
  rest /= heads;
  w.b = (int)(rest % A.B);
  w.a = (int)(rest / A.B);
  w.q_rank = A.host_lo + w.a;
  int kr = (w.q_rank - A.kv_shift) % A.P;
  w.kv_rank = kr < 0 ? kr + A.P : kr;
  if (heads == A.H) {
    w.h = hh;
    w.hkv = hh / (A.H / A.Hkv);
  } else {
    w.hkv = hh;
    w.h = hh * (A.H / A.Hkv);
  }
  return w;
}

// Row of key j of the pair's kv block in the array the kernels read: the
// host-major staging buffer (the host's current block, compact) or the
// natural-order array.
__device__ __forceinline__ int64_t kv_read_row(const BwdArgs& G, const Work& w, int64_t j) {
  const StepArgs& A = G.s;
  const int64_t plane = (int64_t)w.b * A.Hkv + w.hkv;
  if (G.kv_staged) return ((int64_t)(w.q_rank - G.stage_host0) * A.B * A.Hkv + plane) * A.Lkv + j;
  return plane * G.n_tok + host_row(A.layout, w.kv_rank, j, A.Lkv, A.P);
}

// Row of query i (head h) of the pair's query host in q, dout, dq and the
// row statistics: the natural-order arrays, or the host's compact block.
__device__ __forceinline__ int64_t q_read_row(const BwdArgs& G, const Work& w, int h, int64_t i) {
  const StepArgs& A = G.s;
  const int64_t plane = (int64_t)w.b * A.H + h;
  if (G.q_compact) return plane * A.Lq + i;
  return plane * G.n_tok + host_row(A.layout, w.q_rank, i, A.Lq, A.P);
}

// Add `v` (this launch's contribution to one element) into its fp32
// accumulator; the first launch writes instead of adding, and the last
// launch that touches the row writes the total to the output instead.
__device__ __forceinline__ void emit(float* acc, float* out, int64_t idx, float v, bool first, bool fin) {
  const float x = first ? v : acc[idx] + v;
  if (fin) out[idx] = x;
  else acc[idx] = x;
}

// dQ: one wavefront per query row of each active host, against the visible
// keys of its paired kv block.
template <int D>
__global__ __launch_bounds__(64 * kWaves) void bwd_dq_f32_kernel(BwdArgs G, int64_t n_rows) {
  constexpr int NC = D / 64;
  const StepArgs& A = G.s;
  const int lane = threadIdx.x & 63;
  const int64_t gw = (int64_t)blockIdx.x * kWaves + (threadIdx.x >> 6);
  if (gw >= n_rows) return;
  const int64_t i = gw % A.Lq;
  const Work w = pair_work(A, gw / A.Lq, A.H);
  const int64_t lim = key_limit(A, w, i);
  const int64_t qrow = q_read_row(G, w, w.h, i);
  const float* q = static_cast<const float*>(A.q) + qrow * D;
  const float* go = static_cast<const float*>(G.dout) + qrow * D;
  const float* kb = static_cast<const float*>(A.k);
  const float* vb = static_cast<const float*>(A.v);
  float qv[NC], ov[NC], dq[NC];
#pragma unroll
  for (int e = 0; e < NC; ++e) {
    qv[e] = q[lane + 64 * e];
    ov[e] = go[lane + 64 * e];
    dq[e] = 0.f;
  }
  const float lse2 = G.rowstat[2 * qrow], delta = G.rowstat[2 * qrow + 1];
  const float c = A.scale_log2;
  for (int64_t j = 0; j <= lim; ++j) {
    const int64_t kr = kv_read_row(G, w, j) * D;
    float kv[NC], s = 0.f, dp = 0.f;
#pragma unroll
    for (int e = 0; e < NC; ++e) {
      kv[e] = kb[kr + lane + 64 * e];
      s += qv[e] * kv[e];
      dp += ov[e] * vb[kr + lane + 64 * e];
    }
    s = wave_sum(s);
    dp = wave_sum(dp);
    const float p = fast_exp2(__builtin_fmaf(s, c, -lse2));
    const float ds = p * (dp - delta);
#pragma unroll
    for (int e = 0; e < NC; ++e) dq[e] += ds * kv[e];
  }
  const bool first = G.first != 0, fin = ((G.q_fin >> w.q_rank) & 1ull) != 0;
#pragma unroll
  for (int e = 0; e < NC; ++e) emit(G.dq_acc, G.dq_out_f32, qrow * D + lane + 64 * e, G.scale * dq[e], first, fin);
}

// dK / dV: one wavefront per key of each active kv block, against every
// query of the paired host (all query heads of the kv head's group) that
// sees it.  The causal limit does not decrease along the query rows in any
// layout, so the queries that see key j are the rows from the first one
// whose limit reaches j.
template <int D>
__global__ __launch_bounds__(64 * kWaves) void bwd_dkdv_f32_kernel(BwdArgs G, int64_t n_rows) {
  constexpr int NC = D / 64;
  const StepArgs& A = G.s;
  const int lane = threadIdx.x & 63;
  const int64_t gw = (int64_t)blockIdx.x * kWaves + (threadIdx.x >> 6);
  if (gw >= n_rows) return;
  const int64_t j = gw % A.Lkv;
  Work w = pair_work(A, gw / A.Lkv, A.Hkv);
  const int group = A.H / A.Hkv;
  const int64_t plane = (int64_t)w.b * A.Hkv + w.hkv;
  const int64_t kr = kv_read_row(G, w, j) * D;
  const int64_t acc_row =
      G.kv_compact ? plane * A.Lkv + j : plane * G.n_tok + host_row(A.layout, w.kv_rank, j, A.Lkv, A.P);
  float kv[NC], vv[NC], dk[NC], dv[NC];
#pragma unroll
  for (int e = 0; e < NC; ++e) {
    kv[e] = static_cast<const float*>(A.k)[kr + lane + 64 * e];
    vv[e] = static_cast<const float*>(A.v)[kr + lane + 64 * e];
    dk[e] = dv[e] = 0.f;
  }
  int64_t i0 = 0;
  if (A.causal) {
    int64_t lo = 0, hi = A.Lq;
    while (lo < hi) {
      const int64_t mid = (lo + hi) >> 1;
      if (key_limit(A, w, mid) >= j) hi = mid; else lo = mid + 1;
    }
    i0 = lo;
  }
  const float c = A.scale_log2;
  for (int g = 0; g < group; ++g) {
    const int h = w.hkv * group + g;
    for (int64_t i = i0; i < A.Lq; ++i) {
      const int64_t qrow = q_read_row(G, w, h, i);
      const float* q = static_cast<const float*>(A.q) + qrow * D;
      const float* go = static_cast<const float*>(G.dout) + qrow * D;
      float qv[NC], ov[NC], s = 0.f, dp = 0.f;
#pragma unroll
      for (int e = 0; e < NC; ++e) {
        qv[e] = q[lane + 64 * e];
        ov[e] = go[lane + 64 * e];
        s += qv[e] * kv[e];
        dp += ov[e] * vv[e];
      }
      s = wave_sum(s);
      dp = wave_sum(dp);
      const float p = fast_exp2(__builtin_fmaf(s, c, -G.rowstat[2 * qrow]));
      const float ds = p * (dp - G.rowstat[2 * qrow + 1]);
#pragma unroll
      for (int e = 0; e < NC; ++e) {
        dv[e] += p * ov[e];
        dk[e] += ds * qv[e];
      }
    }
  }
  const bool first = G.kv_first != 0, fin = ((G.kv_fin >> w.kv_rank) & 1ull) != 0;
#pragma unroll
  for (int e = 0; e < NC; ++e) {
    const int64_t idx = acc_row * D + lane + 64 * e;
    emit(G.dk_acc, G.dk_out_f32, idx, G.scale * dk[e], first, fin);
    emit(G.dv_acc, G.dv_out_f32, idx, dv[e], first, fin);
  }
}

template <typename K>
hipError_t launch_rows(K kernel, const BwdArgs& a, int64_t n_rows, hipStream_t s) {
  if (n_rows <= 0) return hipSuccess;
  const int64_t g = (n_rows + kWaves - 1) / kWaves;
  if (g > 0x7fffffffLL) return hipErrorInvalidValue;
  hipLaunchKernelGGL(kernel, dim3((unsigned)g), dim3(64 * kWaves), 0, s, a, n_rows);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_bwd_prep_f32(const float* out, const float* dout, const float* lse, float* rowstat, int64_t rows,
                               int d, hipStream_t s) {
  if (rows <= 0) return hipSuccess;
  const int64_t g = (rows + kWaves - 1) / kWaves;
  if (g > 0x7fffffffLL) return hipErrorInvalidValue;
  if (d == 128)
    hipLaunchKernelGGL(bwd_prep_f32_kernel<128>, dim3((unsigned)g), dim3(64 * kWaves), 0, s, out, dout, lse, rowstat,
                       rows);
  else if (d == 64)
    hipLaunchKernelGGL(bwd_prep_f32_kernel<64>, dim3((unsigned)g), dim3(64 * kWaves), 0, s, out, dout, lse, rowstat,
                       rows);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

hipError_t launch_bwd_dkdv_f32(const BwdArgs& a, int d, hipStream_t s) {
  const int64_t n = (int64_t)a.s.n_hosts * a.s.B * a.s.Hkv * a.s.Lkv;
  if (d == 128) return launch_rows(bwd_dkdv_f32_kernel<128>, a, n, s);
  if (d == 64) return launch_rows(bwd_dkdv_f32_kernel<64>, a, n, s);
  return hipErrorInvalidValue;
}

hipError_t launch_bwd_dq_f32(const BwdArgs& a, int d, hipStream_t s) {
  const int64_t n = (int64_t)a.s.n_hosts * a.s.B * a.s.H * a.s.Lq;
  if (d == 128) return launch_rows(bwd_dq_f32_kernel<128>, a, n, s);
  if (d == 64) return launch_rows(bwd_dq_f32_kernel<64>, a, n, s);
  return hipErrorInvalidValue;
}

}  // namespace ra

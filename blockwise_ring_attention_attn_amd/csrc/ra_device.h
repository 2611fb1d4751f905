// Device-side helpers shared by the forward and backward attention kernels:
// vector types, token positions of the ring layouts, work decode, causal key
// limits, row addressing, cross-half reductions and LDS access helpers.
//
// Pages cited (by title; section named alone):
//   [TKG] "RingAttention 심층 아키텍처 ..." (techknowgenie.com): §2 sequence
//         sharding, §7 causal mask and striped sharding.
//   [CML] "Makale Bülteni — RingAttention" (cmlonder.com), "İddia ve
//         Gerçeklik": striped and zigzag schedules.
#pragma once
#include <type_traits>
#include <utility>

#include "ra_internal.h"

namespace ra {
namespace dev {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kTau = 8.0f;   // lazy-rescale threshold, base-2 units
constexpr float kSumCap = 65536.0f;  // largest accepted per-lane weight sum of a tile against a stale reference max
constexpr float kNegInf = -__builtin_huge_valf();

// Global token position of row i of host `rank`'s block (blk rows):
// contiguous rank*blk + i; striped i*P + rank; zigzag: the block is chunks
// rank and 2P-1-rank of 2P chunks of blk/2 tokens.
__device__ __forceinline__ int64_t host_row(int layout, int rank, int64_t i, int blk, int P) {
  if (layout == 0) return (int64_t)rank * blk + i;
  if (layout == 1) return i * P + rank;
  const int64_t c = blk >> 1;
  return i < c ? (int64_t)rank * c + i : (int64_t)(2 * P - 1 - rank) * c + (i - c);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float fast_log2(float x) { return __builtin_amdgcn_logf(x); }

// Value of the same query held by the lane 32 apart (the two halves of a
// wave hold the same 32 queries and disjoint keys / dims).
__device__ __forceinline__ float partner_max(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float partner_sum(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Work decomposition shared by both kernels.
struct Work {
  int a, b, h, hkv, qtile;
  int q_rank, kv_rank;
};

__device__ __forceinline__ Work decode_work(const StepArgs& A) {
  // XCD-aware remap: consecutive workgroup ids are dealt round-robin to the
  // 8 XCDs; give each XCD a contiguous range of logical work so the
  // workgroups that share one kv plane sit behind the same L2.
  const int G = gridDim.x, bid = blockIdx.x;
  const int xcd = bid & 7, idx = bid >> 3;
  const int qq = G >> 3, rr = G & 7;
  const int Lw = xcd * qq + (xcd < rr ? xcd : rr) + idx;
  const int group = A.H / A.Hkv;
  const int per_plane = group * A.n_qtiles;
  const int plane = Lw / per_plane;          // (a, b, hkv)
  const int rem = Lw - plane * per_plane;
  const int t = rem / group;                 // heaviest (last) query tile first
  Work w;
  const int hg = rem - t * group;
  w.qtile = A.n_qtiles - 1 - t;
  w.hkv = plane % A.Hkv;
  const int ab = plane / A.Hkv;
  w.b = ab % A.B;
  w.a = ab / A.B;
  w.h = w.hkv * group + hg;
  w.q_rank = A.host_lo + w.a;
  int kr = (w.q_rank - A.kv_shift) % A.P;
  w.kv_rank = kr < 0 ? kr + A.P : kr;
  return w;
}

// Largest visible key index (within the kv block) for query row i of the
// block, or -1 if none; clamped to Lkv - 1.
__device__ __forceinline__ int64_t key_limit(const StepArgs& A, const Work& w, int64_t i) {
  int64_t lim;
  if (!A.causal) {
    lim = A.Lkv - 1;
  } else if (A.layout == 0) {
    lim = (int64_t)w.q_rank * A.Lq + i - (int64_t)w.kv_rank * A.Lkv;
  } else if (A.layout == 1) {
    lim = i - (w.kv_rank > w.q_rank ? 1 : 0);
  } else {
    // zigzag: the kv block's positions increase with the row index (its
    // low chunk precedes its high chunk), so the visible keys are a prefix
    // whose length counts the keys of each chunk at or before the query.
    const int64_t c = A.Lkv >> 1;
    const int64_t pos = host_row(2, w.q_rank, i, A.Lq, A.P);
    int64_t na = pos - (int64_t)w.kv_rank * c + 1;
    int64_t nb = pos - (int64_t)(2 * A.P - 1 - w.kv_rank) * c + 1;
    na = na < 0 ? 0 : (na > c ? c : na);
    nb = nb < 0 ? 0 : (nb > c ? c : nb);
    lim = na + nb - 1;
  }
  if (lim > A.Lkv - 1) lim = A.Lkv - 1;
  if (lim < -1) lim = -1;
  return lim;
}

__device__ __forceinline__ int64_t q_row_index(const StepArgs& A, const Work& w, int64_t i) {
  const int64_t row = A.q_mode == ROWS_COMPACT ? i : host_row(A.layout, w.q_rank, i, A.Lq, A.P);
  return ((int64_t)w.b * A.H + w.h) * A.q_plane_rows + row;
}

// First row (within the k / v array) of this workgroup's kv block and the
// row stride between consecutive keys of the block.
__device__ __forceinline__ void kv_block_rows(const StepArgs& A, const Work& w, int64_t& first, int64_t& stride) {
  const int64_t plane = (int64_t)w.b * A.Hkv + w.hkv;
  if (A.kv_mode == ROWS_COMPACT) {
    first = plane * A.kv_plane_rows;
    stride = 1;
  } else if (A.kv_mode == ROWS_HOST_MAJOR) {
    first = ((int64_t)w.q_rank * A.B * A.Hkv + plane) * A.kv_plane_rows;
    stride = 1;
  } else {
    // natural-order source (contiguous or striped only; a zigzag block is
    // two separate chunks and is always staged compactly first)
    const int rk = A.kv_mode == ROWS_HOST_Q ? w.q_rank : w.kv_rank;
    first = plane * A.kv_plane_rows + (A.layout == 0 ? (int64_t)rk * A.Lkv : rk);
    stride = A.layout == 0 ? 1 : A.P;
  }
}

__device__ __forceinline__ int64_t kv_row_index(const StepArgs& A, const Work& w, int64_t j) {
  int64_t first, stride;
  kv_block_rows(A, w, first, stride);
  return first + j * stride;
}

__device__ __forceinline__ u32x2 lds_read_tr(const unsigned char* p) {
  typedef short s16x4 __attribute__((ext_vector_type(4)));
  s16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) s16x4*)(const_cast<unsigned char*>(p)));
  return __builtin_bit_cast(u32x2, v);
}

// s_waitcnt vmcnt(N) (at most N vector-memory loads of this wave still in
// flight), leaving expcnt / lgkmcnt unconstrained.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt is 6 bits");
  __builtin_amdgcn_s_waitcnt(0x0F70 | (N & 15) | ((N >> 4) << 14));
}

__device__ __forceinline__ void wait_vmcnt0() {
  // s_waitcnt vmcnt(0), leaving expcnt / lgkmcnt unconstrained
  __builtin_amdgcn_s_waitcnt(0x0F70);
}

__device__ __forceinline__ void wait_lgkmcnt0() {
  // s_waitcnt lgkmcnt(0), leaving vmcnt / expcnt unconstrained
  __builtin_amdgcn_s_waitcnt(0xC07F);
}

// Workgroup barrier without a memory fence.  __syncthreads() is a
// workgroup release/acquire, which waits for every outstanding LDS write of
// the wave, direct-to-LDS buffer loads included (vmcnt(0)), so loads issued
// tiles ahead would be drained at every barrier.  Callers wait explicitly
// (wait_vmcnt<N>) for the loads the other waves must see after the barrier;
// the compiler fences keep memory accesses and instructions on their side.
__device__ __forceinline__ void barrier_no_fence() {
  __builtin_amdgcn_sched_barrier(0);
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
}


// Compile-time loop: f(std::integral_constant<int, I>{}) for I = 0..N-1, so
// every index inside is a constant expression.
template <typename F, int... I>
__device__ __forceinline__ void static_for_impl(F&& f, std::integer_sequence<int, I...>) {
  (f(std::integral_constant<int, I>{}), ...);
}
template <int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  static_for_impl(f, std::make_integer_sequence<int, N>{});
}

}  // namespace dev
}  // namespace ra

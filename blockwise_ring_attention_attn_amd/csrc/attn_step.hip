// Fused block-attention step kernels for gfx950 (CDNA4).
//
// Pages cited (by title; section or equation named alone):
//   [TKG] "RingAttention 심층 아키텍처: 통신-연산 완전 중첩과 블록 단위 온라인
//         소프트맥스로 1,000만 토큰 컨텍스트를 정복한 분산 어텐션 엔지니어링"
//         (techknowgenie.com).
//   [AIT] FlashAttention video summary (aitrends.kr): tiling into on-chip
//         memory, online softmax, Q outer loop / KV inner loop.
//
// One launch performs one ring step for a set of query hosts: every
// workgroup owns BM query rows of one (host, batch, head) and sweeps the
// visible key/value tiles of that host's current kv block, fusing
//   S = Q K^T * scale                          [TKG] §3 equation S
//   causal mask on global positions           [TKG] §7
//   m_new = max(m, rowmax S), alpha, l update  [TKG] §3 m_block / m_new / alpha / l_new
//   O = alpha O + P V                          [TKG] §3 O_new
// and, at the end, merges with the state of earlier ring steps and either
// stores the fp32 state or finalizes (O / l, lse = m + ln l; [TKG] §3
// O_final).  The kernel uses the form P = exp(S - m_new) (the page's beta
// factor folded into P), base-2 exponentials with log2(e) folded into the
// scale, and keeps m stale while the new tile max stays within 2^8 of it
// (skipping the alpha rescale; l and O stay relative to the same m, so the
// result is unchanged).
//
// bf16 path: S^T = K Q^T and O^T = V^T P^T on v_mfma_f32_32x32x16_bf16.
// With K as the A operand every lane ends up owning one query column of
// S^T, so row max / row sum are in-lane reductions plus one permlane32 swap,
// and the output accumulator's rescale is a per-lane scalar.  P^T feeds the
// second MFMA straight from registers: the contraction index is permuted to
// the order the first MFMA left the keys in, and V^T is read from LDS in
// that same order with the gfx950 transposing LDS read.  K and V tiles are
// stored row-major in LDS and double-buffered: the global loads of the next
// tiles are in flight while the current one computes.
#include <type_traits>

#include "ra_device.h"
#include "ra_internal.h"

namespace ra {
namespace {

using namespace dev;

// Epilogue.  Where a launch merges with the state of earlier ring steps at
// the end (the fp32 kernel), the previous state of a row is read once, the
// merge weights are formed once per row, every group of 4 dims is merged
// and written, and only then are the row scalars (m, l or lse) written.
struct RowMerge {
  float ca, cb;      // weights of the stored state and of this launch's partial
  float m_new, l_new;
};

__device__ __forceinline__ RowMerge row_merge(const StepArgs& A, int64_t idx, float m2, float l) {
  RowMerge r{0.f, 1.f, m2, l};
  if (A.has_prev) {
    const float mp = A.m[idx] * kLog2e;
    const float lp = A.l[idx];
    r.m_new = fmaxf(mp, m2);
    r.ca = 0.f;
    r.cb = 0.f;
    if (r.m_new != kNegInf) {
      r.ca = fast_exp2(mp - r.m_new);
      r.cb = fast_exp2(m2 - r.m_new);
    }
    r.l_new = r.ca * lp + r.cb * l;
  }
  return r;
}

template <typename OutT>
__device__ __forceinline__ void store_dims4(const StepArgs& A, int64_t idx, int dim, int D, bool fin,
                                            const RowMerge& rm, const float o[4], bool merge) {
  float oo[4] = {rm.cb * o[0], rm.cb * o[1], rm.cb * o[2], rm.cb * o[3]};
  if (merge) {
    const float4 op = *reinterpret_cast<const float4*>(A.o + idx * D + dim);
    oo[0] += rm.ca * op.x;
    oo[1] += rm.ca * op.y;
    oo[2] += rm.ca * op.z;
    oo[3] += rm.ca * op.w;
  }
  if (fin) {
    const float inv = rm.l_new > 0.f ? 1.f / rm.l_new : 0.f;
    OutT* out = reinterpret_cast<OutT*>(A.out) + idx * D + dim;
    if constexpr (sizeof(OutT) == 2) {
      bf16x2 p0, p1;
      p0[0] = (__bf16)(oo[0] * inv); p0[1] = (__bf16)(oo[1] * inv);
      p1[0] = (__bf16)(oo[2] * inv); p1[1] = (__bf16)(oo[3] * inv);
      u32x2 pk;
      pk[0] = __builtin_bit_cast(unsigned, p0);
      pk[1] = __builtin_bit_cast(unsigned, p1);
      *reinterpret_cast<u32x2*>(out) = pk;
    } else {
      *reinterpret_cast<float4*>(out) = make_float4(oo[0] * inv, oo[1] * inv, oo[2] * inv, oo[3] * inv);
    }
  } else {
    *reinterpret_cast<float4*>(A.o + idx * D + dim) = make_float4(oo[0], oo[1], oo[2], oo[3]);
  }
}

__device__ __forceinline__ void store_row(const StepArgs& A, int64_t idx, bool fin, const RowMerge& rm) {
  if (fin) {
    A.lse[idx] = rm.l_new > 0.f ? (rm.m_new + fast_log2(rm.l_new)) * kLn2 : kNegInf;
  } else {
    A.m[idx] = rm.m_new == kNegInf ? kNegInf : rm.m_new * kLn2;
    A.l[idx] = rm.l_new;
  }
}

// ---------------------------------------------------------------------------
// bf16 MFMA kernel.
//
// Workgroup: 4 waves, BM = 128 query rows (32 per wave, one MFMA column
// block), two workgroups per CU (two waves per SIMD, so one wave's softmax
// overlaps the other's MFMAs).  Key/value tiles of BN = 64 rows go straight
// from HBM into LDS with buffer_load_dwordx4 ... lds (each wave instruction
// fills 1 KiB of LDS, lane l at byte 16 l; the buffer descriptor's bound
// turns rows past the block into zeros), double-buffered: tile j + 1 is in
// flight while tile j computes, one barrier per tile.
//
// LDS rows are unpadded (D * 2 bytes); 16-byte chunks are XOR-swizzled so
// that every read phase covers all 64 LDS banks (ds_read_b128 is served 16
// lanes at a time, ds_read_b64_tr_b16 32 lanes at a time):
//   K row r:  logical chunk c sits in slot c ^ kswz(r)
//   V row k:  logical chunk c sits in slot c ^ vswz(k)
// with kswz(r) = r & 15, vswz(k) = 4 (k & 3) for D = 128 (one row spans the
// 64 banks) and kswz(r) = (r >> 1) & 7, vswz(k) = 4 ((k >> 1) & 1) for D = 64
// (two rows span them).
// K fragments (A operand of S^T = K Q^T) are ds_read_b128 of one row each.
// The V^T operand of O^T = V^T P^T comes from ds_read_b64_tr_b16: in each
// 16-lane group, lane i receives element i%4 of the 8-byte pieces addressed
// by lanes i/4 + 4 j (j = 0..3); pointing lane s at key 4 (s/32) + (s%16)/4
// and dims 16 ((s/16)%2) + 4 (s%4) hands every lane 4 consecutive keys of its
// own dim, in the key order the S^T registers already hold.
// ---------------------------------------------------------------------------
constexpr int kWaves = 4;                 // waves per workgroup (32 query rows each)
constexpr int kThreads = 64 * kWaves;
constexpr int kBM = 32 * kWaves;
constexpr int kBN = 64;
constexpr int kWgPerCu = kWaves == 4 ? 2 : 1;

template <int D>
struct Tile {
  static constexpr int RB = D * 2;              // bytes per LDS row
  static constexpr int CPR = D / 8;             // 16-byte chunks per row
  static constexpr int BYTES = kBN * RB;        // one K (or V) tile
  static constexpr int LDS_BYTES = 4 * BYTES;   // K double buffer, then V double buffer
  static constexpr int VOFF = 2 * BYTES;        // start of the V buffers
  static constexpr int INSTR = BYTES / 1024;    // 1 KiB load instructions per tile per tensor
  static constexpr int PER_WAVE = INSTR / kWaves;
};

template <int D>
__device__ __forceinline__ int kswz(int r) { return D == 128 ? (r & 15) : ((r >> 1) & 7); }
template <int D>
__device__ __forceinline__ int vswz(int k) { return D == 128 ? 4 * (k & 3) : 4 * ((k >> 1) & 1); }

// Issue the direct-to-LDS loads of one K (or V) tile: this wave's share of
// the tile's 1 KiB load instructions.  `soff` is the byte offset of the
// tile's first row inside the block's buffer descriptor.
template <int D>
__device__ __forceinline__ void issue_tile(__amdgpu_buffer_rsrc_t rsrc, unsigned char* buf,
                                          const int (&voff)[Tile<D>::PER_WAVE], int wave_u, unsigned soff) {
#pragma unroll
  for (int u = 0; u < Tile<D>::PER_WAVE; ++u) {
    const int i = wave_u * Tile<D>::PER_WAVE + u;   // instruction index within the tile
    __builtin_amdgcn_raw_ptr_buffer_load_lds(
        rsrc, (__attribute__((address_space(3))) void*)(buf + i * 1024), 16, voff[u], soff, 0, 0);
  }
}

template <int D, typename OutT>
__global__ __launch_bounds__(kThreads, kWgPerCu) void step_bf16_kernel(StepArgs A) {
  using T = Tile<D>;
  const Work w = decode_work(A);
  const int lane = threadIdx.x & 63;
  const int wave_u = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int half = lane >> 5;       // which half of the wave
  const int col = lane & 31;        // query column owned by this lane
  const int64_t row_first = (int64_t)w.qtile * kBM;
  const int64_t row_last = (row_first + kBM < A.Lq ? row_first + kBM : A.Lq) - 1;
  const int64_t my_row = row_first + wave_u * 32 + col;
  const bool row_ok = my_row < A.Lq;
  const int64_t my_lim = key_limit(A, w, row_ok ? my_row : row_last);
  const int64_t kv_end = key_limit(A, w, row_last) + 1;
  const int64_t full_end = key_limit(A, w, row_first) + 1;
  const int ntiles = (int)((kv_end + kBN - 1) / kBN);
  const int lim32 = (int)my_lim;

  // Buffer descriptors covering exactly the kv block's rows of this plane:
  // row j sits at byte j * rstride * RB; rows j >= Lkv read as zero.
  int64_t plane_row, rstride;
  kv_block_rows(A, w, plane_row, rstride);
  const unsigned nrec = (unsigned)(((int64_t)(A.Lkv - 1) * rstride + 1) * T::RB);
  const __amdgpu_buffer_rsrc_t rk = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<unsigned short*>(reinterpret_cast<const unsigned short*>(A.k)) + plane_row * D, 0, nrec,
      0x00020000);
  const __amdgpu_buffer_rsrc_t rv = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<unsigned short*>(reinterpret_cast<const unsigned short*>(A.v)) + plane_row * D, 0, nrec,
      0x00020000);
  const unsigned tile_bytes = (unsigned)(kBN * rstride * T::RB);
  // Per-lane source offsets: lane l of load instruction i fills LDS slot
  // (64 i + l) of the tile, i.e. row r = (64 i + l) / CPR, slot q = l % CPR,
  // which holds logical chunk q ^ swizzle(r).
  int voff_k[T::PER_WAVE], voff_v[T::PER_WAVE];
#pragma unroll
  for (int u = 0; u < T::PER_WAVE; ++u) {
    const int pos = (wave_u * T::PER_WAVE + u) * 64 + lane;
    const int r = pos / T::CPR, q = pos % T::CPR;
    voff_k[u] = (int)(r * rstride * T::RB + 16 * (q ^ kswz<D>(r)));
    voff_v[u] = (int)(r * rstride * T::RB + 16 * (q ^ vswz<D>(r)));
  }

  // Resident query fragment: B operand of S^T = K Q^T (16 dims per MFMA).
  bf16x8 qf[D / 16];
  {
    const unsigned short* Q = reinterpret_cast<const unsigned short*>(A.q);
    const int64_t qi = q_row_index(A, w, row_ok ? my_row : row_first);
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks) {
      u32x4 x = row_ok ? *reinterpret_cast<const u32x4*>(Q + qi * D + ks * 16 + half * 8)
                       : u32x4{0u, 0u, 0u, 0u};
      qf[ks] = __builtin_bit_cast(bf16x8, x);
    }
  }

  // LDS read addresses (bytes within a buffer).
  // K: row kb*32 + col, logical chunk 2 ks + half; kswz(kb*32 + col) = kswz(col).
  int kaddr[D / 16];
#pragma unroll
  for (int ks = 0; ks < D / 16; ++ks) kaddr[ks] = col * T::RB + 16 * ((2 * ks + half) ^ kswz<D>(col));
  // V (transposing reads): lane s -> key 4 half + jp (+ 32 kb + 16 hc, + 8),
  // jp = (s%16)/4, and dims 32 db + 16 g + 4 (s%4), g = (s/16)%2, i.e. chunk
  // 4 db + u, u = 2 g + (s%4)/2, byte 8 (s%2) inside it; vswz of the key
  // depends on jp only.
  const int jp = (lane & 15) >> 2;
  const int ug = 2 * ((lane >> 4) & 1) + ((lane & 3) >> 1);
  int vaddr[D / 32];
#pragma unroll
  for (int db = 0; db < D / 32; ++db)
    vaddr[db] = (4 * half + jp) * T::RB + 16 * ((4 * db + ug) ^ vswz<D>(jp)) + 8 * (lane & 1);

  // Online-softmax state: resumed from the stored (m, l, o) of the earlier
  // ring steps, so the epilogue only stores.  The stored o and l are
  // relative to the stored m; l lives in half 0 (each half sums its own
  // keys and the halves are added at the end).
  f32x16 oacc[D / 32];
  float m_run = kNegInf, l_run = 0.f;
  if (A.has_prev && row_ok) {
    const int64_t idx = q_row_index(A, w, my_row);
    m_run = A.m[idx] * kLog2e;
    l_run = half == 0 ? A.l[idx] : 0.f;
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const float4 x = *reinterpret_cast<const float4*>(A.o + idx * D + db * 32 + 8 * g + 4 * half);
        oacc[db][4 * g] = x.x;
        oacc[db][4 * g + 1] = x.y;
        oacc[db][4 * g + 2] = x.z;
        oacc[db][4 * g + 3] = x.w;
      }
  } else {
#pragma unroll
    for (int db = 0; db < D / 32; ++db) oacc[db] = f32x16{};
  }
  const float c = A.scale_log2;

  // Software pipeline over key tiles: iteration j computes S(j+1) = K(j+1) Q^T
  // on the MFMA pipe while the VALU turns S(j) into P(j), then O += V(j)^T P(j).
  // K tiles therefore run one tile ahead of V tiles: during iteration j the
  // loads of K(j+2) and V(j+1) are in flight, K(j+1) and V(j) are read.
  // Four separate LDS objects, so that reads of one buffer are not ordered
  // behind direct-to-LDS loads that target another.
  __shared__ __align__(1024) unsigned char kbuf0[T::BYTES];
  __shared__ __align__(1024) unsigned char kbuf1[T::BYTES];
  __shared__ __align__(1024) unsigned char vbuf0[T::BYTES];
  __shared__ __align__(1024) unsigned char vbuf1[T::BYTES];

  // The two key blocks' accumulator chains alternate, so consecutive MFMAs
  // never depend on each other.
  auto qk = [&](const unsigned char* kb_lds, f32x16 (&s)[2]) {
    s[0] = f32x16{};
    s[1] = f32x16{};
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks)
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        const unsigned char* p = kb_lds + kaddr[ks] + kb * 32 * T::RB;
        const bf16x8 a = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(p));
        s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[ks], s[kb], 0, 0, 0);
      }
  };

  // Mask, row max and (lazy) rescale of tile jt's scores; returns the
  // reference max to subtract.
  auto prepare = [&](f32x16 (&s)[2], int jt) -> float {
    const int tile0 = jt * kBN;
    if (tile0 + kBN > full_end) {
      // key tile0 + kb*32 + 8*(r/4) + 4*half + r%4 is visible iff its offset
      // in the tile is <= my_lim - tile0; compare the compile-time part of
      // the offset against one per-lane 32-bit bound (block rows < 2^30).
      const int bound = lim32 - tile0 - 4 * half;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          if (kb * 32 + 8 * (r >> 2) + (r & 3) > bound) s[kb][r] = kNegInf;
    }
    float mx = kNegInf;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[kb][r]);
    mx = partner_max(mx);
    const float m_tile = mx * c;
    // Lazily refreshed reference max: rescale only when the tile max exceeds
    // it by more than kTau (base 2).
    const bool need = m_tile > m_run + kTau;
    if (__builtin_amdgcn_ballot_w64(need) != 0ull) {
      const float m_new = fmaxf(m_run, m_tile);
      const float alpha = m_new == kNegInf ? 1.f : fast_exp2(m_run - m_new);
      l_run *= alpha;
#pragma unroll
      for (int db = 0; db < D / 32; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[db][r] *= alpha;
      m_run = m_new;
    }
    return m_run == kNegInf ? 0.f : m_run;
  };

  // P = exp2(S c - m): the row sum takes the fp32 values, the PV product
  // their bf16 rounding (as the page's listing: block sum from the fp32
  // exponentials, P cast to the V dtype for P V).
  auto softmax = [&](const f32x16 (&s)[2], float m_use, bf16x8 (&pk)[2][2]) {
    float lsum0 = 0.f, lsum1 = 0.f;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int hc = 0; hc < 2; ++hc)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float p = fast_exp2(__builtin_fmaf(s[kb][hc * 8 + e], c, -m_use));
          if (e & 1) lsum1 += p; else lsum0 += p;
          pk[kb][hc][e] = (__bf16)p;
        }
    l_run += lsum0 + lsum1;
  };

  // S(j+1) = K(j+1) Q^T interleaved with P(j) = softmax(S(j)): the loop is
  // cut into NSTEP steps (one MFMA each, K fragment read two steps ahead,
  // 32 / NSTEP score elements of the current tile), fenced so the compiler
  // keeps the MFMAs spread across the exponentials.
  auto qk_softmax = [&](const unsigned char* kb_lds, f32x16 (&nxt)[2], const f32x16 (&cur)[2], float m_use,
                        bf16x8 (&pk)[2][2]) {
    constexpr int KS = D / 16;
    constexpr int NSTEP = 2 * KS;            // (kb, ks) pairs
    constexpr int EPS = 32 / NSTEP;          // score elements per step (2 or 4)
    // step i: key block i % 2, dim slice i / 2 (the two chains alternate)
    auto kread = [&](int i) -> bf16x8 {
      const int kb = i & 1, ks = i >> 1;
      return __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(kb_lds + kaddr[ks] + kb * 32 * T::RB));
    };
    nxt[0] = f32x16{};
    nxt[1] = f32x16{};
    bf16x8 kf[3];
    kf[0] = kread(0);
    kf[1] = kread(1);
    float lsum0 = 0.f, lsum1 = 0.f;
#pragma unroll
    for (int i = 0; i < NSTEP; ++i) {
      if (i + 2 < NSTEP) kf[(i + 2) % 3] = kread(i + 2);
      const int kb = i & 1, ks = i >> 1;
      nxt[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[i % 3], qf[ks], nxt[kb], 0, 0, 0);
#pragma unroll
      for (int t = 0; t < EPS; t += 2) {
        const int el = i * EPS + t;          // element pair (el, el + 1) of the current tile
        const int ckb = el / 16, r = el % 16;
        const float p0 = fast_exp2(__builtin_fmaf(cur[ckb][r], c, -m_use));
        const float p1 = fast_exp2(__builtin_fmaf(cur[ckb][r + 1], c, -m_use));
        lsum0 += p0;
        lsum1 += p1;
        pk[ckb][r >> 3][r & 7] = (__bf16)p0;
        pk[ckb][r >> 3][(r & 7) + 1] = (__bf16)p1;
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    l_run += lsum0 + lsum1;
  };

  // O^T += V^T P^T.  Contraction index k = 8*half + e maps to key
  // 16*hc + 8*(e/4) + 4*half + e%4 of key block kb (the S^T register order).
  auto pv = [&](const unsigned char* vb_lds, const bf16x8 (&pk)[2][2]) {
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int hc = 0; hc < 2; ++hc)
#pragma unroll
        for (int db = 0; db < D / 32; ++db) {
          const unsigned char* p0 = vb_lds + vaddr[db] + (kb * 32 + hc * 16) * T::RB;
          const u32x2 lo = lds_read_tr(p0);
          const u32x2 hi = lds_read_tr(p0 + 8 * T::RB);
          const u32x4 av = {lo[0], lo[1], hi[0], hi[1]};
          oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, av), pk[kb][hc],
                                                             oacc[db], 0, 0, 0);
        }
  };

  f32x16 sa[2], sb[2];
  if (ntiles > 0) {
    issue_tile<D>(rk, kbuf0, voff_k, wave_u, 0u);
    issue_tile<D>(rv, vbuf0, voff_v, wave_u, 0u);
    if (ntiles > 1) issue_tile<D>(rk, kbuf1, voff_k, wave_u, tile_bytes);
    wait_vmcnt0();
    __syncthreads();
    qk(kbuf0, sa);
    __syncthreads();  // everyone is done with K(0) before K(2) overwrites it
  }

  // One pipeline stage: tile jt with scores `cur`, producing `nxt` for jt + 1
  // (LAST: tile jt is the final tile, nothing to produce).  K(jt+1) lives in
  // kb_next, V(jt) in vb_cur; K(jt+2) goes to kb_free and V(jt+1) to vb_free.
  auto stage = [&](auto last_tag, int jt, f32x16 (&cur)[2], f32x16 (&nxt)[2], const unsigned char* kb_next,
                   unsigned char* kb_free, const unsigned char* vb_cur, unsigned char* vb_free) {
    constexpr bool LAST = decltype(last_tag)::value;
    if (!LAST) {
      if (jt + 2 < ntiles) issue_tile<D>(rk, kb_free, voff_k, wave_u, (unsigned)(jt + 2) * tile_bytes);
      issue_tile<D>(rv, vb_free, voff_v, wave_u, (unsigned)(jt + 1) * tile_bytes);
    }
    const float m_use = prepare(cur, jt);
    bf16x8 pk[2][2];
    if (!LAST) {
      qk_softmax(kb_next, nxt, cur, m_use, pk);
    } else {
      softmax(cur, m_use, pk);
    }
    pv(vb_cur, pk);
    wait_vmcnt0();
    __syncthreads();
  };

  using Mid = std::integral_constant<bool, false>;
  using Last = std::integral_constant<bool, true>;
  // Two tiles per trip so every buffer address is a compile-time offset.
  int jt = 0;
  for (; jt + 2 < ntiles; jt += 2) {
    stage(Mid{}, jt, sa, sb, kbuf1, kbuf0, vbuf0, vbuf1);
    stage(Mid{}, jt + 1, sb, sa, kbuf0, kbuf1, vbuf1, vbuf0);
  }
  if (jt + 1 < ntiles) {  // two tiles left: jt (buffer parity 0) and the last
    stage(Mid{}, jt, sa, sb, kbuf1, kbuf0, vbuf0, vbuf1);
    stage(Last{}, jt + 1, sb, sa, kbuf0, kbuf1, vbuf1, vbuf0);
  } else if (jt < ntiles) {  // one tile left
    stage(Last{}, jt, sa, sb, kbuf1, kbuf0, vbuf0, vbuf1);
  }

  // Combine the two halves' partial sums (they saw disjoint keys).
  const float l_tot = partner_sum(l_run);
  if (!row_ok) return;
  const bool fin = w.q_rank >= A.fin_lo && w.q_rank < A.fin_hi;
  const int64_t idx = q_row_index(A, w, my_row);
  const RowMerge rm{0.f, 1.f, m_run, l_tot};   // the state already includes earlier steps
#pragma unroll
  for (int db = 0; db < D / 32; ++db)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const float o4[4] = {oacc[db][4 * g], oacc[db][4 * g + 1], oacc[db][4 * g + 2], oacc[db][4 * g + 3]};
      store_dims4<OutT>(A, idx, db * 32 + 8 * g + 4 * half, D, fin, rm, o4, false);
    }
  if (half == 0) store_row(A, idx, fin, rm);
}

// ---------------------------------------------------------------------------
// fp32 kernel: one thread per query row, K/V tiles of 32 rows in LDS.
// Plain fp32 FMA arithmetic (no reduced-precision products).
// ---------------------------------------------------------------------------
constexpr int kF32BM = 64;
constexpr int kF32BN = 32;

template <int D>
__global__ __launch_bounds__(kF32BM) void step_f32_kernel(StepArgs A) {
  __shared__ float Ks[kF32BN][D];
  __shared__ float Vs[kF32BN][D];
  const Work w = decode_work(A);
  const int t = threadIdx.x;
  const int64_t row_first = (int64_t)w.qtile * kF32BM;
  const int64_t row_last = (row_first + kF32BM < A.Lq ? row_first + kF32BM : A.Lq) - 1;
  const int64_t my_row = row_first + t;
  const bool row_ok = my_row < A.Lq;
  const int64_t kv_end = key_limit(A, w, row_last) + 1;
  const int64_t my_lim = key_limit(A, w, row_ok ? my_row : row_last);
  const float* Q = reinterpret_cast<const float*>(A.q);
  const float* K = reinterpret_cast<const float*>(A.k);
  const float* V = reinterpret_cast<const float*>(A.v);

  float q[D], o[D];
  {
    const int64_t qi = q_row_index(A, w, row_ok ? my_row : row_first);
#pragma unroll
    for (int c = 0; c < D; ++c) {
      q[c] = row_ok ? Q[qi * D + c] : 0.f;
      o[c] = 0.f;
    }
  }
  float m_run = kNegInf, l_run = 0.f;
  const float cs = A.scale_log2;
  for (int64_t tile0 = 0; tile0 < kv_end; tile0 += kF32BN) {
    __syncthreads();
    for (int e = t; e < kF32BN * D; e += kF32BM) {
      const int r = e / D, cc = e % D;
      const int64_t j = tile0 + r;
      float kv = 0.f, vv = 0.f;
      if (j < A.Lkv) {
        const int64_t ri = kv_row_index(A, w, j);
        kv = K[ri * D + cc];
        vv = V[ri * D + cc];
      }
      Ks[r][cc] = kv;
      Vs[r][cc] = vv;
    }
    __syncthreads();
    float s[kF32BN];
    float mx = kNegInf;
#pragma unroll
    for (int r = 0; r < kF32BN; ++r) {
      float acc = 0.f;
#pragma unroll
      for (int c2 = 0; c2 < D; ++c2) acc = __builtin_fmaf(q[c2], Ks[r][c2], acc);
      s[r] = (tile0 + r <= my_lim) ? acc * cs : kNegInf;
      mx = fmaxf(mx, s[r]);
    }
    const float m_new = fmaxf(m_run, mx);
    const float m_use = m_new == kNegInf ? 0.f : m_new;
    const float alpha = fast_exp2(m_run - m_use);
    l_run *= alpha;
#pragma unroll
    for (int c2 = 0; c2 < D; ++c2) o[c2] *= alpha;
#pragma unroll
    for (int r = 0; r < kF32BN; ++r) {
      const float p = fast_exp2(s[r] - m_use);
      l_run += p;
#pragma unroll
      for (int c2 = 0; c2 < D; ++c2) o[c2] = __builtin_fmaf(p, Vs[r][c2], o[c2]);
    }
    m_run = m_new;
  }
  if (!row_ok) return;
  const bool fin = w.q_rank >= A.fin_lo && w.q_rank < A.fin_hi;
  const int64_t idx = q_row_index(A, w, my_row);
  const RowMerge rm = row_merge(A, idx, m_run, l_run);
#pragma unroll
  for (int c2 = 0; c2 < D; c2 += 4) {
    const float o4[4] = {o[c2], o[c2 + 1], o[c2 + 2], o[c2 + 3]};
    store_dims4<float>(A, idx, c2, D, fin, rm, o4, A.has_prev);
  }
  store_row(A, idx, fin, rm);
}

}  // namespace

int step_block_rows_bf16(int) { return kBM; }
int step_block_rows_f32(int) { return kF32BM; }

static int grid_size(const StepArgs& a) {
  return a.n_hosts * a.B * a.H * a.n_qtiles;
}

hipError_t launch_step_bf16(const StepArgs& a, int d, hipStream_t s) {
  const int g = grid_size(a);
  if (g <= 0) return hipSuccess;
  if (d == 128) {
    hipLaunchKernelGGL((step_bf16_kernel<128, __bf16>), dim3(g), dim3(kThreads), 0, s, a);
  } else if (d == 64) {
    hipLaunchKernelGGL((step_bf16_kernel<64, __bf16>), dim3(g), dim3(kThreads), 0, s, a);
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_step_f32(const StepArgs& a, int d, hipStream_t s) {
  const int g = grid_size(a);
  if (g <= 0) return hipSuccess;
  if (d == 128) {
    hipLaunchKernelGGL((step_f32_kernel<128>), dim3(g), dim3(kF32BM), 0, s, a);
  } else if (d == 64) {
    hipLaunchKernelGGL((step_f32_kernel<64>), dim3(g), dim3(kF32BM), 0, s, a);
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

// The bf16 kernel needs more than the default 64 KiB of dynamic LDS.
hipError_t step_kernel_setup() {
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(step_bf16_kernel<128, __bf16>),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, Tile<128>::LDS_BYTES);
  if (e != hipSuccess) return e;
  return hipFuncSetAttribute(reinterpret_cast<const void*>(step_bf16_kernel<64, __bf16>),
                             hipFuncAttributeMaxDynamicSharedMemorySize, Tile<64>::LDS_BYTES);
}

}  // namespace ra

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
// scale, and keeps m stale while no score of a new tile exceeds it by more
// than 16 (base 2): the bf16 kernel first exponentiates a tile against the
// current m and takes the row max (and the alpha rescale) only when the
// weights come out too large (the fp32 kernel keeps the exact running
// max).  l and O stay relative to the same m, so the result is unchanged.
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
  float l_norm;      // divisor of the output at finalization
};

__device__ __forceinline__ RowMerge row_merge(const StepArgs& A, int64_t idx, float m2, float l) {
  RowMerge r{0.f, 1.f, m2, l, l};
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
    r.l_norm = r.l_new;
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
    const float inv = rm.l_norm > 0.f ? 1.f / rm.l_norm : 0.f;
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
// Workgroup: 8 waves, BM = 256 query rows (32 per wave), one workgroup per
// CU.  The waves form two groups of four: group 0 owns rows 0..127 of the
// tile, group 1 rows 128..255.  Waves w and w + 4 run on the same SIMD, so
// every SIMD holds one wave of each group.  The work of one key tile is cut
// into two phases:
//   MFMA phase M(j):    S(j) = K(j) Q^T and O += V(j-1)^T P(j-1)  (matrix pipe)
//   softmax phase X(j): mask, row max, lazy rescale, P(j) = exp2(S c - m),
//                       row sums, bf16 packing                     (VALU)
// Group 1 runs one phase behind group 0 and every phase ends at a workgroup
// barrier, so on each SIMD one wave's MFMAs overlap the other wave's
// exponentials instead of waiting for them.
//
// Key/value tiles of BN = 64 rows go straight from HBM into LDS with
// buffer_load_dwordx4 ... lds (each wave instruction fills 1 KiB of LDS,
// lane l at byte 16 l; the buffer descriptor's bound turns rows past the
// block into zeros).  Three buffers per tensor, tile t in buffer t % 3.
// Group 1 issues every tile load: K(j+3) and V(j+2) at the start of its
// softmax phase X(j), and it waits for them at the end of X(j+1), before
// the barrier.  Every wave's first LDS reads of M(j+1) are issued at the end
// of X(j) and stay in flight across the barrier (the barrier does not wait
// for LDS reads; the buffers they read are not reloaded until both groups
// have finished M(j+1)).
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
constexpr int kWaves = 8;                 // two groups of four waves, 32 query rows each
constexpr int kThreads = 64 * kWaves;
constexpr int kGroupRows = 128;
constexpr int kBM = 2 * kGroupRows;
constexpr int kBN = 64;

template <int D>
struct Tile {
  static constexpr int RB = D * 2;              // bytes per LDS row
  static constexpr int CPR = D / 8;             // 16-byte chunks per row
  static constexpr int BYTES = kBN * RB;        // one K (or V) tile
  static constexpr int INSTR = BYTES / 1024;    // 1 KiB load instructions per tile per tensor
  static constexpr int PER_WAVE = INSTR / 4;    // issued by the four waves of group 1
  static constexpr int NDB = D / 32;            // 32-dim output blocks
  static constexpr int NSTEP = 2 * (D / 16);    // S MFMAs per tile (= PV MFMAs per tile)
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
                                          const int (&voff)[Tile<D>::PER_WAVE], int wl, unsigned soff) {
#pragma unroll
  for (int u = 0; u < Tile<D>::PER_WAVE; ++u) {
    const int i = wl * Tile<D>::PER_WAVE + u;   // instruction index within the tile
    __builtin_amdgcn_raw_ptr_buffer_load_lds(
        rsrc, (__attribute__((address_space(3))) void*)(buf + i * 1024), 16, voff[u], soff, 0, 0);
  }
}

template <int D, typename OutT>
__global__ __launch_bounds__(kThreads, 1) void step_bf16_kernel(StepArgs A) {
  using T = Tile<D>;
  constexpr int NSTEP = T::NSTEP;
  constexpr int PF = 3;                 // MFMA steps whose operands are read ahead
  const Work w = decode_work(A);
  const int lane = threadIdx.x & 63;
  const int wave_u = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int grp = wave_u >> 2;          // 0: rows 0..127 of the tile, 1: rows 128..255
  const int wl = wave_u & 3;
  const int half = lane >> 5;           // which half of the wave
  const int col = lane & 31;            // query column owned by this lane
  const int64_t row_first = (int64_t)w.qtile * kBM;
  const int64_t wg_last = (row_first + kBM < A.Lq ? row_first + kBM : A.Lq) - 1;
  const int64_t g_first = row_first + grp * kGroupRows;
  const bool grp_ok = g_first < A.Lq;
  const int64_t g_last = grp_ok ? ((g_first + kGroupRows < A.Lq ? g_first + kGroupRows : A.Lq) - 1) : wg_last;
  const int64_t my_row = g_first + wl * 32 + col;
  const bool row_ok = my_row < A.Lq;
  const int64_t my_lim = key_limit(A, w, row_ok ? my_row : g_last);
  const int64_t kv_end = key_limit(A, w, wg_last) + 1;
  const int ntiles = (int)((kv_end + kBN - 1) / kBN);
  // Group 1 loads every tile of the workgroup, so it runs through all of
  // them (its rows see the most keys); group 0 stops after its own last
  // visible tile.
  const int n_own = (int)((key_limit(A, w, g_last) + 1 + kBN - 1) / kBN);
  const int n_g = grp == 1 ? ntiles : (n_own < ntiles ? n_own : ntiles);
  const int64_t full_end = key_limit(A, w, grp_ok ? g_first : g_last) + 1;
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
  // Per-lane source offsets (group 1): lane l of load instruction i fills
  // LDS slot (64 i + l) of the tile, i.e. row r = (64 i + l) / CPR, slot
  // q = l % CPR, which holds logical chunk q ^ swizzle(r).
  int voff_k[T::PER_WAVE], voff_v[T::PER_WAVE];
#pragma unroll
  for (int u = 0; u < T::PER_WAVE; ++u) {
    const int pos = (wl * T::PER_WAVE + u) * 64 + lane;
    const int r = pos / T::CPR, q = pos % T::CPR;
    voff_k[u] = (int)(r * rstride * T::RB + 16 * (q ^ kswz<D>(r)));
    voff_v[u] = (int)(r * rstride * T::RB + 16 * (q ^ vswz<D>(r)));
  }

  // (The V buffers take the low LDS addresses -- the backend lays the
  // objects out by name -- so that the transposing reads' addresses fit the
  // 16-bit immediate offset of ds_read_b64_tr_b16 and need no address
  // arithmetic.)
  __shared__ __align__(1024) unsigned char av0[T::BYTES];
  __shared__ __align__(1024) unsigned char av1[T::BYTES];
  __shared__ __align__(1024) unsigned char av2[T::BYTES];
  __shared__ __align__(1024) unsigned char bk0[T::BYTES];
  __shared__ __align__(1024) unsigned char bk1[T::BYTES];
  __shared__ __align__(1024) unsigned char bk2[T::BYTES];
  // Six separate LDS objects, selected at compile time, so that reads of
  // one buffer are never ordered behind direct-to-LDS loads into another.
  auto kbuf = [&](auto I) -> unsigned char* {
    constexpr int i = decltype(I)::value % 3;
    if constexpr (i == 0) return bk0;
    else if constexpr (i == 1) return bk1;
    else return bk2;
  };
  auto vbuf = [&](auto I) -> unsigned char* {
    constexpr int i = decltype(I)::value % 3;
    if constexpr (i == 0) return av0;
    else if constexpr (i == 1) return av1;
    else return av2;
  };

  // Tiles K(0), V(0), K(1) first; their loads overlap the query and state loads.
  if (grp == 1 && ntiles > 0) {
    issue_tile<D>(rk, bk0, voff_k, wl, 0u);
    issue_tile<D>(rv, av0, voff_v, wl, 0u);
    if (ntiles > 1) issue_tile<D>(rk, bk1, voff_k, wl, tile_bytes);
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
  // The K buffers sit above the V buffers, partly past the 64 KiB that the
  // 16-bit immediate offset of ds_read_b128 reaches from a zero base, so
  // each lane keeps its K addresses relative to the first K buffer (kept
  // opaque, so that the buffer and key-block offsets stay immediates).
  typedef __attribute__((address_space(3))) const unsigned char lds_u8;
  unsigned kaddr[D / 16];
#pragma unroll
  for (int ks = 0; ks < D / 16; ++ks) {
    kaddr[ks] = (unsigned)(size_t)(lds_u8*)bk0 + col * T::RB + 16 * ((2 * ks + half) ^ kswz<D>(col));
    asm volatile("" : "+v"(kaddr[ks]));
  }
  // V (transposing reads): lane s -> key 4 half + jp (+ 32 kb + 16 hc, + 8),
  // jp = (s%16)/4, and dims 32 db + 16 g + 4 (s%4), g = (s/16)%2, i.e. chunk
  // 4 db + u, u = 2 g + (s%4)/2, byte 8 (s%2) inside it; vswz of the key
  // depends on jp only.
  const int jp = (lane & 15) >> 2;
  const int ug = 2 * ((lane >> 4) & 1) + ((lane & 3) >> 1);
  int vaddr[T::NDB];
#pragma unroll
  for (int db = 0; db < T::NDB; ++db)
    vaddr[db] = (4 * half + jp) * T::RB + 16 * ((4 * db + ug) ^ vswz<D>(jp)) + 8 * (lane & 1);

  // Online-softmax state: resumed from the stored (m, l, o) of the earlier
  // ring steps, so the epilogue only stores.  The stored o and l are
  // relative to the stored m; l lives in half 0 (each half sums its own
  // keys and the halves are added at the end).
  // Two row sums: l_run of the fp32 weights (for lse) and lb_run of their
  // bf16 roundings, the weights the P V product actually applies; the
  // output is normalized by lb, so its error depends on how much the values
  // differ, not on their size.  A stored state keeps o scaled to o l / lb,
  // i.e. o / l is that normalized output.
  f32x16 oacc[T::NDB];
  float m_run = kNegInf, l_run = 0.f;
  float lbr[4] = {0.f, 0.f, 0.f, 0.f};  // running sums of the bf16 weights, four chains
  if (A.has_prev && row_ok) {
    const int64_t idx = q_row_index(A, w, my_row);
    m_run = A.m[idx] * kLog2e;
    l_run = half == 0 ? A.l[idx] : 0.f;
    lbr[0] = l_run;
#pragma unroll
    for (int db = 0; db < T::NDB; ++db)
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
    for (int db = 0; db < T::NDB; ++db) oacc[db] = f32x16{};
  }
  const float c = A.scale_log2;
  wait_vmcnt0();
  __syncthreads();  // K(0), V(0), K(1) are in LDS

  f32x16 s[2];        // S^T of the tile between its MFMA and softmax phases
  bf16x8 pk[2][2];    // P^T of the tile between its softmax phase and the next MFMA phase
  bf16x8 kf[PF];      // K fragments of the first MFMA steps, read ahead
  u32x4 vf[PF];       // V^T fragments of the first MFMA steps, read ahead

  // MFMA step t: S MFMA on key block t & 1, dim slice t >> 1; PV MFMA on
  // output block db = t % NDB, key half hc = (t / NDB) % 2, key block
  // t / (2 NDB).  Consecutive MFMAs never feed each other.
  auto kread = [&](const unsigned char* kb, int t) -> bf16x8 {
    typedef __attribute__((address_space(3))) const u32x4 lds_u32x4;
    const unsigned rel = (unsigned)((lds_u8*)kb - (lds_u8*)bk0) + (t & 1) * 32 * T::RB;
    return __builtin_bit_cast(bf16x8, *(lds_u32x4*)(size_t)(kaddr[t >> 1] + rel));
  };
  // Contraction index k = 8*half + e of the PV MFMA maps to key
  // 16*hc + 8*(e/4) + 4*half + e%4 of its key block (the S^T register order).
  auto vread = [&](const unsigned char* vb, int t) -> u32x4 {
    const int db = t % T::NDB, hc = (t / T::NDB) & 1, kbv = t / (2 * T::NDB);
    const unsigned char* p0 = vb + vaddr[db] + (kbv * 32 + hc * 16) * T::RB;
    const u32x2 lo = lds_read_tr(p0);
    const u32x2 hi = lds_read_tr(p0 + 8 * T::RB);
    return u32x4{lo[0], lo[1], hi[0], hi[1]};
  };

  // MFMA phase; steps 0..PF-1 use the fragments read ahead.  With the PV
  // product it also sums the bf16 weights into lb (v_dot2_f32_bf16 of each
  // packed pair with (1, 1), four chains), using VALU slots the matrix
  // pipe leaves free.
  auto mphase = [&](auto do_s_tag, auto do_pv_tag, const unsigned char* kb, const unsigned char* vb) {
    constexpr bool DO_S = decltype(do_s_tag)::value;
    constexpr bool DO_PV = decltype(do_pv_tag)::value;
    constexpr int NPAIR = 16;                        // packed pairs of P per tile
    constexpr int PAIRS_PER_STEP = NPAIR / NSTEP;    // 1 (d = 128) or 2 (d = 64)
    const bf16x2 ones = {(__bf16)1.f, (__bf16)1.f};
    // The wave in its MFMA phase wins instruction issue over the other
    // group's wave on the same SIMD (otherwise the older wave would).
    __builtin_amdgcn_s_setprio(1);
    if constexpr (DO_S) {
      s[0] = f32x16{};
      s[1] = f32x16{};
    }
    static_for<NSTEP>([&](auto T_) __attribute__((always_inline)) {
      constexpr int t = decltype(T_)::value;
      if constexpr (DO_S) {
        const bf16x8 a = kf[t % PF];
        if constexpr (t + PF < NSTEP) kf[t % PF] = kread(kb, t + PF);
        s[t & 1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[t >> 1], s[t & 1], 0, 0, 0);
      }
      if constexpr (DO_PV) {
        constexpr int db = t % T::NDB, hc = (t / T::NDB) & 1, kbv = t / (2 * T::NDB);
        const u32x4 b = vf[t % PF];
        if constexpr (t + PF < NSTEP) vf[t % PF] = vread(vb, t + PF);
        oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, b), pk[kbv][hc],
                                                           oacc[db], 0, 0, 0);
#pragma unroll
        for (int q = 0; q < PAIRS_PER_STEP; ++q) {
          const int pr = t * PAIRS_PER_STEP + q;       // pair index: (kb, hc, element pair)
          const bf16x2 pair = {pk[pr >> 3][(pr >> 2) & 1][2 * (pr & 3)], pk[pr >> 3][(pr >> 2) & 1][2 * (pr & 3) + 1]};
          lbr[pr & 3] = __builtin_amdgcn_fdot2_f32_bf16(pair, ones, lbr[pr & 3], false);
          asm volatile("" : "+v"(lbr[pr & 3]));   // stays at this step (not sunk into the next phase)
        }
      }
      __builtin_amdgcn_sched_barrier(0);
    });
    __builtin_amdgcn_s_setprio(0);
  };

  // Causal mask of tile jt's scores (only past the all-visible prefix).
  auto mask_tile = [&](int jt) __attribute__((always_inline)) {
    const int tile0 = jt * kBN;
    if (tile0 + kBN > full_end) {
      // key tile0 + kb*32 + 8*(r/4) + 4*half + r%4 is visible iff its offset
      // in the tile is <= my_lim - tile0; compare the compile-time part of
      // the offset against one per-lane 32-bit bound (block rows < 2^30).
      // (One compare into VCC and one select per element, written out so the
      // compiler does not hold a lane mask per element in scalar registers.)
      const int bound = lim32 - tile0 - 4 * half;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          asm volatile("v_cmp_lt_i32 vcc, %1, %2\n\tv_cndmask_b32 %0, %0, %3, vcc"
                       : "+v"(s[kb][r])
                       : "v"(bound), "n"(kb * 32 + 8 * (r >> 2) + (r & 3)), "v"(kNegInf)
                       : "vcc");
    }
  };

  // Row max of the tile's scores; the reference max moves up to it (if
  // higher), rescaling l, lb and O.  Returns the reference to subtract.
  auto refresh_max = [&]() __attribute__((always_inline)) -> float {
    float mx = kNegInf;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[kb][r]);
    const float m_new = fmaxf(m_run, partner_max(mx) * c);
    const float alpha = m_new == kNegInf ? 1.f : fast_exp2(m_run - m_new);
    l_run *= alpha;
#pragma unroll
    for (int i = 0; i < 4; ++i) lbr[i] *= alpha;
#pragma unroll
    for (int db = 0; db < T::NDB; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r) oacc[db][r] *= alpha;
    m_run = m_new;
    return m_run == kNegInf ? 0.f : m_run;
  };

  // P = exp2(S c - m): returns this lane's sum of the fp32 values (for l);
  // the PV product takes their bf16 rounding (P cast to the V dtype, as the
  // page's listing does); the MFMA phase that consumes them also adds them
  // into lb.
  auto softmax = [&](float m_use) __attribute__((always_inline)) -> float {
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
    return lsum0 + lsum1;
  };

  // Softmax of tile jt against the current reference max, without a row
  // max first: the exponentials are accepted when every lane's sum of its
  // 32 weights is at most kSumCap (so that every weight is, i.e. no score
  // exceeds the reference by more than log2 kSumCap; an overflow shows as an
  // infinite sum).  Otherwise, and on a row's first tile (no reference yet),
  // the wave takes the row max, refreshes the reference and redoes them.
  // The reference is only ever moved to a true row max, and l, lb and O
  // stay relative to it, so the result does not depend on which path ran.
  auto tile_softmax = [&](int jt) __attribute__((always_inline)) {
    mask_tile(jt);
    float ls = 0.f;
    bool slow = __builtin_amdgcn_ballot_w64(m_run == kNegInf) != 0ull;
    if (!slow) {
      ls = softmax(m_run);
      slow = __builtin_amdgcn_ballot_w64(!(ls <= kSumCap)) != 0ull;
    }
    if (slow) ls = softmax(refresh_max());
    l_run += ls;
    asm volatile("" : "+v"(l_run));  // the sum finishes in this phase
  };

  // Softmax phase X(j) (j % 3 == JM): group 1 first issues the loads of
  // K(j+3) (into K(j)'s buffer, free since both groups finished M(j)) and
  // V(j+2) (into V(j-1)'s buffer), and at the end waits for the loads it
  // issued in X(j-1); then every wave reads ahead the first fragments of
  // M(j+1): K(j+1) unless j + 1 is the group's last MFMA phase, and V(j).
  auto xphase = [&](auto JM_, int j) {
    using JM = decltype(JM_);
    const bool ld_v = grp == 1 && j + 2 < ntiles;
    const bool ld_k = grp == 1 && j + 3 < ntiles;
    if (ld_v) issue_tile<D>(rv, vbuf(std::integral_constant<int, JM::value + 2>{}), voff_v, wl,
                            (unsigned)(j + 2) * tile_bytes);
    if (ld_k) issue_tile<D>(rk, kbuf(JM{}), voff_k, wl, (unsigned)(j + 3) * tile_bytes);
    tile_softmax(j);
    // Keep the bf16 packing in this phase (the compiler would otherwise sink
    // it past the barrier, next to its use in the MFMA phase).
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int hc = 0; hc < 2; ++hc) asm volatile("" : "+v"(pk[kb][hc]));
    if (grp == 1) {
      if (ld_k) wait_vmcnt<2 * T::PER_WAVE>();
      else if (ld_v) wait_vmcnt<T::PER_WAVE>();
      else wait_vmcnt0();
    }
    if (j + 1 < n_g) {
      const unsigned char* kb = kbuf(std::integral_constant<int, JM::value + 1>{});
#pragma unroll
      for (int t = 0; t < PF; ++t) kf[t] = kread(kb, t);
    }
    {
      const unsigned char* vb = vbuf(JM{});
#pragma unroll
      for (int t = 0; t < PF; ++t) vf[t] = vread(vb, t);
    }
    barrier_no_fence();
  };

  using Yes = std::integral_constant<bool, true>;
  using No = std::integral_constant<bool, false>;
  using I0 = std::integral_constant<int, 0>;
  using I1 = std::integral_constant<int, 1>;
  using I2 = std::integral_constant<int, 2>;
  // M(j) for j % 3 == JM reads K(j) and V(j-1).
  auto mboth = [&](auto JM_) {
    using JM = decltype(JM_);
    mphase(Yes{}, Yes{}, kbuf(JM{}), vbuf(std::integral_constant<int, JM::value + 2>{}));
    asm volatile("" : "+v"(s[0]), "+v"(s[1]));
    barrier_no_fence();
  };

  if (n_g > 0) {
#pragma unroll
    for (int t = 0; t < PF; ++t) kf[t] = kread(bk0, t);
    if (grp == 1) {
      // Group 1 starts one phase late; meanwhile it loads K(2) and V(1).
      if (ntiles > 1) issue_tile<D>(rv, av1, voff_v, wl, tile_bytes);
      if (ntiles > 2) issue_tile<D>(rk, bk2, voff_k, wl, 2u * tile_bytes);
      barrier_no_fence();
    }
    mphase(Yes{}, No{}, bk0, nullptr);   // M(0): S(0) only
    barrier_no_fence();
    xphase(I0{}, 0);
    int j = 1;
    for (; j + 2 < n_g; j += 3) {
      mboth(I1{});
      xphase(I1{}, j);
      mboth(I2{});
      xphase(I2{}, j + 1);
      mboth(I0{});
      xphase(I0{}, j + 2);
    }
    if (j < n_g) {  // j % 3 == 1
      mboth(I1{});
      xphase(I1{}, j);
      ++j;
      if (j < n_g) {
        mboth(I2{});
        xphase(I2{}, j);
      }
    }
    // M(n_g): O += V(n_g - 1)^T P(n_g - 1) only.
    const int jl = (n_g - 1) % 3;
    if (jl == 0) mphase(No{}, Yes{}, nullptr, av0);
    else if (jl == 1) mphase(No{}, Yes{}, nullptr, av1);
    else mphase(No{}, Yes{}, nullptr, av2);
    // Group 0 matches group 1's last barrier, so group 1's final MFMA phase
    // overlaps group 0's stores.
    if (grp == 0) barrier_no_fence();
  }
  // Every wave passes the same number of barriers: a group that processed
  // n > 0 tiles passed 2 n + 1 after the first one.  Group 0 stops early
  // when its rows see fewer tiles and waits out group 1's remaining phases.
  if (grp == 0) {
    const int extra = (ntiles > 0 ? 2 * ntiles + 1 : 0) - (n_g > 0 ? 2 * n_g + 1 : 0);
    for (int b = 0; b < extra; ++b) barrier_no_fence();
  }

  // Combine the two halves' partial sums (they saw disjoint keys).
  const float l_tot = partner_sum(l_run);
  const float lb_tot = partner_sum((lbr[0] + lbr[1]) + (lbr[2] + lbr[3]));
  if (!row_ok) return;
  const bool fin = w.q_rank >= A.fin_lo && w.q_rank < A.fin_hi;
  const int64_t idx = q_row_index(A, w, my_row);
  // The state already includes earlier steps: finalize with O = o / lb, or
  // store o l / lb (so that o / l is the normalized output) with l.
  const RowMerge rm{0.f, fin || !(lb_tot > 0.f) ? 1.f : l_tot / lb_tot, m_run, l_tot, lb_tot};
#pragma unroll
  for (int db = 0; db < T::NDB; ++db)
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


}  // namespace ra

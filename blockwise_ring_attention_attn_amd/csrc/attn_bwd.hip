// Backward pass of blockwise ring attention by recomputation (bf16, gfx950).
//
// Pages cited (by title; section or equation named alone):
//   [TKG] "RingAttention 심층 아키텍처: 통신-연산 완전 중첩과 블록 단위 온라인
//         소프트맥스로 1,000만 토큰 컨텍스트를 정복한 분산 어텐션 엔지니어링"
//         (techknowgenie.com).  §3 (S, the online softmax statistics),
//         §7 "활성화 체크포인팅과 메모리 재연산": the backward pass keeps only
//         the queries and the row statistics of each block, sends the
//         key/value blocks around the ring the other way and recomputes the
//         attention map in place.
//
// One ring step pairs query host r with kv block (r + s) mod P.  For every
// such pair the kernels recompute, tile by tile,
//   S = scale Q K^T,  P = exp(S - lse)      (lse = m + ln l of the forward,
//                                            taken in base 2 as lse2)
//   dP = dO V^T,      dS = P (dP - delta)   (delta_i = dO_i . O_i)
// and add
//   dV += P^T dO,  dK += scale dS^T Q       (bwd_dkdv_kernel, one key tile
//                                            per workgroup)
//   dQ += scale dS K                         (bwd_dq_kernel, one query tile
//                                            per workgroup)
// into fp32 accumulators; each kernel owns its outputs, so no atomics.
// These are the chain-rule derivatives of the forward definition (the
// pages name the strategy, not the formulas).
//
// MFMA orientation.  The dK/dV kernel keeps one key per lane column: it
// computes S and dP as [queries x keys] with the key tile's K and V rows
// resident in registers (the B operands), so P and dS come out with one key
// per lane and feed dV^T = dO^T P and dK^T = Q^T dS directly from registers
// (contraction over queries, in the register order; dO^T and Q^T come from
// transposing LDS reads).  The dQ kernel mirrors the forward step: S^T and
// dP^T as [keys x queries] with Q and dO resident, dQ^T = K^T dS^T with K^T
// from transposing LDS reads.  Tiles that are read both by rows
// (ds_read_b128) and transposed (ds_read_b64_tr_b16) use one XOR swizzle
// that serves both patterns (dswz below).
#include "ra_device.h"
#include "ra_internal.h"

namespace ra {
namespace {

using namespace dev;

constexpr int kThreads = 256;   // 4 waves
constexpr int kRows = 32;       // rows per streamed tile (queries for dK/dV, keys for dQ)
constexpr int kDkdvKeys = 128;  // keys per dK/dV workgroup (32 per wave)
constexpr int kDqRows = 128;    // queries per dQ workgroup (32 per wave)

// 16-byte chunk c of tile row r sits in slot c ^ dswz(r).  A 16-lane
// ds_read_b128 phase reads 16 consecutive rows at one logical chunk: dswz
// is a bijection on r mod 16 (D = 128, one row spans the 64 banks) or on
// (r / 2) mod 8 (D = 64, two rows span them).  A 32-lane transposing-read
// phase reads rows c0 + {0..3} (c0 a multiple of 4) at chunks 4 db + {0..3}:
// bits 2-3 (D = 128) or bit 2 (D = 64) of dswz vary with those rows, so the
// slots cover all banks.
template <int D>
__device__ __forceinline__ int dswz(int r) {
  return D == 128 ? ((4 * (r & 3)) | ((r >> 2) & 3)) : ((4 * ((r >> 1) & 1)) | ((r >> 2) & 3));
}

template <int D>
struct RowTile {
  static constexpr int RB = 2 * D;                  // bytes per LDS row
  static constexpr int CPR = D / 8;                 // 16-byte chunks per row
  static constexpr int BYTES = kRows * RB;
  static constexpr int PER_THREAD = kRows * CPR / kThreads;
};

// Token position of row i of host `rank`'s block (blk rows) for a layout
// fixed at compile time (0 contiguous, 1 striped, 2 zigzag); positions fit
// in 32 bits (blocks are at most 2^30 rows and N / P == blk).
template <int LAYOUT>
__device__ __forceinline__ int lrow(int rank, int i, int blk, int P) {
  if constexpr (LAYOUT == 0) {
    return rank * blk + i;
  } else if constexpr (LAYOUT == 1) {
    return i * P + rank;
  } else {
    const int c = blk >> 1;
    return i < c ? rank * c + i : (2 * P - 1 - rank) * c + (i - c);
  }
}

// Largest visible key (index in the kv block) of query row i, clamped to
// [-1, Lkv - 1]: the same limit as the forward's, for a compile-time layout.
template <int LAYOUT>
__device__ __forceinline__ int llim(const StepArgs& A, int q_rank, int kv_rank, int i) {
  if (!A.causal) return A.Lkv - 1;
  int lim;
  if constexpr (LAYOUT == 0) {
    lim = q_rank * A.Lq + i - kv_rank * A.Lkv;
  } else if constexpr (LAYOUT == 1) {
    lim = i - (kv_rank > q_rank ? 1 : 0);
  } else {
    const int c = A.Lkv >> 1;
    const int pos = lrow<2>(q_rank, i, A.Lq, A.P);
    const int na = min(max(pos - kv_rank * c + 1, 0), c);
    const int nb = min(max(pos - (2 * A.P - 1 - kv_rank) * c + 1, 0), c);
    lim = na + nb - 1;
  }
  return min(max(lim, -1), A.Lkv - 1);
}

// Natural-order row of host `rank`'s block row i in plane `plane` of an
// array with n_tok rows per plane.
template <int LAYOUT>
__device__ __forceinline__ int64_t nat_row(const StepArgs& A, int64_t plane, int64_t n_tok, int rank, int i, int blk) {
  return plane * n_tok + lrow<LAYOUT>(rank, i, blk, A.P);
}

// Per-lane LDS offsets.  Row-fragment reads (A operand, lane l: row l % 32,
// dims 16 ks + 8 (l / 32) .. + 7): roff[ks].  Transposing reads for the
// contraction over the tile's rows (A operand, lane l: dim 32 db + l % 32,
// rows 16 hc + 8 (e / 4) + 4 (l / 32) + e % 4 for e = 0..7, the register
// order of the accumulators): toff[db][hi] for the two 8-row halves; the
// row block hc adds 16 hc rows.
template <int D>
struct LdsOffsets {
  int roff[D / 16];
  int toff[D / 32][2];
  __device__ __forceinline__ LdsOffsets(int lane) {
    using T = RowTile<D>;
    const int col = lane & 31, half = lane >> 5;
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks) roff[ks] = col * T::RB + 16 * ((2 * ks + half) ^ dswz<D>(col));
    // transposing read: in each 16-lane group lane i gets element i % 4 of
    // the 8-byte pieces of lanes i / 4 + 4 j; lane s points at row
    // 4 half + (s % 16) / 4 (+ 8 hi) and dims 16 ((s / 16) % 2) + 4 (s % 4)
    const int jp = (lane & 15) >> 2;
    const int ug = 2 * ((lane >> 4) & 1) + ((lane & 3) >> 1);
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int hi = 0; hi < 2; ++hi) {
        const int r = 4 * half + jp + 8 * hi;
        toff[db][hi] = r * T::RB + 16 * ((4 * db + ug) ^ dswz<D>(r)) + 8 * (lane & 1);
      }
  }
};

template <int D>
__device__ __forceinline__ bf16x8 read_rowfrag(const unsigned char* lds, const LdsOffsets<D>& o, int ks) {
  return __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(lds + o.roff[ks]));
}

template <int D>
__device__ __forceinline__ bf16x8 read_trfrag(const unsigned char* lds, const LdsOffsets<D>& o, int db, int hc) {
  using T = RowTile<D>;
  const u32x2 lo = lds_read_tr(lds + o.toff[db][0] + hc * 16 * T::RB);
  const u32x2 hi = lds_read_tr(lds + o.toff[db][1] + hc * 16 * T::RB);
  return __builtin_bit_cast(bf16x8, u32x4{lo[0], lo[1], hi[0], hi[1]});
}

__device__ __forceinline__ bf16x8 pack8(const f32x16& x, int base) {
  bf16x8 r;
#pragma unroll
  for (int e = 0; e < 8; ++e) r[e] = (__bf16)x[base + e];
  return r;
}

// Direct-to-LDS buffer loads (16 or 4 bytes per lane) at a vector offset
// plus a scalar offset.
__device__ __forceinline__ void lds_load16(__amdgpu_buffer_rsrc_t r, unsigned char* lds, int voff, unsigned soff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)lds, 16, voff, soff, 0, 0);
}
__device__ __forceinline__ void lds_load4(__amdgpu_buffer_rsrc_t r, void* lds, int voff, unsigned soff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)lds, 4, voff, soff, 0, 0);
}

// One LDS buffer per (use, slot): a distinct object for every slot.  The
// compiler tracks direct-to-LDS loads per LDS object and makes a read wait
// for every load in flight into the same object, so slots of one array
// would make each tile's reads wait for the loads just issued for a later
// tile.
template <int TAG, int SLOT, int BYTES>
__device__ __forceinline__ unsigned char* slot_buf() {
  __shared__ __align__(1024) unsigned char b[BYTES];
  return b;
}
template <int I>
using IC = std::integral_constant<int, I>;

// Resident fragment of one row of a natural-order bf16 array for MFMA B
// operands: lane l holds dims 16 ks + 8 (l / 32) .. + 7 of its row.
template <int D>
__device__ __forceinline__ void load_row_frags(bf16x8 (&f)[D / 16], const unsigned short* base, int64_t row, bool ok,
                                               int half) {
#pragma unroll
  for (int ks = 0; ks < D / 16; ++ks) {
    const u32x4 x = ok ? *reinterpret_cast<const u32x4*>(base + row * D + 16 * ks + 8 * half) : u32x4{0u, 0u, 0u, 0u};
    f[ks] = __builtin_bit_cast(bf16x8, x);
  }
}

// Emit a [32 x 32] accumulator block (rows = dims 32 db + 8 (r / 4) + 4 half
// + r % 4, column = this lane's row) times `mul` into an fp32 row of D
// floats: added to the row, or written over it on the first launch; on the
// last launch that touches the row the sum is rounded to bf16 and written to
// the output row instead.
__device__ __forceinline__ void emit_block(float* acc_row, __bf16* out_row, const f32x16& acc, int db, int half,
                                           float mul, bool first, bool fin) {
#pragma unroll
  for (int g = 0; g < 4; ++g) {
    const int c = 32 * db + 8 * g + 4 * half;
    float4 x = first ? make_float4(0.f, 0.f, 0.f, 0.f) : *reinterpret_cast<const float4*>(acc_row + c);
    x.x += mul * acc[4 * g];
    x.y += mul * acc[4 * g + 1];
    x.z += mul * acc[4 * g + 2];
    x.w += mul * acc[4 * g + 3];
    if (fin) {
      bf16x2 lo, hi;
      lo[0] = (__bf16)x.x; lo[1] = (__bf16)x.y;
      hi[0] = (__bf16)x.z; hi[1] = (__bf16)x.w;
      u32x2 pk;
      pk[0] = __builtin_bit_cast(unsigned, lo);
      pk[1] = __builtin_bit_cast(unsigned, hi);
      *reinterpret_cast<u32x2*>(out_row + c) = pk;
    } else {
      *reinterpret_cast<float4*>(acc_row + c) = x;
    }
  }
}

// ---------------------------------------------------------------------------
// dK / dV: one workgroup per (query host, batch, kv head, 128-key tile).  It
// sweeps, for every query head of the kv head's group, the 32-row query
// tiles that see any of its keys.
//
// Eight waves in producer / consumer pairs: waves p and p + 4 (p = 0..3)
// share a SIMD and the 32 keys key0 + 32 p ... .  The producer (wave p)
// keeps the keys' K and V rows in registers and, for query tile t,
// computes S = Q K^T and dP = dO V^T (MFMA), then P = exp2(S c - lse2) and
// dS = P (dP - delta) (VALU), and hands P and dS to its consumer through
// LDS.  The consumer (wave p + 4) holds the fp32 dV^T and dK^T accumulators
// and adds dO^T P and Q^T dS (MFMA, dO^T and Q^T from transposing LDS reads)
// one phase later, while the producer computes the next tile.  So on every
// SIMD one wave's MFMAs run beside the other wave's exponentials, and each
// wave stays within half the register file (the accumulators and the
// resident K / V rows would not fit one wave at two waves per SIMD).
// Phase k: producers on tile k, consumers on tile k - 1; one barrier per
// phase.  The consumers also issue the tile loads (Q, dO and the row
// statistics, straight into LDS, LOOK tiles ahead).
// ---------------------------------------------------------------------------
constexpr int kDkdvThreads = 512;

template <int D, int LAYOUT>
__global__ __launch_bounds__(kDkdvThreads, 1) void bwd_dkdv_kernel(BwdArgs G) {
  using T = RowTile<D>;
  constexpr int KS = D / 16, NDB = D / 32;
  const StepArgs& A = G.s;
  // work decode: XCD-aware remap, then (host, batch, kv head) plane major
  const int Gn = gridDim.x, bid = blockIdx.x;
  const int xcd = bid & 7, idx = bid >> 3;
  const int Lw = xcd * (Gn >> 3) + (xcd < (Gn & 7) ? xcd : (Gn & 7)) + idx;
  const int plane = Lw / G.n_kvtiles;
  const int kt = Lw - plane * G.n_kvtiles;
  Work w;
  w.hkv = plane % A.Hkv;
  w.b = (plane / A.Hkv) % A.B;
  w.a = plane / (A.Hkv * A.B);
  w.q_rank = A.host_lo + w.a;
  {
    int kr = (w.q_rank - A.kv_shift) % A.P;
    w.kv_rank = kr < 0 ? kr + A.P : kr;
  }
  w.h = 0;
  w.qtile = 0;
  const int group = A.H / A.Hkv;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const bool producer = wave < 4;
  const int pw = wave & 3;              // the pair: keys key0 + 32 pw ...
  const int cw = wave - 4;              // consumer index 0..3 (consumers only)
  const int half = lane >> 5, col = lane & 31;
  const float c = A.scale_log2;

  // this lane's key and the pair's key range
  const int key0 = kt * kDkdvKeys;
  const int my_key = key0 + pw * 32 + col;
  const bool key_ok = my_key < A.Lkv;
  const int64_t kv_plane = (int64_t)w.b * A.Hkv + w.hkv;
  // this key's row in the dK / dV accumulators and outputs (and in the
  // natural-order K / V when they are read in place)
  const int64_t key_row = !key_ok        ? 0
                          : G.kv_compact ? kv_plane * A.Lkv + my_key
                                         : nat_row<LAYOUT>(A, kv_plane, G.n_tok, w.kv_rank, my_key, A.Lkv);

  // first query row that sees any key of the workgroup (the limit is
  // non-decreasing in the row)
  int i0 = 0;
  if (A.causal) {
    int lo = 0, hi = A.Lq;
    while (lo < hi) {
      const int mid = (lo + hi) >> 1;
      if (llim<LAYOUT>(A, w.q_rank, w.kv_rank, mid) >= key0) hi = mid; else lo = mid + 1;
    }
    i0 = lo;
  }
  const int qt0 = i0 / kRows;
  const int nqt = (A.Lq + kRows - 1) / kRows - qt0;   // query tiles per head
  const int total = nqt > 0 ? nqt * group : 0;

  // LDS: NSLOT slots for the streamed (Q, dO, row statistics) tiles (tile k
  // is read by the producers in phase k and by the consumers in phase k + 1,
  // and the loads of tile k + LOOK are issued in phase k), and two exchange
  // buffers of packed P and dS per pair (written in phase k, read in k + 1).
  constexpr int LOOK = 2, NSLOT = LOOK + 2;
  constexpr int ROWS_PER_INSTR = 1024 / T::RB;        // tile rows per 1 KiB load instruction
  constexpr int INSTR = T::BYTES / 1024;              // per tensor per tile
  constexpr int PER_WAVE = INSTR / 4;                 // per consumer wave
  static_assert(PER_WAVE >= 1 && INSTR % 4 == 0, "tile must split over the four consumer waves");
  auto qbuf = [](auto I) { return slot_buf<0, decltype(I)::value % NSLOT, T::BYTES>(); };
  auto obuf = [](auto I) { return slot_buf<1, decltype(I)::value % NSLOT, T::BYTES>(); };
  auto rsb = [](auto I) { return reinterpret_cast<float(*)[2]>(slot_buf<2, decltype(I)::value % NSLOT, 8 * kRows>()); };
  // exchange buffer: per pair 4 KiB (packed P and dS of the pair's tile)
  auto xbuf = [](auto I) { return slot_buf<3, decltype(I)::value % 2, 4 * 4096>(); };
  const LdsOffsets<D> off(lane);

  // ---- consumer side: the tile loads -------------------------------------
  // Tile it: head hkv*group + it / nqt, query tile qt0 + it % nqt, issued in
  // order, so the next call's head and query tile are kept (no division per
  // tile).  Lane l of load instruction i fills LDS slot 64 i + l of the tile:
  // row ROWS_PER_INSTR i + l / CPR, chunk slot l % CPR holding logical chunk
  // (l % CPR) ^ dswz(row).  Q, dO and the row statistics are read from the
  // natural-order arrays (N rows per plane) or, for one device's share, from
  // the host's compact block (Lq rows per plane, block row i at row i).
  // Contiguous and striped tiles, and every compact tile, are arithmetic
  // sequences of rows: the row base goes into the scalar offset and
  // each lane's vector offset is a constant.  Zigzag tiles and a head's ragged
  // last tile take per-lane offsets, rows past the block out of the buffer's
  // range (they read zeros); a tile index past the last one loads zeros.
  // Consumer 0 also loads the tile's row statistics (lse2, delta): 256 bytes,
  // lane l: row l / 2, statistic l % 2.
  const bool qc = G.q_compact != 0;
  const int64_t q_plane_rows = qc ? (int64_t)A.Lq : G.n_tok;   // rows per (b, h) plane of q, dout, row statistics
  const int64_t plane_elems = q_plane_rows * D;
  const unsigned rec_rows = (unsigned)(q_plane_rows * T::RB);
  const unsigned rec_rs = (unsigned)(q_plane_rows * 8);
  constexpr bool kAffine = LAYOUT != 2;
  const int row_stride = (LAYOUT == 1 && !qc) ? A.P : 1;
  int voff_row[PER_WAVE], rr_row[PER_WAVE], qchunk[PER_WAVE];
#pragma unroll
  for (int u = 0; u < PER_WAVE; ++u) {
    const int ins = cw * PER_WAVE + u;
    rr_row[u] = ins * ROWS_PER_INSTR + lane / T::CPR;
    qchunk[u] = 16 * ((lane % T::CPR) ^ dswz<D>(rr_row[u]));
    voff_row[u] = rr_row[u] * row_stride * T::RB + qchunk[u];
  }
  const int voff_rs = (lane >> 1) * row_stride * 8 + 4 * (lane & 1);
  int is_qt = 0;
  const int64_t qplane0 = (int64_t)w.b * A.H + w.hkv * group;
  unsigned short* qbase = const_cast<unsigned short*>(reinterpret_cast<const unsigned short*>(A.q)) + qplane0 * plane_elems;
  unsigned short* obase =
      const_cast<unsigned short*>(reinterpret_cast<const unsigned short*>(G.dout)) + qplane0 * plane_elems;
  float* rbase = const_cast<float*>(G.rowstat) + qplane0 * q_plane_rows * 2;
  auto issue = [&](int it, auto slot) __attribute__((always_inline)) {
    const bool valid = it < total;
    const int row0 = (qt0 + is_qt) * kRows;
    const __amdgpu_buffer_rsrc_t rq = __builtin_amdgcn_make_buffer_rsrc(qbase, 0, rec_rows, 0x00020000);
    const __amdgpu_buffer_rsrc_t ro = __builtin_amdgcn_make_buffer_rsrc(obase, 0, rec_rows, 0x00020000);
    const __amdgpu_buffer_rsrc_t rr = __builtin_amdgcn_make_buffer_rsrc(rbase, 0, rec_rs, 0x00020000);
    if (kAffine && valid && row0 + kRows <= A.Lq) {
      const unsigned nat0 = qc ? (unsigned)row0
                               : LAYOUT == 0 ? (unsigned)(w.q_rank * A.Lq + row0) : (unsigned)(row0 * A.P + w.q_rank);
#pragma unroll
      for (int u = 0; u < PER_WAVE; ++u) {
        const int ins = cw * PER_WAVE + u;
        lds_load16(rq, qbuf(slot) + ins * 1024, voff_row[u], nat0 * T::RB);
        lds_load16(ro, obuf(slot) + ins * 1024, voff_row[u], nat0 * T::RB);
      }
      if (cw == 0) lds_load4(rr, &rsb(slot)[0][0], voff_rs, nat0 * 8);
    } else {
#pragma unroll
      for (int u = 0; u < PER_WAVE; ++u) {
        const int ins = cw * PER_WAVE + u;
        const int i = row0 + rr_row[u];
        const int src = qc ? i : lrow<LAYOUT>(w.q_rank, i, A.Lq, A.P);
        const int voff = (valid && i < A.Lq) ? src * T::RB + qchunk[u] : (int)rec_rows;
        lds_load16(rq, qbuf(slot) + ins * 1024, voff, 0u);
        lds_load16(ro, obuf(slot) + ins * 1024, voff, 0u);
      }
      if (cw == 0) {
        const int i = row0 + (lane >> 1);
        const int src = qc ? i : lrow<LAYOUT>(w.q_rank, i, A.Lq, A.P);
        const int voff = (valid && i < A.Lq) ? src * 8 + 4 * (lane & 1) : (int)rec_rs;
        lds_load4(rr, &rsb(slot)[0][0], voff, 0u);
      }
    }
    if (valid && ++is_qt == nqt) {
      is_qt = 0;
      qbase += plane_elems;
      obase += plane_elems;
      rbase += q_plane_rows * 2;
    }
  };
  // Loads a consumer may leave in flight at the end of a phase: those of the
  // LOOK - 1 newest tiles (consumer 0 also loads each tile's row statistics).
  constexpr int LOADS = 2 * PER_WAVE;
  auto wait_landed = [&]() __attribute__((always_inline)) {
    if (cw == 0) wait_vmcnt<(LOOK - 1) * (LOADS + 1)>();
    else wait_vmcnt<(LOOK - 1) * LOADS>();
  };

  // Each role runs its own copy of the phase loop (same phases, same
  // barriers), so that the producers' resident K / V rows and the
  // consumers' accumulators are never live in the same code and the
  // register allocator gives each role the whole per-wave budget.
  // Phase k (0 <= k <= total): producers produce tile k (k < total) into
  // exchange buffer k % 2; consumers consume tile k - 1 (k >= 1) and issue the
  // loads of tile k + LOOK.  The slot of tile k is k % NSLOT.
  const int n_phases = total > 0 ? total + 1 : 0;
  auto run_phases = [&](auto&& phase) __attribute__((always_inline)) {
    int k = 0;
    for (; k + NSLOT <= n_phases; k += NSLOT)
      static_for<NSLOT>([&](auto i) __attribute__((always_inline)) { phase(i, k + decltype(i)::value); });
    static_for<NSLOT - 1>([&](auto i) __attribute__((always_inline)) {
      if (k + decltype(i)::value < n_phases) phase(i, k + decltype(i)::value);
    });
  };

  if (producer) {
    // ---- producer: S, dP, P, dS ------------------------------------------
    bf16x8 kf[KS], vf[KS];
    {
      const int64_t src_row =
          G.kv_staged ? ((int64_t)(w.q_rank - G.stage_host0) * A.B * A.Hkv + kv_plane) * A.Lkv + (key_ok ? my_key : 0)
                      : key_row;
      load_row_frags<D>(kf, reinterpret_cast<const unsigned short*>(A.k), src_row, key_ok, half);
      load_row_frags<D>(vf, reinterpret_cast<const unsigned short*>(A.v), src_row, key_ok, half);
    }
    // Causal mask: -inf where this lane's key lies past the row's limit
    // (register r holds query row 8 (r / 4) + 4 half + r % 4); only for tiles
    // whose first row does not see every key of the pair.
    const int pair_last_key = min(key0 + pw * 32 + 31, A.Lkv - 1);
    int cs_qt = 0;  // query tile (within its head) of the tile being produced
    auto produce = [&](auto slot, auto xs) __attribute__((always_inline)) {
      const int row0 = (qt0 + cs_qt) * kRows;
      cs_qt = cs_qt + 1 == nqt ? 0 : cs_qt + 1;
      // Q and dO fragments read two MFMA steps (four MFMAs) ahead of use
      constexpr int RA = 2;
      f32x16 sc = f32x16{}, dpc = f32x16{};
      bf16x8 qa[RA], oa[RA];
      static_for<RA>([&](auto I) __attribute__((always_inline)) {
        qa[decltype(I)::value] = read_rowfrag<D>(qbuf(slot), off, decltype(I)::value);
        oa[decltype(I)::value] = read_rowfrag<D>(obuf(slot), off, decltype(I)::value);
      });
      // the tile's row statistics, read now so that their latency hides
      // under the MFMAs: rows 8 g + 4 half + {0, 1} and + {2, 3}
      float4 rsa[4], rsb4[4];
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int q0 = 8 * g + 4 * half;
        rsa[g] = *reinterpret_cast<const float4*>(&rsb(slot)[q0][0]);
        rsb4[g] = *reinterpret_cast<const float4*>(&rsb(slot)[q0 + 2][0]);
      }
      static_for<KS>([&](auto T_) __attribute__((always_inline)) {
        constexpr int t = decltype(T_)::value;
        const bf16x8 a = qa[t % RA], o = oa[t % RA];
        if constexpr (t + RA < KS) {
          qa[t % RA] = read_rowfrag<D>(qbuf(slot), off, t + RA);
          oa[t % RA] = read_rowfrag<D>(obuf(slot), off, t + RA);
        }
        sc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, kf[t], sc, 0, 0, 0);
        dpc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(o, vf[t], dpc, 0, 0, 0);
        __builtin_amdgcn_sched_barrier(0);
      });
      if (A.causal && llim<LAYOUT>(A, w.q_rank, w.kv_rank, row0) < pair_last_key) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int i = row0 + 8 * (r >> 2) + 4 * half + (r & 3);
          const int lim = i < A.Lq ? llim<LAYOUT>(A, w.q_rank, w.kv_rank, i) : -1;
          if (my_key > lim) sc[r] = kNegInf;
        }
      }
      bf16x8 pb[2], dsb[2];
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        // row statistics of rows 8 g + 4 half + e
        const float4 a4 = rsa[g];
        const float4 b4 = rsb4[g];
        const float lv[4] = {a4.x, a4.z, b4.x, b4.z};
        const float dv[4] = {a4.y, a4.w, b4.y, b4.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int r = 4 * g + e;
          const float pr = fast_exp2(__builtin_fmaf(sc[r], c, -lv[e]));   // 0 where masked (S = -inf)
          const float ds = pr * (dpc[r] - dv[e]);
          pb[r >> 3][r & 7] = (__bf16)pr;
          dsb[r >> 3][r & 7] = (__bf16)ds;
        }
      }
      // hand P, dS to the consumer: four 1 KiB rows (P halves, dS halves),
      // 16 bytes per lane, consecutive lanes at consecutive 16-byte chunks
      unsigned char* xb = xbuf(xs) + pw * 4096;
      *reinterpret_cast<bf16x8*>(xb + lane * 16) = pb[0];
      *reinterpret_cast<bf16x8*>(xb + 1024 + lane * 16) = pb[1];
      *reinterpret_cast<bf16x8*>(xb + 2048 + lane * 16) = dsb[0];
      *reinterpret_cast<bf16x8*>(xb + 3072 + lane * 16) = dsb[1];
    };
    if (n_phases > 0) barrier_no_fence();   // the consumers' first tile loads have landed
    run_phases([&](auto kc, int k) __attribute__((always_inline)) {
      constexpr int K = decltype(kc)::value;   // k % NSLOT (NSLOT is even: k % 2 == K % 2)
      if (k < total) produce(IC<K>{}, IC<K>{});
      wait_lgkmcnt0();   // exchange writes done, slot reads done
      barrier_no_fence();
    });
    return;
  }

  // ---- consumer: dV^T += dO^T P, dK^T += Q^T dS; the tile loads ----------
  f32x16 dvT[NDB], dkT[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) dvT[db] = dkT[db] = f32x16{};
  auto consume = [&](auto slot, auto xs) __attribute__((always_inline)) {
    const unsigned char* xb = xbuf(xs) + pw * 4096;
    const bf16x8 pb0 = *reinterpret_cast<const bf16x8*>(xb + lane * 16);
    const bf16x8 pb1 = *reinterpret_cast<const bf16x8*>(xb + 1024 + lane * 16);
    const bf16x8 ds0 = *reinterpret_cast<const bf16x8*>(xb + 2048 + lane * 16);
    const bf16x8 ds1 = *reinterpret_cast<const bf16x8*>(xb + 3072 + lane * 16);
    // dO^T and Q^T fragments read two steps (four MFMAs) ahead of use
    constexpr int NST = 2 * NDB, RA = 2;
    bf16x8 ta[RA], tb[RA];
    static_for<RA>([&](auto I) __attribute__((always_inline)) {
      constexpr int st = decltype(I)::value;
      ta[st] = read_trfrag<D>(obuf(slot), off, st % NDB, st / NDB);
      tb[st] = read_trfrag<D>(qbuf(slot), off, st % NDB, st / NDB);
    });
    static_for<NST>([&](auto T_) __attribute__((always_inline)) {
      constexpr int st = decltype(T_)::value, db = st % NDB, hc = st / NDB;
      const bf16x8 a = ta[st % RA], b = tb[st % RA];
      if constexpr (st + RA < NST) {
        ta[st % RA] = read_trfrag<D>(obuf(slot), off, (st + RA) % NDB, (st + RA) / NDB);
        tb[st % RA] = read_trfrag<D>(qbuf(slot), off, (st + RA) % NDB, (st + RA) / NDB);
      }
      dvT[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, hc ? pb1 : pb0, dvT[db], 0, 0, 0);
      dkT[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(b, hc ? ds1 : ds0, dkT[db], 0, 0, 0);
      __builtin_amdgcn_sched_barrier(0);
    });
  };
  if (n_phases > 0) {
    static_for<LOOK>([&](auto I) __attribute__((always_inline)) { issue(decltype(I)::value, I); });
    wait_landed();     // tile 0 is in LDS
    barrier_no_fence();
    run_phases([&](auto kc, int k) __attribute__((always_inline)) {
      constexpr int K = decltype(kc)::value;
      issue(k + LOOK, IC<K + LOOK>{});
      if (k >= 1) consume(IC<K + NSLOT - 1>{}, IC<K + 1>{});
      wait_landed();     // tile k + 1 is in LDS for the producers' next phase
      wait_lgkmcnt0();   // exchange and slot reads done before they are rewritten
      barrier_no_fence();
    });
    wait_vmcnt0();       // loads past the end (zeros into free slots)
  }

  // (A key tile no query sees still writes its zeros on the first launch
  // and its final values on the last.)
  const bool first = G.kv_first != 0;
  const bool fin = ((G.kv_fin >> w.kv_rank) & 1ull) != 0;
  if (!key_ok || (total == 0 && !first && !fin)) return;
  float* dk_row = G.dk_acc + key_row * D;
  float* dv_row = G.dv_acc + key_row * D;
#pragma unroll
  for (int db = 0; db < NDB; ++db) {
    emit_block(dk_row, G.dk_out + key_row * D, dkT[db], db, half, G.scale, first, fin);
    emit_block(dv_row, G.dv_out + key_row * D, dvT[db], db, half, 1.f, first, fin);
  }
}

// ---------------------------------------------------------------------------
// dQ: one workgroup per (query host, batch, query head, 128-row query tile),
// sweeping the visible 32-key tiles of the paired kv block.
// ---------------------------------------------------------------------------
template <int D, int LAYOUT>
__global__ __launch_bounds__(kThreads, 2) void bwd_dq_kernel(BwdArgs G) {
  using T = RowTile<D>;
  constexpr int KS = D / 16, NDB = D / 32;
  const StepArgs& A = G.s;
  const Work w = decode_work(A);   // n_qtiles counts 128-row query tiles
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int half = lane >> 5, col = lane & 31;
  const float c = A.scale_log2;
  const int row_first = w.qtile * kDqRows;
  const int row_last = (row_first + kDqRows < A.Lq ? row_first + kDqRows : A.Lq) - 1;
  const int my_row = row_first + wave * 32 + col;
  const bool row_ok = my_row < A.Lq;
  const int lim32 = llim<LAYOUT>(A, w.q_rank, w.kv_rank, row_ok ? my_row : row_last);
  // limit of the wave's first row: keys up to it are visible to all its rows
  const int wave_first = row_first + wave * 32;
  const int wave_first_lim = llim<LAYOUT>(A, w.q_rank, w.kv_rank, wave_first < A.Lq ? wave_first : row_last);
  const int kv_end = llim<LAYOUT>(A, w.q_rank, w.kv_rank, row_last) + 1;
  const int ntiles = (int)((kv_end + kRows - 1) / kRows);

  const int64_t qplane = (int64_t)w.b * A.H + w.h;
  const int64_t qrow = !row_ok ? 0
                       : G.q_compact ? qplane * A.Lq + my_row
                                     : nat_row<LAYOUT>(A, qplane, G.n_tok, w.q_rank, my_row, A.Lq);
  bf16x8 qf[KS], of[KS];
  load_row_frags<D>(qf, reinterpret_cast<const unsigned short*>(A.q), qrow, row_ok, half);
  load_row_frags<D>(of, reinterpret_cast<const unsigned short*>(G.dout), qrow, row_ok, half);
  const float lse2 = row_ok ? G.rowstat[2 * qrow] : __builtin_huge_valf();   // past the block: P = 0
  const float del = row_ok ? G.rowstat[2 * qrow + 1] : 0.f;

  f32x16 dqT[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) dqT[db] = f32x16{};

  // Four LDS slots for the K / V tiles; tile t+3 is loaded straight into
  // LDS while tile t computes (two tiles of time for each load to land).
  constexpr int NSLOT = 4, LOOK = 3;
  constexpr int ROWS_PER_INSTR = 1024 / T::RB;
  constexpr int INSTR = T::BYTES / 1024;
  constexpr int PER_WAVE = INSTR / 4;
  constexpr int LOADS = 2 * PER_WAVE;   // vector loads per wave per tile
  static_assert(PER_WAVE >= 1 && INSTR % 4 == 0, "tile must split over the four waves");
  auto kbuf = [](auto I) { return slot_buf<5, decltype(I)::value % NSLOT, T::BYTES>(); };
  auto vbuf = [](auto I) { return slot_buf<6, decltype(I)::value % NSLOT, T::BYTES>(); };
  const LdsOffsets<D> off(lane);
  const int64_t kv_plane = (int64_t)w.b * A.Hkv + w.hkv;
  // K / V rows: in place, the plane of the natural-order arrays (block row j
  // at its token's row); staged, the host's compact block (row j at j)
  const bool staged = G.kv_staged != 0;
  const int64_t kv_base =
      staged ? ((int64_t)(w.q_rank - G.stage_host0) * A.B * A.Hkv + kv_plane) * A.Lkv : kv_plane * G.n_tok;
  const unsigned rec_rows = (unsigned)((staged ? (int64_t)A.Lkv : G.n_tok) * T::RB);
  const __amdgpu_buffer_rsrc_t rk = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<unsigned short*>(reinterpret_cast<const unsigned short*>(A.k)) + kv_base * D, 0, rec_rows,
      0x00020000);
  const __amdgpu_buffer_rsrc_t rv = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<unsigned short*>(reinterpret_cast<const unsigned short*>(A.v)) + kv_base * D, 0, rec_rows,
      0x00020000);
  // Lane l of load instruction i fills LDS slot 64 i + l of the tile: row
  // ROWS_PER_INSTR i + l / CPR, chunk slot l % CPR holding logical chunk
  // (l % CPR) ^ dswz(row); keys past the block read as zeros.
  auto issue = [&](int t, auto slot) __attribute__((always_inline)) {
#pragma unroll
    for (int u = 0; u < PER_WAVE; ++u) {
      const int ins = wave * PER_WAVE + u;
      const int r = ins * ROWS_PER_INSTR + lane / T::CPR;
      const int q = lane % T::CPR;
      const int j = t * kRows + r;
      const int src = staged ? j : lrow<LAYOUT>(w.kv_rank, j, A.Lkv, A.P);
      const int voff = j < A.Lkv ? src * T::RB + 16 * (q ^ dswz<D>(r)) : (int)rec_rows;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rk, (__attribute__((address_space(3))) void*)(kbuf(slot) + ins * 1024),
                                               16, voff, 0, 0, 0);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rv, (__attribute__((address_space(3))) void*)(vbuf(slot) + ins * 1024),
                                               16, voff, 0, 0, 0);
    }
  };

  static_for<LOOK>([&](auto I) __attribute__((always_inline)) {
    if (decltype(I)::value < ntiles) issue(decltype(I)::value, I);
  });
  // tile t: S^T = K Q^T and dP^T = V dO^T ([32 keys x 32 queries], one query
  // per lane column; register r holds key 32 t + 8 (r / 4) + 4 half + r % 4),
  // dS^T, then dQ^T += K^T dS^T (contraction over the tile's keys)
  auto body = [&](auto slot_tag, int t) __attribute__((always_inline)) {
    constexpr int SL = decltype(slot_tag)::value;
    constexpr int SF = (SL + LOOK) % NSLOT;
    // tile t must have landed: only the loads of tiles t+1, t+2 may remain
    if (t + 2 < ntiles) wait_vmcnt<2 * LOADS>();
    else if (t + 1 < ntiles) wait_vmcnt<LOADS>();
    else wait_vmcnt0();
    barrier_no_fence();
    if (t + LOOK < ntiles) issue(t + LOOK, IC<SF>{});   // its slot held tile t-1, done before the barrier
    const unsigned char* kt = kbuf(IC<SL>{});
    const unsigned char* vt = vbuf(IC<SL>{});
    // K and V fragments read two MFMA steps (four MFMAs) ahead of use
    constexpr int RA = 2;
    f32x16 s = f32x16{}, dp = f32x16{};
    bf16x8 ka[RA], va[RA];
    static_for<RA>([&](auto I) __attribute__((always_inline)) {
      ka[decltype(I)::value] = read_rowfrag<D>(kt, off, decltype(I)::value);
      va[decltype(I)::value] = read_rowfrag<D>(vt, off, decltype(I)::value);
    });
    static_for<KS>([&](auto T_) __attribute__((always_inline)) {
      constexpr int t = decltype(T_)::value;
      const bf16x8 a = ka[t % RA], b = va[t % RA];
      if constexpr (t + RA < KS) {
        ka[t % RA] = read_rowfrag<D>(kt, off, t + RA);
        va[t % RA] = read_rowfrag<D>(vt, off, t + RA);
      }
      s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[t], s, 0, 0, 0);
      dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(b, of[t], dp, 0, 0, 0);
      __builtin_amdgcn_sched_barrier(0);
    });
    // causal limit per element, only on the tiles past the wave's fully
    // visible prefix (the limits do not decrease along the rows)
    if (t * kRows + kRows - 1 > wave_first_lim) {
      const int bound = lim32 - t * kRows - 4 * half;
#pragma unroll
      for (int r = 0; r < 16; ++r)
        if (8 * (r >> 2) + (r & 3) > bound) s[r] = kNegInf;
    }
    f32x16 dsf;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const float p = fast_exp2(__builtin_fmaf(s[r], c, -lse2));
      dsf[r] = p * (dp[r] - del);
    }
#pragma unroll
    for (int hc = 0; hc < 2; ++hc) {
      const bf16x8 db8 = pack8(dsf, 8 * hc);
#pragma unroll
      for (int db = 0; db < NDB; ++db)
        dqT[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(read_trfrag<D>(kt, off, db, hc), db8, dqT[db], 0, 0, 0);
    }
  };
  int t = 0;
  for (; t + NSLOT <= ntiles; t += NSLOT)
    static_for<NSLOT>([&](auto k) __attribute__((always_inline)) {
      body(std::integral_constant<int, decltype(k)::value>{}, t + decltype(k)::value);
    });
  static_for<NSLOT - 1>([&](auto k) __attribute__((always_inline)) {
    if (t + decltype(k)::value < ntiles) body(std::integral_constant<int, decltype(k)::value>{}, t + decltype(k)::value);
  });
  const bool first = G.first != 0;
  const bool fin = ((G.q_fin >> w.q_rank) & 1ull) != 0;
  if (!row_ok || (ntiles == 0 && !first && !fin)) return;
  float* dq_row = G.dq_acc + qrow * D;
#pragma unroll
  for (int db = 0; db < NDB; ++db) emit_block(dq_row, G.dq_out + qrow * D, dqT[db], db, half, G.scale, first, fin);
}

// Row statistics (lse2_i, delta_i), interleaved per row: delta_i =
// sum_c dO_ic O_ic and the base-2 lse the kernels subtract, lse2_i = lse_i
// log2(e), +inf for a row without visible keys (so that its P is 0).  A row is d/8 lanes, each with one 16-byte chunk of O and of dO
// (read once: nontemporal loads); the lanes of a row are an aligned group,
// so the butterfly stays inside it.
__global__ __launch_bounds__(256) void bwd_prep_kernel(const __bf16* out, const __bf16* dout, const float* lse,
                                                        float* rowstat, int64_t rows, int d) {
  const int cpr = d >> 3;                       // 8 or 16 lanes per row
  const int t = (int)threadIdx.x;
  const int64_t row = (int64_t)blockIdx.x * (256 / cpr) + t / cpr;
  const int c = t % cpr;
  const bool ok = row < rows;
  float acc = 0.f;
  if (ok) {
    const bf16x8 o = __builtin_bit_cast(
        bf16x8, __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(out + row * d) + c));
    const bf16x8 g = __builtin_bit_cast(
        bf16x8, __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(dout + row * d) + c));
#pragma unroll
    for (int e = 0; e < 8; ++e) acc += (float)o[e] * (float)g[e];
  }
  for (int m = cpr >> 1; m >= 1; m >>= 1) acc += __shfl_xor(acc, m);
  if (ok && c == 0) {
    const float l = lse[row];
    *reinterpret_cast<float2*>(rowstat + 2 * row) = make_float2(l == kNegInf ? __builtin_huge_valf() : l * kLog2e, acc);
  }
}

}  // namespace

int bwd_dq_rows() { return kDqRows; }
int bwd_dkdv_rows() { return kDkdvKeys; }

hipError_t launch_bwd_prep(const void* out, const void* dout, const float* lse, float* rowstat, int64_t rows, int d,
                           hipStream_t s) {
  if (rows <= 0) return hipSuccess;
  if (d != 64 && d != 128) return hipErrorInvalidValue;
  const int64_t per_block = 256 / (d / 8);      // rows per workgroup
  const int64_t g = (rows + per_block - 1) / per_block;
  if (g > 0x7fffffffLL) return hipErrorInvalidValue;
  hipLaunchKernelGGL(bwd_prep_kernel, dim3((unsigned)g), dim3(256), 0, s,
                     reinterpret_cast<const __bf16*>(out), reinterpret_cast<const __bf16*>(dout), lse, rowstat, rows, d);
  return hipGetLastError();
}

template <int D, int L>
hipError_t launch_dkdv_t(const BwdArgs& a, unsigned g, hipStream_t s) {
  hipLaunchKernelGGL((bwd_dkdv_kernel<D, L>), dim3(g), dim3(kDkdvThreads), 0, s, a);
  return hipGetLastError();
}

template <int D, int L>
hipError_t launch_dq_t(const BwdArgs& a, unsigned g, hipStream_t s) {
  hipLaunchKernelGGL((bwd_dq_kernel<D, L>), dim3(g), dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

template <int D>
hipError_t launch_dkdv_d(const BwdArgs& a, unsigned g, hipStream_t s) {
  switch (a.s.layout) {
    case 0: return launch_dkdv_t<D, 0>(a, g, s);
    case 1: return launch_dkdv_t<D, 1>(a, g, s);
    case 2: return launch_dkdv_t<D, 2>(a, g, s);
    default: return hipErrorInvalidValue;
  }
}

template <int D>
hipError_t launch_dq_d(const BwdArgs& a, unsigned g, hipStream_t s) {
  switch (a.s.layout) {
    case 0: return launch_dq_t<D, 0>(a, g, s);
    case 1: return launch_dq_t<D, 1>(a, g, s);
    case 2: return launch_dq_t<D, 2>(a, g, s);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_bwd_dkdv(const BwdArgs& a, int d, hipStream_t s) {
  const int64_t g = (int64_t)a.s.n_hosts * a.s.B * a.s.Hkv * a.n_kvtiles;
  if (g <= 0) return hipSuccess;
  if (g > 0x7fffffffLL) return hipErrorInvalidValue;
  if (d == 128) return launch_dkdv_d<128>(a, (unsigned)g, s);
  if (d == 64) return launch_dkdv_d<64>(a, (unsigned)g, s);
  return hipErrorInvalidValue;
}

hipError_t launch_bwd_dq(const BwdArgs& a, int d, hipStream_t s) {
  const int64_t g = (int64_t)a.s.n_hosts * a.s.B * a.s.H * a.s.n_qtiles;
  if (g <= 0) return hipSuccess;
  if (g > 0x7fffffffLL) return hipErrorInvalidValue;
  if (d == 128) return launch_dq_d<128>(a, (unsigned)g, s);
  if (d == 64) return launch_dq_d<64>(a, (unsigned)g, s);
  return hipErrorInvalidValue;
}

}  // namespace ra

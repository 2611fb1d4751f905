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

// v_mfma_f32_32x32x16_bf16 as volatile inline asm, so that it keeps its
// place among a step's other instructions (the builtin is a pure function
// the optimizer moves freely, and in the dK/dV loop it gathered the MFMAs
// at the end of the tile, after all the exponentials).  The accumulator
// lives in VGPRs (_v) or AGPRs (_a); _z starts it from zero.  The compiler
// does not know these are MFMAs, so a VALU read of the result must come
// after mfma_settle (18 wait states cover the longest MFMA).
// (The zero-start form marks its result early-clobber: an MFMA must not
// write registers it still reads.)
__device__ __forceinline__ void mfma_v_z(f32x16& acc, const bf16x8& a, const bf16x8& b) {
  asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, 0" : "=&v"(acc) : "v"(a), "v"(b));
}
__device__ __forceinline__ void mfma_v(f32x16& acc, const bf16x8& a, const bf16x8& b) {
  asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(acc) : "v"(a), "v"(b));
}
__device__ __forceinline__ void mfma_a(f32x16& acc, const bf16x8& a, const bf16x8& b) {
  asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+a"(acc) : "v"(a), "v"(b));
}
__device__ __forceinline__ void mfma_settle() { asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory"); }

// ---------------------------------------------------------------------------
// dK / dV: one workgroup per (query host, batch, kv head, 128-key tile).  It
// sweeps, for every query head of the kv head's group, the 32-row query
// tiles that see any of its keys.
// ---------------------------------------------------------------------------
template <int D, int LAYOUT>
__global__ __launch_bounds__(kThreads, 1) void bwd_dkdv_kernel(BwdArgs G) {
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
  const int half = lane >> 5, col = lane & 31;
  const float c = A.scale_log2;

  // this lane's key and the wave's key range
  const int key0 = kt * kDkdvKeys;
  const int my_key = key0 + wave * 32 + col;
  const bool key_ok = my_key < A.Lkv;
  const int64_t kv_plane = (int64_t)w.b * A.Hkv + w.hkv;
  const int64_t key_row = key_ok ? nat_row<LAYOUT>(A, kv_plane, G.n_tok, w.kv_rank, my_key, A.Lkv) : 0;

  bf16x8 kf[KS], vf[KS];
  load_row_frags<D>(kf, reinterpret_cast<const unsigned short*>(A.k), key_row, key_ok, half);
  load_row_frags<D>(vf, reinterpret_cast<const unsigned short*>(A.v), key_row, key_ok, half);

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

  f32x16 dvT[NDB], dkT[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) dvT[db] = dkT[db] = f32x16{};

  // Five LDS slots for the streamed (Q, dO, lse, delta, limit) tiles.  Tile
  // t+3 is loaded straight into LDS (buffer_load ... lds, no registers)
  // while tile t is consumed, so each load has two tiles of time to land.
  constexpr int NSLOT = 5, LOOK = 3;
  constexpr int ROWS_PER_INSTR = 1024 / T::RB;        // tile rows per 1 KiB load instruction
  constexpr int INSTR = T::BYTES / 1024;              // per tensor per tile
  constexpr int PER_WAVE = INSTR / 4;                 // per wave
  constexpr int LOADS = 2 * PER_WAVE + 2;             // vector loads per wave per tile (Q, dO, lse, delta)
  static_assert(PER_WAVE >= 1 && INSTR % 4 == 0, "tile must split over the four waves");
  // Per slot: the Q and dO tiles; lse / delta, where wave w loads rows
  // 8 w .. 8 w + 7 with 4-byte lanes (every lane of the load owns a float of
  // the wave's 64-float area; lanes 8..63 read out of range and write zeros
  // there); the causal limits of the tile's rows.
  auto qbuf = [](auto I) { return slot_buf<0, decltype(I)::value % NSLOT, T::BYTES>(); };
  auto obuf = [](auto I) { return slot_buf<1, decltype(I)::value % NSLOT, T::BYTES>(); };
  auto lseb = [](auto I) { return reinterpret_cast<float(*)[64]>(slot_buf<2, decltype(I)::value % NSLOT, 1024>()); };
  auto delb = [](auto I) { return reinterpret_cast<float(*)[64]>(slot_buf<3, decltype(I)::value % NSLOT, 1024>()); };
  auto lims = [](auto I) { return reinterpret_cast<int*>(slot_buf<4, decltype(I)::value % NSLOT, 4 * kRows>()); };
  const LdsOffsets<D> off(lane);
  const int64_t plane_elems = G.n_tok * D;
  const unsigned rec_rows = (unsigned)(G.n_tok * T::RB);   // bytes of one (b, h) plane
  const unsigned rec_vec = (unsigned)(G.n_tok * 4);

  // tile it: head hkv*group + it / nqt, query tile qt0 + it % nqt.  Lane
  // l of load instruction i fills LDS slot 64 i + l of the tile: row
  // ROWS_PER_INSTR i + l / CPR, chunk slot l % CPR holding logical chunk
  // (l % CPR) ^ dswz(row).  Rows past the block read as zeros (offset out
  // of the buffer's range).
  // A tile index past the last one issues the same loads with every offset
  // out of range (they write zeros into the slot and touch no memory), so
  // that the loop body has no branch: the compiler would otherwise sink the
  // MFMAs of a step into the block after it, away from the exponentials
  // they are meant to overlap.
  auto issue = [&](int it_in, auto slot) __attribute__((always_inline)) {
    const bool valid = it_in < total;
    const int it = valid ? it_in : 0;
    const int h = w.hkv * group + it / nqt;
    const int row0 = (qt0 + it % nqt) * kRows;
    const int64_t qplane = (int64_t)w.b * A.H + h;
    const __amdgpu_buffer_rsrc_t rq = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<unsigned short*>(reinterpret_cast<const unsigned short*>(A.q)) + qplane * plane_elems, 0,
        rec_rows, 0x00020000);
    const __amdgpu_buffer_rsrc_t ro = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<unsigned short*>(reinterpret_cast<const unsigned short*>(G.dout)) + qplane * plane_elems, 0,
        rec_rows, 0x00020000);
#pragma unroll
    for (int u = 0; u < PER_WAVE; ++u) {
      const int ins = wave * PER_WAVE + u;
      const int r = ins * ROWS_PER_INSTR + lane / T::CPR;
      const int q = lane % T::CPR;
      const int i = row0 + r;
      const int voff = (valid && i < A.Lq) ? lrow<LAYOUT>(w.q_rank, i, A.Lq, A.P) * T::RB + 16 * (q ^ dswz<D>(r))
                                           : (int)rec_rows;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rq, (__attribute__((address_space(3))) void*)(qbuf(slot) + ins * 1024),
                                               16, voff, 0, 0, 0);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(ro, (__attribute__((address_space(3))) void*)(obuf(slot) + ins * 1024),
                                               16, voff, 0, 0, 0);
    }
    // lse and delta: wave w loads rows 8 w .. 8 w + 7 (lanes 0..7)
    const __amdgpu_buffer_rsrc_t rl = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<float*>(G.lse2) + qplane * G.n_tok, 0, rec_vec, 0x00020000);
    const __amdgpu_buffer_rsrc_t rd = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<float*>(G.delta) + qplane * G.n_tok, 0, rec_vec, 0x00020000);
    {
      const int i = row0 + 8 * wave + lane;
      const int voff = (valid && lane < 8 && i < A.Lq) ? lrow<LAYOUT>(w.q_rank, i, A.Lq, A.P) * 4 : (int)rec_vec;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rl, (__attribute__((address_space(3))) void*)(&lseb(slot)[wave][0]),
                                               4, voff, 0, 0, 0);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rd, (__attribute__((address_space(3))) void*)(&delb(slot)[wave][0]),
                                               4, voff, 0, 0, 0);
    }
    if (threadIdx.x < kRows) {
      const int i = row0 + threadIdx.x;
      lims(slot)[threadIdx.x] = i < A.Lq ? llim<LAYOUT>(A, w.q_rank, w.kv_rank, i) : -1;
    }
  };

  // S and dP of a tile: [32 queries x 32 keys], one key per lane column;
  // register r holds query 8 (r / 4) + 4 half + r % 4 of the tile.
  f32x16 sc = f32x16{}, dpc = f32x16{};
  if (total > 0) {
    static_for<LOOK>([&](auto I) __attribute__((always_inline)) {
      if (decltype(I)::value < total) issue(decltype(I)::value, I);
    });
    wait_vmcnt0();
    __syncthreads();
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      sc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(read_rowfrag<D>(qbuf(IC<0>{}), off, ks), kf[ks], sc, 0, 0, 0);
      dpc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(read_rowfrag<D>(obuf(IC<0>{}), off, ks), vf[ks], dpc, 0, 0, 0);
    }
  }

  // One iteration per query tile t, cut into one-MFMA-pair steps fenced with
  // sched_barrier.  Step i issues
  //   S(t+1) (even i) or dP(t+1) (odd i): one MFMA, 2 accumulators;
  //   dV^T += dO^T P(t-1) (even i) or dK^T += Q^T dS(t-1) (odd i): one MFMA,
  //   2 NDB accumulators;
  // and the VALU turns one element of S(t), dP(t) into P(t), dS(t).  The
  // MFMA pipe therefore always has 2 + 2 NDB independent chains in flight
  // and the exponentials hide under them.  Tile t's slot keeps (Q, dO)
  // until the dV/dK products of iteration t+1, so five slots are needed:
  // t-1 (transposed reads), t (row statistics), t+1 (row reads), t+2
  // (landing), t+3 (loading).
  bf16x8 pbp[2], dsbp[2];   // packed P(t-1), dS(t-1)
  auto body = [&](auto slot_tag, auto hasb_tag, int t) __attribute__((always_inline)) {
    bf16x8 pbn[2], dsbn[2];  // packed P(t), dS(t), filled pair by pair
    float p_prev = 0.f, ds_prev = 0.f;
    constexpr int SL = decltype(slot_tag)::value;          // t % NSLOT
    constexpr int SN = (SL + 1) % NSLOT;                   // tile t+1
    constexpr int SP = (SL + NSLOT - 1) % NSLOT;           // tile t-1
    constexpr int SF = (SL + LOOK) % NSLOT;                // tile t+3 (the slot held t-2)
    constexpr bool HASB = decltype(hasb_tag)::value;       // t >= 1
    issue(t + LOOK, IC<SF>{});
    // (S(t+1), dP(t+1) are computed even for the last tile: the slot holds
    // stale rows then and the results are not used.)
    f32x16 sn, dpn;
    constexpr int NA = 2 * KS;        // S / dP MFMAs per tile
    constexpr int NB = 4 * NDB;       // dV / dK MFMAs per tile
    static_assert(NA == NB, "one S/dP and one dV/dK MFMA per step");
    constexpr int PFA = 4, PFB = 3;   // steps whose operands are read ahead
    auto afrag = [&](int i) __attribute__((always_inline)) -> bf16x8 {
      return (i & 1) ? read_rowfrag<D>(obuf(IC<SN>{}), off, i >> 1) : read_rowfrag<D>(qbuf(IC<SN>{}), off, i >> 1);
    };
    // dV on even steps, dK on odd ones; (db, hc) = ((j / 2) % NDB, (j / 2) / NDB)
    auto bfrag = [&](int j) __attribute__((always_inline)) -> bf16x8 {
      const int db = (j >> 1) % NDB, hc = (j >> 1) / NDB;
      return (j & 1) ? read_trfrag<D>(qbuf(IC<SP>{}), off, db, hc) : read_trfrag<D>(obuf(IC<SP>{}), off, db, hc);
    };
    bf16x8 fa[PFA], fb[PFB];
#pragma unroll
    for (int i = 0; i < PFA; ++i) fa[i] = afrag(i);
    if constexpr (HASB) {
#pragma unroll
      for (int j = 0; j < PFB; ++j) fb[j] = bfrag(j);
    }
    // Row statistics of tile t (lse2, delta, causal limit) in groups of four
    // rows, each group read one group ahead of its use.
    float lv[2][4], dv[2][4];
    int lm[2][4];
    auto rowstats = [&](int g, int k) __attribute__((always_inline)) {
      const int q0 = 8 * g + 4 * half;   // rows q0 .. q0 + 3 (loaded by wave g)
      const float4 l4 = *reinterpret_cast<const float4*>(&lseb(IC<SL>{})[g][4 * half]);
      const float4 d4 = *reinterpret_cast<const float4*>(&delb(IC<SL>{})[g][4 * half]);
      const int4 m4 = *reinterpret_cast<const int4*>(&lims(IC<SL>{})[q0]);
      lv[k][0] = l4.x; lv[k][1] = l4.y; lv[k][2] = l4.z; lv[k][3] = l4.w;
      dv[k][0] = d4.x; dv[k][1] = d4.y; dv[k][2] = d4.z; dv[k][3] = d4.w;
      lm[k][0] = m4.x; lm[k][1] = m4.y; lm[k][2] = m4.z; lm[k][3] = m4.w;
    };
    rowstats(0, 0);
    static_for<NA>([&](auto ic) __attribute__((always_inline)) {
      constexpr int i = decltype(ic)::value;
      {
        const bf16x8 a = fa[i % PFA];
        if constexpr (i + PFA < NA) fa[i % PFA] = afrag(i + PFA);
        if constexpr (i == 0) mfma_v_z(sn, a, kf[0]);
        else if constexpr (i == 1) mfma_v_z(dpn, a, vf[0]);
        else if constexpr ((i & 1) == 0) mfma_v(sn, a, kf[i >> 1]);
        else mfma_v(dpn, a, vf[i >> 1]);
      }
      if constexpr (HASB) {
        constexpr int db = (i >> 1) % NDB, hc = (i >> 1) / NDB;
        const bf16x8 b = fb[i % PFB];
        if constexpr (i + PFB < NB) fb[i % PFB] = bfrag(i + PFB);
        if constexpr ((i & 1) == 0) mfma_a(dvT[db], b, pbp[hc]);
        else mfma_a(dkT[db], b, dsbp[hc]);
      }
      // VALU: the 16 elements of tile t spread over the NA steps.  The causal
      // limit is applied to every element (a row's limit is at least every
      // key of an unmasked tile, so the test is a no-op there); testing per
      // element keeps the step free of branches.
      static_for<16>([&](auto rc) __attribute__((always_inline)) {
        constexpr int r = decltype(rc)::value;
        if constexpr (r * NA / 16 == i) {
          constexpr int g = r >> 2, k = g & 1;
          if constexpr ((r & 3) == 0 && g + 1 < 4) rowstats(g + 1, k ^ 1);
          float x = sc[r];
          asm volatile("" : "+v"(x));   // (keeps the element's arithmetic in this step)
          float p = fast_exp2(__builtin_fmaf(x, c, -lv[k][r & 3]));
          p = my_key > lm[k][r & 3] ? 0.f : p;
          float ds = p * (dpc[r] - dv[k][r & 3]);
          asm volatile("" : "+v"(p), "+v"(ds));
          if constexpr (r & 1) {
            pbn[r >> 3][(r & 7) - 1] = (__bf16)p_prev;
            pbn[r >> 3][r & 7] = (__bf16)p;
            dsbn[r >> 3][(r & 7) - 1] = (__bf16)ds_prev;
            dsbn[r >> 3][r & 7] = (__bf16)ds;
          } else {
            p_prev = p;
            ds_prev = ds;
          }
        }
      });
      __builtin_amdgcn_sched_barrier(0);
    });
    mfma_settle();   // S(t+1), dP(t+1) are read by the VALU from here on
#pragma unroll
    for (int hc = 0; hc < 2; ++hc) {
      pbp[hc] = pbn[hc];
      dsbp[hc] = dsbn[hc];
    }
    sc = sn;
    dpc = dpn;
    // tile t+2 must have landed before the next iteration reads it: only
    // tile t+3's loads (issued above) may still be in flight (and the causal
    // limits written with ds_write are visible)
    wait_vmcnt<LOADS>();
    wait_lgkmcnt0();
    barrier_no_fence();
  };
  // The dV / dK products of the last tile, alone.
  auto drain = [&](auto slot_tag) __attribute__((always_inline)) {
    constexpr int SP = decltype(slot_tag)::value;
    constexpr int NB = 4 * NDB;
    static_for<NB>([&](auto jc) __attribute__((always_inline)) {
      constexpr int j = decltype(jc)::value;
      constexpr int db = (j >> 1) % NDB, hc = (j >> 1) / NDB;
      if constexpr ((j & 1) == 0)
        dvT[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(read_trfrag<D>(obuf(IC<SP>{}), off, db, hc), pbp[hc],
                                                          dvT[db], 0, 0, 0);
      else
        dkT[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(read_trfrag<D>(qbuf(IC<SP>{}), off, db, hc), dsbp[hc],
                                                          dkT[db], 0, 0, 0);
    });
  };

  using Yes = std::integral_constant<bool, true>;
  using No = std::integral_constant<bool, false>;
  if (total > 0) {
    body(IC<0>{}, No{}, 0);
    int t = 1;
    for (; t + NSLOT - 1 < total; t += NSLOT)   // t % NSLOT == 1
      static_for<NSLOT>([&](auto k) __attribute__((always_inline)) {
        body(IC<(decltype(k)::value + 1) % NSLOT>{}, Yes{}, t + decltype(k)::value);
      });
    static_for<NSLOT - 1>([&](auto k) __attribute__((always_inline)) {
      if (t + decltype(k)::value < total) body(IC<(decltype(k)::value + 1) % NSLOT>{}, Yes{}, t + decltype(k)::value);
    });
    switch ((total - 1) % NSLOT) {
      case 0: drain(IC<0>{}); break;
      case 1: drain(IC<1>{}); break;
      case 2: drain(IC<2>{}); break;
      case 3: drain(IC<3>{}); break;
      default: drain(IC<4>{}); break;
    }
    wait_vmcnt0();   // the last iterations' loads past the end (zeros into free slots)
  }
  // (A key tile no query sees still writes its zeros on the first launch
  // and its final values on the last.)
  const bool first = G.first != 0;
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
  const int kv_end = llim<LAYOUT>(A, w.q_rank, w.kv_rank, row_last) + 1;
  const int ntiles = (int)((kv_end + kRows - 1) / kRows);

  const int64_t qplane = (int64_t)w.b * A.H + w.h;
  const int64_t qrow = row_ok ? nat_row<LAYOUT>(A, qplane, G.n_tok, w.q_rank, my_row, A.Lq) : 0;
  bf16x8 qf[KS], of[KS];
  load_row_frags<D>(qf, reinterpret_cast<const unsigned short*>(A.q), qrow, row_ok, half);
  load_row_frags<D>(of, reinterpret_cast<const unsigned short*>(G.dout), qrow, row_ok, half);
  const float lse2 = row_ok ? G.lse2[qrow] : __builtin_huge_valf();   // past the block: P = 0
  const float del = row_ok ? G.delta[qrow] : 0.f;

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
  const unsigned rec_rows = (unsigned)(G.n_tok * T::RB);
  const __amdgpu_buffer_rsrc_t rk = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<unsigned short*>(reinterpret_cast<const unsigned short*>(A.k)) + kv_plane * G.n_tok * D, 0, rec_rows,
      0x00020000);
  const __amdgpu_buffer_rsrc_t rv = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<unsigned short*>(reinterpret_cast<const unsigned short*>(A.v)) + kv_plane * G.n_tok * D, 0, rec_rows,
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
      const int voff = j < A.Lkv ? lrow<LAYOUT>(w.kv_rank, j, A.Lkv, A.P) * T::RB + 16 * (q ^ dswz<D>(r)) : (int)rec_rows;
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
    f32x16 s = f32x16{}, dp = f32x16{};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(read_rowfrag<D>(kt, off, ks), qf[ks], s, 0, 0, 0);
      dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(read_rowfrag<D>(vt, off, ks), of[ks], dp, 0, 0, 0);
    }
    // causal limit per element, branch free (a no-op on unmasked tiles)
    const int bound = lim32 - t * kRows - 4 * half;
    f32x16 dsf;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      float p = fast_exp2(__builtin_fmaf(s[r], c, -lse2));
      p = 8 * (r >> 2) + (r & 3) > bound ? 0.f : p;
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

// delta_i = sum_c dO_ic O_ic and the base-2 lse the kernels subtract:
// lse2_i = lse_i log2(e), +inf for a row without visible keys (so that its P
// is 0).  A row is d/8 lanes, each with one 16-byte chunk of O and of dO
// (read once: nontemporal loads); the lanes of a row are an aligned group,
// so the butterfly stays inside it.
__global__ __launch_bounds__(256) void bwd_prep_kernel(const __bf16* out, const __bf16* dout, const float* lse,
                                                        float* delta, float* lse2, int64_t rows, int d) {
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
    delta[row] = acc;
    const float l = lse[row];
    lse2[row] = l == kNegInf ? __builtin_huge_valf() : l * kLog2e;
  }
}

}  // namespace

int bwd_dq_rows() { return kDqRows; }
int bwd_dkdv_rows() { return kDkdvKeys; }

hipError_t launch_bwd_prep(const void* out, const void* dout, const float* lse, float* delta, float* lse2,
                           int64_t rows, int d, hipStream_t s) {
  if (rows <= 0) return hipSuccess;
  if (d != 64 && d != 128) return hipErrorInvalidValue;
  const int64_t per_block = 256 / (d / 8);      // rows per workgroup
  hipLaunchKernelGGL(bwd_prep_kernel, dim3((unsigned)((rows + per_block - 1) / per_block)), dim3(256), 0, s,
                     reinterpret_cast<const __bf16*>(out), reinterpret_cast<const __bf16*>(dout), lse, delta, lse2,
                     rows, d);
  return hipGetLastError();
}

template <int D, int L>
hipError_t launch_dkdv_t(const BwdArgs& a, unsigned g, hipStream_t s) {
  hipLaunchKernelGGL((bwd_dkdv_kernel<D, L>), dim3(g), dim3(kThreads), 0, s, a);
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
  if (d == 128) return launch_dkdv_d<128>(a, (unsigned)g, s);
  if (d == 64) return launch_dkdv_d<64>(a, (unsigned)g, s);
  return hipErrorInvalidValue;
}

hipError_t launch_bwd_dq(const BwdArgs& a, int d, hipStream_t s) {
  const int64_t g = (int64_t)a.s.n_hosts * a.s.B * a.s.H * a.s.n_qtiles;
  if (g <= 0) return hipSuccess;
  if (d == 128) return launch_dq_d<128>(a, (unsigned)g, s);
  if (d == 64) return launch_dq_d<64>(a, (unsigned)g, s);
  return hipErrorInvalidValue;
}

}  // namespace ra

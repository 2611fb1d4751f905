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
//   S = scale Q K^T,  P = exp(S - lse)      (lse = m + ln l of the forward)
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

// Natural-order row of host `rank`'s block row i in plane `plane` of an
// array with n_tok rows per plane.
__device__ __forceinline__ int64_t nat_row(const StepArgs& A, int64_t plane, int64_t n_tok, int rank, int64_t i,
                                           int blk) {
  return plane * n_tok + host_row(A.layout, rank, i, blk, A.P);
}

// Global -> register prefetch and register -> LDS store of one 32-row tile
// of a natural-order bf16 array; rows at or beyond `valid` read as zero.
template <int D>
struct TileRegs {
  u32x4 v[RowTile<D>::PER_THREAD];
};

template <int D, typename RowFn>
__device__ __forceinline__ void tile_fetch(TileRegs<D>& t, const unsigned short* base, int64_t row0, int valid,
                                           RowFn&& row_of) {
  using T = RowTile<D>;
#pragma unroll
  for (int u = 0; u < T::PER_THREAD; ++u) {
    const int ch = u * kThreads + threadIdx.x;
    const int r = ch / T::CPR, c = ch % T::CPR;
    const int64_t i = row0 + r;
    t.v[u] = i < valid ? *reinterpret_cast<const u32x4*>(base + row_of(i) * D + 8 * c) : u32x4{0u, 0u, 0u, 0u};
  }
}

template <int D>
__device__ __forceinline__ void tile_store(const TileRegs<D>& t, unsigned char* lds) {
  using T = RowTile<D>;
#pragma unroll
  for (int u = 0; u < T::PER_THREAD; ++u) {
    const int ch = u * kThreads + threadIdx.x;
    const int r = ch / T::CPR, c = ch % T::CPR;
    *reinterpret_cast<u32x4*>(lds + r * T::RB + 16 * (c ^ dswz<D>(r))) = t.v[u];
  }
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

// Add a [32 x 32] accumulator block (rows = dims 32 db + 8 (r / 4) + 4 half +
// r % 4, column = this lane's row) times `mul` into an fp32 row of D floats.
__device__ __forceinline__ void add_block(float* dst_row, const f32x16& acc, int db, int half, float mul) {
#pragma unroll
  for (int g = 0; g < 4; ++g) {
    float4* p = reinterpret_cast<float4*>(dst_row + 32 * db + 8 * g + 4 * half);
    float4 x = *p;
    x.x += mul * acc[4 * g];
    x.y += mul * acc[4 * g + 1];
    x.z += mul * acc[4 * g + 2];
    x.w += mul * acc[4 * g + 3];
    *p = x;
  }
}

// ---------------------------------------------------------------------------
// dK / dV: one workgroup per (query host, batch, kv head, 128-key tile).  It
// sweeps, for every query head of the kv head's group, the 32-row query
// tiles that see any of its keys.
// ---------------------------------------------------------------------------
template <int D>
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
  const int64_t key0 = (int64_t)kt * kDkdvKeys;
  const int64_t my_key = key0 + wave * 32 + col;
  const bool key_ok = my_key < A.Lkv;
  const int64_t kv_plane = (int64_t)w.b * A.Hkv + w.hkv;
  const int64_t key_row = key_ok ? nat_row(A, kv_plane, G.n_tok, w.kv_rank, my_key, A.Lkv) : 0;
  const int64_t wave_last = (key0 + wave * 32 + 31 < A.Lkv ? key0 + wave * 32 + 31 : A.Lkv - 1);

  bf16x8 kf[KS], vf[KS];
  load_row_frags<D>(kf, reinterpret_cast<const unsigned short*>(A.k), key_row, key_ok, half);
  load_row_frags<D>(vf, reinterpret_cast<const unsigned short*>(A.v), key_row, key_ok, half);

  // first query row that sees any key of the workgroup (key_limit is
  // non-decreasing in the row)
  int i0 = 0;
  if (A.causal) {
    int lo = 0, hi = A.Lq;
    while (lo < hi) {
      const int mid = (lo + hi) >> 1;
      if (key_limit(A, w, mid) >= key0) hi = mid; else lo = mid + 1;
    }
    i0 = lo;
  }
  const int qt0 = i0 / kRows;
  const int nqt = (A.Lq + kRows - 1) / kRows - qt0;   // query tiles per head
  const int total = nqt > 0 ? nqt * group : 0;

  f32x16 dvT[NDB], dkT[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) dvT[db] = dkT[db] = f32x16{};

  __shared__ __align__(1024) unsigned char qbuf[2][T::BYTES];
  __shared__ __align__(1024) unsigned char obuf[2][T::BYTES];
  __shared__ __align__(16) float lse2s[2][kRows];
  __shared__ __align__(16) float dels[2][kRows];
  __shared__ __align__(16) int lims[2][kRows];
  const LdsOffsets<D> off(lane);
  const unsigned short* Qb = reinterpret_cast<const unsigned short*>(A.q);
  const unsigned short* Ob = reinterpret_cast<const unsigned short*>(G.dout);

  // iteration it: head g*group + it / nqt, query tile qt0 + it % nqt
  auto tile_of = [&](int it, int& h, int64_t& row0) {
    h = w.hkv * group + it / nqt;
    row0 = (int64_t)(qt0 + it % nqt) * kRows;
  };
  TileRegs<D> rq, ro;
  float pre_lse = 0.f, pre_del = 0.f;
  int pre_lim = -1;
  auto fetch = [&](int it) {
    int h;
    int64_t row0;
    tile_of(it, h, row0);
    const int64_t qplane = (int64_t)w.b * A.H + h;
    auto rowf = [&](int64_t i) { return nat_row(A, qplane, G.n_tok, w.q_rank, i, A.Lq); };
    tile_fetch<D>(rq, Qb, row0, A.Lq, rowf);
    tile_fetch<D>(ro, Ob, row0, A.Lq, rowf);
    if (threadIdx.x < kRows) {
      const int64_t i = row0 + threadIdx.x;
      if (i < A.Lq) {
        const int64_t r = rowf(i);
        const float l = G.lse[r];
        pre_lse = l == kNegInf ? __builtin_huge_valf() : l * kLog2e;   // no visible key: P = 0
        pre_del = G.delta[r];
        pre_lim = (int)key_limit(A, w, i);
      } else {
        pre_lse = __builtin_huge_valf();   // no such query: P = 0
        pre_del = 0.f;
        pre_lim = -1;
      }
    }
  };
  auto stash = [&](int buf) {
    tile_store<D>(rq, qbuf[buf]);
    tile_store<D>(ro, obuf[buf]);
    if (threadIdx.x < kRows) {
      lse2s[buf][threadIdx.x] = pre_lse;
      dels[buf][threadIdx.x] = pre_del;
      lims[buf][threadIdx.x] = pre_lim;
    }
  };

  if (total > 0) {
    fetch(0);
    stash(0);
    if (total > 1) fetch(1);
    __syncthreads();
  }
  for (int it = 0; it < total; ++it) {
    const int buf = it & 1;
    if (it + 1 < total) {
      stash(buf ^ 1);                 // tile it+1 (its buffer was freed by the last barrier)
      if (it + 2 < total) fetch(it + 2);
    }
    const unsigned char* qt = qbuf[buf];
    const unsigned char* ot = obuf[buf];
    // S = Q K^T and dP = dO V^T, [32 queries x 32 keys], one key per lane column
    f32x16 s = f32x16{}, dp = f32x16{};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(read_rowfrag<D>(qt, off, ks), kf[ks], s, 0, 0, 0);
      dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(read_rowfrag<D>(ot, off, ks), vf[ks], dp, 0, 0, 0);
    }
    // register r holds query 8 (r / 4) + 4 half + r % 4 of the tile
    const bool masked = A.causal && lims[buf][0] < wave_last;
    f32x16 pf, dsf;
#pragma unroll
    for (int g4 = 0; g4 < 4; ++g4) {
      const int q0 = 8 * g4 + 4 * half;
      const float4 l4 = *reinterpret_cast<const float4*>(&lse2s[buf][q0]);
      const float4 d4 = *reinterpret_cast<const float4*>(&dels[buf][q0]);
      const float lv[4] = {l4.x, l4.y, l4.z, l4.w};
      const float dv[4] = {d4.x, d4.y, d4.z, d4.w};
      int lm[4] = {0, 0, 0, 0};
      if (masked) {
        const int4 m4 = *reinterpret_cast<const int4*>(&lims[buf][q0]);
        lm[0] = m4.x; lm[1] = m4.y; lm[2] = m4.z; lm[3] = m4.w;
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int r = 4 * g4 + e;
        float p = fast_exp2(__builtin_fmaf(s[r], c, -lv[e]));
        if (masked && my_key > lm[e]) p = 0.f;
        pf[r] = p;
        dsf[r] = p * (dp[r] - dv[e]);
      }
    }
    // dV^T += dO^T P and dK^T += Q^T dS (contraction over the tile's queries)
#pragma unroll
    for (int hc = 0; hc < 2; ++hc) {
      const bf16x8 pb = pack8(pf, 8 * hc);
      const bf16x8 db8 = pack8(dsf, 8 * hc);
#pragma unroll
      for (int db = 0; db < NDB; ++db) {
        dvT[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(read_trfrag<D>(ot, off, db, hc), pb, dvT[db], 0, 0, 0);
        dkT[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(read_trfrag<D>(qt, off, db, hc), db8, dkT[db], 0, 0, 0);
      }
    }
    __syncthreads();
  }
  if (!key_ok || total == 0) return;
  float* dk_row = G.dk_acc + key_row * D;
  float* dv_row = G.dv_acc + key_row * D;
#pragma unroll
  for (int db = 0; db < NDB; ++db) {
    add_block(dk_row, dkT[db], db, half, G.scale);
    add_block(dv_row, dvT[db], db, half, 1.f);
  }
}

// ---------------------------------------------------------------------------
// dQ: one workgroup per (query host, batch, query head, 128-row query tile),
// sweeping the visible 32-key tiles of the paired kv block.
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(kThreads, 2) void bwd_dq_kernel(BwdArgs G) {
  using T = RowTile<D>;
  constexpr int KS = D / 16, NDB = D / 32;
  const StepArgs& A = G.s;
  const Work w = decode_work(A);   // n_qtiles counts 128-row query tiles
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int half = lane >> 5, col = lane & 31;
  const float c = A.scale_log2;
  const int64_t row_first = (int64_t)w.qtile * kDqRows;
  const int64_t row_last = (row_first + kDqRows < A.Lq ? row_first + kDqRows : A.Lq) - 1;
  const int64_t wave_first = row_first + wave * 32 < row_last ? row_first + wave * 32 : row_last;
  const int64_t my_row = row_first + wave * 32 + col;
  const bool row_ok = my_row < A.Lq;
  const int lim32 = (int)key_limit(A, w, row_ok ? my_row : row_last);
  const int64_t kv_end = key_limit(A, w, row_last) + 1;
  const int64_t full_end = key_limit(A, w, wave_first) + 1;
  const int ntiles = (int)((kv_end + kRows - 1) / kRows);

  const int64_t qplane = (int64_t)w.b * A.H + w.h;
  const int64_t qrow = row_ok ? nat_row(A, qplane, G.n_tok, w.q_rank, my_row, A.Lq) : 0;
  bf16x8 qf[KS], of[KS];
  load_row_frags<D>(qf, reinterpret_cast<const unsigned short*>(A.q), qrow, row_ok, half);
  load_row_frags<D>(of, reinterpret_cast<const unsigned short*>(G.dout), qrow, row_ok, half);
  const float lse_in = row_ok ? G.lse[qrow] : kNegInf;
  const float lse2 = lse_in == kNegInf ? __builtin_huge_valf() : lse_in * kLog2e;   // no visible key: P = 0
  const float del = row_ok ? G.delta[qrow] : 0.f;

  f32x16 dqT[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) dqT[db] = f32x16{};

  __shared__ __align__(1024) unsigned char kbuf[2][T::BYTES];
  __shared__ __align__(1024) unsigned char vbuf[2][T::BYTES];
  const LdsOffsets<D> off(lane);
  const unsigned short* Kb = reinterpret_cast<const unsigned short*>(A.k);
  const unsigned short* Vb = reinterpret_cast<const unsigned short*>(A.v);
  const int64_t kv_plane = (int64_t)w.b * A.Hkv + w.hkv;
  auto rowf = [&](int64_t j) { return nat_row(A, kv_plane, G.n_tok, w.kv_rank, j, A.Lkv); };
  TileRegs<D> rk, rv;
  auto fetch = [&](int t) {
    tile_fetch<D>(rk, Kb, (int64_t)t * kRows, A.Lkv, rowf);
    tile_fetch<D>(rv, Vb, (int64_t)t * kRows, A.Lkv, rowf);
  };
  auto stash = [&](int buf) {
    tile_store<D>(rk, kbuf[buf]);
    tile_store<D>(rv, vbuf[buf]);
  };

  if (ntiles > 0) {
    fetch(0);
    stash(0);
    if (ntiles > 1) fetch(1);
    __syncthreads();
  }
  for (int t = 0; t < ntiles; ++t) {
    const int buf = t & 1;
    if (t + 1 < ntiles) {
      stash(buf ^ 1);
      if (t + 2 < ntiles) fetch(t + 2);
    }
    const unsigned char* kt = kbuf[buf];
    const unsigned char* vt = vbuf[buf];
    // S^T = K Q^T and dP^T = V dO^T, [32 keys x 32 queries], one query per lane column
    f32x16 s = f32x16{}, dp = f32x16{};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(read_rowfrag<D>(kt, off, ks), qf[ks], s, 0, 0, 0);
      dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(read_rowfrag<D>(vt, off, ks), of[ks], dp, 0, 0, 0);
    }
    // register r holds key t*32 + 8 (r / 4) + 4 half + r % 4
    const bool masked = t * kRows + kRows > full_end;
    const int bound = lim32 - t * kRows - 4 * half;
    f32x16 dsf;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      float p = fast_exp2(__builtin_fmaf(s[r], c, -lse2));
      if (masked && 8 * (r >> 2) + (r & 3) > bound) p = 0.f;
      dsf[r] = p * (dp[r] - del);
    }
    // dQ^T += K^T dS^T (contraction over the tile's keys)
#pragma unroll
    for (int hc = 0; hc < 2; ++hc) {
      const bf16x8 db8 = pack8(dsf, 8 * hc);
#pragma unroll
      for (int db = 0; db < NDB; ++db)
        dqT[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(read_trfrag<D>(kt, off, db, hc), db8, dqT[db], 0, 0, 0);
    }
    __syncthreads();
  }
  if (!row_ok || ntiles == 0) return;
  float* dq_row = G.dq_acc + qrow * D;
#pragma unroll
  for (int db = 0; db < NDB; ++db) add_block(dq_row, dqT[db], db, half, G.scale);
}

// delta_i = sum_c dO_ic O_ic (one wavefront per row), bf16 inputs.
__global__ __launch_bounds__(256) void bwd_prep_kernel(const __bf16* out, const __bf16* dout, float* delta,
                                                        int64_t rows, int d) {
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (row >= rows) return;
  float acc = 0.f;
  for (int cc = lane; cc < d; cc += 64) acc += (float)out[row * d + cc] * (float)dout[row * d + cc];
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) acc += __shfl_xor(acc, o);
  if (lane == 0) delta[row] = acc;
}

__global__ __launch_bounds__(256) void fill_zero_kernel(float* p, int64_t n) {
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256) p[i] = 0.f;
}

__global__ __launch_bounds__(256) void to_bf16_kernel(const float* src, __bf16* dst, int64_t n) {
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256)
    dst[i] = (__bf16)src[i];
}

unsigned elementwise_grid(int64_t n) {
  int64_t g = (n + 255) / 256;
  return (unsigned)(g < 8192 ? (g < 1 ? 1 : g) : 8192);
}

}  // namespace

int bwd_dq_rows() { return kDqRows; }
int bwd_dkdv_rows() { return kDkdvKeys; }

hipError_t launch_bwd_prep(const void* out, const void* dout, float* delta, int64_t rows, int d, hipStream_t s) {
  if (rows <= 0) return hipSuccess;
  hipLaunchKernelGGL(bwd_prep_kernel, dim3((unsigned)((rows + 3) / 4)), dim3(256), 0, s,
                     reinterpret_cast<const __bf16*>(out), reinterpret_cast<const __bf16*>(dout), delta, rows, d);
  return hipGetLastError();
}

hipError_t launch_fill_zero(float* p, int64_t n, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(fill_zero_kernel, dim3(elementwise_grid(n)), dim3(256), 0, s, p, n);
  return hipGetLastError();
}

hipError_t launch_to_bf16(const float* src, void* dst, int64_t n, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(to_bf16_kernel, dim3(elementwise_grid(n)), dim3(256), 0, s, src,
                     reinterpret_cast<__bf16*>(dst), n);
  return hipGetLastError();
}

hipError_t launch_bwd_dkdv(const BwdArgs& a, int d, hipStream_t s) {
  const int64_t g = (int64_t)a.s.n_hosts * a.s.B * a.s.Hkv * a.n_kvtiles;
  if (g <= 0) return hipSuccess;
  if (d == 128) hipLaunchKernelGGL(bwd_dkdv_kernel<128>, dim3((unsigned)g), dim3(kThreads), 0, s, a);
  else if (d == 64) hipLaunchKernelGGL(bwd_dkdv_kernel<64>, dim3((unsigned)g), dim3(kThreads), 0, s, a);
  else return hipErrorInvalidValue;
  return hipGetLastError();
}

hipError_t launch_bwd_dq(const BwdArgs& a, int d, hipStream_t s) {
  const int64_t g = (int64_t)a.s.n_hosts * a.s.B * a.s.H * a.s.n_qtiles;
  if (g <= 0) return hipSuccess;
  if (d == 128) hipLaunchKernelGGL(bwd_dq_kernel<128>, dim3((unsigned)g), dim3(kThreads), 0, s, a);
  else if (d == 64) hipLaunchKernelGGL(bwd_dq_kernel<64>, dim3((unsigned)g), dim3(kThreads), 0, s, a);
  else return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace ra

// Split-KV decode for gfx950: one query token per sequence against a long
// key/value cache split into P ring blocks, each block into chunks.
//
// Pages cited: "RingAttention 심층 아키텍처 ..." (techknowgenie.com) §3 for
// the online-softmax update and §3 O_final; the RingAttention newsletter
// (cmlonder.com) for the decode-time KV-cache footprint that makes this
// pass bound by HBM bandwidth.
//
// The pass streams every key/value row from HBM once per sub-group of 16
// query heads of its group (once in all for H/Hkv <= 16) and uses it for
// all heads of the sub-group.  Scores S^T = K Q^T run on
// v_mfma_f32_16x16x32_bf16 with K as the A operand loaded straight from
// global memory (16 contiguous bytes per lane) and the sub-group's query
// heads as the 16 MFMA columns (the columns past the group are zero).  V goes through a
// per-wave LDS transpose so that O^T = V^T P^T runs on the same MFMA with P
// taken straight from the score registers.  Each wavefront writes one
// normalized partial (O, lse); a second kernel merges the partials of each
// ring block and then the ring blocks.
#include <mutex>

#include "ra_internal.h"

namespace ra {

// Static scratch of ring_attn_decode_noalloc (the per-wavefront partials
// that ring_attn_decode keeps in the caller's workspace), for callers that
// cannot allocate.  Each GPU the library runs on holds its own copy until
// the process ends.  In host code `scratch` names a host-side stand-in:
// kernels get the device address that hipGetSymbolAddress returns for it
// (decode_scratch below), never the name itself.
__device__ __align__(256) unsigned char scratch[kDecodeScratchBytes];

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kTau = 8.0f;
constexpr float kNegInf = -__builtin_huge_valf();
constexpr int kWaves = 4;
constexpr int kTile = 32;       // keys per wave iteration
constexpr int kVP = kTile + 4;  // V^T LDS pitch (bf16 elements)

__device__ __forceinline__ float xor_max(float x, int m) { return fmaxf(x, __shfl_xor(x, m)); }

template <int D>
__global__ __launch_bounds__(256, 2) void decode_partial_kernel(DecodeArgs A) {
  __shared__ __align__(16) unsigned short vt_all[kWaves][D * kVP];
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int lg = lane >> 4;    // lane group 0..3
  const int lc = lane & 15;    // MFMA column = query head within the group
  unsigned short* vt = vt_all[wave];

  // blockIdx -> (b, hkv, sub-group, split) with the split index fastest; a
  // sub-group is 16 query heads of the kv head's group (the MFMA columns).
  const int S_blk = A.P * A.chunks_per_block;
  const int split = blockIdx.x % S_blk;
  const int rest = blockIdx.x / S_blk;
  const int sg = rest % A.sub_groups;
  const int bh = rest / A.sub_groups;
  const int hkv = bh % A.Hkv;
  const int b = bh / A.Hkv;
  const int hq = sg * 16 + lc;   // this lane column's query head within the group
  const int p = split / A.chunks_per_block;
  const int cidx = split % A.chunks_per_block;
  int64_t k_begin = (int64_t)p * A.block + (int64_t)cidx * A.chunk;
  int64_t k_end = k_begin + A.chunk;
  const int64_t blk_end = (int64_t)(p + 1) * A.block;
  if (k_end > blk_end) k_end = blk_end;

  const unsigned short* Kp = reinterpret_cast<const unsigned short*>(A.k) +
                             ((int64_t)b * A.Hkv + hkv) * A.L * D;
  const unsigned short* Vp = reinterpret_cast<const unsigned short*>(A.v) +
                             ((int64_t)b * A.Hkv + hkv) * A.L * D;

  // Query heads of the group as B operand columns (zero beyond the group).
  bf16x8 qf[D / 32];
  {
    const bool live = hq < A.group;
    const int h = hkv * A.group + (live ? hq : 0);
    const unsigned short* Q = reinterpret_cast<const unsigned short*>(A.q) +
                              ((int64_t)b * A.H + h) * D;
#pragma unroll
    for (int ks = 0; ks < D / 32; ++ks) {
      u32x4 x = live ? *reinterpret_cast<const u32x4*>(Q + ks * 32 + lg * 8) : u32x4{0u, 0u, 0u, 0u};
      qf[ks] = __builtin_bit_cast(bf16x8, x);
    }
  }

  f32x4 oacc[D / 16];
#pragma unroll
  for (int db = 0; db < D / 16; ++db) oacc[db] = f32x4{};
  float m_run = kNegInf, l_run = 0.f, lb_run = 0.f;
  const float c = A.scale_log2;

  constexpr int CPR = D / 8;                       // 16-byte chunks per row
  constexpr int VUNITS = (kTile / 4) * CPR;        // 4-key x 8-dim units per tile
  constexpr int VU = VUNITS / 64;

  // The loads of a wave's next tile are issued before the current tile's
  // arithmetic (two register sets, the loop unrolled by two).
  // Every K and V row is read once (its query heads share the wave), so the
  // loads are nontemporal: streaming reads measured 6.0 TB/s with ordinary
  // loads and 6.6 TB/s with nontemporal ones.
  auto load_tile = [&](int64_t t0, u32x4 (&kr)[2][D / 32], u32x4 (&vr)[VU][4]) __attribute__((always_inline)) {
    // K as A operand: lane holds key t0 + 16*kg + lc, dims 32*ks + 8*lg.
#pragma unroll
    for (int kg = 0; kg < 2; ++kg) {
      const int64_t j = t0 + kg * 16 + lc;
#pragma unroll
      for (int ks = 0; ks < D / 32; ++ks)
        kr[kg][ks] = j < k_end ? __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(Kp + j * D + ks * 32 + lg * 8))
                               : u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int u = 0; u < VU; ++u) {
      const int unit = lane + u * 64;
      const int dg = unit % CPR, kq = unit / CPR;
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        const int64_t j = t0 + kq * 4 + kk;
        vr[u][kk] = j < k_end ? __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(Vp + j * D + dg * 8))
                              : u32x4{0u, 0u, 0u, 0u};
      }
    }
  };

  auto tile = [&](int64_t t0, const u32x4 (&kr)[2][D / 32], const u32x4 (&vr)[VU][4]) __attribute__((always_inline)) {
    f32x4 s[2];
#pragma unroll
    for (int kg = 0; kg < 2; ++kg) {
      s[kg] = f32x4{};
#pragma unroll
      for (int ks = 0; ks < D / 32; ++ks)
        s[kg] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, kr[kg][ks]),
                                                        qf[ks], s[kg], 0, 0, 0);
    }
    // s[kg][r] = S^T[key t0 + 16 kg + 4 lg + r][head lc]
    if (t0 + kTile > k_end) {
#pragma unroll
      for (int kg = 0; kg < 2; ++kg)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          if (t0 + kg * 16 + 4 * lg + r >= k_end) s[kg][r] = kNegInf;
    }
    float mx = fmaxf(fmaxf(fmaxf(s[0][0], s[0][1]), fmaxf(s[0][2], s[0][3])),
                     fmaxf(fmaxf(s[1][0], s[1][1]), fmaxf(s[1][2], s[1][3])));
    mx = xor_max(mx, 16);
    mx = xor_max(mx, 32);
    const float m_tile = mx * c;
    const bool need = m_tile > m_run + kTau;
    if (__builtin_amdgcn_ballot_w64(need) != 0ull) {
      const float m_new = fmaxf(m_run, m_tile);
      const float alpha = m_new == kNegInf ? 1.f : __builtin_amdgcn_exp2f(m_run - m_new);
      l_run *= alpha;
      lb_run *= alpha;
#pragma unroll
      for (int db = 0; db < D / 16; ++db)
#pragma unroll
        for (int r = 0; r < 4; ++r) oacc[db][r] *= alpha;
      m_run = m_new;
    }
    const float m_use = m_run == kNegInf ? 0.f : m_run;
    // B operand: contraction index k = 8*lg + e <-> key 16*(e/4) + 4*lg + e%4.
    // fp32 weights for the row sum l (lse), their bf16 rounding for P V and
    // for the sum lb that normalizes the output (the weights P V applies).
    bf16x8 pb;
    float lsum = 0.f, lbsum = 0.f;
    const bf16x2 ones = {(__bf16)1.f, (__bf16)1.f};
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float pe = __builtin_amdgcn_exp2f(__builtin_fmaf(s[e >> 2][e & 3], c, -m_use));
      lsum += pe;
      pb[e] = (__bf16)pe;
    }
#pragma unroll
    for (int e = 0; e < 8; e += 2) {
      const bf16x2 pair = {pb[e], pb[e + 1]};
      lbsum = __builtin_amdgcn_fdot2_f32_bf16(pair, ones, lbsum, false);
    }
    l_run += lsum;
    lb_run += lbsum;

    // V tile -> V^T in this wave's LDS slice.
#pragma unroll
    for (int u = 0; u < VU; ++u) {
      const int unit = lane + u * 64;
      const int dg = unit % CPR, kq = unit / CPR;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const unsigned sel = (i & 1) ? 0x07060302u : 0x05040100u;
        const int dw = i >> 1;
        u32x2 pr;
        pr[0] = __builtin_amdgcn_perm(vr[u][1][dw], vr[u][0][dw], sel);
        pr[1] = __builtin_amdgcn_perm(vr[u][3][dw], vr[u][2][dw], sel);
        *reinterpret_cast<u32x2*>(vt + (dg * 8 + i) * kVP + kq * 4) = pr;
      }
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
    for (int db = 0; db < D / 16; ++db) {
      const unsigned short* row = vt + (db * 16 + lc) * kVP + 4 * lg;
      u32x2 lo = *reinterpret_cast<const u32x2*>(row);
      u32x2 hi = *reinterpret_cast<const u32x2*>(row + 16);
      u32x4 av = {lo[0], lo[1], hi[0], hi[1]};
      oacc[db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, av), pb,
                                                         oacc[db], 0, 0, 0);
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  };

  const int64_t stride = (int64_t)kWaves * kTile;
  u32x4 krA[2][D / 32], vrA[VU][4], krB[2][D / 32], vrB[VU][4];
  int64_t t0 = k_begin + (int64_t)wave * kTile;
  if (t0 < k_end) load_tile(t0, krA, vrA);
  for (; t0 < k_end; t0 += 2 * stride) {
    if (t0 + stride < k_end) load_tile(t0 + stride, krB, vrB);
    tile(t0, krA, vrA);
    if (t0 + stride >= k_end) break;
    if (t0 + 2 * stride < k_end) load_tile(t0 + 2 * stride, krA, vrA);
    tile(t0 + stride, krB, vrB);
  }

  // l: the four lane groups hold disjoint keys of the same head.
  float l_tot = l_run + __shfl_xor(l_run, 16);
  l_tot += __shfl_xor(l_tot, 32);
  float lb_tot = lb_run + __shfl_xor(lb_run, 16);
  lb_tot += __shfl_xor(lb_tot, 32);
  if (hq >= A.group) return;
  const int h = hkv * A.group + hq;
  const int S_all = A.S;
  const int sidx = split * kWaves + wave;
  const int64_t pidx = ((int64_t)b * A.H + h) * S_all + sidx;
  const float inv = lb_tot > 0.f ? 1.f / lb_tot : 0.f;
  float* op = A.o_part + pidx * D;
#pragma unroll
  for (int db = 0; db < D / 16; ++db)
    *reinterpret_cast<float4*>(op + db * 16 + 4 * lg) =
        make_float4(oacc[db][0] * inv, oacc[db][1] * inv, oacc[db][2] * inv, oacc[db][3] * inv);
  if (lg == 0) A.lse_part[pidx] = l_tot > 0.f ? (m_run + __builtin_amdgcn_logf(l_tot)) * kLn2 : kNegInf;
}

// Merge: one workgroup per (b, h).  Wave w merges the partials of ring
// blocks w, w + 4, ... into each block's (O, lse); wave 0 then merges the
// ring blocks in order.  (The arithmetic and its order per (b, h) are those
// of a single wave doing both in turn; the four waves only run the block
// merges side by side.)
constexpr int kMaxRingBlocks = 64;
template <int D, bool kBf16>
__global__ __launch_bounds__(256) void decode_merge_kernel(DecodeArgs A) {
  const int64_t bh = blockIdx.x;
  const int wave = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  constexpr int PER = D / 64;  // dims per lane
  __shared__ float blk_o[kMaxRingBlocks][D];
  __shared__ float blk_lse[kMaxRingBlocks];
  const int per_block = A.chunks_per_block * kWaves;
  const float* lp = A.lse_part + bh * A.S;
  const float* op = A.o_part + bh * A.S * D;
  for (int p = wave; p < A.P; p += kWaves) {
    float M = kNegInf;
    for (int i = 0; i < per_block; ++i) M = fmaxf(M, lp[p * per_block + i]);
    float blk[PER];
    for (int e = 0; e < PER; ++e) blk[e] = 0.f;
    float W = 0.f;
    if (M != kNegInf) {
      for (int i = 0; i < per_block; ++i) {
        const int si = p * per_block + i;
        const float w = __builtin_amdgcn_exp2f((lp[si] - M) * kLog2e);
        W += w;
        for (int e = 0; e < PER; ++e) blk[e] += w * op[(int64_t)si * D + lane * PER + e];
      }
    }
    const float lse_b = W > 0.f ? M + __builtin_amdgcn_logf(W) * kLn2 : kNegInf;
    if (W > 0.f) {
      const float inv = 1.f / W;
      for (int e = 0; e < PER; ++e) blk[e] *= inv;
    }
    for (int e = 0; e < PER; ++e) blk_o[p][lane * PER + e] = blk[e];
    if (lane == 0) blk_lse[p] = lse_b;
  }
  __syncthreads();
  if (wave != 0) return;
  float acc[PER];
  for (int e = 0; e < PER; ++e) acc[e] = 0.f;
  float lse_run = kNegInf;
  for (int p = 0; p < A.P; ++p) {
    // ring merge: (acc, lse_run) <- merge((acc, lse_run), (block p's O, lse))
    const float lse_b = blk_lse[p];
    const float MM = fmaxf(lse_run, lse_b);
    if (MM != kNegInf) {
      float wa = __builtin_amdgcn_exp2f((lse_run - MM) * kLog2e);
      float wb = __builtin_amdgcn_exp2f((lse_b - MM) * kLog2e);
      const float tot = wa + wb;
      const float inv = 1.f / tot;
      for (int e = 0; e < PER; ++e) acc[e] = (wa * acc[e] + wb * blk_o[p][lane * PER + e]) * inv;
      lse_run = MM + __builtin_amdgcn_logf(tot) * kLn2;
    }
  }
  for (int e = 0; e < PER; ++e) {
    if constexpr (kBf16) reinterpret_cast<__bf16*>(A.out)[bh * D + lane * PER + e] = (__bf16)acc[e];
    else reinterpret_cast<float*>(A.out)[bh * D + lane * PER + e] = acc[e];
  }
  if (lane == 0) A.lse[bh] = lse_run;
}

}  // namespace

hipError_t decode_scratch(void** ptr, size_t* bytes) {
  // Looked up once per device, with that device current (the first call on
  // it), and kept: every device holds the array at its own address.
  constexpr int kMaxDev = 64;
  static std::mutex mu;
  static void* addr[kMaxDev] = {};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDev) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lk(mu);
  if (!addr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    addr[dev] = p;
  }
  *ptr = addr[dev];
  *bytes = kDecodeScratchBytes;
  return hipSuccess;
}

hipError_t launch_decode_partial(const DecodeArgs& a, int d, int bf16, hipStream_t s) {
  if (!bf16) return hipErrorInvalidValue;
  const int64_t g = (int64_t)a.B * a.Hkv * a.sub_groups * a.P * a.chunks_per_block;
  if (g <= 0) return hipSuccess;
  if (d == 128) hipLaunchKernelGGL(decode_partial_kernel<128>, dim3((unsigned)g), dim3(256), 0, s, a);
  else if (d == 64) hipLaunchKernelGGL(decode_partial_kernel<64>, dim3((unsigned)g), dim3(256), 0, s, a);
  else return hipErrorInvalidValue;
  return hipGetLastError();
}

hipError_t launch_decode_merge(const DecodeArgs& a, int d, int bf16, hipStream_t s) {
  const int64_t g = (int64_t)a.B * a.H;
  if (g <= 0) return hipSuccess;
  if (a.P > kMaxRingBlocks) return hipErrorInvalidValue;
  if (d == 128) {
    if (bf16) hipLaunchKernelGGL((decode_merge_kernel<128, true>), dim3((unsigned)g), dim3(256), 0, s, a);
    else hipLaunchKernelGGL((decode_merge_kernel<128, false>), dim3((unsigned)g), dim3(256), 0, s, a);
  } else if (d == 64) {
    if (bf16) hipLaunchKernelGGL((decode_merge_kernel<64, true>), dim3((unsigned)g), dim3(256), 0, s, a);
    else hipLaunchKernelGGL((decode_merge_kernel<64, false>), dim3((unsigned)g), dim3(256), 0, s, a);
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace ra

// Host side of the ring-attention library: argument checks, the mask-aware
// step scheduler, the ring-step driver (two HIP streams, events, staging
// double buffer) and the C ABI of include/ring_attn.h.
//
// Pages cited (by title; section named alone):
//   [TKG] "RingAttention 심층 아키텍처 ..." (techknowgenie.com): §2 sequence
//         sharding and the KV ring, §4 compute/communication overlap,
//         §5 the per-rank step loop with a dedicated communication stream and
//         a double-buffered KV block, §7 causal imbalance and striping.
//
// The P ranks of the page are P virtual hosts on one GPU.  The page's
// send-to-next / receive-from-previous exchange becomes a device-to-device
// copy on a second stream: at step s host r computes with the kv block of
// host (r - s) mod P, which sits at host r's own row positions of the
// staging buffer used at step s; the copy for step s + 1 shifts that buffer
// by one host into the other staging buffer while step s computes.
// Ordering (both directions, unlike a one-way wait):
//   copy(s+1)    waits for compute(s-1)  (it overwrites what step s-1 read)
//   compute(s)   waits for copy(s)
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdint>
#include <initializer_list>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <string>
#include <vector>

#include "ra_internal.h"
#include "ring_attn.h"

using namespace ra;

namespace {

thread_local std::string g_err;

ra_status fail(ra_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_err = buf;
  return st;
}

ra_status hip_fail(hipError_t e, const char* what) {
  return fail(RA_EHIP, "%s: %s", what, hipGetErrorString(e));
}

#define RA_HIP(call, what)                          \
  do {                                              \
    hipError_t _e = (call);                         \
    if (_e != hipSuccess) return hip_fail(_e, what); \
  } while (0)

constexpr int kMaxDevices = 64;
constexpr int kMaxP = 64;
constexpr size_t kAlign = 256;

struct DeviceCtx {
  bool ready = false;
  std::mutex enqueue;  // one multi-stream call at a time per device (shared events)
  hipStream_t copy = nullptr;
  hipEvent_t fork = nullptr, join = nullptr;
  hipEvent_t copied[2] = {nullptr, nullptr};
  hipEvent_t done[2] = {nullptr, nullptr};
};

std::mutex g_mu;
DeviceCtx g_dev[kMaxDevices];
int g_delay_compute_us = 0, g_delay_copy_us = 0;  // test hook (ra_debug_set_delays)
bool g_staging = true;  // ring exchange through staging copies (ra_debug_set_staging)

ra_status get_ctx(DeviceCtx** out) {
  int dev = 0;
  RA_HIP(hipGetDevice(&dev), "hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices) return fail(RA_EUNSUPPORTED, "device index %d out of range", dev);
  std::lock_guard<std::mutex> lk(g_mu);
  DeviceCtx& c = g_dev[dev];
  if (!c.ready) {
    RA_HIP(hipStreamCreateWithFlags(&c.copy, hipStreamNonBlocking), "hipStreamCreateWithFlags");
    RA_HIP(hipEventCreateWithFlags(&c.fork, hipEventDisableTiming), "hipEventCreate");
    RA_HIP(hipEventCreateWithFlags(&c.join, hipEventDisableTiming), "hipEventCreate");
    for (int i = 0; i < 2; ++i) {
      RA_HIP(hipEventCreateWithFlags(&c.copied[i], hipEventDisableTiming), "hipEventCreate");
      RA_HIP(hipEventCreateWithFlags(&c.done[i], hipEventDisableTiming), "hipEventCreate");
    }
    c.ready = true;
  }
  *out = &c;
  return RA_OK;
}

// ---------------------------------------------------------------------------
// Profiling: timing events around the fused step / decode kernels.
// ---------------------------------------------------------------------------
struct ProfRec {
  hipEvent_t a, b;
  double work;
  int kind;  // 0 step kernel, 1 decode kernel
};
struct Prof {
  bool on = false;
  std::vector<ProfRec> recs;
  std::vector<hipEvent_t> pool;
  double acc[6] = {0, 0, 0, 0, 0, 0};
} g_prof;

hipEvent_t prof_event() {
  if (!g_prof.pool.empty()) {
    hipEvent_t e = g_prof.pool.back();
    g_prof.pool.pop_back();
    return e;
  }
  // Timing-only events: no system-scope fence when they complete (nothing
  // synchronizes with them except the elapsed-time query after a device
  // synchronization), so recording them around a kernel costs little.
  hipEvent_t e = nullptr;
  if (hipEventCreateWithFlags(&e, hipEventDisableSystemFence) != hipSuccess) return nullptr;
  return e;
}

struct ProfScope {
  hipEvent_t a = nullptr, b = nullptr;
  hipStream_t s;
  double work;
  int kind;
  ProfScope(hipStream_t st, double w, int k) : s(st), work(w), kind(k) {
    if (!g_prof.on) return;
    std::lock_guard<std::mutex> lk(g_mu);
    a = prof_event();
    b = prof_event();
    if (a) hipEventRecord(a, s);
  }
  ~ProfScope() {
    if (!a || !b) return;
    hipEventRecord(b, s);
    std::lock_guard<std::mutex> lk(g_mu);
    g_prof.recs.push_back({a, b, work, kind});
  }
};

// ---------------------------------------------------------------------------
// Scheduler: which query hosts have visible work at a ring step, and the
// exact number of visible (query, key) pairs of a block pair.
// ---------------------------------------------------------------------------
int64_t clamp_prefix(int64_t x, int64_t M) {
  // F(x) = sum_{t=0}^{x-1} clamp(t, 0, M), F(x) = 0 for x <= 0.
  if (x <= 0) return 0;
  if (x <= M + 1) return x * (x - 1) / 2;
  return M * (M + 1) / 2 + (x - M - 1) * M;
}

// Visible (query, key) pairs between two chunks of c tokens at global chunk
// indices a (queries) and b (keys): all when b < a, the lower triangle with
// the diagonal when b == a, none when b > a.
int64_t chunk_pairs(int64_t a, int64_t b, int64_t c) {
  return b < a ? c * c : (b == a ? c * (c + 1) / 2 : 0);
}

// Visible pairs between query block q_rank (Lq rows) and kv block kv_rank
// (Lkv rows): query i sees keys j <= lim(i), lim(i) = i + c0 - 1.
int64_t visible_pairs(int layout, int causal, int P, int q_rank, int kv_rank, int64_t Lq, int64_t Lkv) {
  if (!causal) return Lq * Lkv;
  if (layout == RA_ZIGZAG) {
    // blocks of two chunks each: q_rank and 2P-1-q_rank, kv_rank and 2P-1-kv_rank
    const int64_t c = Lq / 2;
    const int64_t qa = q_rank, qb = 2 * P - 1 - q_rank, ka = kv_rank, kb = 2 * P - 1 - kv_rank;
    return chunk_pairs(qa, ka, c) + chunk_pairs(qa, kb, c) + chunk_pairs(qb, ka, c) + chunk_pairs(qb, kb, c);
  }
  int64_t c0 = layout == RA_CONTIGUOUS ? (int64_t)q_rank * Lq - (int64_t)kv_rank * Lkv + 1
                                       : 1 - (kv_rank > q_rank ? 1 : 0);
  // sum_{i=0}^{Lq-1} clamp(i + c0, 0, Lkv)
  return clamp_prefix(c0 + Lq, Lkv) - clamp_prefix(c0, Lkv);
}

// Does query host q_rank see anything of kv host kv_rank?
bool pair_active(int layout, int causal, int P, int q_rank, int kv_rank, int64_t Lq, int64_t Lkv) {
  return visible_pairs(layout, causal, P, q_rank, kv_rank, Lq, Lkv) > 0;
}

struct StepPlan {
  int host_lo, n_hosts;  // contiguous range of query hosts with work
  int fin_lo, fin_hi;    // hosts whose last active step this is
};

// Hosts r with work at step s (kv = (r - s) mod P).  For a contiguous causal
// ring these are r = s .. P-1 and host s finishes at step s ([TKG] §7: the
// later hosts see more of the past); for striped or unmasked rings every host
// works at every step and all finish at step P-1.
StepPlan plan_step(int layout, int causal, int P, int s, int64_t Bl) {
  StepPlan p{0, 0, 0, 0};
  int lo = -1, hi = -1;
  for (int r = 0; r < P; ++r) {
    const int kv = ((r - s) % P + P) % P;
    if (pair_active(layout, causal, P, r, kv, Bl, Bl)) {
      if (lo < 0) lo = r;
      hi = r;
    }
  }
  if (lo < 0) return p;
  p.host_lo = lo;
  p.n_hosts = hi - lo + 1;
  // last active step of each host in [lo, hi]
  int flo = P, fhi = -1;
  for (int r = lo; r <= hi; ++r) {
    int last = -1;
    for (int t = 0; t < P; ++t) {
      const int kv = ((r - t) % P + P) % P;
      if (pair_active(layout, causal, P, r, kv, Bl, Bl)) last = t;
    }
    if (last == s) {
      if (r < flo) flo = r;
      if (r > fhi) fhi = r;
    }
  }
  if (fhi >= flo) {
    p.fin_lo = flo;
    p.fin_hi = fhi + 1;
  }
  return p;
}


size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

// Tensor rows are read and written as 16-byte vectors (a row of d = 64 or 128
// elements keeps the base's alignment); per-row fp32 statistics as 4-byte words.
bool misaligned(const void* p, uintptr_t a) { return reinterpret_cast<uintptr_t>(p) % a != 0; }
ra_status check_tensor_align(std::initializer_list<const void*> vec16, std::initializer_list<const void*> word4) {
  for (const void* p : vec16)
    if (misaligned(p, 16)) return fail(RA_EINVAL, "tensor pointers must be 16-byte aligned");
  for (const void* p : word4)
    if (misaligned(p, 4)) return fail(RA_EINVAL, "fp32 statistics pointers must be 4-byte aligned");
  return RA_OK;
}
size_t esize(ra_dtype t) { return t == RA_BF16 ? 2 : 4; }
bool dtype_ok(int t) { return t == RA_F32 || t == RA_BF16; }
bool layout_ok(int l) { return l == RA_CONTIGUOUS || l == RA_STRIPED || l == RA_ZIGZAG; }

// Zigzag blocks are two chunks of N / (2P) tokens.  With one host the block
// is the whole sequence in natural order, i.e. the contiguous layout.
ra_status check_layout(int layout, long long N, int P) {
  if (!layout_ok(layout)) return fail(RA_EINVAL, "unknown layout %d", layout);
  if (layout == RA_ZIGZAG && N % (2LL * P))
    return fail(RA_EINVAL, "zigzag layout needs N (%lld) to be a multiple of 2P (%d)", N, 2 * P);
  return RA_OK;
}
int effective_layout(int layout, int P) { return (layout == RA_ZIGZAG && P == 1) ? RA_CONTIGUOUS : layout; }

ra_status check_common(int B, int H, int Hkv, long long N, int d, int P, ra_dtype dtype, float scale) {
  if (B < 1 || H < 1 || Hkv < 1) return fail(RA_EINVAL, "B, H, Hkv must be >= 1 (got %d, %d, %d)", B, H, Hkv);
  if (H % Hkv) return fail(RA_EINVAL, "H (%d) must be a multiple of Hkv (%d)", H, Hkv);
  if (d != 64 && d != 128) return fail(RA_EINVAL, "head dim d must be 64 or 128 (got %d)", d);
  if (P < 1 || P > kMaxP) return fail(RA_EINVAL, "P must be in [1, %d] (got %d)", kMaxP, P);
  if (N < 1) return fail(RA_EINVAL, "N must be >= 1");
  if (N % P) return fail(RA_EINVAL, "N (%lld) must be a multiple of P (%d)", N, P);
  if (N / P > (1LL << 30)) return fail(RA_EINVAL, "block length N/P too large");
  if (!dtype_ok(dtype)) return fail(RA_EINVAL, "unknown dtype %d", (int)dtype);
  if (!(scale > 0.f) || !std::isfinite(scale)) return fail(RA_EINVAL, "scale must be finite and > 0");
  return RA_OK;
}

// The bf16 step kernel reads a key/value block through a buffer descriptor
// with 32-bit offsets: one block of one (batch, kv head) plane must stay
// below 2 GiB.  (A striped ring whose whole plane is larger stages its first
// step's blocks instead of reading them in place; see stage_first_block.)
constexpr uint64_t kSpanLimit = 1ull << 31;
ra_status check_block_span(long long rows, int d, ra_dtype dtype) {
  if (dtype == RA_BF16 && (uint64_t)rows * d * esize(dtype) >= kSpanLimit)
    return fail(RA_EINVAL, "one key/value block of one head (%lld rows x %d) must stay below 2 GiB", rows, d);
  return RA_OK;
}

// Does the first ring step need its key/value blocks staged (compact) rather
// than read in place from the natural-order k / v?  Zigzag blocks are two
// separate chunks; a striped block read in place spans the whole plane,
// which the bf16 kernel's 32-bit buffer offsets reach only below 2 GiB.
bool stage_first_block(int layout, long long N, int d, int P, ra_dtype dtype) {
  if (layout == RA_ZIGZAG) return true;
  return layout == RA_STRIPED && P > 1 && dtype == RA_BF16 && (uint64_t)N * d * esize(dtype) >= kSpanLimit;
}

// Workspace sizes are computed in 64 bits with overflow checks.  Device
// virtual addresses are 48 bits wide, so anything at or above 2^48 bytes
// cannot be allocated: the size queries return SIZE_MAX and the launches
// RA_ENOMEM.
constexpr uint64_t kMaxAllocBytes = 1ull << 48;
struct SizeAcc {
  uint64_t total = 0;
  bool bad = false;
  // appends a region of n1 * n2 * ... bytes (aligned), returns its offset
  size_t add(std::initializer_list<uint64_t> factors) {
    uint64_t x = 1;
    for (uint64_t f : factors)
      if (__builtin_mul_overflow(x, f, &x)) bad = true;
    if (x >= kMaxAllocBytes) bad = true;
    const size_t off = (size_t)total;
    if (!bad) {
      x = (x + kAlign - 1) / kAlign * kAlign;
      if (__builtin_add_overflow(total, x, &total) || total >= kMaxAllocBytes) bad = true;
    }
    return off;
  }
};

struct FwdWs {
  size_t stage_bytes;  // one staging buffer (K and V)
  size_t kv_bytes;     // K (or V) part of a staging buffer
  size_t off_stage[2], off_m, off_l, off_o, total;
  bool overflow;       // the sizes do not fit a device allocation
};

FwdWs fwd_ws_layout(int B, int H, int Hkv, long long Nq, long long Nkv_stage, int d, int P, ra_dtype dtype) {
  FwdWs w{};
  if (P == 1) return w;  // single block: no staging, no state
  SizeAcc a;
  w.off_stage[0] = a.add({(uint64_t)B, (uint64_t)Hkv, (uint64_t)Nkv_stage, (uint64_t)d, esize(dtype)});
  const size_t k_end = (size_t)a.total;
  w.kv_bytes = k_end - w.off_stage[0];
  a.add({(uint64_t)B, (uint64_t)Hkv, (uint64_t)Nkv_stage, (uint64_t)d, esize(dtype)});
  w.stage_bytes = (size_t)a.total - w.off_stage[0];
  w.off_stage[1] = a.add({2, w.kv_bytes});
  w.off_m = a.add({(uint64_t)B, (uint64_t)H, (uint64_t)Nq, 4});
  w.off_l = a.add({(uint64_t)B, (uint64_t)H, (uint64_t)Nq, 4});
  w.off_o = a.add({(uint64_t)B, (uint64_t)H, (uint64_t)Nq, (uint64_t)d, 4});
  w.total = (size_t)a.total;
  w.overflow = a.bad;
  return w;
}

// Workspace check shared by the launches: RA_ENOMEM for sizes no device can
// hold, RA_EINVAL for a missing, short or misaligned workspace.
ra_status check_ws(bool overflow, size_t need, const void* ws, size_t ws_bytes) {
  if (overflow) return fail(RA_ENOMEM, "workspace size exceeds the 48-bit device address space");
  if (ws_bytes < need) return fail(RA_EINVAL, "workspace too small: need %zu bytes, got %zu", need, ws_bytes);
  if (need && !ws) return fail(RA_EINVAL, "null workspace");
  if (need && (reinterpret_cast<uintptr_t>(ws) % kAlign)) return fail(RA_EINVAL, "workspace must be 256-byte aligned");
  return RA_OK;
}

hipError_t launch_step(const StepArgs& a, int d, ra_dtype dtype, hipStream_t s, double flops) {
  ProfScope ps(s, flops, 0);
  return dtype == RA_BF16 ? launch_step_bf16(a, d, s) : launch_step_f32(a, d, s);
}

int block_rows(ra_dtype dtype, int d) {
  return dtype == RA_BF16 ? step_block_rows_bf16(d) : step_block_rows_f32(d);
}

double step_flops(const StepArgs& a, int d) {
  if (!g_prof.on) return 0.0;
  double pairs = 0;
  for (int i = 0; i < a.n_hosts; ++i) {
    const int qr = a.host_lo + i;
    const int kr = ((qr - a.kv_shift) % a.P + a.P) % a.P;
    pairs += (double)visible_pairs(a.layout, a.causal, a.P, qr, kr, a.Lq, a.Lkv);
  }
  return 4.0 * d * pairs * a.B * a.H;
}

// Staging copy helpers (2-D copies on the copy stream).
hipError_t copy2d(void* dst, size_t dpitch, const void* src, size_t spitch, size_t width, size_t height,
                  hipStream_t s) {
  if (width == 0 || height == 0) return hipSuccess;
  return hipMemcpy2DAsync(dst, dpitch, src, spitch, width, height, hipMemcpyDeviceToDevice, s);
}

// Staging buffers of ring_attn_fwd are host-major: [P hosts][planes][Bl][d],
// host r's current kv block contiguous at r * host_bytes.
//
// First hand-off: staging[r] <- host (r-1) mod P's block of the natural-order
// array, for receivers r in [r_lo, P).
hipError_t ring_gather_first(void* dst, const void* src, int layout, int64_t planes, int64_t N, int64_t Bl,
                             int P, int r_lo, size_t row_bytes, hipStream_t s) {
  char* D = static_cast<char*>(dst);
  const char* S = static_cast<const char*>(src);
  const size_t host_bytes = (size_t)planes * Bl * row_bytes;
  for (int r = r_lo; r < P; ++r) {
    const int from = (r + P - 1) % P;
    hipError_t e;
    if (layout == RA_CONTIGUOUS) {
      e = copy2d(D + r * host_bytes, (size_t)Bl * row_bytes, S + (size_t)from * Bl * row_bytes,
                 (size_t)N * row_bytes, (size_t)Bl * row_bytes, planes, s);
    } else {
      e = copy2d(D + r * host_bytes, row_bytes, S + (size_t)from * row_bytes, (size_t)P * row_bytes, row_bytes,
                 (size_t)planes * Bl, s);
    }
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

// Later hand-offs: dst[r] <- src[r-1] for receivers r in [r_lo, P) (one
// contiguous move), and dst[0] <- src[P-1] when host 0 receives.
hipError_t ring_shift(void* dst, const void* src, int64_t planes, int64_t Bl, int P, int r_lo, size_t row_bytes,
                      hipStream_t s) {
  char* D = static_cast<char*>(dst);
  const char* S = static_cast<const char*>(src);
  const size_t host_bytes = (size_t)planes * Bl * row_bytes;
  const int lo = r_lo > 1 ? r_lo : 1;
  hipError_t e = hipSuccess;
  if (lo < P) e = hipMemcpyAsync(D + lo * host_bytes, S + (lo - 1) * host_bytes, (P - lo) * host_bytes,
                                 hipMemcpyDeviceToDevice, s);
  if (e != hipSuccess || r_lo > 0) return e;
  return hipMemcpyAsync(D, S + (size_t)(P - 1) * host_bytes, host_bytes, hipMemcpyDeviceToDevice, s);
}

// dst (compact [planes, Bl, d]) <- block `kv` of src (natural [planes, N, d]).
hipError_t gather_block(void* dst, const void* src, int layout, int64_t planes, int64_t N, int64_t Bl,
                        int P, int kv, size_t row_bytes, hipStream_t s) {
  char* D = static_cast<char*>(dst);
  const char* S = static_cast<const char*>(src);
  if (layout == RA_CONTIGUOUS) {
    return copy2d(D, (size_t)Bl * row_bytes, S + (size_t)kv * Bl * row_bytes, (size_t)N * row_bytes,
                  (size_t)Bl * row_bytes, planes, s);
  }
  if (layout == RA_ZIGZAG) {
    const int64_t c = Bl / 2;
    const size_t cb = (size_t)c * row_bytes;
    hipError_t e = copy2d(D, (size_t)Bl * row_bytes, S + (size_t)kv * cb, (size_t)N * row_bytes, cb, planes, s);
    if (e != hipSuccess) return e;
    return copy2d(D + cb, (size_t)Bl * row_bytes, S + (size_t)(2 * P - 1 - kv) * cb, (size_t)N * row_bytes, cb,
                  planes, s);
  }
  return copy2d(D, row_bytes, S + (size_t)kv * row_bytes, (size_t)P * row_bytes, row_bytes,
                (size_t)planes * Bl, s);
}

// Host-major staging of every host's own block: dst[r] <- block r of src
// (used by layouts whose blocks the kernel cannot read in place).
hipError_t ring_gather_own(void* dst, const void* src, int layout, int64_t planes, int64_t N, int64_t Bl, int P,
                           size_t row_bytes, hipStream_t s) {
  char* D = static_cast<char*>(dst);
  const size_t host_bytes = (size_t)planes * Bl * row_bytes;
  for (int r = 0; r < P; ++r) {
    hipError_t e = gather_block(D + r * host_bytes, src, layout, planes, N, Bl, P, r, row_bytes, s);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace

// ===========================================================================
// C ABI
// ===========================================================================
extern "C" {

const char* ra_last_error(void) { return g_err.c_str(); }
const char* ra_version(void) { return "ring_attn 0.1 gfx950"; }

// The size queries apply the launch's own checks to the arguments they take
// and return SIZE_MAX (with a message for ra_last_error) when those fail or
// the size cannot be allocated; 0 means that no workspace is needed.
size_t ring_attn_fwd_ws_bytes(int B, int H, int Hkv, long long N, int d, int P, ra_dtype dtype) {
  g_err.clear();
  if (check_common(B, H, Hkv, N, d, P, dtype, 1.f) != RA_OK || check_block_span(N / P, d, dtype) != RA_OK)
    return SIZE_MAX;
  const FwdWs W = fwd_ws_layout(B, H, Hkv, N, N, d, P, dtype);
  if (W.overflow) {
    fail(RA_ENOMEM, "workspace size exceeds the 48-bit device address space");
    return SIZE_MAX;
  }
  return W.total;
}

size_t ring_attn_fwd_share_ws_bytes(int B, int H, int Hkv, long long N, int d, int P, ra_dtype dtype) {
  g_err.clear();
  if (check_common(B, H, Hkv, N, d, P, dtype, 1.f) != RA_OK || check_block_span(N / P, d, dtype) != RA_OK)
    return SIZE_MAX;
  const FwdWs W = fwd_ws_layout(B, H, Hkv, N / P, N / P, d, P, dtype);
  if (W.overflow) {
    fail(RA_ENOMEM, "workspace size exceeds the 48-bit device address space");
    return SIZE_MAX;
  }
  return W.total;
}

ra_status ring_attn_fwd(const void* q, const void* k, const void* v, void* out, float* lse, int B, int H,
                        int Hkv, long long N, int d, int P, int causal, ra_layout layout, float scale,
                        ra_dtype dtype, void* stream, void* ws, size_t ws_bytes) {
  g_err.clear();
  if (!q || !k || !v || !out || !lse) return fail(RA_EINVAL, "null tensor pointer");
  ra_status st = check_common(B, H, Hkv, N, d, P, dtype, scale);
  if (st != RA_OK) return st;
  if ((st = check_layout(layout, N, P)) != RA_OK) return st;
  if ((st = check_block_span(N / P, d, dtype)) != RA_OK) return st;
  const int lay = effective_layout(layout, P);
  const bool stage_own = stage_first_block(lay, N, d, P, dtype);  // step 0 reads staged blocks too
  const FwdWs W = fwd_ws_layout(B, H, Hkv, N, N, d, P, dtype);
  if ((st = check_ws(W.overflow, W.total, ws, ws_bytes)) != RA_OK) return st;
  if ((st = check_tensor_align({q, k, v, out}, {lse})) != RA_OK) return st;
  const int64_t Bl = N / P;
  const int BM = block_rows(dtype, d);
  const int64_t nqt = (Bl + BM - 1) / BM;
  if ((int64_t)P * B * H * nqt > 0x7fffffffLL) return fail(RA_EINVAL, "problem too large for one launch");
  DeviceCtx* ctx = nullptr;
  if ((st = get_ctx(&ctx)) != RA_OK) return st;
  std::lock_guard<std::mutex> enq(ctx->enqueue);
  hipStream_t cs = static_cast<hipStream_t>(stream);
  const size_t row_bytes = (size_t)d * esize(dtype);
  char* wsb = static_cast<char*>(ws);

  StepArgs a{};
  a.q = q;
  a.out = out;
  a.lse = lse;
  a.q_plane_rows = N;
  a.kv_plane_rows = N;
  a.B = B; a.H = H; a.Hkv = Hkv;
  a.Lq = (int)Bl; a.Lkv = (int)Bl;
  a.P = P;
  a.layout = lay;
  a.q_mode = ROWS_HOST_Q;
  a.kv_mode = ROWS_HOST_Q;
  a.causal = causal ? 1 : 0;
  a.n_qtiles = (int)nqt;
  a.scale_log2 = scale * 1.4426950408889634f;
  if (P > 1) {
    a.m = reinterpret_cast<float*>(wsb + W.off_m);
    a.l = reinterpret_cast<float*>(wsb + W.off_l);
    a.o = reinterpret_cast<float*>(wsb + W.off_o);
  }

  // With the exchange switched off (ra_debug_set_staging(0)) every step
  // reads its blocks in place where the kernel can address them.
  const bool staged = P > 1 && (g_staging || stage_own);
  auto kbuf = [&](int s) -> const void* {
    return (s == 0 && !stage_own) || !staged ? k : static_cast<const void*>(wsb + W.off_stage[s & 1]);
  };
  auto vbuf = [&](int s) -> const void* {
    return (s == 0 && !stage_own) || !staged ? v : static_cast<const void*>(wsb + W.off_stage[s & 1] + W.kv_bytes);
  };
  const int64_t planes = (int64_t)B * Hkv;

  if (staged) {
    RA_HIP(hipEventRecord(ctx->fork, cs), "hipEventRecord");
    RA_HIP(hipStreamWaitEvent(ctx->copy, ctx->fork, 0), "hipStreamWaitEvent");
  }
  if (stage_own) {
    // Every host's own block into staging buffer 0 before step 0.
    RA_HIP(launch_spin(g_delay_copy_us, ctx->copy), "delay");
    RA_HIP(ring_gather_own(wsb + W.off_stage[0], k, lay, planes, N, Bl, P, row_bytes, ctx->copy), "staging copy");
    RA_HIP(ring_gather_own(wsb + W.off_stage[0] + W.kv_bytes, v, lay, planes, N, Bl, P, row_bytes, ctx->copy),
           "staging copy");
    RA_HIP(hipEventRecord(ctx->copied[0], ctx->copy), "hipEventRecord");
  }
  for (int s = 0; s < P; ++s) {
    // Copy stream: stage the blocks of step s + 1 while step s computes.
    if (staged && s + 1 < P) {
      if (s >= 1) RA_HIP(hipStreamWaitEvent(ctx->copy, ctx->done[(s - 1) & 1], 0), "hipStreamWaitEvent");
      void* kd = wsb + W.off_stage[(s + 1) & 1];
      void* vd = wsb + W.off_stage[(s + 1) & 1] + W.kv_bytes;
      // Receivers that still have work at step s + 1 (all hosts unless the
      // ring is contiguous and causal, where hosts below s + 1 are done;
      // their staging slots are never read again).
      const StepPlan nxt = plan_step(lay, a.causal, P, s + 1, Bl);
      const int r_lo = (lay == RA_CONTIGUOUS && a.causal) ? nxt.host_lo : 0;
      RA_HIP(launch_spin(g_delay_copy_us, ctx->copy), "delay");
      if (s == 0 && !stage_own) {
        RA_HIP(ring_gather_first(kd, k, lay, planes, N, Bl, P, r_lo, row_bytes, ctx->copy), "staging copy");
        RA_HIP(ring_gather_first(vd, v, lay, planes, N, Bl, P, r_lo, row_bytes, ctx->copy), "staging copy");
      } else {
        RA_HIP(ring_shift(kd, kbuf(s), planes, Bl, P, r_lo, row_bytes, ctx->copy), "staging copy");
        RA_HIP(ring_shift(vd, vbuf(s), planes, Bl, P, r_lo, row_bytes, ctx->copy), "staging copy");
      }
      RA_HIP(hipEventRecord(ctx->copied[(s + 1) & 1], ctx->copy), "hipEventRecord");
    }
    // Compute stream: step s.
    if (staged && (s >= 1 || stage_own)) RA_HIP(hipStreamWaitEvent(cs, ctx->copied[s & 1], 0), "hipStreamWaitEvent");
    const StepPlan sp = plan_step(lay, a.causal, P, s, Bl);
    const bool in_place = (s == 0 && !stage_own) || !staged;
    a.k = kbuf(s);
    a.v = vbuf(s);
    a.kv_mode = in_place ? ROWS_HOST_KV : ROWS_HOST_MAJOR;
    a.kv_plane_rows = in_place ? N : Bl;
    a.host_lo = sp.host_lo;
    a.n_hosts = sp.n_hosts;
    a.kv_shift = s;
    a.has_prev = s > 0 ? 1 : 0;
    a.fin_lo = sp.fin_lo;
    a.fin_hi = sp.fin_hi;
    if (sp.n_hosts > 0) {
      RA_HIP(launch_spin(g_delay_compute_us, cs), "delay");
      RA_HIP(launch_step(a, d, dtype, cs, step_flops(a, d)), "step kernel launch");
    }
    if (staged && s + 2 < P) RA_HIP(hipEventRecord(ctx->done[s & 1], cs), "hipEventRecord");
  }
  return RA_OK;
}

ra_status ring_attn_fwd_share(const void* q, const void* k, const void* v, void* out, float* lse, int B,
                              int H, int Hkv, long long N, int d, int P, int rank, int causal,
                              ra_layout layout, float scale, ra_dtype dtype, void* stream, void* ws,
                              size_t ws_bytes) {
  g_err.clear();
  if (!q || !k || !v || !out || !lse) return fail(RA_EINVAL, "null tensor pointer");
  ra_status st = check_common(B, H, Hkv, N, d, P, dtype, scale);
  if (st != RA_OK) return st;
  if ((st = check_layout(layout, N, P)) != RA_OK) return st;
  if ((st = check_block_span(N / P, d, dtype)) != RA_OK) return st;
  const int lay = effective_layout(layout, P);
  const bool stage_first = stage_first_block(lay, N, d, P, dtype);  // the first block is not read in place
  if (rank < 0 || rank >= P) return fail(RA_EINVAL, "rank %d out of [0, %d)", rank, P);
  const int64_t Bl = N / P;
  const FwdWs W = fwd_ws_layout(B, H, Hkv, Bl, Bl, d, P, dtype);
  if ((st = check_ws(W.overflow, W.total, ws, ws_bytes)) != RA_OK) return st;
  if ((st = check_tensor_align({q, k, v, out}, {lse})) != RA_OK) return st;
  const int BM = block_rows(dtype, d);
  const int64_t nqt = (Bl + BM - 1) / BM;
  if ((int64_t)B * H * nqt > 0x7fffffffLL) return fail(RA_EINVAL, "problem too large for one launch");
  DeviceCtx* ctx = nullptr;
  if ((st = get_ctx(&ctx)) != RA_OK) return st;
  std::lock_guard<std::mutex> enq(ctx->enqueue);
  hipStream_t cs = static_cast<hipStream_t>(stream);
  const size_t row_bytes = (size_t)d * esize(dtype);
  char* wsb = static_cast<char*>(ws);

  // Steps with visible work, in ring order.
  std::vector<int> steps;
  for (int s = 0; s < P; ++s) {
    const int kv = ((rank - s) % P + P) % P;
    if (pair_active(lay, causal ? 1 : 0, P, rank, kv, Bl, Bl)) steps.push_back(s);
  }

  StepArgs a{};
  a.q = q;
  a.out = out;
  a.lse = lse;
  a.q_plane_rows = Bl;
  a.B = B; a.H = H; a.Hkv = Hkv;
  a.Lq = (int)Bl; a.Lkv = (int)Bl;
  a.P = P;
  a.layout = lay;
  a.q_mode = ROWS_COMPACT;
  a.causal = causal ? 1 : 0;
  a.n_qtiles = (int)nqt;
  a.scale_log2 = scale * 1.4426950408889634f;
  a.host_lo = rank;
  a.n_hosts = 1;
  if (P > 1) {
    a.m = reinterpret_cast<float*>(wsb + W.off_m);
    a.l = reinterpret_cast<float*>(wsb + W.off_l);
    a.o = reinterpret_cast<float*>(wsb + W.off_o);
  }
  const int n = (int)steps.size();
  const int64_t planes = (int64_t)B * Hkv;
  // With the exchange switched off (ra_debug_set_staging(0)) every step
  // reads its block in place where the kernel can address it.
  const bool staged = g_staging || stage_first;
  if (staged && (n > 1 || (n > 0 && stage_first))) {
    RA_HIP(hipEventRecord(ctx->fork, cs), "hipEventRecord");
    RA_HIP(hipStreamWaitEvent(ctx->copy, ctx->fork, 0), "hipStreamWaitEvent");
  }
  if (n > 0 && stage_first) {
    const int kv0 = ((rank - steps[0]) % P + P) % P;
    RA_HIP(launch_spin(g_delay_copy_us, ctx->copy), "delay");
    RA_HIP(gather_block(wsb + W.off_stage[0], k, lay, planes, N, Bl, P, kv0, row_bytes, ctx->copy), "staging copy");
    RA_HIP(gather_block(wsb + W.off_stage[0] + W.kv_bytes, v, lay, planes, N, Bl, P, kv0, row_bytes, ctx->copy),
           "staging copy");
    RA_HIP(hipEventRecord(ctx->copied[0], ctx->copy), "hipEventRecord");
  }
  // Step index i uses staging buffer i & 1 (i >= 1); the first step reads
  // its block in place from the natural-order k / v (contiguous, striped)
  // or from staging buffer 0 (zigzag).
  for (int i = 0; i < n; ++i) {
    const int s = steps[i];
    if (staged && i + 1 < n) {
      const int s1 = steps[i + 1];
      const int kv1 = ((rank - s1) % P + P) % P;
      if (i >= 1) RA_HIP(hipStreamWaitEvent(ctx->copy, ctx->done[(i - 1) & 1], 0), "hipStreamWaitEvent");
      void* kd = wsb + W.off_stage[(i + 1) & 1];
      void* vd = wsb + W.off_stage[(i + 1) & 1] + W.kv_bytes;
      RA_HIP(launch_spin(g_delay_copy_us, ctx->copy), "delay");
      RA_HIP(gather_block(kd, k, lay, planes, N, Bl, P, kv1, row_bytes, ctx->copy), "staging copy");
      RA_HIP(gather_block(vd, v, lay, planes, N, Bl, P, kv1, row_bytes, ctx->copy), "staging copy");
      RA_HIP(hipEventRecord(ctx->copied[(i + 1) & 1], ctx->copy), "hipEventRecord");
    }
    if (staged && (i >= 1 || stage_first)) RA_HIP(hipStreamWaitEvent(cs, ctx->copied[i & 1], 0), "hipStreamWaitEvent");
    if ((i == 0 && !stage_first) || !staged) {
      a.k = k;
      a.v = v;
      a.kv_mode = ROWS_HOST_KV;
      a.kv_plane_rows = N;
    } else {
      a.k = wsb + W.off_stage[i & 1];
      a.v = wsb + W.off_stage[i & 1] + W.kv_bytes;
      a.kv_mode = ROWS_COMPACT;
      a.kv_plane_rows = Bl;
    }
    a.kv_shift = s;
    a.has_prev = i > 0 ? 1 : 0;
    a.fin_lo = (i == n - 1) ? rank : 0;
    a.fin_hi = (i == n - 1) ? rank + 1 : 0;
    RA_HIP(launch_spin(g_delay_compute_us, cs), "delay");
    RA_HIP(launch_step(a, d, dtype, cs, step_flops(a, d)), "step kernel launch");
    if (staged && i + 2 < n) RA_HIP(hipEventRecord(ctx->done[i & 1], cs), "hipEventRecord");
  }
  if (n == 0) {
    // Nothing visible (cannot happen for a causal ring: a host sees itself).
    return fail(RA_EINVAL, "no visible keys for rank %d", rank);
  }
  return RA_OK;
}

// ---------------------------------------------------------------------------
// Backward by recomputation ([TKG] §7, "활성화 체크포인팅과 메모리 재연산"):
// the forward's lse (= m + ln l) and the queries stay put; at step s host r
// recomputes its attention against kv block (r + s) mod P (the kv blocks
// travel the other way round the ring) and adds that pair's dQ, dK, dV.
// On one GPU the dK / dV accumulators that would travel with their kv block
// stay at the block's rows; each kv block meets exactly one host per step,
// so the kernels of one step never write the same rows.
// ---------------------------------------------------------------------------
struct BwdWs {
  size_t off_stage[2], kv_bytes;  // staging buffers (K then V) and the K part's size
  size_t off_rowstat, off_dq, off_dk, off_dv, total;
  bool overflow;
};

static BwdWs bwd_ws_layout(int B, int H, int Hkv, long long N, int d, int P, ra_dtype dtype) {
  BwdWs w{};
  SizeAcc a;
  // two staging buffers of K and V for the reverse ring (input dtype, host-major)
  if (P > 1) {
    const uint64_t es = esize(dtype);
    w.off_stage[0] = a.add({(uint64_t)B, (uint64_t)Hkv, (uint64_t)N, (uint64_t)d, es});
    w.kv_bytes = a.add({(uint64_t)B, (uint64_t)Hkv, (uint64_t)N, (uint64_t)d, es}) - w.off_stage[0];
    w.off_stage[1] = a.add({2, w.kv_bytes});
  }
  w.off_rowstat = a.add({(uint64_t)B, (uint64_t)H, (uint64_t)N, 8});
  w.off_dq = a.add({(uint64_t)B, (uint64_t)H, (uint64_t)N, (uint64_t)d, 4});
  w.off_dk = a.add({(uint64_t)B, (uint64_t)Hkv, (uint64_t)N, (uint64_t)d, 4});
  w.off_dv = a.add({(uint64_t)B, (uint64_t)Hkv, (uint64_t)N, (uint64_t)d, 4});
  w.total = (size_t)a.total;
  w.overflow = a.bad;
  return w;
}

// The bf16 backward kernels read q, dO and the row statistics of a whole
// (batch, head) plane through buffer descriptors with 32-bit offsets; the
// fp32 kernels use plain 64-bit addressing.
ra_status bwd_args(int B, int H, int Hkv, long long N, int d, int P, ra_dtype dtype, float scale) {
  ra_status st = check_common(B, H, Hkv, N, d, P, dtype, scale);
  if (st != RA_OK) return st;
  if (dtype == RA_BF16 && (uint64_t)N * d * esize(dtype) >= kSpanLimit)
    return fail(RA_EINVAL, "the bf16 backward needs one head plane (N * d elements) below 2 GiB");
  return RA_OK;
}

size_t ring_attn_bwd_ws_bytes(int B, int H, int Hkv, long long N, int d, int P, ra_dtype dtype) {
  g_err.clear();
  if (bwd_args(B, H, Hkv, N, d, P, dtype, 1.f) != RA_OK) return SIZE_MAX;
  const BwdWs W = bwd_ws_layout(B, H, Hkv, N, d, P, dtype);
  if (W.overflow) {
    fail(RA_ENOMEM, "workspace size exceeds the 48-bit device address space");
    return SIZE_MAX;
  }
  return W.total;
}

ra_status ring_attn_bwd(const void* q, const void* k, const void* v, const void* out, const void* dout,
                        const float* lse, void* dq, void* dk, void* dv, int B, int H, int Hkv, long long N, int d,
                        int P, int causal, ra_layout layout, float scale, ra_dtype dtype, void* stream, void* ws,
                        size_t ws_bytes) {
  g_err.clear();
  if (!q || !k || !v || !out || !dout || !lse || !dq || !dk || !dv) return fail(RA_EINVAL, "null tensor pointer");
  ra_status st = bwd_args(B, H, Hkv, N, d, P, dtype, scale);
  if (st != RA_OK) return st;
  if ((st = check_layout(layout, N, P)) != RA_OK) return st;
  const BwdWs W = bwd_ws_layout(B, H, Hkv, N, d, P, dtype);
  if ((st = check_ws(W.overflow, W.total, ws, ws_bytes)) != RA_OK) return st;
  if ((st = check_tensor_align({q, k, v, out, dout, dq, dk, dv}, {lse})) != RA_OK) return st;
  const bool f32 = dtype == RA_F32;
  const int64_t Bl = N / P;
  const int64_t nqt = (Bl + bwd_dq_rows() - 1) / bwd_dq_rows();
  const int64_t nkt = (Bl + bwd_dkdv_rows() - 1) / bwd_dkdv_rows();
  if ((int64_t)P * B * H * nqt > 0x7fffffffLL || (int64_t)P * B * Hkv * nkt > 0x7fffffffLL ||
      (f32 && (int64_t)P * B * H * Bl / 4 >= 0x7fffffffLL))
    return fail(RA_EINVAL, "problem too large for one launch");
  const int lay = effective_layout(layout, P);
  hipStream_t cs = static_cast<hipStream_t>(stream);
  char* wsb = static_cast<char*>(ws);

  BwdArgs a{};
  a.s.q = q;
  a.s.k = k;
  a.s.v = v;
  a.s.q_plane_rows = N;
  a.s.kv_plane_rows = N;
  a.s.B = B; a.s.H = H; a.s.Hkv = Hkv;
  a.s.Lq = (int)Bl; a.s.Lkv = (int)Bl;
  a.s.P = P;
  a.s.layout = lay;
  a.s.q_mode = ROWS_HOST_Q;
  a.s.kv_mode = ROWS_HOST_KV;
  a.s.causal = causal ? 1 : 0;
  a.s.n_qtiles = (int)nqt;
  a.s.scale_log2 = scale * 1.4426950408889634f;
  a.dout = dout;
  a.rowstat = reinterpret_cast<float*>(wsb + W.off_rowstat);
  a.dq_acc = reinterpret_cast<float*>(wsb + W.off_dq);
  a.dk_acc = reinterpret_cast<float*>(wsb + W.off_dk);
  a.dv_acc = reinterpret_cast<float*>(wsb + W.off_dv);
  a.n_tok = N;
  a.scale = scale;
  a.n_kvtiles = (int)nkt;

  if (f32) {
    a.dq_out_f32 = static_cast<float*>(dq);
    a.dk_out_f32 = static_cast<float*>(dk);
    a.dv_out_f32 = static_cast<float*>(dv);
  } else {
    a.dq_out = static_cast<__bf16*>(dq);
    a.dk_out = static_cast<__bf16*>(dk);
    a.dv_out = static_cast<__bf16*>(dv);
  }

  // Launch plan: step s pairs query host r with kv block (r + s) mod P; a
  // launch covers the hosts lo .. hi that have visible work at that step.
  // Step 0 (every host against its own block, which holds the diagonal)
  // has work for every host, so its launch writes the accumulators instead
  // of adding to them, and the last active step of a host (kv block) writes
  // its dQ (dK, dV) in the output dtype: no separate clear or conversion pass.
  static_assert(kMaxP <= 64, "the last-step masks hold one bit per host");
  std::vector<int> lo_s(P, -1), hi_s(P, -1), last_q(P, -1), last_kv(P, -1);
  for (int s = 0; s < P; ++s)
    for (int r = 0; r < P; ++r) {
      const int kv = (r + s) % P;
      if (pair_active(lay, a.s.causal, P, r, kv, Bl, Bl)) {
        if (lo_s[s] < 0) lo_s[s] = r;
        hi_s[s] = r;
        last_q[r] = s;
        last_kv[kv] = s;
      }
    }
  if (lo_s[0] != 0 || hi_s[0] != P - 1) return fail(RA_EUNSUPPORTED, "internal: a host has no diagonal work");
  // Reverse ring: step s pairs host r with kv block (r + s) mod P.  Step 0
  // (every host's own block) reads K and V in place; for each later step
  // the copy stream moves every working host's block into its slot of a
  // host-major staging buffer (two buffers, alternating) while the
  // previous step computes: from the slot of the host that held the block
  // at the previous step when that slot was filled (the block moves one
  // host down the ring), else from the natural-order arrays.  The dK / dV
  // accumulators stay at the blocks' rows.
  std::vector<int> steps;
  for (int s = 0; s < P; ++s)
    if (lo_s[s] >= 0) steps.push_back(s);
  const int n = (int)steps.size();
  const bool staged = g_staging && P > 1 && n > 1;
  DeviceCtx* ctx = nullptr;
  if (staged && (st = get_ctx(&ctx)) != RA_OK) return st;
  std::unique_lock<std::mutex> enq;
  if (staged) enq = std::unique_lock<std::mutex>(ctx->enqueue);
  const size_t row_bytes = (size_t)d * esize(dtype);
  const int64_t planes = (int64_t)B * Hkv;
  const size_t host_bytes = (size_t)planes * Bl * row_bytes;
  if (f32)
    RA_HIP(launch_bwd_prep_f32(static_cast<const float*>(out), static_cast<const float*>(dout), lse,
                               const_cast<float*>(a.rowstat), (int64_t)B * H * N, d, cs),
           "prep launch");
  else
    RA_HIP(launch_bwd_prep(out, dout, lse, const_cast<float*>(a.rowstat), (int64_t)B * H * N, d, cs),
           "prep launch");
  if (staged) {
    RA_HIP(hipEventRecord(ctx->fork, cs), "hipEventRecord");
    RA_HIP(hipStreamWaitEvent(ctx->copy, ctx->fork, 0), "hipStreamWaitEvent");
  }
  std::vector<char> filled_prev(P, 0), filled(P, 0);
  for (int i = 0; i < n; ++i) {
    const int s = steps[i];
    if (staged && i + 1 < n) {
      // copy stream: the blocks of step i + 1 into staging buffer (i + 1) & 1
      const int s1 = steps[i + 1];
      if (i >= 1) RA_HIP(hipStreamWaitEvent(ctx->copy, ctx->done[(i - 1) & 1], 0), "hipStreamWaitEvent");
      RA_HIP(launch_spin(g_delay_copy_us, ctx->copy), "delay");
      char* kd = wsb + W.off_stage[(i + 1) & 1];
      char* vd = kd + W.kv_bytes;
      const char* ks = wsb + W.off_stage[i & 1];
      const char* vs = ks + W.kv_bytes;
      std::fill(filled.begin(), filled.end(), 0);
      for (int r = lo_s[s1]; r <= hi_s[s1]; ++r) {
        const int blk = (r + s1) % P;
        const int from = ((blk - s) % P + P) % P;  // host that held the block at step s
        if (i >= 1 && filled_prev[from]) {
          RA_HIP(hipMemcpyAsync(kd + r * host_bytes, ks + from * host_bytes, host_bytes, hipMemcpyDeviceToDevice,
                                ctx->copy), "staging copy");
          RA_HIP(hipMemcpyAsync(vd + r * host_bytes, vs + from * host_bytes, host_bytes, hipMemcpyDeviceToDevice,
                                ctx->copy), "staging copy");
        } else {
          RA_HIP(gather_block(kd + r * host_bytes, k, lay, planes, N, Bl, P, blk, row_bytes, ctx->copy), "staging copy");
          RA_HIP(gather_block(vd + r * host_bytes, v, lay, planes, N, Bl, P, blk, row_bytes, ctx->copy), "staging copy");
        }
        filled[r] = 1;
      }
      filled_prev.swap(filled);
      RA_HIP(hipEventRecord(ctx->copied[(i + 1) & 1], ctx->copy), "hipEventRecord");
    }
    if (staged && i >= 1) RA_HIP(hipStreamWaitEvent(cs, ctx->copied[i & 1], 0), "hipStreamWaitEvent");
    a.s.host_lo = lo_s[s];
    a.s.n_hosts = hi_s[s] - lo_s[s] + 1;
    a.s.kv_shift = -s;
    a.first = a.kv_first = s == 0;
    a.q_fin = a.kv_fin = 0;
    for (int r = 0; r < P; ++r) {
      if (last_q[r] == s) a.q_fin |= 1ull << r;
      if (last_kv[r] == s) a.kv_fin |= 1ull << r;
    }
    const bool use_stage = staged && i >= 1;
    a.kv_staged = use_stage ? 1 : 0;
    a.s.k = use_stage ? static_cast<const void*>(wsb + W.off_stage[i & 1]) : k;
    a.s.v = use_stage ? static_cast<const void*>(wsb + W.off_stage[i & 1] + W.kv_bytes) : v;
    RA_HIP(launch_spin(staged ? g_delay_compute_us : 0, cs), "delay");
    RA_HIP(f32 ? launch_bwd_dkdv_f32(a, d, cs) : launch_bwd_dkdv(a, d, cs), "dK/dV kernel launch");
    RA_HIP(f32 ? launch_bwd_dq_f32(a, d, cs) : launch_bwd_dq(a, d, cs), "dQ kernel launch");
    if (staged && i + 2 < n) RA_HIP(hipEventRecord(ctx->done[i & 1], cs), "hipEventRecord");
  }
  return RA_OK;
}

// One device's share of the backward: host `rank` keeps its query block
// (q, out, dout, lse, dq: compact [B, H, Bl, ...]) and meets kv block
// (rank + s) mod P at step s; dk, dv [B, Hkv, N, d] receive this host's
// contribution to every key (the sum over the P shares is the full dK, dV;
// a block the host never sees gets zeros).  Each step writes a different
// kv block, so the dK / dV kernels write their results directly; dQ is
// accumulated in fp32 over the host's active steps.  Blocks after the
// host's own are staged into one of two slot buffers on the copy stream
// while the previous step computes, as in the forward share.
struct BwdShareWs {
  size_t off_stage[2], kv_bytes;
  size_t off_rowstat, off_dq, total;
  bool overflow;
};

static BwdShareWs bwd_share_ws_layout(int B, int H, int Hkv, long long N, int d, int P, ra_dtype dtype) {
  BwdShareWs w{};
  SizeAcc a;
  const uint64_t Bl = (uint64_t)(N / P);
  if (P > 1) {
    const uint64_t es = esize(dtype);
    w.off_stage[0] = a.add({(uint64_t)B, (uint64_t)Hkv, Bl, (uint64_t)d, es});
    w.kv_bytes = a.add({(uint64_t)B, (uint64_t)Hkv, Bl, (uint64_t)d, es}) - w.off_stage[0];
    w.off_stage[1] = a.add({2, w.kv_bytes});
  }
  w.off_rowstat = a.add({(uint64_t)B, (uint64_t)H, Bl, 8});
  w.off_dq = a.add({(uint64_t)B, (uint64_t)H, Bl, (uint64_t)d, 4});
  w.total = (size_t)a.total;
  w.overflow = a.bad;
  return w;
}

size_t ring_attn_bwd_share_ws_bytes(int B, int H, int Hkv, long long N, int d, int P, ra_dtype dtype) {
  g_err.clear();
  if (bwd_args(B, H, Hkv, N, d, P, dtype, 1.f) != RA_OK) return SIZE_MAX;
  const BwdShareWs W = bwd_share_ws_layout(B, H, Hkv, N, d, P, dtype);
  if (W.overflow) {
    fail(RA_ENOMEM, "workspace size exceeds the 48-bit device address space");
    return SIZE_MAX;
  }
  return W.total;
}

ra_status ring_attn_bwd_share(const void* q, const void* k, const void* v, const void* out, const void* dout,
                              const float* lse, void* dq, void* dk, void* dv, int B, int H, int Hkv, long long N,
                              int d, int P, int rank, int causal, ra_layout layout, float scale, ra_dtype dtype,
                              void* stream, void* ws, size_t ws_bytes) {
  g_err.clear();
  if (!q || !k || !v || !out || !dout || !lse || !dq || !dk || !dv) return fail(RA_EINVAL, "null tensor pointer");
  ra_status st = bwd_args(B, H, Hkv, N, d, P, dtype, scale);
  if (st != RA_OK) return st;
  if ((st = check_layout(layout, N, P)) != RA_OK) return st;
  if (rank < 0 || rank >= P) return fail(RA_EINVAL, "rank %d out of [0, %d)", rank, P);
  const BwdShareWs W = bwd_share_ws_layout(B, H, Hkv, N, d, P, dtype);
  if ((st = check_ws(W.overflow, W.total, ws, ws_bytes)) != RA_OK) return st;
  if ((st = check_tensor_align({q, k, v, out, dout, dq, dk, dv}, {lse})) != RA_OK) return st;
  const bool f32 = dtype == RA_F32;
  const int64_t Bl = N / P;
  const int64_t nqt = (Bl + bwd_dq_rows() - 1) / bwd_dq_rows();
  const int64_t nkt = (Bl + bwd_dkdv_rows() - 1) / bwd_dkdv_rows();
  if ((int64_t)B * H * nqt > 0x7fffffffLL || (int64_t)B * Hkv * nkt > 0x7fffffffLL ||
      (f32 && (int64_t)B * H * Bl / 4 >= 0x7fffffffLL))
    return fail(RA_EINVAL, "problem too large for one launch");
  const int lay = effective_layout(layout, P);
  hipStream_t cs = static_cast<hipStream_t>(stream);
  char* wsb = static_cast<char*>(ws);

  BwdArgs a{};
  a.s.q = q;
  a.s.q_plane_rows = Bl;
  a.s.kv_plane_rows = N;
  a.s.B = B; a.s.H = H; a.s.Hkv = Hkv;
  a.s.Lq = (int)Bl; a.s.Lkv = (int)Bl;
  a.s.P = P;
  a.s.layout = lay;
  a.s.q_mode = ROWS_COMPACT;
  a.s.kv_mode = ROWS_HOST_KV;
  a.s.causal = causal ? 1 : 0;
  a.s.n_qtiles = (int)nqt;
  a.s.scale_log2 = scale * 1.4426950408889634f;
  a.s.host_lo = rank;
  a.s.n_hosts = 1;
  a.dout = dout;
  a.rowstat = reinterpret_cast<float*>(wsb + W.off_rowstat);
  a.dq_acc = reinterpret_cast<float*>(wsb + W.off_dq);
  a.n_tok = N;
  a.scale = scale;
  a.n_kvtiles = (int)nkt;
  a.q_compact = 1;
  a.kv_first = 1;
  a.stage_host0 = rank;
  if (f32) {
    a.dq_out_f32 = static_cast<float*>(dq);
    a.dk_out_f32 = static_cast<float*>(dk);
    a.dv_out_f32 = static_cast<float*>(dv);
  } else {
    a.dq_out = static_cast<__bf16*>(dq);
    a.dk_out = static_cast<__bf16*>(dk);
    a.dv_out = static_cast<__bf16*>(dv);
  }

  // Every step launches the dK / dV kernel (a block the host does not see
  // gets its zeros from it); the dQ kernel runs on the active steps only.
  std::vector<int> active;
  for (int s = 0; s < P; ++s)
    if (pair_active(lay, a.s.causal, P, rank, (rank + s) % P, Bl, Bl)) active.push_back(s);
  if (active.empty() || active[0] != 0) return fail(RA_EUNSUPPORTED, "internal: host %d has no diagonal work", rank);
  const int n = (int)active.size();
  const bool staged = g_staging && n > 1;
  DeviceCtx* ctx = nullptr;
  if (staged && (st = get_ctx(&ctx)) != RA_OK) return st;
  std::unique_lock<std::mutex> enq;
  if (staged) enq = std::unique_lock<std::mutex>(ctx->enqueue);
  const size_t row_bytes = (size_t)d * esize(dtype);
  const int64_t planes = (int64_t)B * Hkv;
  if (f32)
    RA_HIP(launch_bwd_prep_f32(static_cast<const float*>(out), static_cast<const float*>(dout), lse,
                               const_cast<float*>(a.rowstat), (int64_t)B * H * Bl, d, cs),
           "prep launch");
  else
    RA_HIP(launch_bwd_prep(out, dout, lse, const_cast<float*>(a.rowstat), (int64_t)B * H * Bl, d, cs),
           "prep launch");
  if (staged) {
    RA_HIP(hipEventRecord(ctx->fork, cs), "hipEventRecord");
    RA_HIP(hipStreamWaitEvent(ctx->copy, ctx->fork, 0), "hipStreamWaitEvent");
  }
  int i = 0;  // index of the next active step
  for (int s = 0; s < P; ++s) {
    const int blk = (rank + s) % P;
    const bool on = i < n && active[i] == s;
    if (on && staged && i + 1 < n) {
      // copy stream: the block of the next active step into slot (i + 1) & 1
      const int blk1 = (rank + active[i + 1]) % P;
      if (i >= 1) RA_HIP(hipStreamWaitEvent(ctx->copy, ctx->done[(i - 1) & 1], 0), "hipStreamWaitEvent");
      RA_HIP(launch_spin(g_delay_copy_us, ctx->copy), "delay");
      char* kd = wsb + W.off_stage[(i + 1) & 1];
      RA_HIP(gather_block(kd, k, lay, planes, N, Bl, P, blk1, row_bytes, ctx->copy), "staging copy");
      RA_HIP(gather_block(kd + W.kv_bytes, v, lay, planes, N, Bl, P, blk1, row_bytes, ctx->copy), "staging copy");
      RA_HIP(hipEventRecord(ctx->copied[(i + 1) & 1], ctx->copy), "hipEventRecord");
    }
    if (on && staged && i >= 1) RA_HIP(hipStreamWaitEvent(cs, ctx->copied[i & 1], 0), "hipStreamWaitEvent");
    const bool use_stage = on && staged && i >= 1;
    a.kv_staged = use_stage ? 1 : 0;
    a.s.k = use_stage ? static_cast<const void*>(wsb + W.off_stage[i & 1]) : k;
    a.s.v = use_stage ? static_cast<const void*>(wsb + W.off_stage[i & 1] + W.kv_bytes) : v;
    a.s.kv_shift = -s;
    a.first = i == 0;
    a.q_fin = (on && i == n - 1) ? 1ull << rank : 0;
    a.kv_fin = 1ull << blk;
    RA_HIP(launch_spin(on && staged ? g_delay_compute_us : 0, cs), "delay");
    RA_HIP(f32 ? launch_bwd_dkdv_f32(a, d, cs) : launch_bwd_dkdv(a, d, cs), "dK/dV kernel launch");
    if (on) {
      RA_HIP(f32 ? launch_bwd_dq_f32(a, d, cs) : launch_bwd_dq(a, d, cs), "dQ kernel launch");
      if (staged && i + 2 < n) RA_HIP(hipEventRecord(ctx->done[i & 1], cs), "hipEventRecord");
      ++i;
    }
  }
  return RA_OK;
}

// Checks of a (query block, kv block) pair's description shared by the
// forward and backward step calls.
static ra_status check_mask_desc(const ra_mask_desc* md) {
  if (md->B < 1 || md->H < 1 || md->Hkv < 1 || md->H % md->Hkv)
    return fail(RA_EINVAL, "bad head counts B=%d H=%d Hkv=%d", md->B, md->H, md->Hkv);
  if (md->d != 64 && md->d != 128) return fail(RA_EINVAL, "head dim d must be 64 or 128 (got %d)", md->d);
  if (md->Lq < 1 || md->Lkv < 1 || md->Lq > (1LL << 30) || md->Lkv > (1LL << 30))
    return fail(RA_EINVAL, "block lengths must be in [1, 2^30]");
  if (!dtype_ok(md->dtype)) return fail(RA_EINVAL, "unknown dtype %d", (int)md->dtype);
  if (!layout_ok(md->layout)) return fail(RA_EINVAL, "unknown layout %d", (int)md->layout);
  if (md->layout == RA_ZIGZAG && md->causal && (md->Lq != md->Lkv || md->Lq % 2))
    return fail(RA_EINVAL, "zigzag causal blocks must have Lq == Lkv and an even length");
  if (md->P < 1 || md->P > kMaxP || md->q_rank < 0 || md->q_rank >= md->P || md->kv_rank < 0 ||
      md->kv_rank >= md->P)
    return fail(RA_EINVAL, "bad ring description P=%d q_rank=%d kv_rank=%d", md->P, md->q_rank, md->kv_rank);
  if (md->layout == RA_STRIPED && md->causal && md->Lq != md->Lkv)
    return fail(RA_EINVAL, "striped causal blocks must have Lq == Lkv");
  {
    const ra_status sp = check_block_span(md->Lkv, md->d, md->dtype);
    if (sp != RA_OK) return sp;
  }
  if (!(md->scale > 0.f) || !std::isfinite(md->scale)) return fail(RA_EINVAL, "scale must be finite and > 0");
  return RA_OK;
}

ra_status ring_attn_step(const void* q_blk, ra_kv_block kv_blk, float* m, float* l, float* o,
                         const ra_mask_desc* md, void* stream) {
  g_err.clear();
  if (!md) return fail(RA_EINVAL, "null mask_desc");
  if (!q_blk || !kv_blk.k || !kv_blk.v || !m || !l || !o) return fail(RA_EINVAL, "null tensor pointer");
  {
    const ra_status mdst = check_mask_desc(md);
    if (mdst != RA_OK) return mdst;
  }
  {
    const ra_status al = check_tensor_align({q_blk, kv_blk.k, kv_blk.v, o}, {m, l});
    if (al != RA_OK) return al;
  }
  const int BM = block_rows(md->dtype, md->d);
  const int64_t nqt = (md->Lq + BM - 1) / BM;
  if ((int64_t)md->B * md->H * nqt > 0x7fffffffLL) return fail(RA_EINVAL, "problem too large for one launch");
  if (!pair_active(md->layout, md->causal, md->P, md->q_rank, md->kv_rank, md->Lq, md->Lkv)) return RA_OK;
  DeviceCtx* ctx = nullptr;
  ra_status st = get_ctx(&ctx);
  if (st != RA_OK) return st;
  StepArgs a{};
  a.q = q_blk;
  a.k = kv_blk.k;
  a.v = kv_blk.v;
  a.m = m; a.l = l; a.o = o;
  a.q_plane_rows = md->Lq;
  a.kv_plane_rows = md->Lkv;
  a.B = md->B; a.H = md->H; a.Hkv = md->Hkv;
  a.Lq = (int)md->Lq; a.Lkv = (int)md->Lkv;
  a.P = md->P;
  a.layout = md->layout;
  a.host_lo = md->q_rank;
  a.n_hosts = 1;
  a.kv_shift = md->q_rank - md->kv_rank;
  a.q_mode = ROWS_COMPACT;
  a.kv_mode = ROWS_COMPACT;
  a.causal = md->causal ? 1 : 0;
  a.has_prev = 1;
  a.fin_lo = a.fin_hi = 0;
  a.n_qtiles = (int)nqt;
  a.scale_log2 = md->scale * 1.4426950408889634f;
  RA_HIP(launch_step(a, md->d, md->dtype, static_cast<hipStream_t>(stream), step_flops(a, md->d)),
         "step kernel launch");
  return RA_OK;
}

ra_status ring_attn_finalize(const float* m, const float* l, const float* o, void* out, float* lse,
                             long long rows, int d, ra_dtype out_dtype, void* stream) {
  g_err.clear();
  if (rows < 0 || d < 1 || d > 1024) return fail(RA_EINVAL, "bad rows/d");
  if (!dtype_ok(out_dtype)) return fail(RA_EINVAL, "unknown dtype %d", (int)out_dtype);
  if (rows == 0) return RA_OK;  // nothing to do; empty tensors may carry null pointers
  if (!m || !l || !o || !out || !lse) return fail(RA_EINVAL, "null tensor pointer");
  FinalizeArgs a{m, l, o, out, lse, rows, d};
  RA_HIP(launch_finalize(a, out_dtype == RA_BF16, static_cast<hipStream_t>(stream)), "finalize launch");
  return RA_OK;
}

ra_status lse_merge(float* o_a, float* lse_a, const float* o_b, const float* lse_b, long long rows, int d,
                    void* stream) {
  g_err.clear();
  if (rows < 0 || d < 1 || d > 1024) return fail(RA_EINVAL, "bad rows/d");
  if (rows == 0) return RA_OK;  // nothing to do; empty tensors may carry null pointers
  if (!o_a || !lse_a || !o_b || !lse_b) return fail(RA_EINVAL, "null tensor pointer");
  MergeArgs a{o_a, lse_a, o_b, lse_b, rows, d};
  RA_HIP(launch_lse_merge(a, static_cast<hipStream_t>(stream)), "lse_merge launch");
  return RA_OK;
}

// ---------------------------------------------------------------------------
// Backward building blocks for a caller's own ring ([TKG] §7): the row
// statistics of a query block, then one (query block, kv block) pair's
// gradient contributions added into caller-owned fp32 accumulators.
// ---------------------------------------------------------------------------
ra_status ring_attn_bwd_prep(const void* out, const void* dout, const float* lse, float* rowstat, long long rows,
                             int d, ra_dtype dtype, void* stream) {
  g_err.clear();
  if (rows < 0) return fail(RA_EINVAL, "rows must be >= 0");
  if (d != 64 && d != 128) return fail(RA_EINVAL, "head dim d must be 64 or 128 (got %d)", d);
  if (!dtype_ok(dtype)) return fail(RA_EINVAL, "unknown dtype %d", (int)dtype);
  if (rows == 0) return RA_OK;  // nothing to do; empty tensors may carry null pointers
  if (!out || !dout || !lse || !rowstat) return fail(RA_EINVAL, "null tensor pointer");
  {
    const ra_status al = check_tensor_align({out, dout, rowstat}, {lse});
    if (al != RA_OK) return al;
  }
  hipStream_t cs = static_cast<hipStream_t>(stream);
  if (dtype == RA_F32)
    RA_HIP(launch_bwd_prep_f32(static_cast<const float*>(out), static_cast<const float*>(dout), lse, rowstat,
                               (int64_t)rows, d, cs),
           "prep launch");
  else
    RA_HIP(launch_bwd_prep(out, dout, lse, rowstat, (int64_t)rows, d, cs), "prep launch");
  return RA_OK;
}

ra_status ring_attn_bwd_step(const void* q_blk, const void* dout_blk, const float* rowstat, ra_kv_block kv_blk,
                             float* dq_acc, float* dk_acc, float* dv_acc, const ra_mask_desc* md, void* stream) {
  g_err.clear();
  if (!md) return fail(RA_EINVAL, "null mask_desc");
  if (!q_blk || !dout_blk || !rowstat || !kv_blk.k || !kv_blk.v || !dq_acc || !dk_acc || !dv_acc)
    return fail(RA_EINVAL, "null tensor pointer");
  {
    const ra_status mdst = check_mask_desc(md);
    if (mdst != RA_OK) return mdst;
  }
  // the bf16 kernels read a query block's plane (Q, dO) through 32-bit
  // buffer offsets, as they read a key/value block
  if (md->dtype == RA_BF16 && (uint64_t)md->Lq * md->d * esize(md->dtype) >= kSpanLimit)
    return fail(RA_EINVAL, "the bf16 backward needs one query block plane (Lq * d elements) below 2 GiB");
  {
    const ra_status al = check_tensor_align({q_blk, dout_blk, rowstat, kv_blk.k, kv_blk.v, dq_acc, dk_acc, dv_acc}, {});
    if (al != RA_OK) return al;
  }
  const bool f32 = md->dtype == RA_F32;
  const int64_t nqt = (md->Lq + bwd_dq_rows() - 1) / bwd_dq_rows();
  const int64_t nkt = (md->Lkv + bwd_dkdv_rows() - 1) / bwd_dkdv_rows();
  if ((int64_t)md->B * md->H * nqt > 0x7fffffffLL || (int64_t)md->B * md->Hkv * nkt > 0x7fffffffLL ||
      (f32 && ((int64_t)md->B * md->H * md->Lq / 4 >= 0x7fffffffLL ||
               (int64_t)md->B * md->Hkv * md->Lkv / 4 >= 0x7fffffffLL)))
    return fail(RA_EINVAL, "problem too large for one launch");
  if (!pair_active(md->layout, md->causal, md->P, md->q_rank, md->kv_rank, md->Lq, md->Lkv)) return RA_OK;
  BwdArgs a{};
  a.s.q = q_blk;
  a.s.k = kv_blk.k;
  a.s.v = kv_blk.v;
  a.s.q_plane_rows = md->Lq;
  a.s.kv_plane_rows = md->Lkv;
  a.s.B = md->B; a.s.H = md->H; a.s.Hkv = md->Hkv;
  a.s.Lq = (int)md->Lq; a.s.Lkv = (int)md->Lkv;
  a.s.P = md->P;
  a.s.layout = md->layout;
  a.s.host_lo = md->q_rank;
  a.s.n_hosts = 1;
  a.s.kv_shift = md->q_rank - md->kv_rank;
  a.s.q_mode = ROWS_COMPACT;
  a.s.kv_mode = ROWS_COMPACT;
  a.s.causal = md->causal ? 1 : 0;
  a.s.n_qtiles = (int)nqt;
  a.s.scale_log2 = md->scale * 1.4426950408889634f;
  a.dout = dout_blk;
  a.rowstat = rowstat;
  a.dq_acc = dq_acc;
  a.dk_acc = dk_acc;
  a.dv_acc = dv_acc;
  a.n_tok = md->Lkv;
  a.scale = md->scale;
  a.n_kvtiles = (int)nkt;
  a.first = a.kv_first = 0;   // add into the caller's accumulators
  a.q_fin = a.kv_fin = 0;     // and keep the sums in fp32
  a.kv_staged = 1;            // the kv block is compact, as a staged block
  a.stage_host0 = md->q_rank;
  a.q_compact = 1;
  a.kv_compact = 1;
  hipStream_t cs = static_cast<hipStream_t>(stream);
  RA_HIP(f32 ? launch_bwd_dkdv_f32(a, md->d, cs) : launch_bwd_dkdv(a, md->d, cs), "dK/dV kernel launch");
  RA_HIP(f32 ? launch_bwd_dq_f32(a, md->d, cs) : launch_bwd_dq(a, md->d, cs), "dQ kernel launch");
  return RA_OK;
}

}  // extern "C"

namespace {
constexpr int kDecodeTargetWgs = 4096;
constexpr int kDecodeWaves = 4;
constexpr int64_t kDecodeQuantum = 128;  // keys per workgroup iteration (4 waves x 32)

void decode_split(int B, int Hkv, long long L, int P, int64_t* chunk, int* cpb) {
  const int64_t block = L / P;
  int64_t c = (kDecodeTargetWgs + (int64_t)B * Hkv * P - 1) / ((int64_t)B * Hkv * P);
  if (c < 1) c = 1;
  int64_t ch = (block + c - 1) / c;
  ch = (ch + kDecodeQuantum - 1) / kDecodeQuantum * kDecodeQuantum;
  if (ch < kDecodeQuantum) ch = kDecodeQuantum;
  *chunk = ch;
  *cpb = (int)((block + ch - 1) / ch);
}

ra_status decode_args(int B, int H, int Hkv, long long L, int d, int P, ra_dtype dtype, float scale) {
  ra_status st = check_common(B, H, Hkv, L, d, P, dtype, scale);
  if (st != RA_OK) return st;
  return RA_OK;
}

// Decode workspace: per-wavefront partials o_part [B, H, S, d] and
// lse_part [B, H, S] (fp32), S = P x chunks per ring block x 4 waves.
struct DecodeWs {
  int64_t chunk;
  int cpb, S;
  size_t off_o, off_lse, total;
  bool overflow;
};

// Query heads per kv head are processed in sub-groups of 16 (the MFMA
// columns of the bf16 partial pass); each sub-group reads its kv head's rows.
int decode_sub_groups(int H, int Hkv) { return (H / Hkv + 15) / 16; }

DecodeWs decode_ws_layout(int B, int H, int Hkv, long long L, int d, int P) {
  DecodeWs w{};
  decode_split(B, Hkv * decode_sub_groups(H, Hkv), L, P, &w.chunk, &w.cpb);
  const int64_t S = (int64_t)P * w.cpb * kDecodeWaves;
  w.S = S > 0x7fffffffLL ? 0 : (int)S;
  SizeAcc a;
  w.off_o = a.add({(uint64_t)B, (uint64_t)H, (uint64_t)S, (uint64_t)d, 4});
  w.off_lse = a.add({(uint64_t)B, (uint64_t)H, (uint64_t)S, 4});
  w.total = (size_t)a.total;
  w.overflow = a.bad || S > 0x7fffffffLL;
  return w;
}

// Shared by ring_attn_decode and ring_attn_decode_noalloc: argument checks
// past the workspace, then the partial and merge launches on `stream`.
ra_status decode_launch(const void* q, const void* k, const void* v, void* out, float* lse, int B, int H, int Hkv,
                        long long L, int d, int P, float scale, ra_dtype dtype, const DecodeWs& W, void* wsb_,
                        void* stream) {
  ra_status st = check_tensor_align({q, k, v, out}, {lse});
  if (st != RA_OK) return st;
  if ((int64_t)B * Hkv * decode_sub_groups(H, Hkv) * P * W.cpb > 0x7fffffffLL)
    return fail(RA_EINVAL, "problem too large");
  DeviceCtx* ctx = nullptr;
  if ((st = get_ctx(&ctx)) != RA_OK) return st;
  DecodeArgs a{};
  a.q = q; a.k = k; a.v = v;
  a.S = W.S;
  char* wsb = static_cast<char*>(wsb_);
  a.o_part = reinterpret_cast<float*>(wsb + W.off_o);
  a.lse_part = reinterpret_cast<float*>(wsb + W.off_lse);
  a.out = out; a.lse = lse;
  a.B = B; a.H = H; a.Hkv = Hkv; a.group = H / Hkv;
  a.sub_groups = decode_sub_groups(H, Hkv);
  a.L = L;
  a.chunk = W.chunk;
  a.block = L / P;
  a.chunks_per_block = W.cpb;
  a.P = P;
  a.scale_log2 = scale * 1.4426950408889634f;
  hipStream_t cs = static_cast<hipStream_t>(stream);
  {
    const double es = (double)esize(dtype);
    const double bytes = 2.0 * B * Hkv * (double)L * d * es + (double)B * H * d * es +
                         (double)B * H * a.S * (d + 1) * 4;
    ProfScope ps(cs, bytes, 1);
    if (dtype == RA_BF16) RA_HIP(launch_decode_partial(a, d, 1, cs), "decode partial launch");
    else RA_HIP(launch_decode_partial_f32(a, d, cs), "decode partial launch");
  }
  RA_HIP(launch_decode_merge(a, d, dtype == RA_BF16 ? 1 : 0, cs), "decode merge launch");
  return RA_OK;
}

}  // namespace

extern "C" {

size_t ring_attn_decode_ws_bytes(int B, int H, int Hkv, long long L, int d, int P) {
  g_err.clear();
  if (decode_args(B, H, Hkv, L, d, P, RA_BF16, 1.f) != RA_OK) return SIZE_MAX;
  const DecodeWs W = decode_ws_layout(B, H, Hkv, L, d, P);
  if (W.overflow) {
    fail(RA_ENOMEM, "workspace size exceeds the 48-bit device address space");
    return SIZE_MAX;
  }
  return W.total;
}

ra_status ring_attn_decode(const void* q, const void* k, const void* v, void* out, float* lse, int B, int H,
                           int Hkv, long long L, int d, int P, float scale, ra_dtype dtype, void* stream,
                           void* ws, size_t ws_bytes) {
  g_err.clear();
  if (!q || !k || !v || !out || !lse) return fail(RA_EINVAL, "null tensor pointer");
  ra_status st = decode_args(B, H, Hkv, L, d, P, dtype, scale);
  if (st != RA_OK) return st;
  const DecodeWs W = decode_ws_layout(B, H, Hkv, L, d, P);
  if ((st = check_ws(W.overflow, W.total, ws, ws_bytes)) != RA_OK) return st;
  if (!ws) return fail(RA_EINVAL, "null workspace");
  return decode_launch(q, k, v, out, lse, B, H, Hkv, L, d, P, scale, dtype, W, ws, stream);
}

ra_status ring_attn_decode_noalloc(const void* q, const void* k, const void* v, void* out, float* lse, int B,
                                   int H, int Hkv, long long L, int d, int P, float scale, ra_dtype dtype,
                                   void* stream) {
  g_err.clear();
  if (!q || !k || !v || !out || !lse) return fail(RA_EINVAL, "null tensor pointer");
  ra_status st = decode_args(B, H, Hkv, L, d, P, dtype, scale);
  if (st != RA_OK) return st;
  const DecodeWs W = decode_ws_layout(B, H, Hkv, L, d, P);
  if (W.overflow || W.total > kDecodeScratchBytes)
    return fail(RA_EINVAL, "decode needs %zu bytes of scratch; the static scratch holds %zu (use ring_attn_decode "
                "with a caller workspace)", W.total, kDecodeScratchBytes);
  if ((st = check_tensor_align({q, k, v, out}, {lse})) != RA_OK) return st;
  void* scratch = nullptr;
  size_t scratch_bytes = 0;
  RA_HIP(decode_scratch(&scratch, &scratch_bytes), "hipGetSymbolAddress(decode scratch)");
  return decode_launch(q, k, v, out, lse, B, H, Hkv, L, d, P, scale, dtype, W, scratch, stream);
}

ra_status ra_debug_set_delays(int compute_us, int copy_us) {
  if (compute_us < 0 || copy_us < 0 || compute_us > 100000 || copy_us > 100000)
    return fail(RA_EINVAL, "delays must be in [0, 100000] us");
  std::lock_guard<std::mutex> lk(g_mu);
  g_delay_compute_us = compute_us;
  g_delay_copy_us = copy_us;
  return RA_OK;
}

ra_status ra_diag_mfma_loop(int workgroups, int iters, void* stream, double* mfma_count) {
  g_err.clear();
  if (!mfma_count) return fail(RA_EINVAL, "null output");
  if (workgroups < 1 || workgroups > (1 << 20) || iters < 1 || iters > (1 << 24))
    return fail(RA_EINVAL, "workgroups must be in [1, 2^20] and iters in [1, 2^24]");
  RA_HIP(launch_mfma_loop(workgroups, iters, static_cast<hipStream_t>(stream), mfma_count), "calibration launch");
  return RA_OK;
}

ra_status ra_debug_set_staging(int on) {
  std::lock_guard<std::mutex> lk(g_mu);
  g_staging = on != 0;
  return RA_OK;
}

ra_status ra_prof_enable(int on) {
  std::lock_guard<std::mutex> lk(g_mu);
  g_prof.on = on != 0;
  return RA_OK;
}

ra_status ra_prof_reset(void) {
  std::lock_guard<std::mutex> lk(g_mu);
  for (auto& r : g_prof.recs) {
    hipEventSynchronize(r.b);
    g_prof.pool.push_back(r.a);
    g_prof.pool.push_back(r.b);
  }
  g_prof.recs.clear();
  for (double& x : g_prof.acc) x = 0;
  return RA_OK;
}

ra_status ra_prof_read(double* out6) {
  if (!out6) return fail(RA_EINVAL, "null output");
  std::lock_guard<std::mutex> lk(g_mu);
  for (auto& r : g_prof.recs) {
    RA_HIP(hipEventSynchronize(r.b), "hipEventSynchronize");
    float ms = 0.f;
    RA_HIP(hipEventElapsedTime(&ms, r.a, r.b), "hipEventElapsedTime");
    if (r.kind == 0) {
      g_prof.acc[0] += ms;
      g_prof.acc[1] += 1;
      g_prof.acc[4] += r.work;
    } else {
      g_prof.acc[2] += ms;
      g_prof.acc[3] += 1;
      g_prof.acc[5] += r.work;
    }
    g_prof.pool.push_back(r.a);
    g_prof.pool.push_back(r.b);
  }
  g_prof.recs.clear();
  for (int i = 0; i < 6; ++i) out6[i] = g_prof.acc[i];
  return RA_OK;
}

}  // extern "C"

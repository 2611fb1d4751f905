// Internal types shared by the host driver and the HIP kernels.
// Not part of the public ABI (see include/ring_attn.h).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ra {

// How a row index inside a host block maps to a row of the backing array.
enum RowMode : int {
  ROWS_COMPACT = 0,   // row = i                        (a compact block)
  ROWS_HOST_Q = 1,    // row = host_row(q_rank, i)      (natural order array)
  ROWS_HOST_KV = 2,   // row = host_row(kv_rank, i)     (natural order array)
  ROWS_HOST_MAJOR = 3 // row = i of plane (q_rank * B + b) * Hkv + hkv (host-major staging)
};

// One launch of the fused block-attention step kernel.  A launch covers
// `n_hosts` query hosts q_rank = host_lo .. host_lo + n_hosts - 1, each
// against the kv block of host kv_rank = (q_rank - kv_shift) mod P.
struct StepArgs {
  const void* q;        // element type per kernel instantiation
  const void* k;
  const void* v;
  float* m;             // state rows follow q's row mode / plane
  float* l;
  float* o;
  void* out;            // final output (element type), same rows as q
  float* lse;
  int64_t q_plane_rows;   // rows per (b, h) plane of q / out / state
  int64_t kv_plane_rows;  // rows per (b, hkv) plane of k / v
  int B, H, Hkv;
  int Lq, Lkv;            // rows per host block (query / key)
  int P;
  int layout;             // 0 contiguous, 1 striped, 2 zigzag
  int host_lo, n_hosts;
  int kv_shift;           // kv_rank = (q_rank - kv_shift) mod P
  int q_mode;             // RowMode for q / out / state (COMPACT or HOST_Q)
  int kv_mode;            // RowMode for k / v
  int causal;
  int has_prev;           // merge with the state already in (m, l, o)
  int fin_lo, fin_hi;     // query hosts in [fin_lo, fin_hi) finalize (write out / lse);
                          // the others store the fp32 state
  int n_qtiles;           // ceil(Lq / BM)
  float scale_log2;       // scale * log2(e)
};

// One backward ring step (bf16): the fields of `s` describe the (query
// host, kv block) pairs exactly as for the forward step, with q / k / v read
// in natural token order (q_mode = ROWS_HOST_Q, per-row kv addressing).
// The kernels add this step's contributions into fp32 accumulators in
// natural row order.
struct BwdArgs {
  StepArgs s;
  const void* dout;       // [B, H, N, d], same rows as q
  const float* rowstat;   // [B, H, N][2]: lse of the forward times log2(e) (+inf: no visible key),
                          // then rowsum(dO * O)
  float* dq_acc;          // [B, H, N, d]
  float* dk_acc;          // [B, Hkv, N, d]
  float* dv_acc;          // [B, Hkv, N, d]
  int64_t n_tok;          // N (rows per plane of every natural-order array)
  float scale;
  int n_kvtiles;          // ceil(Lkv / rows per dK/dV workgroup)
  // Accumulation: on the first launch (first != 0) the kernels write their
  // rows of the fp32 accumulators instead of adding to them; on the last
  // launch that touches a query host's rows (bit q_rank of q_fin) or a kv
  // block's rows (bit kv_rank of kv_fin) they write the final bf16 value to
  // dq_out / dk_out / dv_out instead.
  __bf16* dq_out;
  __bf16* dk_out;
  __bf16* dv_out;
  int first;
  unsigned long long q_fin, kv_fin;
  // Where the kernels read K and V: 0 in place from the natural-order
  // arrays (rows of kv block kv_rank); 1 from a host-major staging buffer
  // (s.k / s.v), where query host q_rank's current block is plane
  // ((q_rank - stage_host0) * B + b) * Hkv + hkv of Lkv rows, in block
  // order.  The dK / dV accumulators stay at the natural rows of the block
  // unless kv_compact is set.
  int kv_staged;
  // fp32 backward: the final fp32 gradients (the bf16 outputs above unused)
  float* dq_out_f32;
  float* dk_out_f32;
  float* dv_out_f32;
  // One device's share (ring_attn_bwd_share): q, dout, dq and the row
  // statistics hold only the query host's rows, compact (plane stride Lq
  // rows, row i of the block at i) when q_compact != 0; the kv side writes
  // instead of adding when kv_first != 0 (the full backward sets it equal to
  // `first`); a staging buffer's first slot belongs to host stage_host0.
  int q_compact;
  int kv_first;
  int stage_host0;
  // Rows of the dK / dV accumulators: 0 the natural rows of the block
  // (n_tok per plane); 1 compact, Lkv per plane and block row j at row j
  // (one ring step on caller-owned block accumulators, ring_attn_bwd_step).
  int kv_compact;
};

struct MergeArgs {
  float* o_a; float* lse_a; const float* o_b; const float* lse_b;
  int64_t rows; int d;
};

struct FinalizeArgs {
  const float* m; const float* l; const float* o; void* out; float* lse;
  int64_t rows; int d;
};

// Split-KV decode: partial pass writes one normalized (O, lse) per
// (b, h, split); splits are ordered ring block major, chunk minor.
struct DecodeArgs {
  const void* q; const void* k; const void* v;
  float* o_part;          // [B, H, S, d]
  float* lse_part;        // [B, H, S]
  void* out; float* lse;  // [B, H, d], [B, H]
  int B, H, Hkv, group;
  int64_t L;              // keys per sequence
  int64_t chunk;          // keys per split (last split of a ring block may be shorter)
  int64_t block;          // keys per ring block (L / P)
  int chunks_per_block, P, S;
  float scale_log2;
  int sub_groups;         // ceil(group / 16): query heads per kv head in sub-groups of 16
};

// Launchers (return hipError_t of the launch).
hipError_t launch_step_bf16(const StepArgs& a, int d, hipStream_t s);
hipError_t launch_step_f32(const StepArgs& a, int d, hipStream_t s);
int step_block_rows_bf16(int d);  // BM of the bf16 kernel
int step_block_rows_f32(int d);   // BM of the f32 kernel
hipError_t launch_lse_merge(const MergeArgs& a, hipStream_t s);
hipError_t launch_finalize(const FinalizeArgs& a, int out_bf16, hipStream_t s);
hipError_t launch_decode_partial(const DecodeArgs& a, int d, int bf16, hipStream_t s);
hipError_t launch_decode_merge(const DecodeArgs& a, int d, int bf16, hipStream_t s);
// fp32 partial pass: the same grid, split order and partial layout as
// launch_decode_partial (four waves per split, one partial per wave).
hipError_t launch_decode_partial_f32(const DecodeArgs& a, int d, hipStream_t s);
// Size of the static decode scratch (ring_attn_decode_noalloc).
constexpr size_t kDecodeScratchBytes = 64ull << 20;
// Device address and size of the static decode scratch on the current
// device (looked up with hipGetSymbolAddress on the first call per device).
hipError_t decode_scratch(void** ptr, size_t* bytes);
hipError_t launch_spin(int microseconds, hipStream_t s);  // bounded busy wait (test hook)
// Counter calibration: `workgroups` x 4 waves, each issuing iters x 8 bf16
// 32x32x16 MFMAs from registers; *mfma_count receives the total issued.
hipError_t launch_mfma_loop(int workgroups, int iters, hipStream_t s, double* mfma_count);

// Backward (bf16): delta = rowsum(dO * O); dK/dV and dQ step kernels (the
// first step writes the fp32 accumulators, a row's last step its bf16 result).
int bwd_dq_rows();     // query rows per dQ workgroup
int bwd_dkdv_rows();   // keys per dK/dV workgroup
hipError_t launch_bwd_prep(const void* out, const void* dout, const float* lse, float* rowstat, int64_t rows, int d,
                           hipStream_t s);
hipError_t launch_bwd_dkdv(const BwdArgs& a, int d, hipStream_t s);
hipError_t launch_bwd_dq(const BwdArgs& a, int d, hipStream_t s);
// Backward (fp32): the same steps with fp32 inputs, arithmetic and outputs
// (one wavefront per row; k / v rows in place or in host-major staging).
hipError_t launch_bwd_prep_f32(const float* out, const float* dout, const float* lse, float* rowstat, int64_t rows,
                               int d, hipStream_t s);
hipError_t launch_bwd_dkdv_f32(const BwdArgs& a, int d, hipStream_t s);
hipError_t launch_bwd_dq_f32(const BwdArgs& a, int d, hipStream_t s);

}  // namespace ra

/*
 * ring_attn.h -- C ABI of the MI355X (gfx950) blockwise ring-attention library.
 *
 * Pages cited (by title; the section, equation or table is named alone):
 *   [TKG] "RingAttention 심층 아키텍처: 통신-연산 완전 중첩과 블록 단위 온라인
 *         소프트맥스로 1,000만 토큰 컨텍스트를 정복한 분산 어텐션 엔지니어링"
 *         (techknowgenie.com).
 *   [AIT] FlashAttention video summary (aitrends.kr).
 *   [CML] RingAttention paper newsletter (cmlonder.com, "Makale Bülteni").
 *
 * Conventions shared by every call
 * --------------------------------
 *  - Tensors are row-major and contiguous, in natural token order:
 *      q, out  [B, H,   Nq, d]   (element type `dtype`)
 *      k, v    [B, Hkv, N,  d]   (element type `dtype`)
 *      lse     [B, H,   Nq]      float32, natural log of the scaled logits
 *    Query head h reads kv head floor(h * Hkv / H) (grouped-query attention,
 *    consecutive groups).  d must be 64 or 128.
 *  - All pointers named q, k, v, out, lse, m, l, o, dout, dq, dk, dv, ws are
 *    DEVICE pointers owned by the caller; the library never allocates device
 *    memory inside a call and never frees caller memory.  Scratch state lives in `ws`, a
 *    caller-allocated device workspace of at least the size reported by the
 *    matching *_ws_bytes() query, aligned to 256 bytes.  Tensor pointers
 *    (q, k, v, out, o, dout, dq, dk, dv) must be 16-byte aligned and the
 *    fp32 row statistics (lse, m, l) 4-byte aligned: rows are moved as
 *    16-byte vectors.  Other pointers return RA_EINVAL.
 *  - `stream` is a hipStream_t (passed as void*; NULL = the null stream).
 *    Every call is asynchronous with respect to the host.  Calls that use a
 *    second stream internally fork it from `stream` and join it back before
 *    returning, so callers see ordinary single-stream semantics.  A call
 *    allocates, frees, synchronizes and clears nothing once the library has
 *    set up its per-device stream and events (on the first call that stages
 *    key/value blocks), so a later call may be captured into a HIP graph on
 *    `stream`; the second stream joins the capture through the fork event.
 *    The graph replays the call with the pointers and sizes it was captured
 *    with.
 *  - Errors: a call returns RA_OK or an error code BEFORE launching anything
 *    when an argument is invalid (RA_EINVAL: null pointer, N % P != 0,
 *    H % Hkv != 0, unsupported d, workspace too small, ...).  RA_ENOMEM:
 *    the workspace the arguments need would not fit a device allocation
 *    (its size overflows, or reaches 2^48 bytes, the width of the device's
 *    virtual addresses).  A failed HIP runtime call returns RA_EHIP.
 *    ra_last_error() then gives a message (thread-local).  Faults inside
 *    kernels surface at the caller's next synchronization, as with any HIP
 *    kernel.  No call aborts the process.
 *  - Workspace size queries (*_ws_bytes) apply the launch's checks to the
 *    arguments they take.  They return the size in bytes (0: the call needs
 *    no workspace), or SIZE_MAX when the arguments are invalid or the size
 *    cannot be allocated; ra_last_error() then says which.
 *  - Sizes: block lengths N / P up to 2^30 tokens.  The bf16 step kernel
 *    reads a key/value block through 32-bit buffer offsets, so one block of
 *    one (batch, kv head) plane must stay below 2 GiB (N / P * d * 2 bytes);
 *    whole planes may be larger (a striped ring whose plane is 2 GiB or more
 *    stages its first step's blocks instead of reading them in place).
 *    The bf16 ring_attn_bwd and ring_attn_bwd_share need one head plane
 *    (N * d * 2 bytes) below 2 GiB; the fp32 backward and decode have no
 *    such limit (64-bit addressing).
 */
#ifndef RING_ATTN_H
#define RING_ATTN_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum { RA_OK = 0, RA_EINVAL = 1, RA_ENOMEM = 2, RA_EHIP = 3, RA_EUNSUPPORTED = 4 } ra_status;

/* Which tokens each of the P virtual hosts owns ([TKG] §2 sequence sharding,
 * §7 round-robin striping; [CML] "İddia ve Gerçeklik" names striped and
 * zigzag schedules as the cures for the causal load imbalance):
 *   RA_CONTIGUOUS: host r owns tokens r*Bl .. r*Bl + Bl - 1   (Bl = N / P)
 *   RA_STRIPED:    host r owns tokens r, r + P, r + 2P, ...
 *   RA_ZIGZAG:     the sequence is cut into 2P chunks of C = N / (2P) tokens
 *                  and host r owns chunks r and 2P-1-r, in that order
 *                  (rows 0..C-1 of its block are tokens r*C .., rows C..2C-1
 *                  are tokens (2P-1-r)*C ..).  Needs N % (2P) == 0.      */
typedef enum { RA_CONTIGUOUS = 0, RA_STRIPED = 1, RA_ZIGZAG = 2 } ra_layout;

/* Element type of q, k, v and out.  RA_BF16: bfloat16 inputs, bf16 MFMA
 * products with fp32 accumulation.  RA_F32: float32 throughout.          */
typedef enum { RA_F32 = 0, RA_BF16 = 1 } ra_dtype;

/* ------------------------------------------------------------------------
 * ring_attn_fwd -- full attention by the ring method over P virtual hosts
 * that share this GPU ([TKG] §2-§5).
 *
 * Host r keeps its query block resident and, at ring step s = 0..P-1,
 * attends to the key/value block of host (r - s) mod P ([TKG] §5: every
 * host sends to (r + 1) mod P and receives from (r - 1) mod P).  Each step
 * fuses S = Q K^T * scale, the causal mask, the online-softmax update of the
 * running row max m and row sum l with rescaling of the output accumulator,
 * and the P V product ([TKG] §3, equations S, m_block, m_new, alpha, l_new,
 * O_new); the last step normalizes (O_final = O / l) and writes lse = m +
 * ln l.  The next step's key/value blocks are moved into a staging buffer
 * on a second stream while the current step computes ([TKG] §4 overlap).
 *
 * causal: key j is visible to query i iff pos(j) <= pos(i) on global token
 * positions ([TKG] §7); 0 = no mask.  layout only decides which tokens each
 * host owns; inputs and outputs stay in natural order, so the result does
 * not depend on layout or P (up to rounding).  scale: usually 1/sqrt(d)
 * ([TKG] §3 equation S).  Requires N % P == 0 (N % 2P == 0 for RA_ZIGZAG)
 * and 1 <= P <= 64.  With RA_ZIGZAG every host's block is first gathered
 * into the staging buffer (it is two separate chunks of the sequence).
 * ws: at least ring_attn_fwd_ws_bytes(...) bytes.
 * ---------------------------------------------------------------------- */
size_t ring_attn_fwd_ws_bytes(int B, int H, int Hkv, long long N, int d, int P, ra_dtype dtype);
ra_status ring_attn_fwd(const void* q, const void* k, const void* v, void* out, float* lse,
                        int B, int H, int Hkv, long long N, int d, int P, int causal,
                        ra_layout layout, float scale, ra_dtype dtype, void* stream,
                        void* ws, size_t ws_bytes);

/* ------------------------------------------------------------------------
 * ring_attn_fwd_share -- one device's share of a P-host ring: the query
 * block of host `rank` against all P key/value blocks, visited in ring order
 * rank, rank-1, ..., rank-P+1 (mod P), each next block staged on a second
 * stream while the current one computes ([TKG] §2, §5).
 *
 * q, out [B, H, N/P, d] hold the rank's Nq = N/P query tokens (in the order
 * the layout gives them: contiguous r*Bl + i, striped i*P + r, zigzag chunk
 * r then chunk 2P-1-r); lse is
 * [B, H, N/P].  k, v [B, Hkv, N, d] hold the whole sequence in natural
 * order (the blocks the other hosts would send).  ws: at least
 * ring_attn_fwd_share_ws_bytes(...) bytes.
 * ---------------------------------------------------------------------- */
size_t ring_attn_fwd_share_ws_bytes(int B, int H, int Hkv, long long N, int d, int P,
                                    ra_dtype dtype);
ra_status ring_attn_fwd_share(const void* q, const void* k, const void* v, void* out, float* lse,
                              int B, int H, int Hkv, long long N, int d, int P, int rank,
                              int causal, ra_layout layout, float scale, ra_dtype dtype,
                              void* stream, void* ws, size_t ws_bytes);

/* ------------------------------------------------------------------------
 * ring_attn_step -- one ring step for one (query block, key/value block)
 * pair, updating caller-owned online-softmax state in place ([TKG] §3).
 *
 * q_blk [B, H, Lq, d]; kv_blk.k, kv_blk.v [B, Hkv, Lkv, d] (compact blocks,
 * element type mask_desc->dtype).  State, float32, caller-owned:
 *   m [B, H, Lq]      the row's REFERENCE max of the scaled logits seen so
 *                     far (natural units): the running max of [TKG] §3
 *                     equation m_new, or up to 16 / log2(e) below it
 *   l [B, H, Lq]      sum over keys seen so far of exp(s - m)
 *   o [B, H, Lq, d]   sum over keys seen so far of exp(s - m) * v
 * Initialize with m = -inf, l = 0, o = 0.  After the call (m, l, o) describe
 * the keys seen before plus this block.  The bf16 kernel moves the reference
 * up to the true running max only when a tile's weights exp(s - m) would
 * exceed 2^16 (it skips the rescale otherwise); l and o are always relative
 * to the stored m.  So O = o / l and lse = m + ln l are exact, and so is a
 * merge of two such states by the [TKG] §3 update (m_new = max(m_a, m_b),
 * alpha = e^(m_a - m_new), beta = e^(m_b - m_new), l = alpha l_a + beta l_b,
 * o = alpha o_a + beta o_b): it needs l and o relative to their m, not m
 * to be the true max.  (The fp32 kernel keeps the true running max.)
 *
 * Positions for the causal mask come from mask_desc: contiguous
 * pos_q(i) = q_rank*Lq + i, pos_k(j) = kv_rank*Lkv + j; striped
 * pos_q(i) = i*P + q_rank, pos_k(j) = j*P + kv_rank (needs Lq == Lkv when
 * causal); zigzag with C = Lq/2: pos_q(i) = q_rank*C + i for i < C, else
 * (2P-1-q_rank)*C + i - C, likewise for keys (needs Lq == Lkv, even, when
 * causal).  A query row with no visible key in the block leaves its state
 * unchanged.
 * ---------------------------------------------------------------------- */
typedef struct { const void* k; const void* v; } ra_kv_block;
typedef struct {
  int B, H, Hkv, d;
  long long Lq, Lkv;
  float scale;
  ra_dtype dtype;
  int causal;
  ra_layout layout;
  int P, q_rank, kv_rank;
} ra_mask_desc;
ra_status ring_attn_step(const void* q_blk, ra_kv_block kv_blk, float* m, float* l, float* o,
                         const ra_mask_desc* mask_desc, void* stream);

/* ring_attn_finalize -- O_final = o / l ([TKG] §3 equation O_final) cast to
 * out_dtype, and lse = m + ln l, for `rows` independent rows of width d.
 * A row with l == 0 (no visible key) gives out = 0 and lse = -inf.
 * rows == 0 is a no-op (the pointers are not checked then).              */
ra_status ring_attn_finalize(const float* m, const float* l, const float* o, void* out,
                             float* lse, long long rows, int d, ra_dtype out_dtype,
                             void* stream);

/* ------------------------------------------------------------------------
 * lse_merge -- merge two normalized partial attention results over disjoint
 * key sets, in place into (o_a, lse_a):
 *   lse = ln(e^lse_a + e^lse_b)
 *   o_a = e^(lse_a - lse) * o_a + e^(lse_b - lse) * o_b
 * This is the [TKG] §3 m_new / alpha / beta / l_new / O_new update applied to
 * two partial states written as (O, lse).  A row whose two lse are -inf
 * gets o = 0, lse = -inf.  o_a, o_b [rows, d] and lse_a, lse_b [rows],
 * float32; d any positive value up to 1024.  rows == 0 is a no-op (the
 * pointers are not checked then).
 * ---------------------------------------------------------------------- */
ra_status lse_merge(float* o_a, float* lse_a, const float* o_b, const float* lse_b,
                    long long rows, int d, void* stream);

/* ------------------------------------------------------------------------
 * ring_attn_decode -- split-KV decode: one new query token per sequence
 * against a key/value cache split into P ring blocks ([CML]: the decode
 * KV-cache footprint of a long prompt).  Each ring block is processed in
 * chunks; every chunk yields a normalized partial (O, lse) that reads each
 * key/value row once for all H/Hkv query heads of its group; the partials
 * are merged with the lse_merge rule, chunks within a ring block first, then
 * the ring blocks in order.
 *
 * q, out [B, H, 1, d]; k, v [B, Hkv, L, d], all of element type dtype;
 * lse [B, H] float32.  RA_BF16: bf16 MFMA products with the weights rounded
 * to bf16 as the P V operand, fp32 accumulation.  RA_F32: fp32 throughout (a
 * plain, untuned partial pass).  The partials are fp32 for both, so the
 * workspace does not depend on dtype.  The query sees every cached key (no
 * mask).  Requires L % P == 0.  The query heads of a kv head are handled in
 * sub-groups of 16, each reading the kv head's rows (so K and V are read
 * once for H / Hkv <= 16, and once per 16 query heads beyond that, e.g.
 * twice for multi-query attention with 32 heads).  ws: at least
 * ring_attn_decode_ws_bytes(...) bytes.
 * ---------------------------------------------------------------------- */
size_t ring_attn_decode_ws_bytes(int B, int H, int Hkv, long long L, int d, int P);
ra_status ring_attn_decode(const void* q, const void* k, const void* v, void* out, float* lse,
                           int B, int H, int Hkv, long long L, int d, int P, float scale,
                           ra_dtype dtype, void* stream, void* ws, size_t ws_bytes);

/* ring_attn_decode_noalloc -- ring_attn_decode for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc): the same kernels and results
 * (bit for bit), with the partials in a static device array of the library
 * (64 MiB, held on every GPU the library runs on until the process ends)
 * instead of a caller workspace.  Allocates nothing.  Arguments as for
 * ring_attn_decode; RA_EINVAL when the partials would need more than the
 * 64 MiB (ring_attn_decode_ws_bytes(...) > 64 MiB; e.g. 16 sequences x 32
 * heads x 262144 keys need 34 MB).  The partials are fully rewritten by
 * every call, so nothing needs clearing; calls that overlap on one GPU
 * (different streams, or threads) race on the shared array. */
ra_status ring_attn_decode_noalloc(const void* q, const void* k, const void* v, void* out, float* lse,
                                   int B, int H, int Hkv, long long L, int d, int P, float scale,
                                   ra_dtype dtype, void* stream);

/* ------------------------------------------------------------------------
 * ring_attn_bwd -- gradients of ring_attn_fwd by recomputation over a
 * reverse ring ([TKG] §7, "활성화 체크포인팅과 메모리 재연산": keep the
 * queries and the row statistics, send the key/value blocks the other way
 * round the ring and recompute the attention map where it is needed).
 *
 * At ring step s = 0..P-1 host r pairs with kv block (r + s) mod P and, tile
 * by tile, recomputes S = scale Q K^T and P = exp(S - lse), then adds
 *   dV += P^T dO,  dK += scale dS^T Q,  dQ += scale dS K,
 *   dS = P * (dO V^T - delta),  delta_i = dO_i . O_i
 * (the chain rule applied to the forward definition).
 *
 * q, out, dout, dq [B, H, N, d]; k, v, dk, dv [B, Hkv, N, d]; lse [B, H, N]
 * float32 as written by ring_attn_fwd for the same inputs (out and lse are
 * the forward's results); all in natural token order, all of element type
 * dtype.  RA_BF16: bf16 MFMA products with P and dS rounded to bf16 as
 * operands, fp32 accumulation, bf16 gradients; one head plane (N * d) must
 * stay below 2 GiB.  RA_F32: fp32 inputs, arithmetic and gradients (a
 * plain, untuned path).  With grouped-query attention dk, dv sum the
 * contributions of every query head of the group.  causal, layout, scale,
 * P: as for ring_attn_fwd; the result does not depend on layout or P up to
 * rounding.  dq, dk, dv are overwritten.  ws: at least
 * ring_attn_bwd_ws_bytes(...) bytes (staging buffers for the reverse ring,
 * fp32 accumulators and the row statistics).
 * ---------------------------------------------------------------------- */
size_t ring_attn_bwd_ws_bytes(int B, int H, int Hkv, long long N, int d, int P, ra_dtype dtype);
ra_status ring_attn_bwd(const void* q, const void* k, const void* v, const void* out, const void* dout,
                        const float* lse, void* dq, void* dk, void* dv, int B, int H, int Hkv, long long N, int d,
                        int P, int causal, ra_layout layout, float scale, ra_dtype dtype, void* stream, void* ws,
                        size_t ws_bytes);

/* ------------------------------------------------------------------------
 * ring_attn_bwd_share -- one device's share of the ring backward
 * ([TKG] §7 with the ring of [TKG] §2): host `rank` keeps its queries, its
 * forward output and row statistics, and meets kv block (rank + s) mod P at
 * step s = 0..P-1, each later block staged on a second stream while the
 * previous step computes.  The gradient formulas are those of
 * ring_attn_bwd, restricted to the host's queries.
 *
 * q, out, dout, dq [B, H, N/P, d] and lse [B, H, N/P] hold the rank's
 * query tokens in the order the layout gives them (as for
 * ring_attn_fwd_share, whose out and lse they are); k, v [B, Hkv, N, d]
 * hold the whole sequence in natural order.  dq is the rank's query
 * gradient.  dk, dv [B, Hkv, N, d] (natural order) receive this rank's
 * contribution to every key's gradient: zeros for keys the rank's queries
 * never see; the sum over rank = 0..P-1 of the shares' dk (dv) is
 * ring_attn_bwd's dk (dv) up to rounding.  In a real ring those partial
 * sums travel with their kv block; here each lands at its block's rows.
 * dtype, causal, layout, scale, P and the bf16 head-plane limit: as for
 * ring_attn_bwd.  dq, dk, dv are overwritten.  ws: at least
 * ring_attn_bwd_share_ws_bytes(...) bytes (two staging slots of one block,
 * the fp32 dq accumulator and the row statistics of the rank's rows).
 * ---------------------------------------------------------------------- */
size_t ring_attn_bwd_share_ws_bytes(int B, int H, int Hkv, long long N, int d, int P, ra_dtype dtype);
ra_status ring_attn_bwd_share(const void* q, const void* k, const void* v, const void* out, const void* dout,
                              const float* lse, void* dq, void* dk, void* dv, int B, int H, int Hkv, long long N,
                              int d, int P, int rank, int causal, ra_layout layout, float scale, ra_dtype dtype,
                              void* stream, void* ws, size_t ws_bytes);

/* ------------------------------------------------------------------------
 * Backward building blocks for a caller's own ring ([TKG] §7), the
 * counterparts of ring_attn_step: each host keeps its query block, its
 * forward output and lse, and as the kv blocks pass by adds one pair's
 * gradient contributions; the dK, dV sums travel on with their block.
 *
 * ring_attn_bwd_prep -- the row statistics a query block's backward steps
 * read: for each of `rows` rows, rowstat[row][0] = lse * log2(e) (+inf where
 * lse = -inf, so that the row contributes nothing) and rowstat[row][1] =
 * delta = sum_c dO[row][c] * O[row][c].  out, dout [rows, d] in `dtype`
 * (16-byte aligned), lse [rows] fp32, rowstat [rows][2] fp32 (16-byte
 * aligned; overwritten).  rows = 0 does nothing.
 *
 * ring_attn_bwd_step -- one (query block, kv block) pair, positions and
 * mask as described by mask_desc (the fields and checks of
 * ring_attn_step), ADDED into caller-owned fp32 accumulators (zero them
 * before the first step):
 *   dq_acc [B, H,   Lq,  d] += scale dS K
 *   dk_acc [B, Hkv, Lkv, d] += scale dS^T Q   (all query heads of the group)
 *   dv_acc [B, Hkv, Lkv, d] += P^T dO
 * with P = exp(S - lse) recomputed from the scores and dS = P (dO V^T -
 * delta), the formulas of ring_attn_bwd.  q_blk, dout_blk [B, H, Lq, d]
 * and k, v of kv_blk [B, Hkv, Lkv, d] in mask_desc->dtype, rowstat
 * [B, H, Lq][2] from ring_attn_bwd_prep on the block's out, dout and lse.
 * Every pointer 16-byte aligned.  bf16: one query or key/value block plane
 * below 2 GiB.  A pair with no visible key launches nothing.  Steps that
 * add into the same accumulators must be ordered (one stream).
 * ---------------------------------------------------------------------- */
ra_status ring_attn_bwd_prep(const void* out, const void* dout, const float* lse, float* rowstat, long long rows,
                             int d, ra_dtype dtype, void* stream);
ra_status ring_attn_bwd_step(const void* q_blk, const void* dout_blk, const float* rowstat, ra_kv_block kv_blk,
                             float* dq_acc, float* dk_acc, float* dv_acc, const ra_mask_desc* mask_desc,
                             void* stream);

/* ------------------------------------------------------------------------
 * Diagnostics.
 * ra_last_error: message of the last failed call on this thread ("" if none).
 * ra_version: library version string.
 * ra_prof_enable(1) makes the library bracket every fused block-attention
 * kernel launch (one per ring step) and every decode-partial launch with
 * HIP events on the stream the kernel runs on; ra_prof_read() synchronizes
 * on the recorded events and returns, since the last ra_prof_reset():
 *   out[0] total step-kernel milliseconds   out[1] step-kernel launches
 *   out[2] total decode-kernel milliseconds out[3] decode-kernel launches
 *   out[4] algorithmic FLOPs of the timed step kernels (4 d per unmasked
 *          query/key pair per query head, [TKG] §4 table)
 *   out[5] algorithmic bytes of the timed decode kernels (K and V once, q,
 *          and the fp32 partials written)
 * Events are created once per process and reused.
 * ---------------------------------------------------------------------- */
const char* ra_last_error(void);
const char* ra_version(void);

/* Test hook for the ring driver's stream ordering: when set, every later
 * ring_attn_fwd / ring_attn_fwd_share call enqueues a bounded spin of about
 * `compute_us` microseconds on the compute stream before each step kernel and
 * of about `copy_us` on the copy stream before each staging copy (0 = none,
 * at most 100000).  Results must not change; only the timeline does. */
ra_status ra_debug_set_delays(int compute_us, int copy_us);

/* Test and measurement hook for the ring exchange: with on = 0, later
 * ring_attn_fwd, ring_attn_fwd_share and ring_attn_bwd calls read every ring
 * step's key/value blocks in place from the natural-order k and v (no staging
 * copies, no second stream) wherever the kernels can address them in place
 * (not zigzag forward blocks, nor a striped forward plane of 2 GiB or more,
 * which are always staged); on = 1 (the default) restores the exchange.  The
 * kernels and their arithmetic are the same either way, so results are
 * bitwise identical; only the timeline changes (it isolates what the staging
 * copies cost the kernels that run beside them). */
ra_status ra_debug_set_staging(int on);
/* Counter calibration: launches `workgroups` workgroups of four waves on
 * `stream`, each wave issuing iters x 8 independent bf16 MFMAs
 * (v_mfma_f32_32x32x16_bf16, 32768 FLOPs each) from registers, and writes
 * the total MFMA count to *mfma_count.  Reads and writes no memory.  A
 * profiler's MFMA counters for this launch divided by that count give the
 * counters' scale; its duration gives the MFMA rate reached in practice.
 * workgroups in [1, 2^20], iters in [1, 2^24], else RA_EINVAL. */
ra_status ra_diag_mfma_loop(int workgroups, int iters, void* stream, double* mfma_count);
ra_status ra_prof_enable(int on);
ra_status ra_prof_reset(void);
ra_status ra_prof_read(double* out6);

#ifdef __cplusplus
}
#endif
#endif /* RING_ATTN_H */

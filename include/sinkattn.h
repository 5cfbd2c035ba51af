/*
 * sinkattn.h -- C ABI of the MI355X (gfx950) sink-GQA attention library.
 *
 * One attention layer of the gpt-oss family on its hot path: YaRN /
 * NTK-by-parts rotary embedding at global positions, an append-only KV cache
 * with snapshot/restore, and grouped-query attention under a full causal
 * mask or a sliding band, with a learned per-head sink logit appended as an
 * extra softmax column that is dropped after normalisation.  Prefill and
 * single-token decode.
 *
 * Sources (page title, section):
 *   "MoE-Xtend" README  -- DESIGN CONTRACTS (global positions, mask alignment,
 *       append-only cache, GQA shape contract), ATTENTION STACK (scores,
 *       causal/window masks, sink column), ROPE + SCALING (YaRN blend and
 *       concentration), KV CACHE (layout, extend, snapshot/restore, sizing),
 *       ARCHITECTURE (prefill writes the prompt KV once; decode appends one
 *       row per step).
 *   "GQA Attention" study note on gpt-oss -- How it works (q_mult grouping,
 *       band p-W < j <= p, sinks per query head, sm_scale = 1/sqrt(d_h)).
 *
 * Conventions shared by every entry point
 *   - Every function returns an sa_status (0 = SA_OK).  On any non-OK status
 *     nothing has been enqueued and no library state has changed;
 *     sa_last_error() returns a message for the calling thread.
 *   - Device pointers are HIP device memory on the current device, owned by
 *     the caller; the library never allocates or frees device memory and
 *     never synchronises.  Work is enqueued on `stream` (a hipStream_t;
 *     NULL = the default stream) and completes asynchronously.
 *   - Tensors are dense and row-major.  Element type is bf16 (SA_BF16) or
 *     fp32 (SA_F32); one call uses one type for all of its activations and
 *     cache rows.  Sinks are always fp32.
 *   - Sizes are element counts unless a name ends in _bytes.
 *   - Every device pointer (activations, cache buffers, workspace) must be
 *     16-byte aligned (SA_ERR_ARG otherwise): the kernels move 16-byte
 *     vectors.
 *
 * Cache memory layout (per layer; C = capacity rows, a multiple of 32):
 *   K: [B, C, n_kv, d_h]                     -- the pages' [B, T_cache, H_kv, d]
 *   V: [B, C/32, n_kv, d_h, 32]              -- V[b, j, g, e] lives at
 *        (((b*(C/32) + j/32)*n_kv + g)*d_h + e)*32 + j%32
 *   The V blocking puts 32 consecutive keys of one (head, coordinate) next
 *   to each other, which is the operand order of the gfx950 matrix cores for
 *   the probability x value product.  Both buffers hold
 *   B*C*n_kv*d_h elements.
 */
#ifndef SINKATTN_H
#define SINKATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  SA_OK = 0,
  SA_ERR_ARG = -1,       /* null pointer, non-positive size, bad parameter   */
  SA_ERR_SHAPE = -2,     /* n_q % n_kv != 0, unsupported d_h, shape differs
                            from the cache's, capacity not a multiple of 32  */
  SA_ERR_DTYPE = -3,     /* unknown dtype, or dtype differs from the cache's */
  SA_ERR_CAPACITY = -4,  /* append past capacity, queries past the rows
                            already in the cache, or keys the queries need
                            below the cache's first position                 */
  SA_ERR_SNAPSHOT = -5,  /* snapshot of another cache, rows below it were
                            rewritten since it was taken, or a ring and its
                            stage out of step                                */
  SA_ERR_HIP = -6        /* a HIP launch error                               */
} sa_status;

typedef enum { SA_BF16 = 0, SA_F32 = 1 } sa_dtype;

/* YaRN / NTK-by-parts parameters ("MoE-Xtend" README, ROPE + SCALING).
 * factor = s (1.0 = plain RoPE, theta_i = base^(-2i/d)); orig_ctx = L_train;
 * ntk_alpha < ntk_beta are the cutpoint turn counts.  Requires d_h even and
 * positive, base > 1, factor >= 1, 0 < ntk_alpha < ntk_beta, orig_ctx > 0. */
typedef struct {
  int32_t d_h;
  double base;
  double factor;
  int64_t orig_ctx;
  double ntk_alpha;
  double ntk_beta;
} sa_yarn;

/* Message describing the calling thread's last non-OK status ("" if none).
 * The pointer stays valid until the thread's next library call. */
const char* sa_last_error(void);

/* Host only.  The blended per-pair angular rates inv_freq[0 .. d_h/2) and
 * the concentration c = 0.1*ln(s) + 1, in fp64 ("MoE-Xtend" README, ROPE +
 * SCALING).  inv_freq: host array of d_h/2 doubles, caller-owned. */
int sa_yarn_inv_freq(const sa_yarn* y, double* inv_freq, double* concentration);

/* Host only.  KV bytes of L layers: 2*L*B*T*H_kv*d*dtype_bytes ("MoE-Xtend"
 * README, KV CACHE, memory scaling).  Returns -1 if an argument is negative
 * or the product overflows int64. */
int64_t sa_kv_cache_bytes(int64_t L, int64_t B, int64_t T, int64_t H_kv,
                          int64_t d, int64_t dtype_bytes);

/* Rotate x in place at global positions offset + t ("MoE-Xtend" README,
 * DESIGN CONTRACTS and ROPE + SCALING).  x: device [B, T, n_heads, d_h] of
 * `dtype`.  Coordinate i pairs with i + d_h/2:
 *   y_i       = c*(x_i cos a - x_{i+d/2} sin a)
 *   y_{i+d/2} = c*(x_{i+d/2} cos a + x_i sin a),  a = (offset+t)*inv_freq_i.
 * Angles, rates and the rotation are evaluated in fp64 and rounded once to
 * `dtype` (round to nearest, ties to even).  Positions are never wrapped.
 * Apply to Q (n_heads = n_q) and K (n_heads = n_kv), never to V.
 * Requires d_h == y->d_h, d_h % 8 == 0, d_h <= 256, offset >= 0. */
int yarn_rope_apply(void* x, int dtype, int B, int T, int n_heads, int d_h,
                    int64_t offset, const sa_yarn* y, void* stream);

/* The same rotation out of place: reads x, writes y (both device
 * [B, T, n_heads, d_h] of `dtype`); y may be x itself but must not partly
 * overlap it (SA_ERR_ARG).  x is not modified unless y == x. */
int yarn_rope(const void* x, void* y, int dtype, int B, int T, int n_heads, int d_h,
              int64_t offset, const sa_yarn* yarn, void* stream);

/* Opaque host-side handle of one layer's cache.  K/V storage is the
 * caller's (layout above); the handle records the shape, the offset (the
 * global position the next append writes; one offset is shared by the
 * batch), and the write log used to validate snapshots.  A linear cache
 * holds position p in row p - base, where base is 0 except for a stage
 * cache filled by kv_ring_stage; a ring cache (kv_ring_create) holds p in
 * row p mod W. */
typedef struct sa_kv_cache sa_kv_cache;

typedef struct {
  int64_t offset;
  uint64_t cache_id;
  uint64_t stamp;
} sa_kv_snapshot;

/* Create a handle over caller-owned buffers k, v (device, B*capacity*n_kv*
 * d_h elements each) ("MoE-Xtend" README, KV CACHE: one preallocated cache
 * per layer, K and V of shape [B, T_cache, H_kv, d], sized
 * min(prompt + max_tokens, max_context) rows by the caller; the V buffer
 * here is blocked as described above).  `offset` rows (0 .. capacity) are
 * taken as already written (a pre-filled prefix; K rows already rotated).
 * capacity must be a positive multiple of 32.  The handle is host memory
 * the library allocates; *out is set only on SA_OK.
 * SA_ERR_ARG: null out/k/v, unaligned k/v, B, n_kv or d_h not positive;
 * SA_ERR_DTYPE: unknown dtype; SA_ERR_SHAPE: capacity not a positive
 * multiple of 32, d_h not a multiple of 8 or above 256; SA_ERR_CAPACITY:
 * offset outside [0, capacity]. */
int kv_cache_create(sa_kv_cache** out, void* k, void* v, int dtype, int B,
                    int64_t capacity, int n_kv, int d_h, int64_t offset);
/* The same call under the name the cache's interface gives its
 * constructor ("MoE-Xtend" README, KV CACHE: init_cache); identical
 * arguments, results and errors. */
int kv_cache_init(sa_kv_cache** out, void* k, void* v, int dtype, int B,
                  int64_t capacity, int n_kv, int d_h, int64_t offset);
/* Free the host handle (the caller's K/V buffers are untouched).  Work
 * already enqueued with the handle is unaffected (kernels take plain
 * pointers).  A null handle is SA_ERR_ARG. */
int kv_cache_destroy(sa_kv_cache* c);
/* Positions written so far: the global position of the next append
 * ("MoE-Xtend" README, KV CACHE: offset advances on extend; DESIGN
 * CONTRACTS: RoPE and masks use this absolute position).  -1 for a null
 * handle. */
int64_t kv_cache_offset(const sa_kv_cache* c);
/* Oldest position the cache holds: base for a linear cache, max(0, offset -
 * W) for a ring of W rows ("GPT-OSS-Lite" README, Why these metrics
 * matter: windowed layers keep only their window); -1 for a null handle. */
int64_t kv_cache_base(const sa_kv_cache* c);

/* Append T_new rows to every sequence ("MoE-Xtend" README, KV CACHE: extend
 * writes [offset, offset+T_new) then advances offset; on a ring, row t goes
 * to its slot and only the last W rows of a longer append are written).
 * k_rot: device
 * [B, T_new, n_kv, d_h], already rotated; v: device [B, T_new, n_kv, d_h],
 * unrotated.  Rows are copied bit for bit (V into its blocked layout).  The
 * offset advances at enqueue time.  A decode step appends T_new = 1.
 * SA_ERR_CAPACITY if a linear cache would pass its capacity (a ring never
 * fills). */
int kv_cache_append(sa_kv_cache* c, const void* k_rot, const void* v,
                    int T_new, void* stream);

/* Rotate and append in one pass ("MoE-Xtend" README, ROPE + SCALING and KV
 * CACHE; DESIGN CONTRACTS: a row's position is its global index, so K row
 * t goes to cache row offset + t rotated at that position).  k: device
 * [B, T_new, n_kv, d_h], unrotated; v as for kv_cache_append; y: YaRN
 * parameters with y->d_h == d_h.  The cache receives exactly the bits that
 * yarn_rope(k, offset = kv_cache_offset(c)) followed by kv_cache_append
 * would write, without the intermediate buffer.  bf16 needs d_h % 16 == 0
 * (SA_ERR_SHAPE otherwise); other errors as for kv_cache_append and
 * yarn_rope. */
int kv_cache_append_rope(sa_kv_cache* c, const void* k, const void* v,
                         int T_new, const sa_yarn* y, void* stream);

/* kv_cache_append_rope that also rotates the layer's queries, which sit at
 * the same positions: q (device [B, T_new, n_q, d_h], unrotated) is written
 * rotated to q_rot (same shape; q_rot == q rotates in place, any other
 * overlap is SA_ERR_ARG), exactly as yarn_rope(q, q_rot, offset =
 * kv_cache_offset(c)) would, sharing the angle tables with K (on a ring,
 * every query row is rotated even where only the last W key rows are kept).
 * q and q_rot both null: same as kv_cache_append_rope. */
int kv_cache_append_rope_qk(sa_kv_cache* c, const void* q, void* q_rot, int n_q,
                            const void* k, const void* v, int T_new,
                            const sa_yarn* y, void* stream);

/* O(1) host bookkeeping ("prefill once, decode many").  A snapshot records
 * the offset; restore rewinds the offset to it.  Restoring is refused with
 * SA_ERR_SNAPSHOT if the snapshot belongs to another cache or if any append
 * made after it started below its offset (its rows were overwritten); on a
 * ring, if anything was appended after it (use kv_ring_save/kv_ring_load).
 * kv_ring_stage starts a stage cache's history afresh: snapshots of the
 * stage taken before are refused. */
int kv_cache_snapshot(const sa_kv_cache* c, sa_kv_snapshot* out);
int kv_cache_restore(sa_kv_cache* c, const sa_kv_snapshot* snap);

/* ---- Ring caches for band layers ----
 * "GPT-OSS-Lite" README, "Why these metrics matter" and "Results": the
 * windowed layers cache only the last W tokens while full layers keep the
 * sequence, which is the architecture's KV-cache reduction (2T/(T+W) for
 * alternating layers); "MoE-Xtend" README, ARCHITECTURE: with a sliding
 * window a decode step's attention is O(W).
 *
 * A ring holds W rows per sequence, W = the layer's window, a positive
 * multiple of 32 (SA_ERR_SHAPE otherwise): position p lives in row p mod W,
 * so appending p overwrites p - W, the key that has just left the band.
 * Buffers (caller-owned, device): K [B, W, n_kv, d_h], V [B, W/32, n_kv,
 * d_h, 32], the cache layout above with C = W.  The ring starts empty.
 *   - The append entry points write each row at its slot.
 *   - sinkattn_decode needs window == W (SA_ERR_ARG otherwise): every slot
 *     the ring holds is in the decode query's band, so min(offset, W) rows
 *     are attended without a mask (in slot order).
 *   - sinkattn_prefill and sinkattn_prefill_rope refuse a ring (SA_ERR_ARG):
 *     a chunk's queries need more than W keys between them.  A chunk goes
 *     through a linear stage cache of the same B, n_kv, d_h and dtype and a
 *     capacity of at least W - 1 + T_q rows:
 *        kv_ring_stage(stage, ring)                    the ring's rows
 *        kv_cache_append_rope_qk(stage, q, q_rot, ..)  the chunk
 *        sinkattn_prefill(q_rot, stage, .., window = W,
 *                         q_offset = kv_cache_offset(ring))
 *        kv_ring_commit(ring, stage)                   the last W rows back
 *     The stage is scratch, not layer state: one stage serves every band
 *     layer in turn, and several chunks may be appended and attended
 *     between a stage and its commit. */
int kv_ring_create(sa_kv_cache** out, void* k, void* v, int dtype, int B, int window,
                   int n_kv, int d_h);

/* Make `stage` (a linear cache) hold the ring's last min(offset, W - 1)
 * positions -- all its keys that a query at position offset can see -- at
 * rows 0.., with base = offset - that count and offset = the ring's offset.
 * Enqueues one small copy.  SA_ERR_ARG if `ring` is not a ring or `stage`
 * is; SA_ERR_SHAPE / SA_ERR_DTYPE if they differ in B, n_kv, d_h or dtype;
 * SA_ERR_CAPACITY if the stage is too small. */
int kv_ring_stage(sa_kv_cache* stage, const sa_kv_cache* ring, void* stream);

/* Copy the stage's positions at or above the ring's offset (at most its
 * last W) into the ring's slots and advance the ring's offset to the
 * stage's.  SA_ERR_SNAPSHOT unless the stage was staged (or last committed)
 * from this ring and the ring has not changed since, or if the stage's
 * offset is below the ring's. */
int kv_ring_commit(sa_kv_cache* ring, sa_kv_cache* stage, void* stream);

/* Snapshot and restore of a ring by copy ("prefill once, decode many" when
 * decode sweeps overwrite slots).  k_save, v_save: caller-owned device
 * buffers of B*W*n_kv*d_h elements each (the ring's buffer sizes), 16-byte
 * aligned.  kv_ring_save enqueues a copy of the ring into them and records
 * the offset in *out; kv_ring_load enqueues the copy back and sets the
 * offset.  The caller keeps the buffers unchanged between the two.
 * SA_ERR_ARG for a non-ring cache; SA_ERR_SNAPSHOT for a snapshot of
 * another cache. */
int kv_ring_save(const sa_kv_cache* ring, void* k_save, void* v_save, sa_kv_snapshot* out,
                 void* stream);
int kv_ring_load(sa_kv_cache* ring, const void* k_save, const void* v_save,
                 const sa_kv_snapshot* snap, void* stream);

/* Sink attention of T_q new queries against the cache ("MoE-Xtend" README,
 * ATTENTION STACK; "GQA Attention" study note, How it works).
 *   q:    device [B, T_q, n_q, d_h], already rotated; query t sits at global
 *         position p = q_offset + t.
 *   sinks: device fp32 [n_q], one logit per query head in scaled-logit
 *         units (not multiplied by sm_scale); -inf disables a head's sink.
 *   out:  device [B, T_q, n_q, d_h].
 * For query head h, KV head g = h / (n_q/n_kv), allowed keys
 *   A(p) = { j : max(0, p - window + 1) <= j <= p }  (window > 0: band of
 *   `window` keys including the diagonal) or { j : 0 <= j <= p } (window
 *   <= 0: full causal), and l_j = sm_scale * <q, K_j>:
 *   out = sum_{j in A} e^{l_j} V_j / (e^{sigma_h} + sum_{j in A} e^{l_j}).
 * Requires q_offset + T_q <= kv_cache_offset(c) (append first) and every
 * allowed key at or above kv_cache_base(c) (SA_ERR_CAPACITY); a ring is
 * refused (SA_ERR_ARG, see kv_ring_stage); n_kv and d_h must equal the
 * cache's.  bf16: d_h in {64, 96, 128},
 * n_q/n_kv <= 128, cache capacity below 2^31 rows (SA_ERR_SHAPE otherwise),
 * matrix-core kernel with fp32 accumulation; fp32: d_h % 8 == 0,
 * d_h <= 256, vector kernel. */
int sinkattn_prefill(const void* q, const sa_kv_cache* c, const float* sinks,
                     void* out, int B, int T_q, int n_q, int n_kv, int d_h,
                     int window, float sm_scale, int64_t q_offset,
                     void* stream);

/* sinkattn_prefill with unrotated queries: q holds raw rows and the kernel
 * rotates each one at its position q_offset + t ("MoE-Xtend" README, ROPE +
 * SCALING) before attending, with yarn_rope's arithmetic, so the result is
 * exactly that of yarn_rope(q, q_offset) followed by sinkattn_prefill, without
 * the rotated copy of Q.  y: YaRN parameters with y->d_h == d_h.  bf16
 * caches only (SA_ERR_DTYPE otherwise); other errors as sinkattn_prefill. */
int sinkattn_prefill_rope(const void* q, const sa_kv_cache* c, const float* sinks,
                          void* out, int B, int T_q, int n_q, int n_kv, int d_h,
                          int window, float sm_scale, int64_t q_offset,
                          const sa_yarn* y, void* stream);

/* ---- The layer's fused qkv projection with RoPE and append ----
 * "GQA Attention" study note on gpt-oss, How it works: after the norm, one
 * fused bf16 linear layer (with bias) of width d_qkv = d_h (n_q + 2 n_kv)
 * produces Q, K and V; rotary embeddings run on Q and K.  "MoE-Xtend"
 * README, ROPE + SCALING and KV CACHE: rotation at the global position,
 * then K and V are appended.
 *
 * Bytes of workspace sinkattn_qkv_rope_append needs for T tokens of head
 * dimension d_h (a per-position fp64 (c cos, c sin) table); 0 on invalid
 * arguments. */
size_t sinkattn_qkv_workspace_bytes(int T, int d_h);

/* qkv = x W^T + b, accumulated in fp32 and rounded once to bf16 (what a
 * bf16 linear layer returns; the fp32 summation order is the kernel's),
 * split [Q | K | V] with each part head-major (column h*d_h + e of a part is
 * coordinate e of head h); then exactly what kv_cache_append_rope_qk(c, Q,
 * q_rot, K, V) does with those bf16 values: Q rotated at positions
 * kv_cache_offset(c) + t into q_rot, K rotated into the cache rows, V
 * appended, the offset advanced by T.
 *   x:      device [B, T, d_model] bf16 (the normed hidden states)
 *   w_qkv:  device [d_qkv, d_model] bf16 (a linear layer's [out, in] weight)
 *   b_qkv:  device [d_qkv] bf16
 *   q_rot:  device [B, T, n_q, d_h] bf16, written
 *   workspace: device scratch of sinkattn_qkv_workspace_bytes(T, d_h)
 *      bytes, overwritten.
 * The cache must be a linear bf16 cache (a ring is SA_ERR_ARG: use its
 * stage) with d_h in {64, 96, 128} (SA_ERR_SHAPE); n_kv and d_h are the
 * cache's; d_model a multiple of 64 (SA_ERR_SHAPE); room for T rows
 * (SA_ERR_CAPACITY); y->d_h == d_h. */
int sinkattn_qkv_rope_append(sa_kv_cache* c, const void* x, const void* w_qkv,
                             const void* b_qkv, void* q_rot, int B, int T, int d_model,
                             int n_q, const sa_yarn* y, void* workspace, size_t ws_bytes,
                             void* stream);

/* ---- MoE layer: top-k router, dispatch, selected SwiGLU experts ----
 * "MoE-Xtend" README, MOE ROUTING: S = X W_r^T, I = topk(S, k), w =
 * softmax over the k selected logits, y = sum_i w_i E_i(x); the batched form
 * groups token rows by expert and evaluates only the selected experts; top-k
 * ties must break consistently.  "GPT-OSS-Lite" visual guide, Architecture
 * Specifications: 8 routed experts, 2 active per token, 1 shared expert,
 * SwiGLU experts (ffn 1536).
 * Shapes: x [N, d_model] bf16 (the normed hidden states); w_router [E,
 * d_model] bf16; w13 [E, 2 ffn, d_model] bf16, the gate rows W1 then the
 * up rows W3 of each expert (linear layers' [out, in] weights); w2 [E,
 * d_model, ffn] bf16.  Limits: 1 <= E <= 64, 1 <= k <= min(8, E), d_model a
 * multiple of 64, ffn a multiple of 128 (SA_ERR_SHAPE otherwise);
 * ceil(N / 256) * E <= 16384 (SA_ERR_ARG).  All
 * device pointers caller-owned and 16-byte aligned. */

/* Router: logits = x W_r^T rounded once to bf16 (logits: device [N, E]
 * bf16, written); per token the k largest logits, largest first, equal
 * logits in increasing expert id (expert_ids: device int32 [N, k]); weights
 * = softmax of those k logits in fp32 (device float [N, k]). */
int moe_route(const void* x, int N, int d_model, const void* w_router, int E, int k,
              void* logits, int32_t* expert_ids, float* weights, void* stream);

/* Bytes of scratch moe_dispatch needs for N tokens and E experts. */
size_t moe_dispatch_workspace_bytes(int N, int E);

/* Group the (token, slot) pairs by expert, deterministically: rows (device
 * int32 [N*k]) lists token*k + slot for expert 0's pairs in token order,
 * then expert 1's, ...; expert_start (device int32 [E+1]) holds the first
 * row of each expert and the total.  expert_ids: device int32 [N, k], the
 * k ids of a token distinct and in [0, E) (ids outside are skipped and
 * leave their rows unwritten). */
int moe_dispatch(const int32_t* expert_ids, int N, int E, int k, int32_t* rows,
                 int32_t* expert_start, void* workspace, size_t ws_bytes, void* stream);

/* Bytes of workspace moe_layer needs (ffn_shared = 0: no shared expert). */
size_t moe_workspace_bytes(int N, int d_model, int E, int k, int ffn, int ffn_shared);

/* The whole layer: moe_route, moe_dispatch, then for each expert's rows
 * h = bf16(silu(a) * b), a = bf16(x W1^T), b = bf16(x W3^T), and
 * o = bf16(h W2^T); y = bf16(sum over the token's slots of w * o, plus the
 * shared expert's o with weight 1 when ffn_shared > 0 (w13_shared [2
 * ffn_shared, d_model], w2_shared [d_model, ffn_shared]; both null and
 * ffn_shared = 0 otherwise)), summed in fp32 in slot order (shared last).
 * y: device [N, d_model] bf16.  The workspace (moe_workspace_bytes) holds
 * the logits, ids, weights, dispatch lists, the gated activations and the
 * per-slot outputs; its contents are overwritten. */
int moe_layer(const void* x, int N, int d_model, const void* w_router, int E, int k,
              const void* w13, const void* w2, int ffn, const void* w13_shared,
              const void* w2_shared, int ffn_shared, void* y, void* workspace,
              size_t ws_bytes, void* stream);

/* ---- Sampling controls: from a row of logits to the next token ----
 * "MoE-Xtend" README, SAMPLING CONTROLS: p = softmax(z / T); top-k keeps
 * the k most probable tokens, top-p the smallest set whose cumulative
 * probability reaches p, min-p drops the tokens less probable than a
 * fraction of the most probable one; logit bias, then repetition, presence
 * and frequency penalties, then the truncations, then the draw; T = 0 is
 * greedy.  The project summary page: sampling is deterministic.
 * Per row, as the library computes it:
 *   z' = z + bias; a token seen c > 0 times gets z' / r (z' > 0) or z' * r
 *   (otherwise), then z' - presence, then z' - frequency * c, each step one
 *   fp32 operation;
 *   T = 0: the largest z', ties to the lower id;
 *   T > 0: relative weights e = exp((z' - max z') / T) (fp32) and integer
 *   masses q = floor(e * 2^40), summed exactly, so the result is
 *   deterministic; every truncation is a threshold on z' and never splits
 *   equal logits: top-k keeps z' >= the k-th largest z', top-p (on the
 *   top-k set) keeps z' >= the logit at which the mass summed in decreasing
 *   z' first reaches ceil(top_p * top-k mass), min-p keeps e >= min_p;
 *   the draw takes the first kept token, in increasing id, whose
 *   cumulative mass exceeds floor(u * kept mass). */
typedef struct {
  float temperature;  /* >= 0; 0: greedy                                    */
  int32_t top_k;      /* >= 0; 0 or >= V: off                               */
  float top_p;        /* (0, 1]; 1: off                                     */
  float min_p;        /* [0, 1]; 0: off                                     */
  float repetition;   /* > 0; 1: off                                        */
  float presence;     /* finite; 0: off                                     */
  float frequency;    /* finite; 0: off                                     */
  int32_t reserved;   /* set to 0                                           */
} sa_sample_params;

/* Add each id of ids (device int32 [B, H], row stride ids_stride >= H) into
 * counts (device int32 [B, V]): counts[b, id] += 1 for 0 <= id < V; other
 * ids are skipped.  Integer atomics: the result does not depend on order. */
int sample_count_tokens(const int32_t* ids, int B, int H, int64_t ids_stride, int32_t* counts,
                        int V, void* stream);

/* Bytes of workspace sample_tokens needs for B rows of V logits (0 on
 * invalid sizes). */
size_t sample_workspace_bytes(int B, int V);

/* One token per row.  logits: device fp32 [B, V], row stride
 * logits_stride >= V; bias: device fp32, row b at bias + b * bias_stride
 * (bias_stride 0: one row for the batch; V or more otherwise), or null;
 * counts: device int32 [B, V] occurrence counts for the penalties, or null
 * (penalties off); params: device [B]; u: device fp32 [B], one uniform in
 * [0, 1) per row (unused by greedy rows).  Outputs: tokens device int32
 * [B]; n_kept device int32 [B] (the size of the kept set; 1 for greedy
 * rows), or null; processed device fp32 [B, V] (z' before temperature), or
 * null.  With update_counts != 0 (counts non-null) counts[b, token] += 1
 * after the draw, so a decode loop's counts stay on the device.
 * 1 <= V <= 262144, 1 <= B <= 65535 (SA_ERR_SHAPE otherwise).  A row with
 * invalid parameters (out of the ranges above, or u outside [0, 1) with
 * T > 0), or with no finite z' when T > 0 (no z' above -inf when greedy),
 * gets token -1 and n_kept 0.  All pointers caller-owned; the workspace's
 * contents are overwritten. */
int sample_tokens(const float* logits, int B, int V, int64_t logits_stride, const float* bias,
                  int64_t bias_stride, int32_t* counts, const sa_sample_params* params,
                  const float* u, int update_counts, int32_t* tokens, int32_t* n_kept,
                  float* processed, void* workspace, size_t ws_bytes, void* stream);

/* Bytes of fp32 workspace that sinkattn_decode needs for any cache offset up
 * to `capacity` with these shapes (0 on invalid arguments). */
size_t sinkattn_decode_workspace_bytes(int B, int n_q, int n_kv, int d_h,
                                       int64_t capacity);

/* One decode step's attention: the single query token of each sequence sits
 * at position p = kv_cache_offset(c) - 1 (its own K/V row appended just
 * before, "MoE-Xtend" README, ARCHITECTURE: append KV at offset=t, then
 * t++).  q: device [B, 1, n_q, d_h]; out: device [B, 1, n_q, d_h];
 * workspace: device scratch of at least
 * sinkattn_decode_workspace_bytes(B, n_q, n_kv, d_h, capacity) bytes, whose
 * contents are overwritten.  The allowed key set is split into chunks
 * reduced in parallel and merged in a fixed order (deterministic), with the
 * sink added once at the merge.  bf16: d_h in {64, 96, 128}, n_q/n_kv <= 16,
 * cache capacity below 2^31 rows (SA_ERR_SHAPE otherwise); fp32: as
 * sinkattn_prefill. */
int sinkattn_decode(const void* q, const sa_kv_cache* c, const float* sinks,
                    void* out, int B, int n_q, int n_kv, int d_h, int window,
                    float sm_scale, void* workspace, size_t ws_bytes,
                    void* stream);

/* A whole decode step in one attention launch (two with the split merge):
 * the token at position p = kv_cache_offset(c) (before the call) has its Q
 * and K rotated at p ("MoE-Xtend" README, ROPE + SCALING), its K/V row
 * appended at offset p ("MoE-Xtend" README, ARCHITECTURE and KV CACHE:
 * append at offset = t, then t++), and its query attends to the cache with
 * that row in it, as sinkattn_decode does.  The results are bit for bit
 * those of kv_cache_append_rope_qk(c, q, q_rot, n_q, k, v, 1, y) followed by
 * sinkattn_decode(q_rot, c, ...): the same rotation arithmetic, the same
 * reduction order.
 *   q:     device [B, 1, n_q, d_h], unrotated; not modified.
 *   q_rot: optional device [B, 1, n_q, d_h] that receives the rotated Q;
 *          NULL: not written.  Must not overlap q or out.
 *   k, v:  device [B, 1, n_kv, d_h], k unrotated.
 *   workspace, ws_bytes, window, sm_scale, sinks, out: as sinkattn_decode.
 * bf16 caches only (SA_ERR_DTYPE otherwise), linear or ring.  Every check
 * (those of kv_cache_append_rope_qk and of sinkattn_decode) runs before
 * anything is enqueued; on an error nothing is enqueued and the cache's
 * offset is unchanged.  On success the offset is p + 1. */
int sinkattn_decode_step(sa_kv_cache* c, const void* q, void* q_rot,
                         const void* k, const void* v, const float* sinks,
                         void* out, int B, int n_q, int n_kv, int d_h,
                         int window, float sm_scale, const sa_yarn* y,
                         void* workspace, size_t ws_bytes, void* stream);

/* Bytes of the static device array that sinkattn_decode_noalloc keeps its
 * split partials in (one copy per GPU, held until the process ends). */
#define SA_DECODE_SCRATCH_BYTES (8u << 20)
size_t sinkattn_decode_scratch_bytes(void);

/* sinkattn_decode with no workspace argument, for callers that cannot
 * allocate device memory: code under HIP graph capture, serving loops that
 * may not call hipMalloc, harnesses that forbid it.  Same arguments (less
 * the workspace), same kernels, same results bit for bit.  The split
 * partials go to a static device array of SA_DECODE_SCRATCH_BYTES (8 MiB)
 * on the current device; its address is looked up (hipGetSymbolAddress)
 * on the first call on each device.  The call allocates and frees nothing.
 * SA_ERR_ARG, with nothing enqueued, when this call's partials need more
 * than the array holds (B * n_q * splits * (d_h + 2) * 4 bytes; e.g. the
 * B = 8, 64/8-head, d_h = 64 long-context decode needs 4.3 MB); spans of at
 * most 256 rows need none.  Every call on one GPU shares that GPU's array
 * and leaves its partials there: calls that overlap on one GPU (other
 * streams, other threads) race and must be ordered by the caller. */
int sinkattn_decode_noalloc(const void* q, const sa_kv_cache* c, const float* sinks,
                            void* out, int B, int n_q, int n_kv, int d_h, int window,
                            float sm_scale, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* SINKATTN_H */

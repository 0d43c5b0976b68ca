/*
 * fa2.h -- C ABI of an MI355X (gfx950) FlashAttention-2 forward pass and its
 * backward pass.
 *
 * The operation (exact attention, computed tile by tile with an online
 * softmax, never writing the N x N score matrix to device memory):
 *
 *   S_ij  = scale * <q_i, k_j>
 *   visible(i, j) = true            (non-causal)
 *                 = (j <= i)        (causal)
 *   m_i   = max_{visible j} S_ij
 *   l_i   = sum_{visible j} exp(S_ij - m_i)
 *   O_i   = sum_{visible j} exp(S_ij - m_i) v_j / l_i
 *   LSE_i = m_i + ln(l_i)
 *
 * Sources: Saraf, "FlashAttention 2: Three Places the Chip Was Still
 * Waiting" -- section 1 (tiles folded into a running result with a running
 * max and denominator, exact), section 2.2 (the max correction every step,
 * the division once per query block), section 2.3 (query blocks as
 * independent units of parallel work), section 2.4 (each wave owns whole
 * query rows); papermap "FlashAttention-2" explainer, Chapter 02 (same
 * outputs as standard attention, the N x N matrix never materialised);
 * Mishra, "FlashAttention-2 and -3: From Algebra to GPU Scheduling", "How
 * to compare kernels honestly" (dtype, head dim, lengths, batch, heads and
 * causal mode are the parameters of a forward call).
 *
 * Conventions shared by every entry point:
 *   - Tensors are dense, row-major, contiguous: q, k, v, o (and dout, dq,
 *     dk, dv) are [B, H, N, d] (d fastest); lse (and delta) are [B, H, N].
 *     Query and key lengths are both N.
 *   - All data pointers are DEVICE pointers on the current HIP device.
 *   - The caller owns every buffer.  The library never allocates, frees or
 *     synchronises; it enqueues its kernels on `stream` and returns.  The
 *     caller observes completion through the stream.
 *   - Outputs are fully overwritten (every row, including ragged tails);
 *     inputs are only read.  Outputs must not alias inputs.
 *   - Arguments are validated before any HIP call; on error nothing is
 *     launched and a negative fa2_status is returned.  No output is printed
 *     and no exception crosses the ABI.
 *   - The library keeps no mutable global state and is re-entrant, with one
 *     exception: fa2_decode_paged_noalloc writes its partial results to a
 *     static buffer of FA2_DECODE_SCRATCH_BYTES per device, shared by all of
 *     its calls on that device.
 */
#ifndef FA2_H
#define FA2_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

#define FA2_VERSION 100 /* major*100 + minor */

typedef enum fa2_dtype {
  FA2_F32 = 0,  /* IEEE binary32 */
  FA2_BF16 = 1  /* bfloat16 (8-bit exponent, 7-bit mantissa) */
} fa2_dtype;

typedef enum fa2_status {
  FA2_OK = 0,
  FA2_ERR_INVALID_ARG = -1, /* null or misaligned pointer, bad size, bad scale, bad dtype code */
  FA2_ERR_UNSUPPORTED = -2, /* valid arguments outside what the kernels implement (head dim, dtype pair) */
  FA2_ERR_NO_DEVICE = -3,   /* no usable HIP device is current */
  FA2_ERR_LAUNCH = -4,      /* the kernel launch was rejected by the runtime */
  FA2_ERR_SCRATCH = -5      /* the call needs more than FA2_DECODE_SCRATCH_BYTES of static scratch */
} fa2_status;

/* Size of the static per-device scratch of fa2_decode_paged_noalloc (16 MiB). */
#define FA2_DECODE_SCRATCH_BYTES ((size_t)16 << 20)

/*
 * fa2_fwd -- attention forward: O and the per-row logsumexp.
 *
 *   q, k, v   device pointers, [B, H, N, d] in `in_dtype`, 16-byte aligned.
 *   o         device pointer, [B, H, N, d] in `o_dtype`, 16-byte aligned.
 *   lse       device pointer, [B, H, N] float32, 4-byte aligned: natural-log
 *             logsumexp of the scaled visible scores of each query row.
 *   B, H, N   batch, heads, sequence length; each >= 1, and B*H*N*d must
 *             fit in a signed 64-bit integer (offsets are 64-bit).
 *   d         head dimension; 64 or 128 (others: FA2_ERR_UNSUPPORTED).
 *   causal    0: every key visible; 1: key j visible to query i iff j <= i.
 *   scale     finite, >= 0; multiplies the raw dot products (typically
 *             1/sqrt(d)).  Negative or non-finite: FA2_ERR_INVALID_ARG.
 *   stream    a hipStream_t cast to void* (NULL = the null stream).
 *   in_dtype  FA2_BF16 or FA2_F32 for q, k and v.
 *   o_dtype   FA2_F32 or FA2_BF16 for o.  bf16 outputs are rounded to
 *             nearest-even from the fp32 result.
 *
 * Arithmetic: bf16 inputs use bf16 matrix-core products with fp32
 * accumulation, the softmax statistics in fp32, and probabilities rounded
 * to bf16 (nearest-even) before the P*V product; O is divided by the sum of
 * those rounded probabilities, the logsumexp uses the sum of the unrounded
 * ones.  fp32 inputs keep every step in fp32.
 *
 * Debug: when the environment variable FA2_DEBUG_POISON is set (and not
 * "0") at the time of the call, the bf16 kernel fills each shared-memory
 * tile slot with NaN before copying a K or V tile into it, so a read that
 * races its copy shows up as NaN in o.  Results are otherwise unchanged.
 *
 * Returns FA2_OK after enqueueing, else a negative fa2_status.
 */
int fa2_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
            int B, int H, int N, int d, int causal, float scale,
            void* stream, int in_dtype, int o_dtype);

/*
 * fa2_fwd_gqa -- fa2_fwd with grouped key/value heads (GQA; MQA when
 * H_kv = 1).
 *
 * The H query heads of a sequence share H_kv key/value heads in equal,
 * consecutive groups: query head h attends with key/value head
 * h / (H / H_kv).  Everything else is fa2_fwd; fa2_fwd(...) is
 * fa2_fwd_gqa(...) with H_kv = H.
 *
 * Source: papermap "FlashAttention-2" explainer, Chapter 03 ("The
 * Downstream Story") and Chapter 05 ("The variant family"): GQA-aware
 * kernels are named among the variants built on FlashAttention-2's
 * partitioning; the grouping is the plain reading of the name.
 *
 *   q, o      [B, H, N, d]; lse [B, H, N].
 *   k, v      [B, H_kv, N, d].
 *   H_kv      >= 1 and dividing H (else FA2_ERR_INVALID_ARG).
 *
 * Returns FA2_OK after enqueueing, else a negative fa2_status.
 */
int fa2_fwd_gqa(const void* q, const void* k, const void* v, void* o, float* lse,
                int B, int H, int H_kv, int N, int d, int causal, float scale,
                void* stream, int in_dtype, int o_dtype);

/*
 * fa2_fwd_window -- fa2_fwd_gqa with a sliding-window (local) mask.
 *
 * Key j is visible to query i iff
 *     i - window_left <= j <= i + window_right,
 * where a bound of -1 means no limit on that side and a bound of N or more
 * is the same as no limit.  (-1, 0) is the causal mask and (-1, -1) no
 * mask: fa2_fwd_gqa(..., causal, ...) is fa2_fwd_window with those bounds.
 * Every query sees at least its own key, so every row is defined.  Key
 * tiles wholly outside a query tile's band are never loaded.
 *
 * Source: papermap "FlashAttention-2" explainer, Chapter 03 ("The
 * Downstream Story") and Chapter 05 ("The variant family"): sliding-window
 * kernels are named among the variants built on FlashAttention-2's
 * partitioning; a band of keys around each query is the plain reading.
 *
 *   window_left, window_right  >= -1 (else FA2_ERR_INVALID_ARG).
 *   in_dtype FA2_F32 supports only (-1, -1) and (-1, 0) (else
 *   FA2_ERR_UNSUPPORTED).
 * All other arguments as fa2_fwd_gqa.  Returns FA2_OK after enqueueing,
 * else a negative fa2_status.
 */
int fa2_fwd_window(const void* q, const void* k, const void* v, void* o, float* lse,
                   int B, int H, int H_kv, int N, int d, int window_left, int window_right,
                   float scale, void* stream, int in_dtype, int o_dtype);

/*
 * fa2_bwd -- attention backward: dQ, dK and dV from the forward's O and LSE.
 *
 * The gradient of a scalar loss through the operation of fa2_fwd, given its
 * gradient dO with respect to O (chain rule through P = softmax of the
 * scaled, masked scores):
 *
 *   P_ij  = exp(S_ij - LSE_i) for visible (i, j), else 0
 *   D_i   = sum_c dO_ic O_ic                (written to `delta`)
 *   dV_j  = sum_i P_ij dO_i
 *   dS_ij = P_ij (dO_i . v_j - D_i)
 *   dQ_i  = scale * sum_j dS_ij k_j
 *   dK_j  = scale * sum_i dS_ij q_i
 *
 * Sources: the pages define the forward pass only.  The backward pass is
 * named as part of the training runs behind the headline numbers (Saraf,
 * "FlashAttention 2: Three Places the Chip Was Still Waiting", section 2.5)
 * and as something a benchmark must say whether it times (Mishra,
 * "FlashAttention-2 and -3: From Algebra to GPU Scheduling", the
 * benchmarking checklist); P is recomputed from q, k and LSE instead of
 * stored (Mishra, the note that a fast kernel may redo arithmetic to avoid
 * moving data).  D_i = sum_j P_ij dP_ij because O_i = sum_j P_ij v_j.
 *
 *   q, k, v, dout  device pointers, [B, H, N, d] in `in_dtype`, 16-byte aligned.
 *   o              device pointer, [B, H, N, d] in `o_dtype`, 16-byte aligned:
 *                  the output fa2_fwd returned for the same q, k, v.
 *   lse            device pointer, [B, H, N] float32: the LSE fa2_fwd returned.
 *   delta          device pointer, [B, H, N] float32, caller-owned workspace;
 *                  overwritten with D.
 *   dq, dk, dv     device pointers, [B, H, N, d] in `grad_dtype`, 16-byte
 *                  aligned; fully overwritten.
 *   B, H, N, d, causal, scale, stream: as for fa2_fwd (same values as the
 *                  forward call).
 *   in_dtype       FA2_BF16 (q, k, v and dout); FA2_F32: FA2_ERR_UNSUPPORTED.
 *   o_dtype        FA2_F32 or FA2_BF16 (the dtype o was written in).
 *   grad_dtype     FA2_F32 or FA2_BF16 for dq, dk, dv (bf16: rounded to
 *                  nearest-even from the fp32 result).
 *   d              64 or 128 (others: FA2_ERR_UNSUPPORTED).
 *
 * Arithmetic: bf16 matrix-core products with fp32 accumulation; P and dS
 * are rounded to bf16 (nearest-even) before the products that consume them
 * (dV, and dQ / dK); D and the softmax terms are fp32.
 *
 * Outputs must not alias inputs or each other; delta must not alias any of
 * them.  Three kernels are enqueued on `stream` (D, then dK/dV, then dQ).
 * Returns FA2_OK after enqueueing, else a negative fa2_status.
 */
int fa2_bwd(const void* q, const void* k, const void* v, const void* o, const void* dout,
            const float* lse, float* delta, void* dq, void* dk, void* dv,
            int B, int H, int N, int d, int causal, float scale,
            void* stream, int in_dtype, int o_dtype, int grad_dtype);

/*
 * fa2_bwd_gqa -- fa2_bwd with grouped key/value heads (see fa2_fwd_gqa).
 *
 * q, o, dout, dq: [B, H, N, d]; lse, delta: [B, H, N]; k, v, dk, dv:
 * [B, H_kv, N, d].  A key/value head is used by every query head of its
 * group, so its dK and dV are the sums over that group's query heads
 * (computed in one pass per key/value head, no atomics).  fa2_bwd(...) is
 * fa2_bwd_gqa(...) with H_kv = H.  Returns FA2_OK after enqueueing, else a
 * negative fa2_status.
 */
int fa2_bwd_gqa(const void* q, const void* k, const void* v, const void* o, const void* dout,
                const float* lse, float* delta, void* dq, void* dk, void* dv,
                int B, int H, int H_kv, int N, int d, int causal, float scale,
                void* stream, int in_dtype, int o_dtype, int grad_dtype);

/*
 * fa2_bwd_window -- fa2_bwd_gqa under a sliding-window mask (see
 * fa2_fwd_window for the bounds).  o and lse must come from fa2_fwd_window
 * with the same bounds.  fa2_bwd_gqa(..., causal, ...) is fa2_bwd_window
 * with (-1, causal ? 0 : -1).  Key tiles (dQ) and query blocks (dK, dV)
 * wholly outside the band are skipped.  Returns FA2_OK after enqueueing,
 * else a negative fa2_status (window bounds below -1: FA2_ERR_INVALID_ARG).
 */
int fa2_bwd_window(const void* q, const void* k, const void* v, const void* o, const void* dout,
                   const float* lse, float* delta, void* dq, void* dk, void* dv,
                   int B, int H, int H_kv, int N, int d, int window_left, int window_right,
                   float scale, void* stream, int in_dtype, int o_dtype, int grad_dtype);

/*
 * fa2_split_item -- one chunk of a split forward schedule: the keys of
 * query tile `tile` (rows 256*tile .. 256*tile + 255) in key tiles
 * [kt_lo, kt_hi) (64 keys each).
 *
 *   slot     partial-result slot the chunk writes, 0 <= slot < n_slots; or
 *            -1 when the chunk is the tile's whole key range and writes o
 *            and lse itself.
 *   slot0    first slot of the tile's chunks (they use slot0 .. slot0 +
 *            n_parts - 1); the item with slot == slot0 also merges them.
 *   n_parts  number of chunks of the tile.
 */
typedef struct fa2_split_item {
  int tile;
  int kt_lo;
  int kt_hi;
  int slot;
  int slot0;
  int n_parts;
} fa2_split_item;

/*
 * fa2_split_plan -- build a forward schedule that cuts the key range of
 * the heaviest query tiles into chunks, so that a grid with too few query
 * tiles to fill the chip (few heads, long sequences, causal) still keeps
 * every compute unit busy.  Host-only; touches no device.
 *
 * Each query tile's visible key tiles (the band of fa2_fwd_window) are cut
 * into chunks of at most C key tiles; chunks are listed longest first (the
 * order the hardware dispatches them in).  With max_chunk_tiles == 0 the
 * library picks C (among chunks of about total/(k*num_units) for k from 1
 * to 8 and those that cut the longest band into 2..8 equal parts), or no
 * split at all, by simulating the dispatch of the
 * B*H*n_items workgroups on `num_units` compute units (one resident
 * workgroup each) under a cost model of the kernels: a per-workgroup
 * start-up cost, one unit per key tile, and the traffic of writing and
 * merging partial results.  Without a split every item has slot -1 and
 * n_slots is 0: fa2_fwd_split then computes exactly what fa2_fwd_window
 * does.
 *
 * Source: Mishra, "FlashAttention-2 and -3: From Algebra to GPU
 * Scheduling", "Another use of mergeable statistics" (the (max, sum)
 * statistics of disjoint key ranges merge exactly, which lets a long key
 * range be cut when the grid is too small); Saraf, "FlashAttention 2:
 * Three Places the Chip Was Still Waiting", section 2.3 (few heads and
 * long sequences leave units idle when a block covers a whole head).
 *
 *   B, H, N, d, in_dtype            as for fa2_fwd (in_dtype FA2_BF16 only,
 *                                   else FA2_ERR_UNSUPPORTED).
 *   window_left, window_right       as for fa2_fwd_window.
 *   num_units        compute units of the device (>= 1; ignored when
 *                    max_chunk_tiles > 0).
 *   max_chunk_tiles  0 = the library's choice; > 0 = cut every tile into
 *                    chunks of at most this many key tiles.
 *   items, max_items host array receiving the schedule; items may be NULL
 *                    (then only the counts are returned).  A non-NULL items
 *                    with max_items < the item count: FA2_ERR_INVALID_ARG.
 *   n_items, n_slots, workspace_bytes  (host, non-NULL) receive the number
 *                    of items, of partial slots per (sequence, head), and
 *                    the workspace size fa2_fwd_split needs (0 if no split).
 *
 * Returns FA2_OK or a negative fa2_status.
 */
int fa2_split_plan(int B, int H, int N, int d, int window_left, int window_right, int in_dtype,
                   int num_units, int max_chunk_tiles, fa2_split_item* items, int max_items,
                   int* n_items, int* n_slots, size_t* workspace_bytes);

/*
 * fa2_fwd_split -- fa2_fwd_window over a schedule from fa2_split_plan.
 *
 * One workgroup per (item, sequence, head) runs the forward kernel over the
 * item's key tiles only.  A chunk of a split tile writes its partial result
 * to the workspace: O normalised by its own sum of (rounded) probabilities
 * and the log of that sum and of the unrounded one, per row; a second
 * kernel on the same stream then combines the chunks of each split tile,
 * weighting each by the exponential of its log-sum, into o and lse.  Tiles
 * that are not split write o and lse directly.
 *
 *   items            DEVICE copy of the schedule (n_items entries, as
 *                    filled by fa2_split_plan for the same B, H, N, d and
 *                    window; 4-byte aligned); read only.  A schedule for
 *                    other sizes cannot make the kernels read or write out
 *                    of bounds (every field is clamped) but gives wrong
 *                    results.
 *   n_items, n_slots as returned by fa2_split_plan.
 *   workspace        device buffer of at least workspace_bytes as returned
 *                    by fa2_split_plan, 16-byte aligned, overwritten (NULL
 *                    allowed when n_slots == 0).  Layout: [B*H][n_slots]
 *                    [256][d] fp32 partial O, then [B*H][n_slots][256] pairs
 *                    of fp32 log-sums.
 *   in_dtype         FA2_BF16 only (else FA2_ERR_UNSUPPORTED).
 * All other arguments as fa2_fwd_window; the buffers must not overlap one
 * another.  Two kernels are enqueued when n_slots > 0.  Returns FA2_OK
 * after enqueueing, else a negative fa2_status.
 */
int fa2_fwd_split(const void* q, const void* k, const void* v, void* o, float* lse,
                  int B, int H, int H_kv, int N, int d, int window_left, int window_right,
                  float scale, void* stream, int in_dtype, int o_dtype,
                  const fa2_split_item* items, int n_items, int n_slots,
                  void* workspace, size_t workspace_bytes);

/*
 * fa2_sparse_plan -- turn a block-sparse mask into the per-query-tile key
 * tile lists fa2_fwd_sparse streams.  Host-only; touches no device.
 *
 * Mask: key j is visible to query i iff
 *     block_mask[L][i / block_q][j / block_k] != 0   (and j <= i if causal),
 * with L the layout of the (sequence, head) (see fa2_fwd_sparse).  A query
 * that sees no key has no softmax: fa2_fwd_sparse writes O = 0 and
 * LSE = -inf for it.
 *
 * Source: papermap "FlashAttention-2" explainer, Chapter 03 ("The
 * Downstream Story") and Chapter 05 ("The variant family"): block-sparse
 * kernels are named among the variants built on FlashAttention-2's
 * partitioning; a mask per (query block, key block) pair is the plain
 * reading.  Key tiles with no visible key are never loaded.
 *
 *   N                  sequence length (>= 1).
 *   block_q, block_k   block sizes: block_q a multiple of 32, block_k a
 *                      multiple of 64 (else FA2_ERR_UNSUPPORTED), so that
 *                      each 32-row slice of a query tile lies in one query
 *                      block and each 64-key tile in one key block.
 *   n_layouts          number of masks (>= 1).
 *   block_mask         host bytes [n_layouts][ceil(N/block_q)][ceil(N/block_k)],
 *                      nonzero = visible block.
 *   causal             0 or 1: also apply j <= i.
 *   tile_ptr           host int[n_layouts * ceil(N/256) + 1] receiving, per
 *                      (layout, 256-row query tile), the offset of its list
 *                      in `entries` (and the total at the end); may be NULL
 *                      together with entries (count only).
 *   entries            host array receiving the lists: key tile index (64
 *                      keys each) in bits 0-23, and in bit 24 + s whether the
 *                      query rows 32s .. 32s+31 of the tile see that key
 *                      tile; ascending key tiles.  NULL: count only.
 *   max_entries        capacity of entries (FA2_ERR_INVALID_ARG if short).
 *   n_entries          (host, non-NULL) receives the number of entries.
 *
 * Returns FA2_OK or a negative fa2_status.
 */
int fa2_sparse_plan(int N, int block_q, int block_k, int n_layouts, const unsigned char* block_mask,
                    int causal, int* tile_ptr, unsigned* entries, int max_entries, int* n_entries);

/*
 * fa2_fwd_sparse -- fa2_fwd_gqa under a block-sparse mask, over the lists
 * fa2_sparse_plan built.
 *
 * Each workgroup streams only its query tile's listed key tiles; a
 * wavefront whose rows do not see a listed tile masks it whole, and the
 * causal mask (if causal) applies inside tiles as in fa2_fwd.  Rows with no
 * visible key get O = 0 and LSE = -inf.
 *
 *   n_layouts          1 (one mask for every head), H (one per query head,
 *                      shared by the batch) or B*H (one per (b, h), index
 *                      b*H + h); else FA2_ERR_INVALID_ARG.  Must match the
 *                      plan.
 *   tile_ptr, entries  DEVICE copies of fa2_sparse_plan's outputs for the
 *                      same N and causal flag (4-byte aligned, read only;
 *                      entries may be NULL when n_entries == 0).  Offsets
 *                      and tile indices are clamped into range, so a plan
 *                      for other sizes cannot make the kernel read or write
 *                      out of bounds, but gives wrong results.
 *   in_dtype           FA2_BF16 only (else FA2_ERR_UNSUPPORTED).
 * All other arguments as fa2_fwd_gqa.  Returns FA2_OK after enqueueing,
 * else a negative fa2_status.
 */
int fa2_fwd_sparse(const void* q, const void* k, const void* v, void* o, float* lse,
                   int B, int H, int H_kv, int N, int d, int causal, float scale,
                   void* stream, int in_dtype, int o_dtype, int n_layouts,
                   const int* tile_ptr, const unsigned* entries, int n_entries);

/*
 * fa2_decode_paged_workspace -- chunk size and workspace of a
 * fa2_decode_paged call.  Host-only; touches no device.
 *
 *   B, H, H_kv, n_q, d, max_context   as for fa2_decode_paged.
 *   split_keys      keys per chunk (a multiple of 64), or 0: the library
 *                   picks the chunk from max_context, B*H_kv and num_units:
 *                   with (H/H_kv)*n_q <= 128 (one wavefront per chunk and
 *                   32 rows of a group), one chunk per wavefront slot (four
 *                   per unit) at the longest context, or four chunks per
 *                   sequence when one chunk's wavefronts alone fill the
 *                   slots; with larger groups about eight workgroups per
 *                   unit at the longest context; at least 256 keys per
 *                   chunk unless the context is shorter.
 *   num_units       compute units of the device (used when split_keys == 0).
 *   split_keys_out, workspace_bytes  (host, non-NULL) receive the chunk
 *                   size and the workspace fa2_decode_paged needs for it.
 * Returns FA2_OK, FA2_ERR_INVALID_ARG or FA2_ERR_UNSUPPORTED (d not 64 or
 * 128, or more than 256 query rows per key/value head: (H/H_kv)*n_q).
 */
int fa2_decode_paged_workspace(int B, int H, int H_kv, int n_q, int d, int max_context, int split_keys,
                               int num_units, int* split_keys_out, size_t* workspace_bytes);

/*
 * fa2_decode_paged -- attention of the newest n_q tokens of each sequence
 * over its keys and values in a paged cache.
 *
 * Sequence b has context_lens[b] keys (its new tokens' own keys included,
 * last); logical key j is stored in physical page page_table[b*max_pages +
 * j/page_size] at slot j % page_size.  New token i (0 <= i < n_q) sits at
 * position context_lens[b] - n_q + i and sees the keys at positions up to
 * its own (causal); a token at a negative position sees none and gets
 * O = 0, LSE = -inf.  Query head h reads key/value head h / (H/H_kv).
 *
 * Source: papermap "FlashAttention-2" explainer, Chapter 03 ("The
 * Downstream Story"): paged-KV decoding is named among the kernels built on
 * FlashAttention-2; Mishra, "Another use of mergeable statistics": the
 * statistics of disjoint key ranges merge exactly, so a long context is
 * cut into chunks processed in parallel and merged.
 *
 * Work: one workgroup per (chunk of split_keys keys, sequence, key/value
 * head) computes the H/H_kv query heads x n_q tokens of the group against
 * its chunk (K and V read once per group) and writes a partial result to
 * the workspace; a second kernel merges each group's chunks into o and lse.
 *
 *   q          device, [B, H, n_q, d] in_dtype.
 *   k_cache, v_cache  device, [n_pages, page_size, H_kv, d] in_dtype.
 *   o          device, [B, H, n_q, d] in o_dtype, fully overwritten.
 *   lse        device fp32 [B, H, n_q], fully overwritten.
 *   page_table device int32 [B, max_pages]; entries are clamped into
 *              [0, n_pages) (a bad entry reads a wrong page, never out of
 *              bounds).  Entries past a sequence's context are not read.
 *   context_lens  device int32 [B]; each is clamped into [0, min(max_context,
 *              max_pages*page_size)].
 *   max_context   >= 1: an upper bound of context_lens (it sizes the grid).
 *   page_size  a multiple of 64 (else FA2_ERR_UNSUPPORTED).
 *   split_keys keys per chunk, a multiple of 64 (from
 *              fa2_decode_paged_workspace).
 *   workspace  device, >= fa2_decode_paged_workspace's bytes for the same
 *              arguments, 16-byte aligned; overwritten.
 *   in_dtype   FA2_BF16 only (else FA2_ERR_UNSUPPORTED); o_dtype FA2_F32 or
 *              FA2_BF16.
 *   (H/H_kv)*n_q <= 256, d 64 or 128 (else FA2_ERR_UNSUPPORTED).
 * Written buffers must not overlap any other buffer.  Returns FA2_OK after
 * enqueueing two kernels on `stream`, else a negative fa2_status.
 */
int fa2_decode_paged(const void* q, const void* k_cache, const void* v_cache, void* o, float* lse,
                     int B, int H, int H_kv, int n_q, int d, float scale,
                     const int* page_table, int max_pages, const int* context_lens, int max_context,
                     int page_size, int n_pages, int split_keys,
                     void* workspace, size_t workspace_bytes, void* stream, int in_dtype, int o_dtype);

/*
 * fa2_decode_paged_noalloc -- fa2_decode_paged without a caller workspace,
 * for callers that cannot allocate device memory (code under HIP graph
 * capture, serving loops that must not call hipMalloc, harnesses that
 * forbid it).  It allocates nothing: the partial results go to a static
 * device buffer of FA2_DECODE_SCRATCH_BYTES that each device the library
 * runs on holds until the process ends (its address is looked up once per
 * device, on the first call with that device current).
 *
 * Arguments, kernels and results are those of fa2_decode_paged with the
 * same split_keys (o and lse are bitwise the same).  A call whose
 * fa2_decode_paged_workspace bytes exceed FA2_DECODE_SCRATCH_BYTES returns
 * FA2_ERR_SCRATCH before any HIP call (use fa2_decode_paged with a
 * workspace, or a larger split_keys).  No part of the scratch needs to
 * start at zero: each call writes every partial it reads.
 *
 * All calls on one device share the scratch: two calls whose kernels
 * overlap in time on the same device (on different streams, or from
 * different host threads without ordering) race and give wrong results.
 * Calls ordered on one stream are safe.
 */
int fa2_decode_paged_noalloc(const void* q, const void* k_cache, const void* v_cache, void* o, float* lse,
                             int B, int H, int H_kv, int n_q, int d, float scale,
                             const int* page_table, int max_pages, const int* context_lens, int max_context,
                             int page_size, int n_pages, int split_keys, void* stream, int in_dtype, int o_dtype);

/*
 * fa2_fp8_pack_workspace -- workspace bytes of fa2_fp8_pack for [B, H, N, .]
 * (B*H*ceil(N/256) floats).  Host-only.  FA2_OK or FA2_ERR_INVALID_ARG.
 */
int fa2_fp8_pack_workspace(int B, int H, int N, size_t* workspace_bytes);

/*
 * fa2_fp8_pack -- rotate and quantize Q (or K) for fa2_fwd_fp8.
 *
 * Each row x (d values) becomes x R with R = diag(signs) H / sqrt(d), H the
 * Sylvester-Hadamard matrix, computed in fp32 in a fixed order: signs, then
 * butterfly stages h = 1, 2, ..., d/2 replacing (a, b) at (i, i + h) of
 * every 2h-block by (a + b, a - b), then one multiply by the fp32 constant
 * 1/sqrt(d).  Each (b, h) block of rotated values is quantized to OCP E4M3
 * (largest finite 448) with scale = amax / 448: codes = E4M3(clamp(x R *
 * (448 / amax), -448, 448)), rounded to nearest even; a block of zeros gets
 * codes 0 and scale 1.
 *
 * Source: Mishra, "FlashAttention-2 and -3: From Algebra to GPU
 * Scheduling", "Low precision changes numerical error": a shared orthogonal
 * mixing transform spreads outliers before quantization and leaves QK^T
 * unchanged in exact arithmetic ((QR)(KR)^T = QK^T); block scaling governs
 * the quantization error.  Use the same signs for Q and K.
 *
 *   x          device bf16 [B, H, N, d] (d 64 or 128, else UNSUPPORTED).
 *   signs      HOST array of d values, each +1 or -1 (else
 *              FA2_ERR_INVALID_ARG); NULL = no rotation (plain per-block
 *              quantization).
 *   codes      device [B, H, N, d] bytes, 16-byte aligned; overwritten.
 *   scales     device fp32 [B, H]; overwritten.
 *   workspace  device, >= fa2_fp8_pack_workspace bytes.
 * Buffers must not overlap.  Returns FA2_OK after enqueueing two kernels on
 * `stream`, else a negative fa2_status.
 */
int fa2_fp8_pack(const void* x, int B, int H, int N, int d, const float* signs, void* codes, float* scales,
                 void* workspace, size_t workspace_bytes, void* stream);

/*
 * fa2_fwd_fp8 -- the forward pass with Q K^T on FP8 matrix cores.
 *
 * q8, k8 are fa2_fp8_pack outputs (E4M3 codes of the rotated Q and K, with
 * q_scale [B, H] and k_scale [B, H_kv]); v is bf16.  The kernel computes
 * S = scale * q_scale * k_scale * (codes_q . codes_k) with E4M3 x E4M3
 * products accumulated in fp32 (v_mfma_scale_f32_32x32x64_f8f6f4), then
 * the same online softmax, bf16 P V product and outputs as fa2_fwd_gqa.
 * Relative to exact attention the result carries the quantization error of
 * Q and K (bounded per score by scale * sum_d (|q_d| e(k_d) + e(q_d) |k_d| +
 * e(q_d) e(k_d)), e(x) = max(2^-4 |x|, 2^-10 * block scale)); relative to
 * exact attention of the dequantized codes it carries only fa2_fwd's
 * rounding.
 *
 *   q8 [B, H, N, d], k8 [B, H_kv, N, d] device bytes, 16-byte aligned.
 *   v [B, H_kv, N, d] device bf16; o, lse, B, H, H_kv, N, d, causal, scale,
 *   stream, o_dtype as for fa2_fwd_gqa.
 * Returns FA2_OK after enqueueing, else a negative fa2_status.
 */
int fa2_fwd_fp8(const void* q8, const float* q_scale, const void* k8, const float* k_scale, const void* v,
                void* o, float* lse, int B, int H, int H_kv, int N, int d, int causal, float scale, void* stream,
                int o_dtype);

/*
 * fa2_plan_t -- the launch geometry fa2_fwd uses (or would use) for a shape,
 * for reporting and tests.  Host-only; touches no device.
 */
typedef struct fa2_plan_t {
  int block_rows;          /* B_r: query rows per workgroup */
  int block_cols;          /* B_c: keys per K/V tile */
  int waves_per_group;     /* wavefronts per workgroup (each owns B_r/waves rows) */
  int query_tiles;         /* ceil(N / B_r): query tiles per (batch, head) */
  long long workgroups;    /* B*H*query_tiles: the grid size */
  long long tile_pairs;    /* (query tile, key tile) pairs the grid executes */
  long long normalisations;/* accumulator divisions: one per query tile */
  double waves_of_groups;  /* workgroups / num_units (0 if num_units == 0) */
  int last_wave_groups;    /* workgroups in the final, partial wave (0 if none/unknown) */
  double flops_executed;   /* matrix-core flops the executed tile pairs cost */
  double flops_credited;   /* 4*B*H*N*N*d, halved when causal */
} fa2_plan_t;

/*
 * fa2_plan -- fill *out with the geometry for a forward call.
 *
 *   block_rows  0 = the library's own tile height for (d, in_dtype);
 *               > 0 = evaluate that tile height instead (analysis only:
 *               fa2_fwd always uses the library's own tiles).
 *   block_cols  0 = the library's own key-tile width; > 0 overrides it.
 *   num_units   number of compute units to express the grid in waves of
 *               workgroups (one resident workgroup per unit); 0 = skip.
 *
 * Saraf, section 2.3: one block per (sequence, head) versus one block per
 * query tile per (sequence, head); section 2.2: one division per query
 * block.  Returns FA2_OK or FA2_ERR_INVALID_ARG / FA2_ERR_UNSUPPORTED under
 * the same size rules as fa2_fwd.
 */
int fa2_plan(int B, int H, int N, int d, int causal, int in_dtype,
             int block_rows, int block_cols, int num_units, fa2_plan_t* out);

/*
 * fa2_clock_probe -- measure the shader clock on the device (a diagnostic
 * for benchmarks, not part of the attention path).
 *
 * Enqueues `workgroups` one-wavefront workgroups on `stream`; each runs a
 * dependent chain of VALU work until the 100 MHz reference counter has
 * advanced by `ticks` (10 ns each), then workgroup g writes to
 * out[3g .. 3g+2] how far the shader cycle counter and the reference
 * counter advanced, and a value that keeps the chain from being optimised
 * away.  The mean clock is 100 MHz * sum(out[3g]) / sum(out[3g+1]).  On a
 * stream of its own, beside other work, a single workgroup measures the
 * clock under that work.
 *
 *   workgroups  1 .. 65536;  ticks  1 .. 10^9 (10 s).
 *   out         device, 8-byte aligned, 3 * workgroups uint64, overwritten.
 * Returns FA2_OK after enqueueing, FA2_ERR_INVALID_ARG, FA2_ERR_NO_DEVICE
 * or FA2_ERR_LAUNCH.
 */
int fa2_clock_probe(int workgroups, unsigned long long ticks, unsigned long long* out, void* stream);

/* fa2_strerror -- static, NUL-terminated description of a status code. */
const char* fa2_strerror(int status);

/* fa2_version -- FA2_VERSION of the built library. */
int fa2_version(void);

#ifdef __cplusplus
}
#endif

#endif /* FA2_H */

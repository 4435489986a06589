/*
 * pgqa.h - paged grouped-query attention hot path for AMD Instinct MI355X (gfx950).
 *
 * C ABI of libpgqa.so.  Every pointer named "device" is a HIP device address on
 * the pool's device; every pointer named "host" is ordinary host memory.  No
 * call allocates device memory except pgqa_pool_create, no call synchronises
 * the device except pgqa_pool_check_errors, and no call copies device data to
 * the host.  Work is enqueued on the caller's HIP stream (passed as void*,
 * NULL = the null stream) and the call returns.
 *
 * Sources (web pages, cited by title and section):
 *   [P1] "perf: Qwen3 offline inference - hybrid attention backend, fused
 *        rms_norm_rope, chunked prefill + prompt-lookup spec decoding"
 *        (InfiniLM pull request 585).
 *   [P2] "Ascend qwen3.6 optimizate baseline" (vllm-plugin-FL pull request 301).
 *   [P3] "[2026春季][T2-1-3]" (InfiniLM issue 498).
 *
 * Shapes: D (head_dim) is 128.  Hq query heads share Hkv key/value heads in
 * contiguous groups of r = Hq / Hkv: query head h reads kv head h / r.
 * bf16 tensors are IEEE bfloat16, rounded to nearest-even when produced.
 *
 * Error behaviour: every call returns a pgqa_status; nothing throws across the
 * ABI; pgqa_last_error() gives a thread-local message for the last failure.
 * Host-visible argument errors are detected before anything is enqueued.
 * Metadata that lives in device memory (positions, block ids, context lengths)
 * is range-checked by the kernels themselves: a bad entry never causes an
 * out-of-bounds access; the affected row is skipped (cache write) or produces a
 * zero output row (attention) and a sticky bit is set in the pool's device
 * error word, read with pgqa_pool_check_errors().
 */
#ifndef PGQA_H
#define PGQA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  PGQA_OK = 0,
  PGQA_ERR_INVALID_ARG = 1,   /* a host argument is out of range or inconsistent */
  PGQA_ERR_UNSUPPORTED = 2,   /* a shape this library does not implement (never a silent fallback) */
  PGQA_ERR_POINTER_KIND = 3,  /* a pointer is not device memory of the pool's device */
  PGQA_ERR_WORKSPACE = 4,     /* workspace missing or smaller than required */
  PGQA_ERR_HIP = 5,           /* the HIP runtime reported an error */
  PGQA_ERR_DEVICE = 6         /* pgqa_pool_check_errors found kernel-detected metadata errors */
} pgqa_status;

/* Bits of the pool's sticky device error word. */
#define PGQA_DEVERR_SEQ_ID   0x1u  /* a seq_id outside [0, num_seqs) */
#define PGQA_DEVERR_POSITION 0x2u  /* a position < 0 or past the end of its block-table row */
#define PGQA_DEVERR_BLOCK_ID 0x4u  /* a block-table entry outside [0, num_blocks) where it is read */
#define PGQA_DEVERR_CONTEXT  0x8u  /* a context length < 0, past its table row, or above max_context_len */
#define PGQA_DEVERR_QUERY    0x10u /* query_start_loc not ascending or not ending at total_q, or a chunk longer than
                                      its context or max_q_len */

/*
 * Paged KV pool configuration.  [P3] Summary and file list: the cache is
 * configured by (num_blocks, block_size, max_batch_size), and the two-argument
 * form (no batch bound) stays valid, here as max_batch_size = 0.
 */
typedef struct {
  int32_t num_blocks;      /* physical blocks in the pool, >= 1 */
  int32_t block_size;      /* tokens per block: 16, 32, 64, 128 or 256 */
  int32_t num_kv_heads;    /* Hkv, >= 1 */
  int32_t head_dim;        /* D: 128 only (else PGQA_ERR_UNSUPPORTED) */
  int32_t max_batch_size;  /* upper bound on batch / segments per call; 0 = no bound */
} pgqa_pool_config;

typedef struct pgqa_pool pgqa_pool;  /* opaque */

/* Bytes of device memory the caller must provide for the pool's K/V storage. */
size_t pgqa_pool_bytes(const pgqa_pool_config* cfg);

/*
 * Create a pool over caller-owned device storage `kv_storage` (device, at
 * least pgqa_pool_bytes(cfg) bytes, 256-byte aligned) on the current HIP
 * device.  The storage layout is owned by the library and reported by
 * pgqa_pool_layout; callers never pass cache strides (the layout mismatch of
 * [P2] section 2.3 cannot arise).  The pool allocates only a small device
 * error word.  The storage is not cleared.
 */
pgqa_status pgqa_pool_create(const pgqa_pool_config* cfg, void* kv_storage, pgqa_pool** out);

/* Release the pool handle and its error word; the K/V storage stays the caller's. */
pgqa_status pgqa_pool_destroy(pgqa_pool* pool);

/*
 * Element strides (and element offsets from kv_storage) of the logical views
 * K[num_blocks][block_size][num_kv_heads][head_dim] (k_strides ordered block,
 * slot, head, dim) and V[num_blocks][block_size / 16][16][num_kv_heads][head_dim]
 * (v_strides ordered block, slot / 16, slot % 16, head, dim: slot = 16 * piece
 * + j), so that a caller can build strided views of the cache.  Within one
 * (block, kv head) the library stores K row-major [slot][dim] followed by V
 * transposed in 16-slot pieces [slot / 16][dim][slot % 16], so that 16
 * consecutive keys of one dim are 32 contiguous bytes and the V of 16
 * consecutive keys is one contiguous 4 KiB run at every block size.
 */
pgqa_status pgqa_pool_layout(const pgqa_pool* pool, int64_t k_strides[4], int64_t* k_offset,
                             int64_t v_strides[5], int64_t* v_offset);

/*
 * Synchronise `stream`, read and clear the pool's sticky device error word.
 * *flags (host) receives the PGQA_DEVERR_* bits.  Returns PGQA_ERR_DEVICE if any
 * bit was set, PGQA_OK otherwise.
 */
pgqa_status pgqa_pool_check_errors(pgqa_pool* pool, void* stream, uint32_t* flags);

/*
 * a1 + a2 + a3: per-head RMSNorm of q and k, neox rotary of the normed q and k,
 * and the write of k' and v into the paged cache, in one launch.
 * [P1] Summary item 2 (per-head RMSNorm fused with RoPE, full rotary) and item 1
 * (block-table paged cache).
 *
 *   q  device bf16 [num_tokens][num_q_heads][128], token stride q_row_stride elements
 *   k  device bf16 [num_tokens][Hkv][128], token stride k_row_stride
 *   v  device bf16 [num_tokens][Hkv][128], token stride v_row_stride
 *      (strides allow q/k/v to be views of one fused projection output; each
 *       stride is >= heads*128 and a multiple of 8, the head/dim axes are dense,
 *       and q, k, v are 16-byte aligned)
 *   q_norm_weight, k_norm_weight  device bf16 [128], shared by all heads, 16-byte aligned
 *   positions  device int32 [num_tokens]: absolute 0-based position of each token
 *   seq_ids    device int32 [num_tokens]: row of block_tables holding its sequence
 *   block_tables device int32 [num_seqs][bt_stride]
 *   eps        RMSNorm epsilon (inside the square root), >= 0
 *   rope_theta rotary base (inverse frequency theta^(-2i/128)), > 0
 *   q_out      device bf16 [num_tokens][num_q_heads][128], dense, 16-byte aligned
 *   (num_q_heads + 2 * Hkv <= 128)
 *
 * For token t: y = x / sqrt(mean(x^2) + eps) * w per head row, then each pair
 * (i, i+64) is rotated by positions[t] * theta^(-2i/128); k' and v go to slot
 * positions[t] % block_size of block block_tables[seq_ids[t]][positions[t] / block_size].
 * Tokens may belong to any mix of sequences; two tokens must not share a slot.
 * num_tokens = 0 is a no-op.
 */
pgqa_status pgqa_rms_norm_rope_cache_write(
    pgqa_pool* pool,
    const void* q, int64_t q_row_stride,
    const void* k, int64_t k_row_stride,
    const void* v, int64_t v_row_stride,
    const void* q_norm_weight, const void* k_norm_weight,
    const int32_t* positions, const int32_t* seq_ids,
    const int32_t* block_tables, int32_t bt_stride, int32_t num_seqs,
    int32_t num_tokens, int32_t num_q_heads,
    float eps, double rope_theta,
    void* q_out, void* stream);

/*
 * Split plan of a decode call: keys of each (sequence, kv head) are cut into
 * splits of split_tokens keys, each processed by one workgroup, then merged by
 * a log-sum-exp combine.  pgqa_plan_decode fills it from host-known sizes only
 * ([P1] Summary item 3: routing decisions are host-side, with no device sync).
 */
typedef struct {
  int32_t split_tokens;     /* keys per split: a multiple of max(block_size, 64), <= 1024 * waves_per_split */
  int32_t max_splits;       /* ceil(max_context_len / split_tokens) */
  int32_t waves_per_split;  /* 64-lane waves per workgroup: 1, 2, 4 or 8 */
  int32_t load_hint;        /* K/V loads: 0 library default (streaming in the dot-product kernel, cached in
                               the matrix-core kernel), 1 cached, 2 streaming (non-temporal) */
  int32_t kernel;           /* split kernel: 0 library default (matrix-core when 8 or more query heads share
                               a kv head, else dot-product), 1 dot-product (VALU) kernel, 2 matrix-core
                               (MFMA) kernel.  Both give the same results up to rounding. */
  const int32_t* host_context_lens;
                            /* optional HOST copy of context_lens ([batch]), NULL if not known.  [P1] Summary
                               item 3: the host knows every sequence's length in a serving loop.  With it the
                               call orders the (sequence, kv head) units (at most 1024) longest first, dealt
                               so that workgroups sharing a CU pair long units with short ones.  Results are
                               bit-identical with and without it; a stale hint only costs balance. */
} pgqa_decode_plan;

/* Host-only: the plan pgqa_paged_decode_attention uses when given plan = NULL,
 * for a device with num_cus compute units. */
pgqa_status pgqa_plan_decode(int32_t num_cus, int32_t block_size, int32_t batch, int32_t num_kv_heads,
                             int32_t num_q_heads, int32_t max_context_len, pgqa_decode_plan* out);

/* Device workspace bytes a decode call with this plan needs (plan = NULL: the default plan). */
size_t pgqa_decode_workspace_bytes(const pgqa_pool* pool, int32_t batch, int32_t num_q_heads,
                                   int32_t max_context_len, const pgqa_decode_plan* plan);

/*
 * a4 + a5: paged split-KV GQA decode attention with log-sum-exp combine.
 * [P1] Summary item 1 (self-written paged split-KV kernel for pure decode).
 *
 *   q            device bf16 [batch][num_q_heads][128] (the q_out of the cache write)
 *   context_lens device int32 [batch]: keys attended by each sequence (its newly
 *                written token included); 0 gives a zero output row
 *   block_tables device int32 [batch][bt_stride]
 *   max_context_len host hint >= every context_lens entry (sizes the split grid)
 *   scale        softmax scale applied to q.k (1/sqrt(128) for Qwen3)
 *   plan         host, optional (NULL = pgqa_plan_decode for this device)
 *   workspace    device scratch of >= pgqa_decode_workspace_bytes(...) bytes for
 *                the split partials (0 bytes, and NULL allowed, when the plan
 *                has one split); no initial contents are needed.  Calls that
 *                share a workspace must be ordered on one stream.
 *   out          device bf16 [batch][num_q_heads][128]
 *
 * out[b][h] = sum_j softmax_j(scale * q[b][h] . K_j) V_j over keys j < n_b of kv
 * head h / r, key j at slot j % block_size of block block_tables[b][j / block_size].
 * Outputs are deterministic for a given plan (fixed combine order).  With more
 * than one split the call enqueues two kernels (splits, then the combine).
 */
pgqa_status pgqa_paged_decode_attention(
    pgqa_pool* pool,
    const void* q, const int32_t* context_lens,
    const int32_t* block_tables, int32_t bt_stride,
    int32_t batch, int32_t num_q_heads, int32_t max_context_len,
    float scale, const pgqa_decode_plan* plan,
    void* workspace, size_t workspace_bytes,
    void* out, void* stream);

/*
 * a1..a5 in one launch for a pure decode batch: each sequence b has one new
 * token at position context_lens[b] - 1 (its cached tokens come first, [P1]
 * Summary item 1's decode route).  The token's raw q, k, v rows are normed
 * (per-head RMSNorm, weights q_norm_weight / k_norm_weight, eps) and rotated
 * (neox, rope_theta) exactly as pgqa_rms_norm_rope_cache_write does (same device
 * code, identical bits), k and v are written into the token's cache slot, and
 * paged decode attention over keys 0 .. context_lens[b] - 1 follows, as in
 * pgqa_paged_decode_attention with the same plan and workspace rules.  The
 * separate write launch and its round trip of q through memory disappear.
 *
 *   q, k, v       device bf16 rows per sequence: [batch][row stride], heads
 *                 contiguous from the row start ([Hq][128] / [Hkv][128])
 *   q_out         device bf16 [batch][Hq][128] for the normed, rotated q, or NULL
 *   out           device bf16 [batch][Hq][128]
 *
 * A sequence with context_lens[b] == 0 has no new token: nothing is written
 * and its output rows are zero.  Metadata errors behave as in the two calls it
 * replaces (flags in the pool's error word, no out-of-bounds access).
 */
pgqa_status pgqa_decode_step(
    pgqa_pool* pool,
    const void* q, int64_t q_row_stride,
    const void* k, int64_t k_row_stride,
    const void* v, int64_t v_row_stride,
    const void* q_norm_weight, const void* k_norm_weight,
    float eps, double rope_theta,
    const int32_t* context_lens, const int32_t* block_tables, int32_t bt_stride,
    int32_t batch, int32_t num_q_heads, int32_t max_context_len,
    float scale, const pgqa_decode_plan* plan,
    void* workspace, size_t workspace_bytes,
    void* q_out, void* out, void* stream);

/*
 * The fused decode step above for callers that cannot allocate device memory
 * or own a workspace: code recorded under HIP graph capture, tight serving
 * loops, harnesses that forbid allocation.  Arguments, results and errors are
 * those of pgqa_decode_step (same kernels, bit-identical outputs for the same
 * plan), without the workspace arguments.
 *
 * The split partials go to a fixed device array of PGQA_NOALLOC_SCRATCH_BYTES
 * that is part of the library's code object: every GPU that loads the library
 * holds one copy until the process ends.  The call allocates and frees
 * nothing; on its first call on a device it looks up that device's copy once.
 * The partials need no initial contents, so nothing is cleared.
 *
 * A plan whose partials (pgqa_decode_workspace_bytes) exceed the array returns
 * PGQA_ERR_WORKSPACE before anything is enqueued.  The library's default plans
 * stay far below it (a batch-1 call at 32768 keys needs about 0.2 MiB).
 * All calls on one GPU share its array: two calls whose kernels may overlap on
 * one GPU (different streams, or graphs replayed concurrently) race on it and
 * give undefined results; order them on one stream.
 */
#define PGQA_NOALLOC_SCRATCH_BYTES ((size_t)8 << 20)

pgqa_status pgqa_decode_step_noalloc(
    pgqa_pool* pool,
    const void* q, int64_t q_row_stride,
    const void* k, int64_t k_row_stride,
    const void* v, int64_t v_row_stride,
    const void* q_norm_weight, const void* k_norm_weight,
    float eps, double rope_theta,
    const int32_t* context_lens, const int32_t* block_tables, int32_t bt_stride,
    int32_t batch, int32_t num_q_heads, int32_t max_context_len,
    float scale, const pgqa_decode_plan* plan,
    void* q_out, void* out, void* stream);

/*
 * Split plan of a chunk call.  Rows are (token, query head) pairs of one kv
 * head.  On the chunk kernels (kernel 0 or 1), a segment with more than 32 rows
 * per kv head (a prefill slice) is cut into groups of 128 rows that read their
 * keys in splits of split_tokens keys; a segment with at most 32 rows per kv
 * head (verify rows, single tokens) reads its keys in splits of
 * short_split_tokens keys.  A call whose segments all have at most 16 rows per
 * kv head can instead run on the matrix-core decode kernel (kernel 2).  Rows
 * with several splits are merged by a log-sum-exp combine.
 */
typedef struct {
  int32_t split_tokens;        /* a multiple of 32, at most 4096 */
  int32_t max_splits;          /* >= ceil(max_context_len / min(split_tokens, short_split_tokens)) */
  int32_t short_split_tokens;  /* a multiple of 32, at most 4096; 0 = split_tokens */
  int32_t kernel;              /* 0 or 1: the chunk kernels (wide / short items, combine);
                                  2: the matrix-core decode kernel with the segment's (token, head) rows
                                  as its 16 MFMA columns, for calls with max_q_len x group <= 16 (verify
                                  rows, single tokens): split_tokens keys per split, a multiple of
                                  max(block_size, 64), at most 4096; short_split_tokens unused.
                                  pgqa_plan_chunk picks 2 whenever a call fits. */
} pgqa_chunk_plan;

/* Host-only: the plan pgqa_paged_chunk_attention uses when given plan = NULL. */
pgqa_status pgqa_plan_chunk(int32_t num_cus, int32_t block_size, int32_t num_segments, int32_t total_q,
                            int32_t num_kv_heads, int32_t num_q_heads, int32_t max_q_len,
                            int32_t max_context_len, pgqa_chunk_plan* out);

/* Device workspace bytes a chunk call with this plan needs (plan = NULL: the default plan). */
size_t pgqa_chunk_workspace_bytes(const pgqa_pool* pool, int32_t num_segments, int32_t total_q,
                                  int32_t num_q_heads, int32_t max_q_len, int32_t max_context_len,
                                  const pgqa_chunk_plan* plan);

/*
 * a6: causal attention of short query chunks over the paged cache: chunked-
 * prefill slices and b x (k+1) speculative-verify rows.  [P1] Summary items 1
 * (varlen path over the same paged cache) and 4 (chunked prefill, fixed
 * b x (k+1) verify shape).
 *
 *   q               device bf16 [total_q][num_q_heads][128]
 *   query_start_loc device int32 [num_segments + 1], ascending, [0] = 0,
 *                   [num_segments] = total_q (cu_seqlens convention, [P2] section 2.1)
 *   context_lens    device int32 [num_segments]: keys of each segment, its own
 *                   q_len tokens included (they must already be in the cache)
 *   block_tables    device int32 [num_segments][bt_stride]
 *   max_q_len, max_context_len  host hints >= the device values
 *   plan            host, optional (NULL = pgqa_plan_chunk for this device)
 *   workspace       device scratch of >= pgqa_chunk_workspace_bytes(...) bytes for
 *                   the split partials (no initial contents needed; NULL when that
 *                   is 0)
 *   out             device bf16 [total_q][num_q_heads][128]
 *
 * Query i of segment s (q_len_s = qsl[s+1] - qsl[s], n_s = context_lens[s]) sits
 * at position n_s - q_len_s + i and attends to keys 0 .. that position.  A
 * segment whose metadata is inconsistent gets zero output rows and sets
 * PGQA_DEVERR_QUERY or PGQA_DEVERR_CONTEXT.  A block id outside the pool sets
 * PGQA_DEVERR_BLOCK_ID; the rows that read it are then unspecified (the key is
 * read as zeros, never out of bounds).  On the chunk kernels the call enqueues
 * the attention kernels for long and short segments (each workgroup derives its
 * own work item from the device metadata); with plan kernel 2, the matrix-core
 * decode kernel over (kv head, segment, split).  With more than one split, the
 * combine follows.
 */
pgqa_status pgqa_paged_chunk_attention(
    pgqa_pool* pool,
    const void* q, const int32_t* query_start_loc, const int32_t* context_lens,
    const int32_t* block_tables, int32_t bt_stride,
    int32_t num_segments, int32_t total_q, int32_t num_q_heads,
    int32_t max_q_len, int32_t max_context_len,
    float scale, const pgqa_chunk_plan* plan,
    void* workspace, size_t workspace_bytes,
    void* out, void* stream);

/*
 * One attention launch for a whole mixed serving step: decode rows, chunked-
 * prefill slices and b x (k+1) speculative-verify rows of one call, from a work
 * list built on the host.  [P1] Summary items 1 (decode and prefill routed on
 * the host over one paged cache), 3 (routing decided on the host, no device
 * synchronisation) and 4 (chunked prefill and the fixed b x (k+1) verify shape
 * in one forward).
 *
 * Semantics are those of pgqa_paged_chunk_attention: segment s owns query rows
 * query_start_loc[s] .. query_start_loc[s+1]-1 and context_lens[s] keys (its
 * own tokens included, already in the cache); query i sits at position
 * n_s - q_len_s + i and attends to keys 0 .. that position.  A decode row is a
 * segment of one token.
 *
 * pgqa_plan_mixed (host only) reads HOST copies of query_start_loc
 * [num_segments + 1] and context_lens [num_segments] (the step planner has
 * them) and writes the work list to `items` (host, PGQA_MIXED_ITEM_INTS int32
 * per item, plan->num_items attention items then plan->num_combine combine
 * items; item_capacity counts items).  With items = NULL it only fills *out,
 * so a caller can size its buffer.  Segments with more than 16 query rows per
 * kv head (q_len x group > 16) become wide items (128 rows over one key split of
 * split_wide keys, matrix cores), the others query-column items (the segment's
 * rows as MFMA columns over one split of split_columns keys).  0 for a split
 * lets the planner choose: it estimates the wide items' matrix-core time and
 * the column items' K/V bytes and gives each kind a share of the CUs' two
 * workgroup slots in proportion (rates measured on MI355X).  The attention
 * items alternate between the two kinds in runs of num_cus.  Returns
 * PGQA_ERR_INVALID_ARG for inconsistent host metadata or a buffer that is too
 * small.
 *
 * The caller copies the items to device memory (with its other per-step
 * metadata) and passes them and the plan to pgqa_paged_mixed_attention, which
 * enqueues one attention kernel (plan->num_items workgroups) and, when some row
 * has several splits, one combine kernel.  The workspace (device, caller-owned)
 * holds >= pgqa_mixed_workspace_bytes bytes of split partials (no initial
 * contents needed; 0 bytes when plan->max_splits is 1).
 *
 * Every item carries the host's offset, length and key count of its segment;
 * the kernels compare them with the device metadata.  A mismatch, or metadata
 * that fails the chunk call's checks, sets PGQA_DEVERR_QUERY (or
 * PGQA_DEVERR_CONTEXT) and zeroes the output rows the item's own offsets
 * address (inside total_q; with wrong offsets these may be rows of another
 * segment): once the flag is set, treat the call's whole output as invalid.
 * Items must come from pgqa_plan_mixed for the same metadata: rows that no item
 * covers are not written.
 */
#define PGQA_MIXED_ITEM_INTS 8

typedef struct {
  int32_t split_wide;     /* keys per split of wide items: a multiple of 32, at most 4096 */
  int32_t split_columns;  /* keys per split of query-column items: a multiple of max(64, block_size), <= 4096 */
  int32_t max_splits;     /* partial slots per query row (1: no partials, no combine) */
  int32_t num_items;      /* attention work items: workgroups of the attention launch */
  int32_t num_combine;    /* combine items that follow them in the list */
} pgqa_mixed_plan;

pgqa_status pgqa_plan_mixed(int32_t num_cus, int32_t block_size, int32_t num_kv_heads, int32_t num_q_heads,
                            int32_t num_segments, const int32_t* query_start_loc, const int32_t* context_lens,
                            int32_t split_wide, int32_t split_columns, int32_t* items, int64_t item_capacity,
                            pgqa_mixed_plan* out);

/* Device workspace bytes of a mixed call with this plan. */
size_t pgqa_mixed_workspace_bytes(const pgqa_mixed_plan* plan, int32_t total_q, int32_t num_q_heads);

pgqa_status pgqa_paged_mixed_attention(
    pgqa_pool* pool,
    const void* q, const int32_t* query_start_loc, const int32_t* context_lens,
    const int32_t* block_tables, int32_t bt_stride,
    int32_t num_segments, int32_t total_q, int32_t num_q_heads,
    int32_t max_q_len, int32_t max_context_len,
    float scale, const pgqa_mixed_plan* plan, const int32_t* items,
    void* workspace, size_t workspace_bytes,
    void* out, void* stream);

/*
 * Measurement helper, not part of the attention path: a plain streaming read of
 * `bytes` bytes at src (device, 16-byte aligned, bytes a multiple of 16) with
 * 16-byte non-temporal loads in a grid-stride loop, two per thread in flight.
 * Each of the grid * 256 threads writes the XOR of the 32-bit words it read to
 * sink (device, >= grid * 256 * 4 bytes = sink_bytes), so the XOR of all sink
 * words is the XOR of all words of the buffer.  grid: 256-thread workgroups,
 * 1 .. 65535, or 0 for three per CU of the current device.  Its rate is the
 * achievable HBM read bandwidth of one launch of that size, the reference for
 * the decode kernels' bandwidth.  Asynchronous on `stream` (a hipStream_t, NULL
 * = default stream); no allocation.  PGQA_ERR_INVALID_ARG / POINTER_KIND for bad
 * arguments.
 */
pgqa_status pgqa_stream_read(const void* src, size_t bytes, void* sink, size_t sink_bytes, int32_t grid,
                             void* stream);

/* Static description of a status code. */
const char* pgqa_status_string(pgqa_status s);

/* Thread-local detail message of the last failing call on this thread ("" if none). */
const char* pgqa_last_error(void);

/* Library version, "major.minor.patch". */
const char* pgqa_version(void);

#ifdef __cplusplus
}
#endif

#endif /* PGQA_H */

/*
 * pgqa_sched.h - host producers of the chunk-attention work (C ABI of libpgqa.so).
 *
 * Page "perf: Qwen3 offline inference - hybrid attention backend, fused
 * rms_norm_rope, chunked prefill + prompt-lookup spec decoding" ([P1]), Summary
 * item 4: chunked prefill and prompt-lookup speculative decoding live in a host
 * scheduling layer; speculation and chunked prefill share one step, and
 * verification is one forward pass of a fixed b x (k+1) shape.  Its results
 * (the decode-stall workload: 8 decode streams and a 6.5k-token prompt injected
 * mid-run) show that feeding a long prompt in chunks cuts the worst inter-token
 * stall of the running streams.
 *
 * Everything here is host code on host memory: it never touches the device.
 * The planner's outputs (query_start_loc, context_lens, token positions and
 * sequence ids, block tables) are the metadata of one pgqa_rms_norm_rope_cache_write
 * call and one pgqa_paged_chunk_attention call (or pgqa_paged_decode_attention
 * when every segment is a single decode token); the caller copies them to the
 * device.  Errors: pgqa_status codes with pgqa_last_error() for the message;
 * the int32 returning functions return -1 on bad arguments.
 */
#ifndef PGQA_SCHED_H
#define PGQA_SCHED_H

#include <stdint.h>

#include "pgqa.h"

#ifdef __cplusplus
extern "C" {
#endif

/*
 * Prompt lookup ([P1] Summary item 4, k draft tokens).  Among the trailing
 * n-grams of tokens[0 .. num_tokens) with n from max_ngram down to min_ngram,
 * the longest one that also occurs earlier (ending before the last token) is
 * taken at its most recent earlier occurrence, and the up to k tokens that
 * followed that occurrence are the draft.  Writes them to draft (host, >= k
 * entries) and returns their count (0 when no n-gram recurs), or -1 on bad
 * arguments (num_tokens < 0, min_ngram < 1, max_ngram < min_ngram, k < 0, or a
 * NULL array that must be read or written).
 */
int32_t pgqa_prompt_lookup(const int32_t* tokens, int32_t num_tokens, int32_t min_ngram, int32_t max_ngram,
                           int32_t k, int32_t* draft);

/*
 * Greedy acceptance of a verified draft ([P1] Summary item 4; greedy output must
 * equal plain decoding token for token).  target[i] (i = 0 .. num_draft) is the
 * target model's greedy token after the context and draft[0 .. i).  The longest
 * prefix of draft that agrees with target is accepted, followed by target at the
 * first disagreement (or target[num_draft] when all agree).  Writes those
 * accepted + 1 tokens to out (host, >= num_draft + 1 entries) and returns
 * accepted + 1, or -1 on bad arguments.
 */
int32_t pgqa_accept_greedy(const int32_t* draft, int32_t num_draft, const int32_t* target, int32_t* out);

/* Step planner configuration. */
typedef struct {
  int32_t token_budget;        /* query tokens per step, all segments together (>= 1) */
  int32_t max_segments;        /* segments per step (>= 1) */
  int32_t chunked_prefill;     /* 1: a prompt may be fed over several steps; 0: whole */
  int32_t block_size;          /* cache block size (tokens per block, >= 1; the pools take 16 .. 256) */
  int32_t max_blocks_per_seq;  /* width of a block-table row */
} pgqa_sched_config;

/* Per-sequence state, owned by the caller; the planner only reads it (and
 * num_blocks, which it advances as it hands out cache blocks). */
typedef struct {
  int32_t cached;       /* tokens whose K/V are already in the cache */
  int32_t prompt_left;  /* prompt tokens still to prefill; 0 = the sequence decodes */
  int32_t num_draft;    /* decoding sequences: draft tokens to verify this step (0 = plain decode) */
  int32_t num_blocks;   /* cache blocks held: the first num_blocks entries of its block-table row */
} pgqa_sched_seq;

#define PGQA_SEG_DECODE  0  /* one new token (q_len 1) */
#define PGQA_SEG_VERIFY  1  /* the last token and num_draft drafts (q_len 1 + num_draft) */
#define PGQA_SEG_PREFILL 2  /* a chunk of the prompt */

typedef struct {
  int32_t seq;          /* index into the sequence array; also its block-table row */
  int32_t kind;         /* PGQA_SEG_* */
  int32_t q_len;        /* query tokens of the segment */
  int32_t context_len;  /* keys once this step's tokens are written (cached + q_len) */
} pgqa_sched_segment;

/*
 * Plans one step over seqs[0 .. num_seqs), in the sequences' (arrival) order:
 *   1. every decoding sequence gets a segment while the budget and the segment
 *      limit allow: a decode row (q_len 1), or a verify row (q_len 1 + num_draft)
 *      when it has drafts; decode streams are served before any prefill, so a
 *      long prompt never stalls them;
 *   2. the budget left goes to prefilling sequences in order: with
 *      chunked_prefill each takes min(prompt_left, budget left) tokens; without
 *      it a prompt runs whole if it fits the budget left, and otherwise waits,
 *      unless the step has no prefill segment yet, in which case it runs whole
 *      past the budget (the long step that stalls the decode streams, which
 *      chunking avoids).  A decoding sequence whose verify row does not fit the
 *      budget left, or cannot get its cache blocks, runs as a plain decode row
 *      (kind PGQA_SEG_DECODE).
 * A segment's new tokens sit at positions cached .. cached + q_len - 1 of its
 * sequence; the cache blocks they need are popped from the free-list stack
 * free_list[0 .. *free_count) (top = last entry; NULL when empty) into row `seq` of block_tables
 * ([num_seqs][max_blocks_per_seq], host); a segment whose blocks cannot be had
 * is left out of the step.  Outputs (host arrays):
 *   segs [max_segments], query_start_loc [max_segments + 1] (cu_seqlens style),
 *   context_lens [max_segments], and per query token, in segment order,
 *   token_pos and token_seq [token_capacity]; *num_segments and *num_tokens.
 * Returns PGQA_ERR_INVALID_ARG for bad arguments, a sequence that would outgrow
 * its block-table row, or a step needing more than token_capacity tokens.
 */
pgqa_status pgqa_sched_plan_step(const pgqa_sched_config* cfg, pgqa_sched_seq* seqs, int32_t num_seqs,
                                 int32_t* block_tables, int32_t* free_list, int32_t* free_count,
                                 pgqa_sched_segment* segs, int32_t* query_start_loc, int32_t* context_lens,
                                 int32_t* token_pos, int32_t* token_seq, int32_t token_capacity,
                                 int32_t* num_segments, int32_t* num_tokens);

/*
 * Applies a planned step's outcome: a prefill chunk moves q_len tokens from
 * prompt_left to cached; a decode row adds 1 to cached; a verify row adds
 * accepted[i] + 1 (accepted: host [num_segments], drafts accepted by segment i;
 * entries of other kinds are ignored, and accepted may be NULL when the step
 * has no verify row).  The cache slots of rejected drafts are simply reused by
 * later tokens.  num_draft of every planned sequence is reset to 0.
 */
pgqa_status pgqa_sched_commit(pgqa_sched_seq* seqs, int32_t num_seqs, const pgqa_sched_segment* segs,
                              int32_t num_segments, const int32_t* accepted);

/*
 * A finished sequence hands its cache blocks back: they are pushed onto the
 * free-list stack (capacity free_capacity entries) and its state is zeroed.
 */
pgqa_status pgqa_sched_release(const pgqa_sched_config* cfg, pgqa_sched_seq* seqs, int32_t num_seqs, int32_t seq,
                               int32_t* block_tables, int32_t* free_list, int32_t* free_count,
                               int32_t free_capacity);

#ifdef __cplusplus
}
#endif

#endif /* PGQA_SCHED_H */

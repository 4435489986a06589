// Host producers of the chunk-attention work: prompt-lookup drafts, greedy
// acceptance, and the token-budget step planner of chunked prefill.
//
// Page "perf: Qwen3 offline inference - hybrid attention backend, fused
// rms_norm_rope, chunked prefill + prompt-lookup spec decoding", Summary item 4
// (a host scheduling layer: chunked prefill, prompt-lookup speculation with k
// drafts, verification as one forward pass of b x (k+1) tokens) and its
// decode-stall results (a long prompt fed in chunks no longer stalls the
// running decode streams).  Plain host code: no device access.
#include <cstring>

#include "../../include/pgqa_sched.h"
#include "errors.hpp"

using namespace pgqa;

namespace {

// Most recent start p < n - len of tokens[p .. p + len) == tokens[n - len .. n), or -1.
int32_t last_earlier_match(const int32_t* t, int32_t n, int32_t len) {
  const int32_t* suffix = t + n - len;
  for (int32_t p = n - len - 1; p >= 0; --p)
    if (std::memcmp(t + p, suffix, sizeof(int32_t) * size_t(len)) == 0) return p;
  return -1;
}

}  // namespace

extern "C" {

int32_t pgqa_prompt_lookup(const int32_t* tokens, int32_t num_tokens, int32_t min_ngram, int32_t max_ngram,
                           int32_t k, int32_t* draft) {
  clear_error();
  if (num_tokens < 0 || min_ngram < 1 || max_ngram < min_ngram || k < 0 || (num_tokens > 0 && !tokens) ||
      (k > 0 && !draft)) {
    fail(PGQA_ERR_INVALID_ARG, "prompt lookup: bad arguments");
    return -1;
  }
  if (k == 0) return 0;
  for (int32_t len = max_ngram < num_tokens - 1 ? max_ngram : num_tokens - 1; len >= min_ngram; --len) {
    const int32_t p = last_earlier_match(tokens, num_tokens, len);
    if (p < 0) continue;
    int32_t cnt = num_tokens - (p + len);
    if (cnt > k) cnt = k;
    std::memcpy(draft, tokens + p + len, sizeof(int32_t) * size_t(cnt));
    return cnt;
  }
  return 0;
}

int32_t pgqa_accept_greedy(const int32_t* draft, int32_t num_draft, const int32_t* target, int32_t* out) {
  clear_error();
  if (num_draft < 0 || !target || !out || (num_draft > 0 && !draft)) {
    fail(PGQA_ERR_INVALID_ARG, "greedy acceptance: bad arguments");
    return -1;
  }
  int32_t a = 0;
  while (a < num_draft && draft[a] == target[a]) {
    out[a] = draft[a];
    ++a;
  }
  out[a] = target[a];
  return a + 1;
}

pgqa_status pgqa_sched_plan_step(const pgqa_sched_config* cfg, pgqa_sched_seq* seqs, int32_t num_seqs,
                                 int32_t* block_tables, int32_t* free_list, int32_t* free_count,
                                 pgqa_sched_segment* segs, int32_t* query_start_loc, int32_t* context_lens,
                                 int32_t* token_pos, int32_t* token_seq, int32_t token_capacity,
                                 int32_t* num_segments, int32_t* num_tokens) {
  clear_error();
  if (!cfg || cfg->token_budget < 1 || cfg->max_segments < 1 || cfg->block_size < 1 || cfg->max_blocks_per_seq < 1)
    return fail(PGQA_ERR_INVALID_ARG, "bad step planner configuration");
  if (num_seqs < 0 || (num_seqs > 0 && (!seqs || !block_tables)) || !free_count || *free_count < 0 ||
      (*free_count > 0 && !free_list) ||
      !segs || !query_start_loc || !context_lens || token_capacity < 0 || (token_capacity > 0 && (!token_pos ||
      !token_seq)) || !num_segments || !num_tokens)
    return fail(PGQA_ERR_INVALID_ARG, "step planner: bad arguments");
  for (int32_t i = 0; i < num_seqs; ++i) {
    const pgqa_sched_seq& q = seqs[i];
    if (q.cached < 0 || q.prompt_left < 0 || q.num_draft < 0 || q.num_blocks < 0 ||
        q.num_blocks > cfg->max_blocks_per_seq)
      return fail(PGQA_ERR_INVALID_ARG, "sequence %d: bad state", i);
  }
  const int32_t bs = cfg->block_size;
  int32_t nseg = 0, ntok = 0, budget = cfg->token_budget;
  query_start_loc[0] = 0;
  // Give sequence i the blocks for `len` more tokens; false if the free list runs dry.
  auto take_blocks = [&](int32_t i, int32_t len) -> pgqa_status {
    pgqa_sched_seq& q = seqs[i];
    const int64_t need = (int64_t(q.cached) + len + bs - 1) / bs;
    if (need > cfg->max_blocks_per_seq)
      return fail(PGQA_ERR_INVALID_ARG, "sequence %d needs %lld blocks, its table row holds %d", i,
                  (long long)need, cfg->max_blocks_per_seq);
    if (need - q.num_blocks > *free_count) return PGQA_ERR_WORKSPACE;  // not enough free blocks
    int32_t* row = block_tables + int64_t(i) * cfg->max_blocks_per_seq;
    while (q.num_blocks < need) row[q.num_blocks++] = free_list[--*free_count];
    return PGQA_OK;
  };
  auto emit = [&](int32_t i, int32_t kind, int32_t len) -> pgqa_status {
    if (ntok + len > token_capacity)
      return fail(PGQA_ERR_INVALID_ARG, "step needs more than token_capacity=%d tokens", token_capacity);
    const pgqa_status st = take_blocks(i, len);
    if (st == PGQA_ERR_WORKSPACE) return PGQA_ERR_WORKSPACE;  // skip this segment
    if (st != PGQA_OK) return st;
    const pgqa_sched_seq& q = seqs[i];
    segs[nseg] = pgqa_sched_segment{i, kind, len, q.cached + len};
    context_lens[nseg] = q.cached + len;
    for (int32_t j = 0; j < len; ++j) {
      token_pos[ntok + j] = q.cached + j;
      token_seq[ntok + j] = i;
    }
    ntok += len;
    ++nseg;
    query_start_loc[nseg] = ntok;
    budget -= len;
    return PGQA_OK;
  };
  // 1. decode and verify rows
  for (int32_t i = 0; i < num_seqs && nseg < cfg->max_segments; ++i) {
    const pgqa_sched_seq& q = seqs[i];
    if (q.prompt_left > 0 || budget < 1) continue;
    pgqa_status st = PGQA_ERR_WORKSPACE;
    if (q.num_draft > 0 && 1 + q.num_draft <= budget) st = emit(i, PGQA_SEG_VERIFY, 1 + q.num_draft);
    if (st == PGQA_ERR_WORKSPACE) st = emit(i, PGQA_SEG_DECODE, 1);  // no drafts, or the verify row does not fit
    if (st != PGQA_OK && st != PGQA_ERR_WORKSPACE) return st;
  }
  // 2. prefill chunks
  bool prefill_done = false;
  for (int32_t i = 0; i < num_seqs && nseg < cfg->max_segments; ++i) {
    const pgqa_sched_seq& q = seqs[i];
    if (q.prompt_left == 0) continue;
    int32_t len;
    if (cfg->chunked_prefill) {
      if (budget < 1) break;
      len = q.prompt_left < budget ? q.prompt_left : budget;
    } else if (q.prompt_left <= budget || !prefill_done) {
      len = q.prompt_left;
    } else {
      continue;
    }
    const pgqa_status st = emit(i, PGQA_SEG_PREFILL, len);
    if (st == PGQA_OK) prefill_done = true;
    else if (st != PGQA_ERR_WORKSPACE) return st;
    if (budget < 0) budget = 0;
  }
  *num_segments = nseg;
  *num_tokens = ntok;
  return PGQA_OK;
}

pgqa_status pgqa_sched_commit(pgqa_sched_seq* seqs, int32_t num_seqs, const pgqa_sched_segment* segs,
                              int32_t num_segments, const int32_t* accepted) {
  clear_error();
  if (num_segments < 0 || (num_segments > 0 && (!seqs || !segs)))
    return fail(PGQA_ERR_INVALID_ARG, "commit: bad arguments");
  for (int32_t s = 0; s < num_segments; ++s) {
    const pgqa_sched_segment& g = segs[s];
    if (g.seq < 0 || g.seq >= num_seqs || g.q_len < 1) return fail(PGQA_ERR_INVALID_ARG, "commit: bad segment %d", s);
    if (g.kind == PGQA_SEG_VERIFY) {
      if (!accepted) return fail(PGQA_ERR_INVALID_ARG, "commit: a verify row needs accepted counts");
      if (accepted[s] < 0 || accepted[s] > g.q_len - 1)
        return fail(PGQA_ERR_INVALID_ARG, "commit: segment %d accepted %d of %d drafts", s, accepted[s], g.q_len - 1);
    } else if (g.kind == PGQA_SEG_PREFILL) {
      if (g.q_len > seqs[g.seq].prompt_left) return fail(PGQA_ERR_INVALID_ARG, "commit: segment %d overruns", s);
    } else if (g.kind != PGQA_SEG_DECODE) {
      return fail(PGQA_ERR_INVALID_ARG, "commit: segment %d has kind %d", s, g.kind);
    }
  }
  for (int32_t s = 0; s < num_segments; ++s) {
    const pgqa_sched_segment& g = segs[s];
    pgqa_sched_seq& q = seqs[g.seq];
    if (g.kind == PGQA_SEG_PREFILL) {
      q.cached += g.q_len;
      q.prompt_left -= g.q_len;
    } else {
      q.cached += g.kind == PGQA_SEG_VERIFY ? accepted[s] + 1 : 1;
    }
    q.num_draft = 0;
  }
  return PGQA_OK;
}

pgqa_status pgqa_sched_release(const pgqa_sched_config* cfg, pgqa_sched_seq* seqs, int32_t num_seqs, int32_t seq,
                               int32_t* block_tables, int32_t* free_list, int32_t* free_count,
                               int32_t free_capacity) {
  clear_error();
  if (!cfg || cfg->max_blocks_per_seq < 1 || !seqs || seq < 0 || seq >= num_seqs || !block_tables ||
      !free_count || *free_count < 0 || (!free_list && free_capacity > 0))
    return fail(PGQA_ERR_INVALID_ARG, "release: bad arguments");
  pgqa_sched_seq& q = seqs[seq];
  if (q.num_blocks < 0 || q.num_blocks > cfg->max_blocks_per_seq || *free_count + q.num_blocks > free_capacity)
    return fail(PGQA_ERR_INVALID_ARG, "release: the free list cannot take %d blocks", q.num_blocks);
  int32_t* row = block_tables + int64_t(seq) * cfg->max_blocks_per_seq;
  for (int32_t j = q.num_blocks - 1; j >= 0; --j) {
    free_list[(*free_count)++] = row[j];
    row[j] = -1;
  }
  q = pgqa_sched_seq{0, 0, 0, 0};
  return PGQA_OK;
}

}  // extern "C"

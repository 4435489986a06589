/*
 * A plain C11 caller of libpgqa's host-only entry points (no GPU needed):
 * version, pool sizing, the decode, chunk and mixed-step planners, error
 * reporting, prompt lookup, greedy acceptance and one step of the token-budget
 * planner.  tests/test_c_consumer.py builds it with gcc against include/ and
 * checks what it prints against the Python binding and the oracle.
 */
#include <stdio.h>

#include "pgqa.h"
#include "pgqa_sched.h"

int main(void) {
  printf("version %s\n", pgqa_version());

  pgqa_pool_config cfg = {32, 16, 8, 128, 0};
  printf("pool_bytes %zu\n", pgqa_pool_bytes(&cfg));

  pgqa_decode_plan dp;
  if (pgqa_plan_decode(256, 16, 64, 8, 16, 2049, &dp) != PGQA_OK) return 1;
  printf("decode_plan %d %d %d %d %d\n", dp.split_tokens, dp.max_splits, dp.waves_per_split, dp.load_hint,
         dp.kernel);
  if (pgqa_plan_decode(256, 16, 1, 8, 16, 32769, &dp) != PGQA_OK) return 1;
  printf("decode_plan %d %d %d %d %d\n", dp.split_tokens, dp.max_splits, dp.waves_per_split, dp.load_hint,
         dp.kernel);

  pgqa_chunk_plan cp;
  if (pgqa_plan_chunk(256, 16, 9, 552, 8, 16, 512, 6656, &cp) != PGQA_OK) return 1;
  printf("chunk_plan %d %d %d %d\n", cp.split_tokens, cp.max_splits, cp.short_split_tokens, cp.kernel);
  if (pgqa_plan_chunk(256, 16, 8, 40, 8, 16, 5, 4096, &cp) != PGQA_OK) return 1;
  printf("chunk_plan %d %d %d %d\n", cp.split_tokens, cp.max_splits, cp.short_split_tokens, cp.kernel);

  /* a mixed step: two decode rows, a verify row of 5 tokens, a 40-token slice */
  static int32_t mitems[4096 * PGQA_MIXED_ITEM_INTS];
  const int32_t mqsl[] = {0, 1, 2, 7, 47};
  const int32_t mctx[] = {300, 1200, 900, 2040};
  pgqa_mixed_plan mp;
  if (pgqa_plan_mixed(256, 16, 8, 16, 4, mqsl, mctx, 0, 0, NULL, 0, &mp) != PGQA_OK) return 3;
  if (mp.num_items + mp.num_combine > 4096) return 3;
  if (pgqa_plan_mixed(256, 16, 8, 16, 4, mqsl, mctx, 0, 0, mitems, 4096, &mp) != PGQA_OK) return 3;
  long long checksum = 0;
  for (long long i = 0; i < (long long)(mp.num_items + mp.num_combine) * PGQA_MIXED_ITEM_INTS; ++i)
    checksum += (i + 1) * mitems[i];
  printf("mixed_plan %d %d %d %d %d %lld\n", mp.split_wide, mp.split_columns, mp.max_splits, mp.num_items,
         mp.num_combine, checksum);

  if (pgqa_plan_decode(0, 16, 1, 8, 16, 10, &dp) != PGQA_ERR_INVALID_ARG) return 2;
  printf("error %s | %s\n", pgqa_status_string(PGQA_ERR_INVALID_ARG), pgqa_last_error());

  const int32_t toks[] = {5, 1, 2, 3, 7, 1, 2, 3};
  int32_t draft[4];
  const int32_t nd = pgqa_prompt_lookup(toks, 8, 1, 3, 4, draft);
  printf("draft %d", nd);
  for (int i = 0; i < nd; ++i) printf(" %d", draft[i]);
  printf("\n");

  const int32_t d[] = {7, 1, 9};
  const int32_t t[] = {7, 1, 2, 4};
  int32_t acc[4];
  const int32_t na = pgqa_accept_greedy(d, 3, t, acc);
  printf("accept %d", na);
  for (int i = 0; i < na; ++i) printf(" %d", acc[i]);
  printf("\n");

  /* one step: sequence 0 decodes with 2 drafts, sequence 1 has a 40-token prompt */
  pgqa_sched_config sc = {16, 4, 1, 16, 4};
  pgqa_sched_seq seqs[2] = {{20, 0, 2, 2}, {0, 40, 0, 0}};
  int32_t tables[2][4] = {{3, 8, -1, -1}, {-1, -1, -1, -1}};
  int32_t free_list[6] = {0, 1, 2, 4, 5, 6};
  int32_t free_count = 6;
  pgqa_sched_segment segs[4];
  int32_t qsl[5], ctx[4], pos[64], sid[64], nseg = 0, ntok = 0;
  if (pgqa_sched_plan_step(&sc, seqs, 2, &tables[0][0], free_list, &free_count, segs, qsl, ctx, pos, sid, 64,
                           &nseg, &ntok) != PGQA_OK)
    return 3;
  printf("plan %d segments %d tokens\n", nseg, ntok);
  for (int i = 0; i < nseg; ++i)
    printf("seg %d %d %d %d\n", segs[i].seq, segs[i].kind, segs[i].q_len, segs[i].context_len);
  printf("tables %d %d %d %d | %d %d %d %d | free %d\n", tables[0][0], tables[0][1], tables[0][2], tables[0][3],
         tables[1][0], tables[1][1], tables[1][2], tables[1][3], free_count);
  return 0;
}

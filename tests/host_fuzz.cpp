// Randomised checks of the library's host-side code: the decode, chunk and
// mixed-step planners, prompt lookup, greedy acceptance, and the step planner
// driven through many plan / commit / release rounds.  Each call gets random
// (mostly valid) arguments; the program checks that outputs stay inside the
// buffers the caller sized (guard words), that the step planner's cache blocks
// are conserved and never handed out twice, and that every accepted plan is
// self-consistent.  It prints one "ok" line per part, or a message and exits 1.
//
// Built by tests/test_host_fuzz.py with g++ against libpgqa.so.  For a run
// under AddressSanitizer and UndefinedBehaviorSanitizer, compile the library's
// host sources (errors.cpp, api.cpp, sched.cpp) and this file with hipcc, each
// sanitizer option preceded by -Xarch_host so that only host code is
// instrumented, and link them with the library's device objects and the same
// two sanitizers.
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <random>
#include <set>
#include <vector>

#include "pgqa.h"
#include "pgqa_sched.h"

static int planners(int iters) {
  std::mt19937_64 rng(12345);
  auto U = [&](int64_t lo, int64_t hi) { return int64_t(std::uniform_int_distribution<int64_t>(lo, hi)(rng)); };
  long ok_mixed = 0, bad_mixed = 0, ok_dec = 0, ok_chk = 0;
  for (int it = 0; it < iters; ++it) {
    // ---- pgqa_plan_mixed
    {
      const int bs_choices[] = {16, 32, 64, 128, 256, 8, 0, -16, 48};
      const int bs = U(0, 20) == 0 ? bs_choices[U(0, 8)] : bs_choices[U(0, 4)];
      const int hkv = int(U(0, 50)) == 0 ? int(U(-2, 3)) : int(1 << U(0, 3));
      const int r = int(1 << U(0, 3));
      const int hq = int(U(0, 50)) == 0 ? int(U(-1, 40)) : hkv * r;
      const int cus = int(U(0, 50)) == 0 ? int(U(-2, 2)) : int(U(1, 320));
      const int N = int(U(0, 50)) == 0 ? int(U(-2, 2)) : int(U(0, U(0, 3) == 0 ? 2000 : 64));
      std::vector<int32_t> qsl(std::max(N, 0) + 1, 0), ctx(std::max(N, 0), 0);
      for (int s = 0; s < N; ++s) {
        int ql = U(0, 8) == 0 ? int(U(0, 4096)) : int(U(0, 1)) ? 1 : int(U(1, 8));
        if (U(0, 5000) == 0) ql = int(U(-5, -1));
        qsl[s + 1] = qsl[s] + ql;
        int n = ql + int(U(0, 20000));
        if (U(0, 5000) == 0) n = int(U(-5, ql));
        ctx[s] = n;
      }
      const int sw = U(0, 4) == 0 ? (U(0, 3) ? int(32 * U(1, 128)) : int(U(-64, 5000))) : 0;
      const int sc = U(0, 4) == 0 ? (U(0, 3) ? int(256 * U(1, 16)) : int(U(-64, 5000))) : 0;
      pgqa_mixed_plan plan{};
      pgqa_status st = pgqa_plan_mixed(cus, bs, hkv, hq, N, N >= 0 ? qsl.data() : nullptr, N >= 0 ? ctx.data() : nullptr,
                                       sw, sc, nullptr, 0, &plan);
      if (st == PGQA_OK) {
        const int64_t n_items = int64_t(plan.num_items) + plan.num_combine;
        int64_t cap = n_items;
        if (U(0, 10) == 0) cap = std::max<int64_t>(0, n_items - U(1, 5));
        std::vector<int32_t> items(size_t(std::max<int64_t>(cap, 1)) * PGQA_MIXED_ITEM_INTS + 8, -7);
        pgqa_mixed_plan plan2{};
        st = pgqa_plan_mixed(cus, bs, hkv, hq, N, qsl.data(), ctx.data(), sw, sc, items.data(), cap, &plan2);
        // the guard words past the capacity stay untouched
        for (int k = 0; k < 8; ++k)
          if (items[size_t(std::max<int64_t>(cap, 1)) * PGQA_MIXED_ITEM_INTS + k] != -7 && cap > 0) {
            fprintf(stderr, "it %d: items written past the capacity\n", it);
            return 1;
          }
        if (st == PGQA_OK) ++ok_mixed; else ++bad_mixed;
      } else {
        ++bad_mixed;
      }
    }
    // ---- pgqa_plan_decode / pgqa_plan_chunk
    {
      pgqa_decode_plan dp{};
      const int bs = int(1 << U(3, 8));
      if (pgqa_plan_decode(int(U(-1, 320)), U(0, 5) ? bs : int(U(-3, 300)), int(U(-1, 5000)), int(U(-1, 16)),
                           int(U(-1, 128)), int(U(-1, 1 << 20)), &dp) == PGQA_OK)
        ++ok_dec;
      pgqa_chunk_plan cp{};
      if (pgqa_plan_chunk(int(U(-1, 320)), U(0, 5) ? bs : int(U(-3, 300)), int(U(-1, 5000)), int(U(-1, 100000)),
                          int(U(-1, 16)), int(U(-1, 128)), int(U(-1, 5000)), int(U(-1, 1 << 20)), &cp) == PGQA_OK)
        ++ok_chk;
    }
    // ---- prompt lookup and greedy acceptance
    {
      const int n = int(U(0, 300));
      std::vector<int32_t> toks(std::max(n, 1));
      for (auto& t : toks) t = int32_t(U(0, 5));
      const int mn = int(U(-1, 6)), mx = int(U(-1, 8)), k = int(U(-1, 10));
      std::vector<int32_t> draft(std::max(k, 0) + 1, -9);
      const int32_t got = pgqa_prompt_lookup(toks.data(), n, mn, mx, k, draft.data());
      if (got > k || (got >= 0 && draft[std::max(k, 0)] != -9 && k >= 0)) {
        fprintf(stderr, "it %d: prompt lookup wrote %d of %d\n", it, got, k);
        return 1;
      }
      const int nd = int(U(-1, 12));
      std::vector<int32_t> d(std::max(nd, 1)), tg(std::max(nd, 0) + 1), out(std::max(nd, 0) + 2, -9);
      for (auto& t : d) t = int32_t(U(0, 3));
      for (auto& t : tg) t = int32_t(U(0, 3));
      const int32_t acc = pgqa_accept_greedy(d.data(), nd, tg.data(), out.data());
      if (acc > nd + 1 || (nd >= 0 && out[std::max(nd, 0) + 1] != -9)) {
        fprintf(stderr, "it %d: acceptance wrote past its output\n", it);
        return 1;
      }
    }
  }
  printf("planners ok: mixed %ld accepted / %ld rejected, decode plans %ld, chunk plans %ld\n", ok_mixed,
         bad_mixed, ok_dec, ok_chk);
  return 0;
}

static int step_planner(int runs) {
  std::mt19937_64 rng(777);
  auto U = [&](int64_t lo, int64_t hi) { return int64_t(std::uniform_int_distribution<int64_t>(lo, hi)(rng)); };
  long steps = 0, rejected = 0;
  for (int run = 0; run < runs; ++run) {
    pgqa_sched_config cfg{};
    cfg.token_budget = int(U(1, 600));
    cfg.max_segments = int(U(1, 40));
    cfg.chunked_prefill = int(U(0, 1));
    const int bs_choices[] = {16, 32, 64, 128, 256, 1, 7};
    cfg.block_size = bs_choices[U(0, 6)];
    cfg.max_blocks_per_seq = U(0, 5) == 0 ? int(U(1, 300)) : int((3000 + 60 * 8) / cfg.block_size + 2 + U(0, 10));
    const int S = int(U(1, 24));
    const int total_blocks = int(U(1, 3000));
    std::vector<pgqa_sched_seq> seqs(S);
    for (auto& q : seqs) {
      q.cached = 0;
      q.prompt_left = int(U(1, 3000));
      q.num_draft = 0;
      q.num_blocks = 0;
    }
    std::vector<int32_t> bt(size_t(S) * cfg.max_blocks_per_seq, -1);
    std::vector<int32_t> free_list(total_blocks);
    for (int i = 0; i < total_blocks; ++i) free_list[i] = total_blocks - 1 - i;
    int32_t free_count = total_blocks;
    const int cap = U(0, 5) == 0 ? int(U(1, 800)) : cfg.token_budget + 8 * cfg.max_segments + 3000;
    std::vector<pgqa_sched_segment> segs(cfg.max_segments);
    std::vector<int32_t> qsl(cfg.max_segments + 1), ctx(cfg.max_segments), pos(cap), sq(cap), acc(cfg.max_segments);
    for (int step = 0; step < 60; ++step) {
      for (auto& q : seqs)
        if (q.prompt_left == 0 && U(0, 2) == 0) q.num_draft = int(U(0, 6));
      int32_t ns = -1, nt = -1;
      pgqa_status st = pgqa_sched_plan_step(&cfg, seqs.data(), S, bt.data(), free_list.data(), &free_count, segs.data(),
                                            qsl.data(), ctx.data(), pos.data(), sq.data(), cap, &ns, &nt);
      if (st != PGQA_OK) { ++rejected; break; }
      ++steps;
      if (ns < 0 || ns > cfg.max_segments || nt < 0 || nt > cap || qsl[ns] != nt) {
        fprintf(stderr, "run %d step %d: bad counts ns=%d nt=%d\n", run, step, ns, nt);
        return 1;
      }
      // blocks: held + free == total, all distinct
      std::set<int32_t> seen;
      long held = 0;
      for (int s = 0; s < S; ++s)
        for (int j = 0; j < seqs[s].num_blocks; ++j) {
          const int32_t b = bt[size_t(s) * cfg.max_blocks_per_seq + j];
          if (b < 0 || b >= total_blocks || !seen.insert(b).second) {
            fprintf(stderr, "run %d step %d: bad or repeated block %d\n", run, step, b);
            return 1;
          }
          ++held;
        }
      for (int i = 0; i < free_count; ++i)
        if (!seen.insert(free_list[i]).second) {
          fprintf(stderr, "run %d step %d: free block %d also held\n", run, step, free_list[i]);
          return 1;
        }
      if (held + free_count != total_blocks) {
        fprintf(stderr, "run %d step %d: %ld held + %d free != %d\n", run, step, held, free_count, total_blocks);
        return 1;
      }
      for (int i = 0; i < ns; ++i) acc[i] = segs[i].kind == PGQA_SEG_VERIFY ? int(U(0, segs[i].q_len - 1)) : 0;
      if (pgqa_sched_commit(seqs.data(), S, segs.data(), ns, acc.data()) != PGQA_OK) {
        fprintf(stderr, "run %d step %d: commit failed: %s\n", run, step, pgqa_last_error());
        return 1;
      }
      // finish some decoding sequences
      for (int s = 0; s < S; ++s)
        if (seqs[s].prompt_left == 0 && U(0, 8) == 0) {
          if (pgqa_sched_release(&cfg, seqs.data(), S, s, bt.data(), free_list.data(), &free_count, total_blocks) !=
              PGQA_OK) {
            fprintf(stderr, "run %d step %d: release failed: %s\n", run, step, pgqa_last_error());
            return 1;
          }
          seqs[s].prompt_left = int(U(1, 3000));
        }
    }
  }
  printf("step planner ok: %ld steps, %ld runs ended by a rejected step\n", steps, rejected);
  return 0;
}

int main(int argc, char** argv) {
  const int iters = argc > 1 ? atoi(argv[1]) : 20000;
  const int runs = argc > 2 ? atoi(argv[2]) : 400;
  if (planners(iters)) return 1;
  return step_planner(runs);
}

"""The C-ABI host producers (include/pgqa_sched.h) against the plain oracle
(oracle/sched.py): exact agreement on random histories, states and whole
multi-step runs, and the error returns.  No GPU."""
import copy

import numpy as np
import pytest

import oracle.sched as S
import paged_gqa_decode_head_amd as pg

from test_oracle_sched import random_state


def test_prompt_lookup_matches_oracle():
    rng = np.random.default_rng(11)
    for _ in range(3000):
        n = int(rng.integers(0, 40))
        t = rng.integers(0, int(rng.integers(2, 6)), size=n)
        lo = int(rng.integers(1, 4))
        hi = lo + int(rng.integers(0, 4))
        k = int(rng.integers(0, 6))
        assert pg.prompt_lookup(t, lo, hi, k).tolist() == S.prompt_lookup(t.tolist(), lo, hi, k)


def test_accept_greedy_matches_oracle():
    rng = np.random.default_rng(12)
    for _ in range(2000):
        d = rng.integers(0, 3, size=int(rng.integers(0, 7)))
        t = rng.integers(0, 3, size=d.size + 1)
        assert pg.accept_greedy(d, t).tolist() == S.accept_greedy(d.tolist(), t.tolist())


def _planner_from(cfg, seqs, tables, free):
    p = pg.StepPlanner(cfg["token_budget"], cfg["max_segments"], cfg["chunked_prefill"], cfg["block_size"],
                       cfg["max_blocks_per_seq"], len(seqs), free)
    for i, s in enumerate(seqs):
        p.seqs[i] = [s["cached"], s["prompt_left"], s["num_draft"], s["num_blocks"]]
    if seqs:
        p.block_tables[:] = np.array(tables, dtype=np.int32)
    return p


def _same(p, r_lib, r_ref, seqs, tables, free):
    assert r_lib["segs"].tolist() == [list(x) for x in r_ref["segs"]]
    for k in ("query_start_loc", "context_lens", "token_pos", "token_seq"):
        assert r_lib[k].tolist() == r_ref[k], k
    assert p.seqs.tolist() == [[s["cached"], s["prompt_left"], s["num_draft"], s["num_blocks"]] for s in seqs]
    if seqs:
        assert p.block_tables.tolist() == tables
    assert p.free_list[: p.free_count.value].tolist() == free


@pytest.mark.parametrize("chunked", [0, 1])
def test_plan_step_matches_oracle(chunked):
    rng = np.random.default_rng(13 + chunked)
    for _ in range(500):
        bs = int(rng.choice([4, 16]))
        cfg = {"token_budget": int(rng.integers(1, 40)), "max_segments": int(rng.integers(1, 10)),
               "chunked_prefill": chunked, "block_size": bs, "max_blocks_per_seq": 8}
        seqs, tables, free = random_state(rng, int(rng.integers(0, 9)), bs, 8, int(rng.integers(0, 12)))
        p = _planner_from(cfg, seqs, tables, free)
        r_ref = S.plan_step(cfg, seqs, tables, free)
        r_lib = p.plan(token_capacity=8 * bs * 9)
        _same(p, r_lib, r_ref, seqs, tables, free)


def test_multi_step_runs_match_oracle():
    """Whole runs: decode streams with drafts, prompts arriving, finished
    sequences released; plan, accept and commit every step on both sides."""
    rng = np.random.default_rng(14)
    for run in range(20):
        bs, width, nseq = 16, 16, 6
        cfg = {"token_budget": int(rng.integers(8, 64)), "max_segments": 6, "chunked_prefill": run % 2,
               "block_size": bs, "max_blocks_per_seq": width}
        seqs = [{"cached": 0, "prompt_left": int(rng.integers(1, 120)), "num_draft": 0, "num_blocks": 0}
                for _ in range(nseq)]
        tables = [[-1] * width for _ in range(nseq)]
        free = list(range(nseq * width))
        p = _planner_from(cfg, seqs, tables, free)
        for step in range(40):
            for i, s in enumerate(seqs):  # drafts for some decoding sequences
                if s["prompt_left"] == 0 and s["cached"] > 0:
                    s["num_draft"] = int(rng.integers(0, 5))
                    s["num_draft"] = min(s["num_draft"], bs * width - s["cached"] - 1)
                    p.seqs[i, 2] = s["num_draft"]
            r_ref = S.plan_step(cfg, seqs, tables, free)
            r_lib = p.plan(token_capacity=bs * width * nseq)
            _same(p, r_lib, r_ref, seqs, tables, free)
            acc = [int(rng.integers(0, q - 1 + 1)) if kind == S.SEG_VERIFY else 0
                   for _, kind, q, _ in r_ref["segs"]]
            S.commit(seqs, r_ref["segs"], acc)
            p.commit(r_lib["segs"], acc)
            for i, s in enumerate(seqs):  # finish sequences that reached a length
                if s["prompt_left"] == 0 and s["cached"] >= 150:
                    S.release(seqs, i, tables, free)
                    p.release(i)
            assert p.seqs.tolist() == [[s["cached"], s["prompt_left"], s["num_draft"], s["num_blocks"]]
                                       for s in seqs]
            assert p.free_list[: p.free_count.value].tolist() == free


def test_errors():
    with pytest.raises(pg.PgqaError):
        pg.prompt_lookup([1, 2], 0, 2, 1)
    with pytest.raises(pg.PgqaError):
        pg.prompt_lookup([1, 2], 3, 2, 1)
    p = pg.StepPlanner(8, 4, False, 16, 2, 1, [0, 1, 2])
    p.seqs[0] = [0, 40, 0, 0]  # a whole prompt longer than the row can hold
    with pytest.raises(pg.PgqaError):
        p.plan(token_capacity=64)
    p = pg.StepPlanner(8, 4, True, 16, 4, 1, [0, 1, 2])
    p.seqs[0] = [0, 8, 0, 0]
    with pytest.raises(pg.PgqaError):
        p.plan(token_capacity=4)  # the step needs 8 token slots
    with pytest.raises(pg.PgqaError):
        pg.StepPlanner(0, 4, True, 16, 4, 1, [0]).plan(token_capacity=4)
    with pytest.raises(pg.PgqaError):  # a verify row needs its accepted counts
        p.commit(np.array([[0, pg.SEG_VERIFY, 3, 3]], dtype=np.int32), None)

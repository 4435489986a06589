"""Pins of the host-producer oracle (oracle/sched.py) to something other than
itself: hand-worked cases, an independent brute-force search for prompt lookup,
and invariants of the step planner on random states."""
import copy
import json
import os

import numpy as np
import pytest

import oracle.sched as S

HERE = os.path.dirname(os.path.abspath(__file__))
GOLD = json.load(open(os.path.join(HERE, "golden", "sched_cases.json")))


@pytest.mark.parametrize("case", GOLD["prompt_lookup"], ids=lambda c: c["why"][:40])
def test_prompt_lookup_hand_worked(case):
    assert S.prompt_lookup(case["tokens"], case["min"], case["max"], case["k"]) == case["draft"]


@pytest.mark.parametrize("case", GOLD["accept_greedy"])
def test_accept_greedy_hand_worked(case):
    assert S.accept_greedy(case["draft"], case["target"]) == case["out"]


@pytest.mark.parametrize("case", GOLD["plan_step"], ids=lambda c: c["why"][:40])
def test_plan_step_hand_worked(case):
    seqs, tables, free = copy.deepcopy(case["seqs"]), copy.deepcopy(case["tables"]), list(case["free"])
    r = S.plan_step(case["cfg"], seqs, tables, free)
    assert [list(x) for x in r["segs"]] == case["segs"]
    for k in ("query_start_loc", "context_lens", "token_pos", "token_seq"):
        assert r[k] == case[k], k
    assert tables == case["tables_after"] and free == case["free_after"]
    if "commit_accepted" in case:
        S.commit(seqs, r["segs"], case["commit_accepted"])
        assert seqs == case["seqs_after_commit"]
        r2 = S.plan_step(case["cfg"], seqs, tables, free)
        assert [list(x) for x in r2["segs"]] == case["next_segs"]
        assert tables == case["next_tables_after"] and free == case["next_free_after"]


def _brute_lookup(t, lo, hi, k):
    """All (n, p) matches of the trailing n-gram by sliding windows, then the rule."""
    t = np.asarray(t, dtype=np.int64)
    n = t.size
    for size in range(hi, lo - 1, -1):
        if size > n - 1:
            continue
        win = np.lib.stride_tricks.sliding_window_view(t[: n - 1], size)  # windows ending before the last token
        hits = np.nonzero((win == t[n - size:]).all(axis=1))[0]
        if hits.size:
            p = int(hits.max())
            return t[p + size: p + size + k].tolist()
    return []


def test_prompt_lookup_matches_brute_force():
    rng = np.random.default_rng(5)
    for _ in range(3000):
        n = int(rng.integers(0, 30))
        t = rng.integers(0, int(rng.integers(2, 5)), size=n).tolist()
        lo = int(rng.integers(1, 4))
        hi = lo + int(rng.integers(0, 4))
        k = int(rng.integers(0, 6))
        assert S.prompt_lookup(t, lo, hi, k) == _brute_lookup(t, lo, hi, k), (t, lo, hi, k)


def test_accept_greedy_is_longest_common_prefix_plus_one():
    rng = np.random.default_rng(6)
    for _ in range(2000):
        d = rng.integers(0, 3, size=int(rng.integers(0, 6))).tolist()
        t = rng.integers(0, 3, size=len(d) + 1).tolist()
        out = S.accept_greedy(d, t)
        a = 0
        while a < len(d) and d[a] == t[a]:
            a += 1
        assert out == d[:a] + [t[a]]


def random_state(rng, nseq, bs, width, nfree):
    seqs, tables = [], []
    ids = list(rng.permutation(nfree + nseq * width))
    for _ in range(nseq):
        cached = int(rng.integers(0, bs * (width - 2) + 1))
        prefill = rng.random() < 0.4
        prompt = int(rng.integers(1, bs * width - cached)) if prefill and cached < bs * width - 1 else 0
        if prompt:  # the prompt must fit the table row
            prompt = min(prompt, bs * width - cached)
        nd = 0 if prompt else int(rng.integers(0, 5))
        nd = min(nd, bs * width - cached - 1) if not prompt else 0
        nb = -(-cached // bs)
        row = [ids.pop() for _ in range(nb)] + [-1] * (width - nb)
        seqs.append({"cached": cached, "prompt_left": prompt, "num_draft": max(nd, 0), "num_blocks": nb})
        tables.append(row)
    free = [ids.pop() for _ in range(min(nfree, len(ids)))]
    return seqs, tables, free


@pytest.mark.parametrize("chunked", [0, 1])
def test_plan_step_invariants(chunked):
    rng = np.random.default_rng(7 + chunked)
    for trial in range(400):
        bs = int(rng.choice([4, 16]))
        width = 8
        cfg = {"token_budget": int(rng.integers(1, 40)), "max_segments": int(rng.integers(1, 10)),
               "chunked_prefill": chunked, "block_size": bs, "max_blocks_per_seq": width}
        seqs, tables, free = random_state(rng, int(rng.integers(0, 9)), bs, width, int(rng.integers(0, 12)))
        before = copy.deepcopy(seqs)
        ids_before = sorted([b for r in tables for b in r if b >= 0] + free)
        r = S.plan_step(cfg, seqs, tables, free)
        segs = r["segs"]
        # each sequence at most once; decode/verify rows before prefill chunks, each in arrival order
        order = [s[0] for s in segs]
        assert len(order) == len(set(order)) and len(segs) <= cfg["max_segments"]
        kinds = [s[1] for s in segs]
        first_prefill = kinds.index(S.SEG_PREFILL) if S.SEG_PREFILL in kinds else len(kinds)
        assert all(k == S.SEG_PREFILL for k in kinds[first_prefill:])
        assert order[:first_prefill] == sorted(order[:first_prefill])
        assert order[first_prefill:] == sorted(order[first_prefill:])
        # token budget
        total = sum(s[2] for s in segs)
        if chunked:
            assert total <= cfg["token_budget"]
        else:
            over = [s for s in segs if s[1] == S.SEG_PREFILL and s[2] > 0]
            assert total - max([s[2] for s in over], default=0) <= cfg["token_budget"]
        # segment shapes
        for i, kind, q_len, n in segs:
            b = before[i]
            assert n == b["cached"] + q_len
            if kind == S.SEG_DECODE:
                assert q_len == 1 and b["prompt_left"] == 0
            elif kind == S.SEG_VERIFY:
                assert q_len == 1 + b["num_draft"] and b["num_draft"] > 0
            else:
                assert 1 <= q_len <= b["prompt_left"] and (chunked or q_len == b["prompt_left"])
            assert seqs[i]["num_blocks"] >= -(-n // bs)
        # metadata
        assert r["query_start_loc"] == list(np.cumsum([0] + [s[2] for s in segs]))
        assert r["context_lens"] == [s[3] for s in segs]
        exp_pos = [p for i, _, q, _ in segs for p in range(before[i]["cached"], before[i]["cached"] + q)]
        assert r["token_pos"] == exp_pos and len(r["token_seq"]) == len(exp_pos)
        # blocks are conserved and never shared
        ids_after = sorted([b for row in tables for b in row if b >= 0] + free)
        assert ids_after == ids_before
        # a decoding sequence is left out only when budget, segments or blocks ran out
        for i, b in enumerate(before):
            if b["prompt_left"] == 0 and i not in order:
                need = -(-(b["cached"] + 1) // bs) - b["num_blocks"]
                assert len(segs) == cfg["max_segments"] or total >= cfg["token_budget"] or need > len(free) or \
                    sum(s[2] for s in segs if s[0] < i) >= cfg["token_budget"]


def test_commit_and_release():
    seqs = [{"cached": 7, "prompt_left": 0, "num_draft": 3, "num_blocks": 2},
            {"cached": 0, "prompt_left": 9, "num_draft": 0, "num_blocks": 1}]
    S.commit(seqs, [(0, S.SEG_VERIFY, 4, 11), (1, S.SEG_PREFILL, 5, 5)], [2, 0])
    assert seqs[0]["cached"] == 10 and seqs[0]["num_draft"] == 0
    assert seqs[1]["cached"] == 5 and seqs[1]["prompt_left"] == 4
    tables, free = [[4, 6, -1], [8, -1, -1]], [1]
    S.release(seqs, 0, tables, free)
    assert free == [1, 6, 4] and tables[0] == [-1, -1, -1] and seqs[0]["num_blocks"] == 0

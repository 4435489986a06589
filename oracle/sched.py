"""Host producers of the chunk-attention work, written out plainly.

TEST INFRASTRUCTURE ONLY (see the package docstring): nothing in the product
path imports this module.

Page "perf: Qwen3 offline inference - hybrid attention backend, fused
rms_norm_rope, chunked prefill + prompt-lookup spec decoding", Summary item 4:
a host scheduling layer runs chunked prefill and prompt-lookup speculative
decoding (k draft tokens, verified in one forward pass of b x (k+1) tokens);
its results section (the decode-stall workload: 8 decode streams with a long
prompt injected) motivates serving decode streams before prefill chunks.  The
page states the features, not their rules; the rules below are the plainest
readings:

* prompt lookup: the longest trailing n-gram (n from max_ngram down to
  min_ngram) that occurred earlier in the sequence, at its most recent earlier
  occurrence, proposes the up to k tokens that followed it;
* greedy acceptance: the longest draft prefix equal to the target's greedy
  tokens is kept, then the target's token at the first disagreement;
* step planning: decode and verify rows of decoding sequences first (a verify
  row that does not fit the budget or its cache blocks becomes a decode row),
  then prefill chunks, under one token budget per step (chunked), or with
  prompts run whole (not chunked: a prompt past the budget runs whole in a
  step that has no other prefill);
* cache blocks come from a free-list stack, top = last element.
"""
from __future__ import annotations

SEG_DECODE, SEG_VERIFY, SEG_PREFILL = 0, 1, 2

__all__ = ["SEG_DECODE", "SEG_VERIFY", "SEG_PREFILL", "prompt_lookup", "accept_greedy", "plan_step", "commit",
           "release"]


def prompt_lookup(tokens, min_ngram: int, max_ngram: int, k: int) -> list[int]:
    """Draft tokens for one sequence from its own history (see the module docstring)."""
    t = [int(x) for x in tokens]
    n = len(t)
    for size in range(max_ngram, min_ngram - 1, -1):
        if size > n - 1:
            continue
        suffix = t[n - size:]
        latest = None
        for p in range(n - size):  # occurrences that end before the last token
            if t[p:p + size] == suffix:
                latest = p
        if latest is not None:
            return t[latest + size: latest + size + k]
    return []


def accept_greedy(draft, target) -> list[int]:
    """Accepted draft prefix plus the target's token after it."""
    out = []
    for i, d in enumerate(draft):
        if int(d) != int(target[i]):
            break
        out.append(int(d))
    out.append(int(target[len(out)]))
    return out


def _ceil_div(a: int, b: int) -> int:
    return -(-a // b)


def plan_step(cfg: dict, seqs: list[dict], tables: list[list[int]], free: list[int]) -> dict:
    """One step.  cfg: token_budget, max_segments, chunked_prefill, block_size,
    max_blocks_per_seq.  seqs: dicts with cached, prompt_left, num_draft,
    num_blocks (num_blocks advanced in place); tables: block-table rows
    (extended in place); free: the free-list stack (popped in place).
    Returns segs [(seq, kind, q_len, context_len)], query_start_loc,
    context_lens, token_pos, token_seq."""
    bs, width = cfg["block_size"], cfg["max_blocks_per_seq"]
    budget = cfg["token_budget"]
    segs = []

    def add(i, kind, q_len):
        nonlocal budget
        s = seqs[i]
        need = _ceil_div(s["cached"] + q_len, bs)
        if need > width:
            raise ValueError(f"sequence {i} outgrows its block-table row")
        if need - s["num_blocks"] > len(free):
            return False  # not enough free blocks: the segment waits
        while s["num_blocks"] < need:
            tables[i][s["num_blocks"]] = free.pop()
            s["num_blocks"] += 1
        segs.append((i, kind, q_len, s["cached"] + q_len))
        budget -= q_len
        return True

    # decode streams first
    for i, s in enumerate(seqs):
        if len(segs) == cfg["max_segments"]:
            break
        if s["prompt_left"] > 0 or budget < 1:
            continue
        verified = s["num_draft"] > 0 and 1 + s["num_draft"] <= budget and add(i, SEG_VERIFY, 1 + s["num_draft"])
        if not verified:  # no drafts, or the verify row does not fit: a plain decode row
            add(i, SEG_DECODE, 1)
    # then prompts
    prefilled = False
    for i, s in enumerate(seqs):
        if len(segs) == cfg["max_segments"]:
            break
        if s["prompt_left"] == 0:
            continue
        if cfg["chunked_prefill"]:
            if budget < 1:
                break
            q_len = min(s["prompt_left"], budget)
        elif s["prompt_left"] <= budget or not prefilled:
            q_len = s["prompt_left"]
        else:
            continue
        if add(i, SEG_PREFILL, q_len):
            prefilled = True
        budget = max(budget, 0)

    qsl, ctx, pos, seq = [0], [], [], []
    for i, kind, q_len, n in segs:
        qsl.append(qsl[-1] + q_len)
        ctx.append(n)
        first = seqs[i]["cached"]
        pos.extend(range(first, first + q_len))
        seq.extend([i] * q_len)
    return {"segs": segs, "query_start_loc": qsl, "context_lens": ctx, "token_pos": pos, "token_seq": seq}


def commit(seqs: list[dict], segs, accepted=None) -> None:
    """A step's outcome: prefill chunks move prompt tokens into the cache, a
    decode row adds one token, a verify row adds its accepted drafts plus one."""
    for j, (i, kind, q_len, _) in enumerate(segs):
        s = seqs[i]
        if kind == SEG_PREFILL:
            s["cached"] += q_len
            s["prompt_left"] -= q_len
        elif kind == SEG_VERIFY:
            s["cached"] += accepted[j] + 1
        else:
            s["cached"] += 1
        s["num_draft"] = 0


def release(seqs: list[dict], i: int, tables: list[list[int]], free: list[int]) -> None:
    """A finished sequence returns its blocks (last held first) to the stack."""
    s = seqs[i]
    for j in range(s["num_blocks"] - 1, -1, -1):
        free.append(tables[i][j])
        tables[i][j] = -1
    s.update(cached=0, prompt_left=0, num_draft=0, num_blocks=0)

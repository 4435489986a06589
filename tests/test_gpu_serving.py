"""Serving steps driven by the host producers (include/pgqa_sched.h): the step
planner feeds the fused norm + rotary + cache write and ONE attention call per
step for the whole mixed batch (prefill chunks, decode rows and prompt-lookup
verify rows together): by default the one-launch mixed call, whose work list
pgqa_plan_mixed builds from the planner's host-side lengths; also the chunk
call.  A step of single decode tokens goes to the fused decode step (norm +
rotary + cache write + decode in one launch).
Every step's output is checked against the fp64 reference on the read-back
cache and the GPU-produced q."""
import numpy as np
import pytest
import torch

import oracle as O
import paged_gqa_decode_head_amd as pg

from harness import SCALE, bits_of, compare, dev_i32

pytestmark = pytest.mark.gpu

NB, BS, HKV, HQ, W = 96, 16, 8, 16, 16
EPS, THETA = 1e-6, 1e6


def _bf16(rng, shape):
    return torch.from_numpy(rng.standard_normal(shape)).to(torch.bfloat16).cuda()


@pytest.mark.parametrize("route", ["mixed", "chunk"])
@pytest.mark.parametrize("chunked", [True, False])
def test_planned_steps_match_reference(chunked, route):
    rng = np.random.default_rng(41 + int(chunked))
    nseq = 5
    pool = pg.Pool(NB, BS, HKV)
    wq = torch.from_numpy(1 + 0.1 * rng.standard_normal(128)).to(torch.bfloat16).cuda()
    wk = torch.from_numpy(1 + 0.1 * rng.standard_normal(128)).to(torch.bfloat16).cuda()
    # periodic token streams, so that prompt lookup finds recurring n-grams
    period = [rng.integers(0, 50, size=int(rng.integers(5, 12))).tolist() for _ in range(nseq)]
    stream = lambda i, j: period[i][j % len(period[i])]
    prompt_lens = [40, 70, 150, 9, 33]
    hist = [[stream(i, j) for j in range(prompt_lens[i])] for i in range(nseq)]
    planner = pg.StepPlanner(64, 8, chunked, BS, W, nseq, rng.permutation(NB))
    for i in range(nseq):
        planner.seqs[i] = [0, prompt_lens[i], 0, 0]
    seen = {pg.SEG_DECODE: 0, pg.SEG_VERIFY: 0, pg.SEG_PREFILL: 0}
    mixed = 0
    for step in range(16):
        drafts = {}
        for i in range(nseq):
            if planner.seqs[i, 1] == 0:  # decoding: propose from its own history
                d = pg.prompt_lookup(hist[i], 1, 3, 4)
                d = d[: max(0, BS * W - int(planner.seqs[i, 0]) - 1)]
                drafts[i] = d
                planner.seqs[i, 2] = d.size
        plan = planner.plan(token_capacity=512)
        segs = plan["segs"]
        if segs.shape[0] == 0:
            break
        kinds = set(segs[:, 1].tolist())
        for kd in kinds:
            seen[kd] += 1
        mixed += len(kinds) > 1
        T = plan["token_pos"].size
        print(f"[serving] chunked={chunked} route={route} step {step}: segments {segs.tolist()}", flush=True)
        q, k, v = _bf16(rng, (T, HQ, 128)), _bf16(rng, (T, HKV, 128)), _bf16(rng, (T, HKV, 128))
        bt_full = dev_i32(planner.block_tables)
        bt_seg = np.ascontiguousarray(planner.block_tables[segs[:, 0]])
        ctx, qsl = plan["context_lens"], plan["query_start_loc"]
        if (segs[:, 2] == 1).all():  # host routing: only single decode tokens -> one fused decode step
            q_out = torch.empty_like(q)
            out = pg.decode_step(pool, q, k, v, wq, wk, dev_i32(ctx), dev_i32(bt_seg), int(ctx.max()), EPS, THETA,
                                 SCALE, q_out=q_out)
        else:
            q_out = pg.rms_norm_rope_cache_write(pool, q, k, v, wq, wk, dev_i32(plan["token_pos"]),
                                                 dev_i32(plan["token_seq"]), bt_full, EPS, THETA)
            if route == "mixed":  # work list built on the host from the planner's lengths, uploaded
                mplan, items = pg.plan_mixed(torch.cuda.get_device_properties(0).multi_processor_count, BS, HKV,
                                             HQ, qsl, ctx)
                out = pg.paged_mixed_attention(pool, q_out, dev_i32(qsl), dev_i32(ctx), dev_i32(bt_seg),
                                               int(segs[:, 2].max()), int(ctx.max()), SCALE, mplan, dev_i32(items))
            else:
                out = pg.paged_chunk_attention(pool, q_out, dev_i32(qsl), dev_i32(ctx), dev_i32(bt_seg),
                                               int(segs[:, 2].max()), int(ctx.max()), SCALE)
        kk, vv = pool.read_logical()
        ref = O.chunk_attention(O.bf16_bits_to_f64(bits_of(q_out)), qsl, kk.numpy().view(np.uint16),
                                vv.numpy().view(np.uint16), bt_seg, ctx, SCALE)
        compare(out, ref, f"step {step}")
        # outcomes: the target continues each periodic stream, with an occasional miss
        accepted = []
        for i, kind, q_len, n in segs.tolist():
            nxt = len(hist[i])
            if kind == pg.SEG_VERIFY:
                target = [stream(i, nxt + j) if rng.random() > 0.15 else 99 for j in range(q_len)]
                got = pg.accept_greedy(drafts[i], target)
                hist[i].extend(got.tolist())
                accepted.append(got.size - 1)
            elif kind == pg.SEG_DECODE:
                hist[i].append(stream(i, nxt))
                accepted.append(0)
            else:
                if q_len == planner.seqs[i, 1]:  # the prompt's last chunk yields the first token
                    hist[i].append(stream(i, nxt))
                accepted.append(0)
        planner.commit(segs, accepted)
        for i in range(nseq):  # the history holds the cached tokens and one pending token once decoding
            assert len(hist[i]) == planner.seqs[i, 0] + (1 if planner.seqs[i, 1] == 0 else planner.seqs[i, 1])
    assert pool.check_errors() == 0
    assert seen[pg.SEG_VERIFY] and seen[pg.SEG_PREFILL] and seen[pg.SEG_DECODE]
    assert mixed > 0

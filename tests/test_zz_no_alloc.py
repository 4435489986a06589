"""The allocation-free decode step (pgqa_decode_step_noalloc) against the
decode step with a caller workspace (pgqa_decode_step): the same kernels and
plan, so outputs, q_out and the cache must agree bit for bit; both against the
fp64 reference chain.  Two calls in a row, the second on a smaller batch with a
different plan, so the second reads a scratch array that still holds the first
call's partials."""
import numpy as np
import pytest
import torch

import oracle as O
import paged_gqa_decode_head_amd as pg
from paged_gqa_decode_head_amd.workloads import Group, StepSpec, make_step

from harness import SCALE, StepRun, bits_of, compact, compare

pytestmark = pytest.mark.gpu


def _note(msg):
    print(msg, flush=True)


def _run_pair(w, plan):
    s = w.spec
    a, b = StepRun(w), StepRun(w)
    mx = int(w.dec_ctx.max())
    qo_a, qo_b = torch.empty_like(a.q), torch.empty_like(b.q)
    out_a = pg.decode_step(a.pool, a.q, a.k, a.v, a.wq, a.wk, a.dec_ctx, a.dec_bt, mx, s.eps, s.rope_theta, SCALE,
                           plan=plan, q_out=qo_a)
    out_b = torch.full_like(out_a, 3.0)
    pg.decode_step_noalloc(b.pool, b.q, b.k, b.v, b.wq, b.wk, b.dec_ctx, b.dec_bt, mx, s.eps, s.rope_theta, SCALE,
                           out_b, plan=plan, q_out=qo_b)
    assert a.pool.check_errors() == 0 and b.pool.check_errors() == 0
    return a, b, out_a, out_b, qo_a, qo_b


def _check(w, plan, tag, uses_scratch=False):
    s = w.spec
    a, b, out_a, out_b, qo_a, qo_b = _run_pair(w, plan)
    if uses_scratch:
        need = pg.decode_workspace_bytes(b.pool, w.num_decode, s.num_q_heads, int(w.dec_ctx.max()), plan)
        assert 0 < need <= pg.NOALLOC_SCRATCH_BYTES
    assert np.array_equal(bits_of(out_b), bits_of(out_a)), tag
    assert np.array_equal(bits_of(qo_b), bits_of(qo_a)), tag
    ka, va = a.pool.read_logical(blocks=w.used_blocks)
    kb, vb = b.pool.read_logical(blocks=w.used_blocks)
    assert np.array_equal(ka.numpy(), kb.numpy()) and np.array_equal(va.numpy(), vb.numpy()), tag
    bt_c = compact(w.block_tables, b.used)
    pk, pv = w.prefix_k[b.used].copy(), w.prefix_v[b.used].copy()
    q_ref, _ = O.fused_norm_rope_write(w.tok_q, w.tok_k, w.tok_v, w.wq, w.wk, w.tok_pos, w.tok_seq, bt_c, s.eps,
                                       s.rope_theta, pk, pv)
    compare(out_b, O.decode_attention(O.bf16_round(q_ref), pk, pv, bt_c, w.dec_ctx, SCALE), tag)


@pytest.mark.parametrize("kernel", [1, 2])
def test_noalloc_step_equals_workspace_step_twice(kernel):
    big = make_step(StepSpec("noalloc-big", 9701, 16, 8, 1400, decode=(Group(12, 200, 1500),)))
    small = make_step(StepSpec("noalloc-small", 9702, 32, 4, 300, decode=(Group(3, 30, 700),)))
    for w, split, tag in ((big, 128, "first call"), (small, 64, "second, smaller call")):
        mx = int(w.dec_ctx.max())
        plan = pg.DecodePlan(split, -(-mx // split), 4, 0, kernel)
        _note(f"[noalloc] kernel {kernel} {tag}: batch {w.num_decode} contexts <= {mx} plan {plan}")
        _check(w, plan, f"kernel {kernel} {tag}", uses_scratch=True)


def test_noalloc_step_default_plan_and_single_split():
    w = make_step(StepSpec("noalloc-default", 9703, 16, 8, 700, decode=(Group(2, 3000, 5000),)))
    _note("[noalloc] default plan, batch 2")
    _check(w, None, "default plan")
    w = make_step(StepSpec("noalloc-one", 9704, 16, 8, 300, decode=(Group(5, 10, 300),)))
    plan = pg.DecodePlan(1024, 1, 4, 0, 1)
    _note("[noalloc] one split")
    _check(w, plan, "one split")


def test_noalloc_step_rejects_partials_beyond_the_scratch():
    w = make_step(StepSpec("noalloc-over", 9705, 16, 8, 200, decode=(Group(4, 10, 100),)))
    s = w.spec
    run = StepRun(w)
    mx = int(w.dec_ctx.max())
    plan = pg.DecodePlan(64, 4000, 4, 0, 1)          # 4000 partial slots per (sequence, kv head)
    assert pg.decode_workspace_bytes(run.pool, w.num_decode, s.num_q_heads, mx, plan) > pg.NOALLOC_SCRATCH_BYTES
    out = torch.full((w.num_decode, s.num_q_heads, 128), 5.0, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(pg.PgqaError) as e:
        pg.decode_step_noalloc(run.pool, run.q, run.k, run.v, run.wq, run.wk, run.dec_ctx, run.dec_bt, mx, s.eps,
                               s.rope_theta, SCALE, out, plan=plan)
    assert e.value.status == 4 and "fixed scratch" in str(e.value)
    torch.cuda.synchronize()
    assert torch.all(out == 5.0)                       # nothing was enqueued
    assert run.pool.check_errors() == 0

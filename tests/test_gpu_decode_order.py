"""The decode calls with a host-side copy of the context lengths
(pgqa_decode_plan.host_context_lens): the (sequence, kv head) units run in a
length-balanced order, and every output, q_out and cache row is bit-identical
to the call without the hint (same plan, same kernels)."""
import numpy as np
import pytest
import torch

import paged_gqa_decode_head_amd as pg
from paged_gqa_decode_head_amd.workloads import SPECS, Group, StepSpec, make_step

from harness import KERNELS, SCALE, StepRun, bits_of, compare, default_plan, with_kernel

pytestmark = pytest.mark.gpu


def _note(msg):
    print(msg, flush=True)


def _hinted(plan, w):
    p = pg.DecodePlan(plan.split_tokens, plan.max_splits, plan.waves_per_split, plan.load_hint, plan.kernel)
    return p.set_host_context_lens(w.dec_ctx)


@pytest.mark.parametrize("kernel", KERNELS)
@pytest.mark.parametrize("name", ["cfg2", "cfg3b", "cfg4"])
def test_hinted_order_is_bit_identical(name, kernel):
    _note(f"[order] {name} kernel {kernel}")
    w = make_step(SPECS[name])
    s = w.spec
    plan = default_plan(w, kernel)
    a, b = StepRun(w), StepRun(w)
    mx = int(w.dec_ctx.max())
    qa, qb = torch.empty_like(a.q), torch.empty_like(b.q)
    oa = pg.decode_step(a.pool, a.q, a.k, a.v, a.wq, a.wk, a.dec_ctx, a.dec_bt, mx, s.eps, s.rope_theta, SCALE,
                        plan=plan, q_out=qa)
    ob = pg.decode_step(b.pool, b.q, b.k, b.v, b.wq, b.wk, b.dec_ctx, b.dec_bt, mx, s.eps, s.rope_theta, SCALE,
                        plan=_hinted(plan, w), q_out=qb)
    assert a.pool.check_errors() == 0 and b.pool.check_errors() == 0
    assert np.array_equal(bits_of(oa), bits_of(ob))
    assert np.array_equal(bits_of(qa), bits_of(qb))
    ka, va = a.pool.read_logical(blocks=w.used_blocks)
    kb, vb = b.pool.read_logical(blocks=w.used_blocks)
    assert np.array_equal(ka.numpy(), kb.numpy()) and np.array_equal(va.numpy(), vb.numpy())
    # plain decode attention on the written cache, with and without the hint
    d1 = pg.paged_decode_attention(b.pool, qb, b.dec_ctx, b.dec_bt, mx, SCALE, plan=plan)
    d2 = pg.paged_decode_attention(b.pool, qb, b.dec_ctx, b.dec_bt, mx, SCALE, plan=_hinted(plan, w))
    assert np.array_equal(bits_of(d1), bits_of(d2))
    compare(d2, b.oracle_decode_on_gpu_inputs(qb), f"{name} hinted")


@pytest.mark.parametrize("nseq,hkv,hq", [(37, 8, 16), (200, 8, 16), (129, 8, 64)])
def test_hinted_order_partial_rounds_and_too_many_units(nseq, hkv, hq):
    """Unit counts that are not a multiple of the CU count, and more units than
    the order holds (the hint is then ignored): still bit-identical."""
    rng = np.random.default_rng(nseq)
    lens = [int(x) for x in rng.integers(0, 700, size=nseq)]
    nb = sum(-(-(L + 1) // 16) for L in lens) + 4
    w = make_step(StepSpec(f"ord{nseq}", 9900 + nseq, hq, hkv, nb, decode=tuple(Group(1, L, L) for L in lens)))
    run = StepRun(w)
    run.write()
    q = run.decode_q()
    mx = int(w.dec_ctx.max())
    for kernel in KERNELS:
        plan = default_plan(w, kernel)
        d1 = run.decode(plan=plan, q=q)
        d2 = run.decode(plan=_hinted(plan, w), q=q)
        assert np.array_equal(bits_of(d1), bits_of(d2)), kernel
    assert run.pool.check_errors() == 0
    compare(d2, run.oracle_decode_on_gpu_inputs(q), "hinted")

"""The fused decode step (pgqa_decode_step: norm + rotary of each sequence's
new token, its cache write, and decode attention in one launch) against the
two calls it replaces, bit for bit (same device code, same plan), and against
the fp64 reference chain."""
import numpy as np
import pytest
import torch

import oracle as O
import paged_gqa_decode_head_amd as pg
from paged_gqa_decode_head_amd.workloads import SPECS, Group, StepSpec, make_step

from harness import KERNELS, SCALE, StepRun, bits_of, compact, compare, default_plan, dev_i32

pytestmark = pytest.mark.gpu


def _note(msg):
    print(msg, flush=True)


def _pair(w, plan):
    """Two identical pools; A: write + decode, B: the fused step.  Returns outputs and pools."""
    s = w.spec
    a, b = StepRun(w), StepRun(w)
    assert w.num_tokens == w.num_decode and np.array_equal(w.tok_pos, w.dec_ctx - 1)
    a.write()
    out_a = a.decode(plan=plan)
    qo_b = torch.empty_like(a.q_out)
    out_b = pg.decode_step(b.pool, b.q, b.k, b.v, b.wq, b.wk, b.dec_ctx, b.dec_bt, int(w.dec_ctx.max()), s.eps,
                           s.rope_theta, SCALE, plan=plan, q_out=qo_b)
    return a, b, out_a, out_b, qo_b


def _bits_equal(a, b, w):
    ka, va = a.pool.read_logical(blocks=w.used_blocks)
    kb, vb = b.pool.read_logical(blocks=w.used_blocks)
    return np.array_equal(ka.numpy(), kb.numpy()) and np.array_equal(va.numpy(), vb.numpy())


@pytest.mark.parametrize("kernel", KERNELS)
@pytest.mark.parametrize("name", ["cfg2", "cfg3a", "cfg3b", "cfg4"])
def test_fused_step_equals_write_then_decode(name, kernel):
    _note(f"[step] {name} kernel={kernel}")
    w = make_step(SPECS[name])
    plan = default_plan(w, kernel)
    a, b, out_a, out_b, qo_b = _pair(w, plan)
    assert a.pool.check_errors() == 0 and b.pool.check_errors() == 0
    assert np.array_equal(bits_of(qo_b), bits_of(a.q_out))
    assert np.array_equal(bits_of(out_b), bits_of(out_a))
    assert _bits_equal(a, b, w)
    compare(out_b, b.oracle_decode_on_gpu_inputs(qo_b), f"{name} fused step")


@pytest.mark.parametrize("hq,hkv,bs", [(16, 8, 16), (32, 4, 16), (8, 8, 32), (8, 1, 64), (16, 4, 256)])
@pytest.mark.parametrize("plan", [None, (64, 1), (256, 4), (4096, 8)])
@pytest.mark.parametrize("kernel", [0] + KERNELS)
def test_fused_step_small_shapes_and_plans(hq, hkv, bs, plan, kernel):
    """kernel 0 with plan None: plan = NULL (the library's default plan)."""
    spec = StepSpec(f"fstep-{hq}-{hkv}-{bs}", 940 + hq + bs, hq, hkv, 256 if bs < 256 else 32,
                    decode=(Group(1, 0, 0), Group(1, 15, 15), Group(1, 16, 16), Group(4, 1, 700)), block_size=bs)
    w = make_step(spec)
    p = None
    if plan is not None:
        split = max(plan[0], bs)
        p = pg.DecodePlan(split, -(-int(w.dec_ctx.max()) // split), plan[1], 0, kernel)
    elif kernel:
        p = default_plan(w, kernel)
    a, b, out_a, out_b, qo_b = _pair(w, p)
    assert b.pool.check_errors() == 0
    assert np.array_equal(bits_of(out_b), bits_of(out_a))
    assert np.array_equal(bits_of(qo_b), bits_of(a.q_out))
    assert _bits_equal(a, b, w)


@pytest.mark.parametrize("kernel", KERNELS)
def test_fused_step_end_to_end_against_fp64_chain(kernel):
    """Row-strided q/k/v taken from one packed projection buffer; the output
    against the fp64 chain (norm, rotary, bf16 cache, attention) on raw inputs."""
    w = make_step(StepSpec("fchain", 961, 16, 8, 64, decode=(Group(3, 20, 200),)))
    s = w.spec
    run = StepRun(w)
    B, hq, hkv = w.num_decode, s.num_q_heads, s.num_kv_heads
    packed = torch.cat([run.q.reshape(B, -1), run.k.reshape(B, -1), run.v.reshape(B, -1)], dim=1).contiguous()
    q = packed[:, : hq * 128].view(B, hq, 128)
    k = packed[:, hq * 128:(hq + hkv) * 128].view(B, hkv, 128)
    v = packed[:, (hq + hkv) * 128:].view(B, hkv, 128)
    out = pg.decode_step(run.pool, q, k, v, run.wq, run.wk, run.dec_ctx, run.dec_bt, int(w.dec_ctx.max()), s.eps,
                         s.rope_theta, SCALE, plan=default_plan(w, kernel))
    assert run.pool.check_errors() == 0
    # fp64 chain: the new tokens written into a reference cache model (bf16 K/V),
    # q rounded to bf16 as the kernel holds it, then attention
    bt_c = compact(w.block_tables, run.used)
    pk, pv = w.prefix_k[run.used].copy(), w.prefix_v[run.used].copy()
    q_ref, _ = O.fused_norm_rope_write(w.tok_q, w.tok_k, w.tok_v, w.wq, w.wk, w.tok_pos, w.tok_seq, bt_c, s.eps,
                                       s.rope_theta, pk, pv)
    ref = O.decode_attention(O.bf16_round(q_ref), pk, pv, bt_c, w.dec_ctx, SCALE)
    compare(out, ref, "fused step vs fp64 chain")


@pytest.mark.parametrize("kernel", KERNELS)
def test_fused_step_zero_context_and_bad_block(kernel):
    w = make_step(StepSpec("fbad", 962, 16, 8, 16, decode=(Group(3, 30, 30),)))
    s = w.spec
    run = StepRun(w)
    ctx = w.dec_ctx.copy()
    ctx[1] = 0  # no new token for sequence 1
    bt = w.dec_block_tables.copy()
    bt[2, (ctx[2] - 1) // 16] = s.num_blocks + 5  # the new token's block id is outside the pool
    out = torch.full((3, 16, 128), 7.0, dtype=torch.bfloat16, device="cuda")
    pg.decode_step(run.pool, run.q, run.k, run.v, run.wq, run.wk, dev_i32(ctx), dev_i32(bt), int(ctx.max()), s.eps,
                   s.rope_theta, SCALE, out=out, plan=default_plan(w, kernel))
    assert run.pool.check_errors() & pg.DEVERR_BLOCK_ID
    assert torch.all(out[1] == 0)
    # sequence 0 is untouched by the others' bad metadata: the fp64 chain on its own token
    assert w.tok_seq[0] == 0 and w.dec_tok[0] == 0
    bt_c = compact(w.block_tables, run.used)
    pk, pv = w.prefix_k[run.used].copy(), w.prefix_v[run.used].copy()
    q_ref, _ = O.fused_norm_rope_write(w.tok_q[:1], w.tok_k[:1], w.tok_v[:1], w.wq, w.wk, w.tok_pos[:1],
                                       w.tok_seq[:1], bt_c, s.eps, s.rope_theta, pk, pv)
    ref = O.decode_attention(O.bf16_round(q_ref), pk, pv, bt_c[:1], w.dec_ctx[:1], SCALE)
    compare(out[:1], ref, "sequence 0 beside a zero context and a bad block id")


@pytest.mark.parametrize("seed", range(32))
def test_fused_step_random_cases_against_fp64_chain(seed):
    """Seeded random combinations of head layout, block size, context lengths
    (single key, block boundaries, long) and split plan: outputs against the
    fp64 chain, the new tokens' cache rows (K within tolerance, V bit-exact)."""
    rng = np.random.default_rng(9000 + seed)
    hq, hkv = [(16, 8), (32, 4), (8, 8), (32, 8), (8, 1), (8, 4)][int(rng.integers(6))]
    bs = int(rng.choice([16, 32, 64, 128, 256]))
    nseq = int(rng.integers(1, 13))
    picks = [0, bs - 1, bs, bs + 1, 2 * bs - 1, int(rng.integers(1, 3000)), int(rng.integers(1, 400))]
    lens = [int(picks[int(rng.integers(len(picks)))]) for _ in range(nseq)]
    nblocks = sum(-(-(L + 1) // bs) for L in lens) + 4
    spec = StepSpec(f"frand-{seed}", 9100 + seed, hq, hkv, nblocks, decode=tuple(Group(1, L, L) for L in lens),
                    block_size=bs)
    w = make_step(spec)
    s = w.spec
    mx = int(w.dec_ctx.max())
    plan = None
    if rng.integers(3):
        gran = max(64, bs)
        split = min(gran * int(rng.integers(1, 9)), 4096 // gran * gran)
        waves = int(rng.choice([1, 2, 4, 8]))
        split = min(split, 1024 * waves // gran * gran)  # a plan covers at most 1024 keys per wave
        plan = pg.DecodePlan(split, -(-mx // split), waves, int(rng.integers(3)), int(rng.integers(3)))
    _note(f"[frand] seed {seed}: heads {hq}/{hkv} bs {bs} contexts {w.dec_ctx.tolist()} plan {plan}")
    run = StepRun(w)
    q_out = torch.empty_like(run.q)
    out = pg.decode_step(run.pool, run.q, run.k, run.v, run.wq, run.wk, run.dec_ctx, run.dec_bt, mx, s.eps,
                         s.rope_theta, SCALE, plan=plan, q_out=q_out)
    assert run.pool.check_errors() == 0
    bt_c = compact(w.block_tables, run.used)
    pk, pv = w.prefix_k[run.used].copy(), w.prefix_v[run.used].copy()
    q_ref, _ = O.fused_norm_rope_write(w.tok_q, w.tok_k, w.tok_v, w.wq, w.wk, w.tok_pos, w.tok_seq, bt_c, s.eps,
                                       s.rope_theta, pk, pv)
    compare(q_out, q_ref, f"seed {seed} q_out")
    compare(out, O.decode_attention(O.bf16_round(q_ref), pk, pv, bt_c, w.dec_ctx, SCALE), f"seed {seed} out")
    kk, vv = run.pool.read_logical(blocks=run.used)
    blk, off = O.slot_of(w.tok_pos, w.tok_seq, bt_c, bs)
    assert np.array_equal(vv.numpy().view(np.uint16)[blk, off], pv[blk, off])
    compare(torch.from_numpy(kk.numpy()[blk, off]).view(torch.bfloat16), O.bf16_bits_to_f64(pk[blk, off]),
            f"seed {seed} new K rows")

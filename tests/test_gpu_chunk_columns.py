"""Chunk calls whose segments all have at most 16 query rows per kv head
(q_len x group <= 16: speculative-verify rows, single tokens) run on the
matrix-core decode kernel with the segment's (token, head) rows as MFMA
columns (chunk plan kernel 2, the planner's choice for such calls).  Parity
against the fp64 reference through the C ABI, and agreement with the chunk
kernels and the decode kernel on the same rows."""
import numpy as np
import pytest
import torch

import oracle as O
import paged_gqa_decode_head_amd as pg
from paged_gqa_decode_head_amd.workloads import Group, StepSpec, make_step

from harness import SCALE, SENTINEL, StepRun, bits_of, compare, dev_bf16, dev_i32

pytestmark = pytest.mark.gpu


def _note(msg):
    print(msg, flush=True)


def _spec(name, seed, hq, hkv, bs, segs, nb):
    return StepSpec(name, seed, hq, hkv, nb, chunks=tuple(Group(1, L, L, ql) for L, ql in segs), block_size=bs)


def _columns_plan(split, max_ctx, bs=16):
    sp = max(split, bs, 64)
    return pg.ChunkPlan(sp, -(-max_ctx // sp), 0, 2)


def _call(run, q, plan=None, out=None):
    w = run.w
    qlens = np.diff(w.chk_qsl)
    return pg.paged_chunk_attention(run.pool, q, run.chk_qsl, run.chk_ctx, run.chk_bt, int(qlens.max()),
                                    int(w.chk_ctx.max()), SCALE, plan=plan, out=out)


def test_planner_picks_columns_only_when_every_segment_fits():
    cus = 256
    assert pg.plan_chunk(cus, 16, 8, 40, 8, 16, 5, 4096).kernel == 2      # verify rows, group 2
    assert pg.plan_chunk(cus, 16, 8, 64, 4, 32, 2, 4096).kernel == 2      # group 8, two tokens
    assert pg.plan_chunk(cus, 16, 8, 72, 4, 32, 3, 4096).kernel == 1      # group 8, three tokens: 24 rows
    assert pg.plan_chunk(cus, 16, 9, 552, 8, 16, 512, 6656).kernel == 1   # a prefill slice in the call


def test_verify_rows_parity():
    """8 verify rows of k+1 = 5 tokens over U[1024, 4096] keys (Qwen3-1.7B
    shapes): the default plan (columns) and the chunk kernels, both against
    the fp64 reference."""
    _note("[columns] verify rows")
    w = make_step(StepSpec("verify", 5, 16, 8, 16384, chunks=(Group(8, 1024, 4096, 5),)))
    run = StepRun(w)
    run.write()
    q = run.chunk_q()
    ref = run.oracle_chunk_on_gpu_inputs(q)
    out = _call(run, q)
    assert run.pool.check_errors() == 0
    ma, mr = compare(out, ref, "verify rows, columns")
    _note(f"  columns max_abs={ma:.2e} mean_rel={mr:.2e}")
    mc = int(w.chk_ctx.max())
    out_k = _call(run, q, plan=pg.ChunkPlan(256, -(-mc // 256), 256, 1))
    compare(out_k, ref, "verify rows, chunk kernels")


SEGS = {1: [(0, 7), (20, 16), (33, 1), (3, 9), (9, 0), (100, 12), (250, 16), (1, 1), (15, 2)],
        2: [(0, 7), (20, 5), (33, 1), (3, 8), (9, 0), (100, 6), (250, 8), (1, 1), (15, 2)],
        4: [(0, 3), (20, 4), (33, 1), (3, 2), (9, 0), (100, 4), (250, 4), (1, 1)],
        8: [(0, 2), (20, 1), (33, 2), (9, 0), (100, 2), (250, 1), (1, 1)]}


@pytest.mark.parametrize("hq,hkv,bs", [(16, 8, 16), (32, 4, 16), (8, 8, 16), (32, 8, 32), (16, 8, 64),
                                       (16, 4, 256), (8, 1, 16)])
@pytest.mark.parametrize("split", [None, 64, 256, 4096])
def test_columns_small_ragged(hq, hkv, bs, split):
    segs = SEGS[hq // hkv]
    spec = _spec(f"cols-{hq}-{hkv}-{bs}", 1700 + hq + bs, hq, hkv, bs, segs, 256 if bs < 256 else 16)
    w = make_step(spec)
    run = StepRun(w)
    run.write()
    q = run.chunk_q()
    plan = None if split is None else _columns_plan(split, int(w.chk_ctx.max()), bs)
    if plan is None:
        cus = torch.cuda.get_device_properties(0).multi_processor_count
        p = pg.plan_chunk(cus, bs, w.num_chunks, int(w.chk_qsl[-1]), hkv, hq, int(np.diff(w.chk_qsl).max()),
                          int(w.chk_ctx.max()))
        assert p.kernel == 2
    out = _call(run, q, plan)
    assert run.pool.check_errors() == 0
    compare(out, run.oracle_chunk_on_gpu_inputs(q), f"{spec.name} split={split}")


@pytest.mark.parametrize("hq,hkv", [(16, 8), (32, 4)])
def test_columns_q_len_one_equals_matrix_core_decode(hq, hkv):
    """Single-token segments on the column route give the bits of the
    matrix-core decode kernel with the same split (one split: no combine)."""
    w = make_step(StepSpec("cols1", 1720, hq, hkv, 512, chunks=(Group(6, 1, 900, 1),)))
    run = StepRun(w)
    run.write()
    q = run.chunk_q()
    mc = int(w.chk_ctx.max())
    out_c = bits_of(_call(run, q, plan=pg.ChunkPlan(1024, 1, 0, 2)))
    out_d = bits_of(pg.paged_decode_attention(run.pool, q, run.chk_ctx, run.chk_bt, mc, SCALE,
                                              plan=pg.DecodePlan(1024, 1, 4, 1, 2)))
    assert np.array_equal(out_c, out_d)
    # with splits: same values up to the combine's summation order
    out_cs = _call(run, q, plan=_columns_plan(128, mc))
    compare(out_cs, run.oracle_chunk_on_gpu_inputs(q), "q_len=1 split 128")


@pytest.mark.parametrize("bs", [16, 32, 64, 256])
def test_columns_ignore_garbage_past_the_context(bs):
    """Every slot outside the attended keys holds a NaN pattern."""
    spec = _spec(f"colgarb-{bs}", 1724, 16, 8, bs, [(10, 7), (50, 8), (0, 3), (200, 5)], 40)
    w = make_step(spec)
    run = StepRun(w, fill_prefix=False)
    s = w.spec
    k = np.full((s.num_blocks, bs, 8, 128), SENTINEL, dtype=np.uint16)
    v = k.copy()
    for row in range(w.num_chunks):
        L = int(w.chk_ctx[row]) - int(np.diff(w.chk_qsl)[row])
        for j in range(L):
            blk, off = w.block_tables[row, j // bs], j % bs
            k[blk, off] = w.prefix_k[blk, off]
            v[blk, off] = w.prefix_v[blk, off]
    run.pool.fill_logical(k.view(np.int16), v.view(np.int16))
    run.write()
    q = run.chunk_q()
    mc = int(w.chk_ctx.max())
    for plan in (None, _columns_plan(64, mc, bs), _columns_plan(4096, mc, bs)):
        out = _call(run, q, plan)
        compare(out, run.oracle_chunk_on_gpu_inputs(q), f"columns garbage bs={bs} plan={plan}")


def test_columns_causal_boundary_probe():
    """A key right after query i's position leaves query i's output
    bit-identical and changes query i+1's (8 tokens x 2 heads = 16 columns)."""
    spec = _spec("colprobe", 1722, 4, 2, 16, [(20, 8)], 8)
    w = make_step(spec)
    run = StepRun(w)
    run.write()
    q = run.chunk_q()
    plan = pg.ChunkPlan(64, 1, 0, 2)
    base = bits_of(_call(run, q, plan))
    i = 5
    j = 20 + i + 1
    blk, off = int(w.block_tables[w.num_decode, j // 16]), j % 16
    kb, vb = run.pool.read_logical(blocks=[blk])
    kk = kb.numpy().view(np.uint16).copy()
    vv = vb.numpy().view(np.uint16).copy()
    kk[0, off] = bits_of(q[i + 1, 0::2] * 40)
    vv[0, off] = O.f64_to_bf16_bits(np.full((2, 128), 50.0))
    run.pool.fill_logical(kk.view(np.int16), vv.view(np.int16), blocks=[blk])
    got = bits_of(_call(run, q, plan))
    assert np.array_equal(got[: i + 1], base[: i + 1])
    assert not np.array_equal(got[i + 1], base[i + 1])


@pytest.mark.parametrize("q_len", [1, 5, 8])
def test_columns_addressing_probe_one_hot_every_position(q_len):
    """Only key j* matches every query strongly: each query that sees j*
    returns V_j* bit-exactly, for every logical position j*, with one and
    many splits."""
    bs, hkv, hq = 16, 2, 4
    prefix = 70
    n = prefix + q_len
    nb = 24
    rng = np.random.default_rng(31 + q_len)
    perm = rng.permutation(nb)
    nblk = -(-n // bs)
    bt = perm[:nblk][None].astype(np.int32)
    pool = pg.Pool(nb, bs, hkv)
    u = np.zeros(128)
    u[:32] = 1.0
    vk = O.f64_to_bf16_bits(rng.standard_normal((nb, bs, hkv, 128)))
    q = dev_bf16(np.broadcast_to(O.f64_to_bf16_bits(u), (q_len, hq, 128)).copy())
    hot = O.f64_to_bf16_bits(15.0 * u)
    qsl, ctx, bt_d = dev_i32(np.array([0, q_len])), dev_i32(np.array([n])), dev_i32(bt)
    for jstar in range(n):
        kk = np.zeros((nb, bs, hkv, 128), dtype=np.uint16)
        kk[bt[0, jstar // bs], jstar % bs] = hot
        pool.fill_logical(kk.view(np.int16), vk.view(np.int16))
        for plan in (pg.ChunkPlan(64, -(-n // 64), 0, 2), pg.ChunkPlan(4096, 1, 0, 2)):
            out = bits_of(pg.paged_chunk_attention(pool, q, qsl, ctx, bt_d, q_len, n, SCALE, plan=plan))
            for i in range(q_len):
                if jstar <= prefix + i:
                    for h in range(hq):
                        assert np.array_equal(out[i, h], vk[bt[0, jstar // bs], jstar % bs, h // 2]), (jstar, i, h)


def test_columns_block_permutation_bit_identical_and_deterministic():
    spec = _spec("colperm", 1723, 16, 8, 16, [(300, 5), (1000, 5), (64, 8), (0, 1)], 200)
    w = make_step(spec)
    run = StepRun(w)
    run.write()
    q = run.chunk_q()
    plan = _columns_plan(256, int(w.chk_ctx.max()))
    a = bits_of(_call(run, q, plan))
    assert np.array_equal(a, bits_of(_call(run, q, plan)))
    pk, pv, bt_c = run.read_pool()
    rng = np.random.default_rng(19)
    new_ids = rng.permutation(w.spec.num_blocks)[: len(run.used)]
    pool2 = pg.Pool(w.spec.num_blocks, 16, 8)
    pool2.fill_logical(pk.view(np.int16), pv.view(np.int16), blocks=new_ids)
    bt2 = np.where(bt_c >= 0, new_ids[np.maximum(bt_c, 0)], -1).astype(np.int32)
    qlens = np.diff(w.chk_qsl)
    b = bits_of(pg.paged_chunk_attention(pool2, q, run.chk_qsl, run.chk_ctx, dev_i32(bt2[w.num_decode:]),
                                         int(qlens.max()), int(w.chk_ctx.max()), SCALE, plan=plan))
    assert np.array_equal(a, b)


def test_columns_bad_metadata_flags_and_zero_rows():
    spec = _spec("colbad", 1725, 16, 8, 16, [(10, 4), (20, 6), (5, 3)], 16)
    w = make_step(spec)
    run = StepRun(w)
    run.write()
    q = run.chunk_q()
    plan = pg.ChunkPlan(64, 1, 0, 2)
    # segment 1 claims fewer keys than query tokens; segment 2 more than its table row holds
    ctx = dev_i32(np.array([14, 3, 16 * run.chk_bt.shape[1] + 1], dtype=np.int32))
    out = torch.full((13, 16, 128), 3.0, dtype=torch.bfloat16, device="cuda")
    big = 16 * run.chk_bt.shape[1] + 1
    pg.paged_chunk_attention(run.pool, q, run.chk_qsl, ctx, run.chk_bt, 6, big, SCALE,
                             plan=pg.ChunkPlan(64, -(-big // 64), 0, 2), out=out)
    f = run.pool.check_errors()
    assert f & pg.DEVERR_QUERY and f & pg.DEVERR_CONTEXT
    assert torch.all(out[4:] == 0)
    good = run.oracle_chunk_on_gpu_inputs(q)
    compare(out[:4], good[:4], "good segment beside bad ones")
    # query_start_loc past total_q: flagged, nothing out of bounds
    qsl = dev_i32(np.array([0, 4, 99, 99], dtype=np.int32))
    pg.paged_chunk_attention(run.pool, q, qsl, run.chk_ctx, run.chk_bt, 6, 26, SCALE, plan=plan, out=out)
    assert run.pool.check_errors() & pg.DEVERR_QUERY
    # block id outside the pool
    bt = run.chk_bt.clone()
    bt[0, 0] = 10_000
    pg.paged_chunk_attention(run.pool, q, run.chk_qsl, run.chk_ctx, bt, 6, 26, SCALE, plan=plan, out=out)
    assert run.pool.check_errors() & pg.DEVERR_BLOCK_ID


def test_columns_plan_rejected_when_segments_do_not_fit():
    w = make_step(_spec("colrej", 1726, 16, 8, 16, [(10, 9)], 16))
    run = StepRun(w)
    run.write()
    q = run.chunk_q()
    for plan in (pg.ChunkPlan(64, 1, 0, 2), pg.ChunkPlan(32, 1, 0, 2), pg.ChunkPlan(64, 1, 0, 3)):
        with pytest.raises(pg.PgqaError) as e:
            _call(run, q, plan)
        assert e.value.status == pg.PGQA_ERR_INVALID_ARG


@pytest.mark.parametrize("seed", range(24))
def test_columns_random_steps(seed):
    """Seeded random verify-like calls: head layouts, block sizes, prefixes at
    block boundaries, q_len up to the 16-column limit (empty and single-token
    segments included), default or random split plans."""
    rng = np.random.default_rng(8300 + seed)
    hq, hkv = [(16, 8), (32, 4), (8, 8), (32, 8), (8, 1), (16, 4)][int(rng.integers(6))]
    r = hq // hkv
    bs = int(rng.choice([16, 32, 64, 128, 256]))
    segs = []
    for _ in range(int(rng.integers(1, 13))):
        q_len = int(rng.integers(0, 16 // r + 1))
        prefix = int(rng.choice([0, bs - 1, bs, int(rng.integers(1, 3000))]))
        segs.append((prefix, q_len))
    if all(q == 0 for _, q in segs):
        segs[0] = (segs[0][0], 1)
    nb = sum(-(-(L + q) // bs) for L, q in segs) + 4
    w = make_step(_spec(f"colrand-{seed}", 8400 + seed, hq, hkv, bs, segs, nb))
    mc = int(w.chk_ctx.max())
    plan = None
    if rng.integers(3):
        plan = _columns_plan(int(rng.choice([64, 128, 256, 512, 1024, 4096])), mc, bs)
    _note(f"[colrand] seed {seed}: heads {hq}/{hkv} bs {bs} segments (prefix, q_len) {segs} plan {plan}")
    run = StepRun(w)
    run.write()
    q = run.chunk_q()
    out = _call(run, q, plan)
    assert run.pool.check_errors() == 0
    compare(out, run.oracle_chunk_on_gpu_inputs(q), f"seed {seed}")


def test_columns_many_splits():
    """Query-column calls with more than 32 splits (merged 32 at a time)."""
    spec = _spec("colmany", 1727, 16, 8, 16, [(3000, 5), (4990, 8), (64, 1), (2047, 3)], 1024)
    w = make_step(spec)
    run = StepRun(w)
    run.write()
    q = run.chunk_q()
    plan = _columns_plan(64, int(w.chk_ctx.max()))
    assert plan.max_splits > 64
    out = _call(run, q, plan)
    assert run.pool.check_errors() == 0
    compare(out, run.oracle_chunk_on_gpu_inputs(q), "columns, many splits")

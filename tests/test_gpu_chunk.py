"""GPU parity of paged causal chunk attention (chunked-prefill slices and
b x (k+1) verify rows) against the fp64 reference, through the C ABI."""
import numpy as np
import pytest
import torch

import oracle as O
import paged_gqa_decode_head_amd as pg
from paged_gqa_decode_head_amd.workloads import SPECS, Group, StepSpec, make_step

from harness import SCALE, SENTINEL, StepRun, bits_of, compare, dev_bf16, dev_i32, f64_of

pytestmark = pytest.mark.gpu


def _note(msg):
    print(msg, flush=True)


def test_cfg5_mixed_step_parity():
    """The mixed Qwen3-1.7B step: 8 decode streams, a 512-token slice at offset
    6144, 8 verify rows of 5 tokens; one write, one decode, one chunk call."""
    _note("[chunk] cfg5")
    w = make_step(SPECS["cfg5"])
    run = StepRun(w)
    run.write()
    qd = run.decode_q()
    out_d = run.decode(q=qd)
    qc = run.chunk_q()
    out_c = run.chunk(q=qc)
    assert run.pool.check_errors() == 0
    compare(out_d, run.oracle_decode_on_gpu_inputs(qd), "cfg5 decode")
    ma, mr = compare(out_c, run.oracle_chunk_on_gpu_inputs(qc), "cfg5 chunk")
    _note(f"  chunk max_abs={ma:.2e} mean_rel={mr:.2e}")


def _chunk_spec(name, seed, hq, hkv, bs, segs, nb):
    groups = tuple(Group(1, L, L, ql) for L, ql in segs)
    return StepSpec(name, seed, hq, hkv, nb, chunks=groups, block_size=bs)


SEGS = [(0, 7), (20, 5), (33, 1), (3, 40), (9, 0), (100, 64), (250, 33), (1, 1), (15, 17)]


@pytest.mark.parametrize("hq,hkv,bs", [(16, 8, 16), (32, 4, 16), (8, 8, 16), (32, 8, 32), (16, 8, 64),
                                       (16, 4, 256), (8, 1, 16)])
@pytest.mark.parametrize("split", [None, 64, 256, 4096])
def test_chunk_small_ragged(hq, hkv, bs, split):
    spec = _chunk_spec(f"chunk-{hq}-{hkv}-{bs}", 700 + hq + bs, hq, hkv, bs, SEGS, 256 if bs < 256 else 16)
    w = make_step(spec)
    run = StepRun(w)
    run.write()
    q = run.chunk_q()
    plan = None
    if split is not None:
        sp = max(split, bs)
        plan = pg.ChunkPlan(sp, -(-int(w.chk_ctx.max()) // sp), 0, 0)
    qlens = np.diff(w.chk_qsl)
    out = pg.paged_chunk_attention(run.pool, q, run.chk_qsl, run.chk_ctx, run.chk_bt, int(qlens.max()),
                                   int(w.chk_ctx.max()), SCALE, plan=plan)
    assert run.pool.check_errors() == 0
    compare(out, run.oracle_chunk_on_gpu_inputs(q), f"{spec.name} split={split}")


def test_chunk_q_len_one_matches_decode():
    spec = StepSpec("chunk1", 720, 16, 8, 256, chunks=(Group(6, 1, 900, 1),))
    w = make_step(spec)
    run = StepRun(w)
    run.write()
    q = run.chunk_q()
    out_c = run.chunk(q=q)
    out_d = pg.paged_decode_attention(run.pool, q, run.chk_ctx, run.chk_bt, int(w.chk_ctx.max()), SCALE)
    ref = run.oracle_chunk_on_gpu_inputs(q)
    compare(out_c, ref, "chunk q_len=1")
    compare(out_d, ref, "decode on the same rows")
    d = np.abs(f64_of(out_c) - f64_of(out_d))
    assert d.max() <= 2e-2


def test_chunk_without_prefix_is_plain_causal_attention():
    spec = _chunk_spec("causal0", 721, 16, 8, 16, [(0, 96), (0, 33)], 32)
    w = make_step(spec)
    run = StepRun(w)
    run.write()
    q = run.chunk_q()
    out = run.chunk(q=q)
    # textbook causal attention over the dense K/V of each segment (torch SDPA, fp64, CPU)
    pk, pv, bt_c = run.read_pool()
    qf = f64_of(q)
    for s in range(w.num_chunks):
        n = int(w.chk_ctx[s])
        K, V = [], []
        for g in range(8):
            kg, vg = O.gather_kv(pk, pv, bt_c[w.num_decode + s], n, g)
            K.append(kg)
            V.append(vg)
        K, V = np.stack(K), np.stack(V)
        q0, q1 = w.chk_qsl[s], w.chk_qsl[s + 1]
        ref = torch.nn.functional.scaled_dot_product_attention(
            torch.from_numpy(qf[q0:q1].transpose(1, 0, 2))[None], torch.from_numpy(K)[None],
            torch.from_numpy(V)[None], is_causal=True, enable_gqa=True)[0].numpy().transpose(1, 0, 2)
        compare(out[q0:q1], ref, f"causal segment {s}")


@pytest.mark.parametrize("q_len,i", [(12, 5), (40, 25)])   # a short segment and a wide one
def test_causal_boundary_probe(q_len, i):
    """A key placed right after a query's position must not change that query's
    output or any earlier one (bit-identical), and must change the next query's."""
    spec = _chunk_spec("probe", 722, 4, 2, 16, [(20, q_len)], 8)
    w = make_step(spec)
    run = StepRun(w)
    run.write()
    q = run.chunk_q()
    n = 20 + q_len
    plan = pg.ChunkPlan(64, 1, 0, 0)
    base = bits_of(pg.paged_chunk_attention(run.pool, q, run.chk_qsl, run.chk_ctx, run.chk_bt, q_len, n, SCALE,
                                            plan=plan))
    # query i sits at position 20 + i
    j = 20 + i + 1                               # the key right after it
    blk, off = int(w.block_tables[w.num_decode, j // 16]), j % 16
    kb, vb = run.pool.read_logical(blocks=[blk])
    kk = kb.numpy().view(np.uint16).copy()
    vv = vb.numpy().view(np.uint16).copy()
    kk[0, off] = bits_of(q[i + 1, 0::2] * 40)   # each kv head: aligned with query i+1, huge score
    vv[0, off] = O.f64_to_bf16_bits(np.full((2, 128), 50.0))
    run.pool.fill_logical(kk.view(np.int16), vv.view(np.int16), blocks=[blk])
    got = bits_of(pg.paged_chunk_attention(run.pool, q, run.chk_qsl, run.chk_ctx, run.chk_bt, q_len, n, SCALE,
                                           plan=plan))
    assert np.array_equal(got[: i + 1], base[: i + 1])
    assert not np.array_equal(got[i + 1], base[i + 1])


def test_chunk_block_permutation_bit_identical_and_deterministic():
    spec = _chunk_spec("cperm", 723, 16, 8, 16, [(300, 40), (1000, 5), (64, 64)], 200)
    w = make_step(spec)
    run = StepRun(w)
    run.write()
    q = run.chunk_q()
    plan = pg.ChunkPlan(256, 5, 0, 0)
    qlens = np.diff(w.chk_qsl)
    call = lambda pool, bt: bits_of(pg.paged_chunk_attention(pool, q, run.chk_qsl, run.chk_ctx, bt,
                                                             int(qlens.max()), int(w.chk_ctx.max()), SCALE,
                                                             plan=plan))
    a = call(run.pool, run.chk_bt)
    assert np.array_equal(a, call(run.pool, run.chk_bt))
    pk, pv, bt_c = run.read_pool()
    rng = np.random.default_rng(9)
    new_ids = rng.permutation(w.spec.num_blocks)[: len(run.used)]
    pool2 = pg.Pool(w.spec.num_blocks, 16, 8)
    pool2.fill_logical(pk.view(np.int16), pv.view(np.int16), blocks=new_ids)
    bt2 = np.where(bt_c >= 0, new_ids[np.maximum(bt_c, 0)], -1).astype(np.int32)
    assert np.array_equal(a, call(pool2, dev_i32(bt2[w.num_decode:])))


@pytest.mark.parametrize("bs", [16, 32, 64, 256])
def test_chunk_ignores_garbage_past_the_context(bs):
    """Every cache slot outside the attended keys holds the sentinel (a NaN):
    split ends inside a block, keys past a wide split's end and the unused
    slots of the last block must not reach the output, at every block size."""
    spec = _chunk_spec(f"cgarb-{bs}", 724, 16, 8, bs, [(10, 7), (50, 30), (0, 3)], 40)
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
    for split in (None, 32, 64):
        plan = None if split is None else pg.ChunkPlan(max(split, bs), -(-80 // split), split, 0)
        out = pg.paged_chunk_attention(run.pool, q, run.chk_qsl, run.chk_ctx, run.chk_bt, 30, 80, SCALE, plan=plan)
        compare(out, run.oracle_chunk_on_gpu_inputs(q), f"chunk garbage bs={bs} split={split}")


def test_chunk_bad_metadata_flags_and_zero_rows():
    spec = _chunk_spec("cbad", 725, 16, 8, 16, [(10, 4), (20, 6)], 16)
    w = make_step(spec)
    run = StepRun(w)
    run.write()
    q = run.chunk_q()
    # second segment claims fewer keys than query tokens
    ctx = dev_i32(np.array([14, 3], dtype=np.int32))
    out = torch.full((10, 16, 128), 3.0, dtype=torch.bfloat16, device="cuda")
    pg.paged_chunk_attention(run.pool, q, run.chk_qsl, ctx, run.chk_bt, 6, 26, SCALE, out=out)
    assert run.pool.check_errors() & pg.DEVERR_QUERY
    assert torch.all(out[4:] == 0)
    assert torch.all(torch.isfinite(out[:4].float()))
    # query_start_loc past total_q
    qsl = dev_i32(np.array([0, 4, 99], dtype=np.int32))
    pg.paged_chunk_attention(run.pool, q, qsl, run.chk_ctx, run.chk_bt, 6, 26, SCALE, out=out)
    assert run.pool.check_errors() & pg.DEVERR_QUERY
    # empty call
    pg.paged_chunk_attention(run.pool, q[:0], run.chk_qsl[:1], run.chk_ctx[:0], run.chk_bt[:0], 0, 0, SCALE,
                             out=out[:0])
    assert run.pool.check_errors() == 0


@pytest.mark.parametrize("bs", [16, 256])
def test_chunk_wide_split_over_several_windows(bs):
    """Wide items whose split is longer than the 1024 keys the lanes hold block
    ids for at a time: the split streams through several windows."""
    spec = _chunk_spec(f"cwin{bs}", 728, 16, 8, bs, [(3000, 64), (1500, 40)], 3200 // bs * 2 + 8)
    w = make_step(spec)
    run = StepRun(w)
    run.write()
    q = run.chunk_q()
    mc = int(w.chk_ctx.max())
    _note(f"[chunk] windows bs={bs}")
    for split in (4096, 2048, 1056):
        out = pg.paged_chunk_attention(run.pool, q, run.chk_qsl, run.chk_ctx, run.chk_bt, 64, mc, SCALE,
                                       plan=pg.ChunkPlan(split, -(-mc // 256), 256, 1))
        assert run.pool.check_errors() == 0
        compare(out, run.oracle_chunk_on_gpu_inputs(q), f"split {split}")


def test_chunk_last_offset_must_equal_total_q():
    """A lone segment whose offsets end before total_q: the host sized the call
    as one wide segment (40 tokens, 80 rows per kv head), the device offsets
    claim 10 tokens (20 rows, one tile).  The segment is flagged and its
    claimed rows zeroed; nothing reads stale partials."""
    spec = _chunk_spec("cend", 726, 16, 8, 16, [(30, 40)], 16)
    w = make_step(spec)
    run = StepRun(w)
    run.write()
    q = run.chunk_q()
    out = torch.full((40, 16, 128), 3.0, dtype=torch.bfloat16, device="cuda")
    qsl = dev_i32(np.array([0, 10], dtype=np.int32))
    _note("[chunk] lone segment ending before total_q")
    pg.paged_chunk_attention(run.pool, q, qsl, run.chk_ctx, run.chk_bt, 40, 70, SCALE, out=out)
    assert run.pool.check_errors() & pg.DEVERR_QUERY
    assert torch.all(out[:10] == 0)
    assert torch.all(out[10:] == 3.0)
    # the same on the query-column route (two short segments, the last ending early)
    spec = _chunk_spec("cend2", 727, 16, 8, 16, [(30, 5), (12, 5)], 16)
    w = make_step(spec)
    run = StepRun(w)
    run.write()
    q = run.chunk_q()
    out = torch.full((10, 16, 128), 3.0, dtype=torch.bfloat16, device="cuda")
    qsl = dev_i32(np.array([0, 5, 8], dtype=np.int32))
    pg.paged_chunk_attention(run.pool, q, qsl, run.chk_ctx, run.chk_bt, 5, 35, SCALE, out=out,
                             plan=pg.ChunkPlan(64, 1, 0, 2))
    assert run.pool.check_errors() & pg.DEVERR_QUERY
    assert torch.all(out[5:8] == 0)
    good = run.oracle_chunk_on_gpu_inputs(q)
    compare(out[:5], good[:5], "good segment before the bad one")


@pytest.mark.parametrize("q_len", [5, 40])  # a short (verify-sized) and a wide segment
def test_chunk_addressing_probe_one_hot_every_position(q_len):
    """Only key j* matches every query strongly: each query that sees j* must
    return V_j* bit-exactly, for every logical position j* (every block-table
    entry and offset), for a short and a wide segment, with one and many splits."""
    bs, hkv, hq = 16, 2, 4
    prefix = 60
    n = prefix + q_len
    nb = 24
    rng = np.random.default_rng(17 + q_len)
    perm = rng.permutation(nb)
    nblk = -(-n // bs)
    bt = np.full((1, nblk), -1, dtype=np.int32)
    bt[0] = perm[:nblk]
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
        for plan in (pg.ChunkPlan(32, -(-n // 32), 32, 0), pg.ChunkPlan(4096, 1, 4096, 0)):
            out = bits_of(pg.paged_chunk_attention(pool, q, qsl, ctx, bt_d, q_len, n, SCALE, plan=plan))
            for i in range(q_len):
                if jstar <= prefix + i:  # query i sees key j*
                    for h in range(hq):
                        assert np.array_equal(out[i, h], vk[bt[0, jstar // bs], jstar % bs, h // 2]), (jstar, i, h)



@pytest.mark.parametrize("seed", range(12))
def test_chunk_random_mixed_steps(seed):
    """Seeded random mixed steps: wide segments (more than 32 rows per kv head)
    and short ones (verify rows, single tokens, empty) in one call, random
    prefixes (block boundaries included), head layouts, block sizes and split
    plans, against the fp64 reference."""
    rng = np.random.default_rng(7300 + seed)
    hq, hkv = [(16, 8), (32, 4), (8, 8), (32, 8), (8, 1), (16, 4)][int(rng.integers(6))]
    bs = int(rng.choice([16, 32, 64, 128, 256]))
    segs = []
    for _ in range(int(rng.integers(1, 9))):
        kind = int(rng.integers(4))
        q_len = [int(rng.integers(17, 160)), int(rng.integers(2, 9)), 1, 0][kind]
        prefix = int(rng.choice([0, bs - 1, bs, int(rng.integers(1, 1500))]))
        segs.append((prefix, q_len))
    if all(q == 0 for _, q in segs):  # at least one query token in the call
        segs[0] = (segs[0][0], 1)
    nb = sum(-(-(L + q) // bs) for L, q in segs) + 4
    spec = _chunk_spec(f"crand-{seed}", 7400 + seed, hq, hkv, bs, segs, nb)
    w = make_step(spec)
    plan = None
    mc = int(w.chk_ctx.max())
    if rng.integers(3):
        wide = int(rng.choice([32, 64, 128, 256, 1024]))
        short = int(rng.choice([0, 32, 64, 256]))
        smallest = min(wide, short) if short else wide
        plan = pg.ChunkPlan(wide, -(-mc // smallest), short, 0)
    _note(f"[crand] seed {seed}: heads {hq}/{hkv} bs {bs} segments (prefix, q_len) {segs} plan {plan}")
    run = StepRun(w)
    run.write()
    q = run.chunk_q()
    qlens = np.diff(w.chk_qsl)
    out = pg.paged_chunk_attention(run.pool, q, run.chk_qsl, run.chk_ctx, run.chk_bt, int(qlens.max()), mc, SCALE,
                                   plan=plan)
    assert run.pool.check_errors() == 0
    compare(out, run.oracle_chunk_on_gpu_inputs(q), f"seed {seed}")


@pytest.mark.parametrize("hq,hkv", [(16, 8), (32, 4)])
def test_chunk_more_than_64_segments(hq, hkv):
    """A call of 70 segments (wide, short, single-token and empty ones) with
    forced short splits: its combine finds items by scanning the metadata
    (the row combine serves calls of at most 64 segments).  Against the fp64
    reference, and the first 64 segments bit-identical to the same segments
    called alone (row combine, same split plan)."""
    rng = np.random.default_rng(9700 + hq)
    bs = 16
    segs = []
    for i in range(70):
        q_len = [40, 3, 1, 0, 24][i % 5]
        segs.append((int(rng.integers(0, 300)), q_len))
    nb = sum(-(-(L + q) // bs) for L, q in segs) + 4
    w = make_step(_chunk_spec(f"cseg70-{hq}", 9710 + hq, hq, hkv, bs, segs, nb))
    run = StepRun(w)
    run.write()
    q = run.chunk_q()
    qsl, ctx = w.chk_qsl, w.chk_ctx
    mq, mc = int(np.diff(qsl).max()), int(ctx.max())
    plan = pg.ChunkPlan(64, -(-mc // 32), 32, 0)
    _note(f"[cseg70] heads {hq}/{hkv}: 70 segments, plan {plan}")
    out = pg.paged_chunk_attention(run.pool, q, run.chk_qsl, run.chk_ctx, run.chk_bt, mq, mc, SCALE, plan=plan)
    assert run.pool.check_errors() == 0
    compare(out, run.oracle_chunk_on_gpu_inputs(q), "70 segments")
    t64 = int(qsl[64])
    out64 = pg.paged_chunk_attention(run.pool, q[:t64].contiguous(), dev_i32(qsl[:65]), dev_i32(ctx[:64]),
                                     run.chk_bt[:64].contiguous(), int(np.diff(qsl[:65]).max()), int(ctx[:64].max()),
                                     SCALE, plan=plan)
    assert run.pool.check_errors() == 0
    assert np.array_equal(bits_of(out64), bits_of(out[:t64]))


def test_chunk_bad_segment_beside_split_rows():
    """A bad segment between two good ones, with every row split: the bad rows
    come back zero with the flag raised, and the combine still merges the good
    rows around them (some combine workgroups hold rows of both kinds)."""
    segs = [(300, 41), (200, 6), (500, 3)]
    nb = sum(-(-(L + q) // 16) for L, q in segs) + 4
    w = make_step(_chunk_spec("cbadsplit", 9740, 16, 8, 16, segs, nb))
    run = StepRun(w)
    run.write()
    q = run.chunk_q()
    ref = run.oracle_chunk_on_gpu_inputs(q)
    qsl = w.chk_qsl
    mq, mc = int(np.diff(qsl).max()), int(w.chk_ctx.max())
    plan = pg.ChunkPlan(64, -(-mc // 64), 64, 0)
    ctx = w.chk_ctx.copy()
    ctx[1] = 2  # fewer keys than the segment's 6 query tokens
    out = torch.full((int(qsl[-1]), 16, 128), 3.0, dtype=torch.bfloat16, device="cuda")
    pg.paged_chunk_attention(run.pool, q, run.chk_qsl, dev_i32(ctx), run.chk_bt, mq, mc, SCALE, out=out, plan=plan)
    assert run.pool.check_errors() & pg.DEVERR_QUERY
    a, b = int(qsl[1]), int(qsl[2])
    assert torch.all(out[a:b] == 0)
    keep = np.r_[0:a, b:int(qsl[-1])]
    compare(out[torch.from_numpy(keep).to(out.device)], ref[keep], "good segments beside a bad one")


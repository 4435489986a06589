"""The mixed-step planner (pgqa_plan_mixed, host only): its work list covers
every (segment, kv head, row, key) exactly once, the combine items cover
exactly the rows with several splits, and the list is ordered as documented.
Checked here against a walk of the definitions, on the CPU."""
import numpy as np
import pytest

import paged_gqa_decode_head_amd as pg

WIDE, COLUMN, COMBINE = 0, 1, 2


def _segments(rng, n_seg, bs):
    qls, ctx = [], []
    for _ in range(n_seg):
        q_len = [int(rng.integers(17, 700)), int(rng.integers(2, 9)), 1, 0][int(rng.integers(4))]
        prefix = int(rng.choice([0, bs - 1, bs, int(rng.integers(1, 9000))]))
        qls.append(q_len)
        ctx.append(prefix + q_len)
    return np.concatenate([[0], np.cumsum(qls)]).astype(np.int32), np.array(ctx, dtype=np.int32)


def _check_plan(plan, items, qsl, ctx, hkv, r, bs, cus=256):
    att, comb = items[: plan.num_items], items[plan.num_items:]
    assert len(comb) == plan.num_combine
    assert plan.split_wide % 32 == 0 and 0 < plan.split_wide <= 4096
    assert plan.split_columns % max(64, bs) == 0 and 0 < plan.split_columns <= 4096
    covered = {}
    for it in att:
        s, kind, g, grp, sp, q0, qlen, n = (int(x) for x in it)
        assert (q0, qlen, n) == (int(qsl[s]), int(qsl[s + 1] - qsl[s]), int(ctx[s]))
        assert kind == (WIDE if qlen * r > 16 else COLUMN) and 0 <= g < hkv
        if kind == WIDE:
            rows = range(grp * 128, min((grp + 1) * 128, qlen * r))
            assert len(rows) > 0
            split = plan.split_wide
        else:
            rows = range(qlen * r)
            assert grp == 0
            split = plan.split_columns
        for rho in rows:
            pos = n - qlen + rho // r                      # the row's query position
            covered.setdefault((s, g, rho), []).append((sp * split, min((sp + 1) * split, n), pos))
    # every row of every segment and kv head: its keys 0 .. pos covered once, in split order
    max_ns = 1
    need_combine = set()
    for s in range(len(ctx)):
        qlen, n = int(qsl[s + 1] - qsl[s]), int(ctx[s])
        for g in range(hkv):
            for rho in range(qlen * r):
                ranges = sorted(covered.pop((s, g, rho)))
                pos = ranges[0][2]
                # the item's rows share one key bound: the last row of its group (wide) or n (column)
                assert ranges[0][0] == 0
                for (a0, a1, _), (b0, _, _) in zip(ranges, ranges[1:]):
                    assert a1 == b0
                end = ranges[-1][1]
                assert end > pos and (end == n or end - ranges[-1][0] <= 4096)
                assert all(a1 > a0 for a0, a1, _ in ranges)
                max_ns = max(max_ns, len(ranges))
                if len(ranges) > 1:
                    need_combine.add((s, g, rho, len(ranges)))
    assert not covered
    assert plan.max_splits == max_ns
    got = set()
    for it in comb:
        s, kind, g, rho0, ns, q0, qlen, n = (int(x) for x in it)
        assert kind == COMBINE and ns >= 2
        for rho in range(rho0, min(rho0 + 8, qlen * r)):
            assert (s, g, rho, ns) not in got
            got.add((s, g, rho, ns))
    assert got == need_combine
    # order: wide and column items alternate in runs of num_cus; wide items
    # keep the kv head fastest (and land on XCD position % 8), column items go
    # most keys first, in (segment, split, kv head) order among equals
    kinds = att[:, 1]
    wide_pos = np.nonzero(kinds == WIDE)[0]
    col_pos = np.nonzero(kinds == COLUMN)[0]
    nw, nc = len(wide_pos), len(col_pos)
    expect = []
    wi = ci = 0
    while wi < nw or ci < nc:
        take = min(cus, nw - wi)
        expect += [WIDE] * take
        wi += take
        take = min(cus, nc - ci)
        expect += [COLUMN] * take
        ci += take
    assert kinds.tolist() == expect
    assert np.array_equal(att[wide_pos, 2], np.arange(nw) % hkv)
    if 8 % hkv == 0:
        assert np.array_equal(att[wide_pos, 2], wide_pos % hkv)
    keys = [min(plan.split_columns, int(it[7]) - int(it[4]) * plan.split_columns) for it in att[col_pos]]
    assert keys == sorted(keys, reverse=True)
    order = [(-k, int(it[0]), int(it[4]), int(it[2])) for k, it in zip(keys, att[col_pos])]
    assert order == sorted(order)


@pytest.mark.parametrize("seed", range(24))
def test_mixed_plan_covers_every_row_and_key_once(seed):
    rng = np.random.default_rng(500 + seed)
    hq, hkv = [(16, 8), (32, 4), (8, 8), (32, 8), (8, 1), (16, 4)][seed % 6]
    bs = [16, 32, 64, 128, 256][seed % 5]
    qsl, ctx = _segments(rng, int(rng.integers(1, 12)), bs)
    splits = [(0, 0), (32, max(64, bs)), (256, 0), (0, 4096 // max(64, bs) * max(64, bs))][seed % 4]
    cus = [256, 8, 80, 304][(seed // 4) % 4]   # runs that end part-way through either list
    plan, items = pg.plan_mixed(cus, bs, hkv, hq, qsl, ctx, *splits)
    _check_plan(plan, items, qsl, ctx, hkv, hq // hkv, bs, cus)


def test_mixed_plan_of_the_qwen3_mixed_step():
    from paged_gqa_decode_head_amd.workloads import SPECS, make_step

    w = make_step(SPECS["cfg5"])
    qsl = np.concatenate([[0], np.cumsum(np.concatenate([np.ones(w.num_decode, dtype=np.int64),
                                                         np.diff(w.chk_qsl)]))]).astype(np.int32)
    ctx = np.concatenate([w.dec_ctx, w.chk_ctx]).astype(np.int32)
    plan, items = pg.plan_mixed(256, 16, 8, 16, qsl, ctx)
    _check_plan(plan, items, qsl, ctx, 8, 2, 16)
    # the wide work (8 row groups x 8 kv heads, up to 6656 keys) and the columns'
    # K/V split the slots about evenly: one wide item per CU, 4 splits of 1664 keys
    assert (plan.split_wide, int((items[: plan.num_items, 1] == WIDE).sum())) == (1664, 8 * 8 * 4)


def test_mixed_plan_rejects_bad_host_metadata_and_small_buffers():
    L = pg.lib()
    import ctypes

    plan = pg.MixedPlan()
    for qsl, ctx in (([1, 3], [4]), ([0, 5, 3], [6, 6]), ([0, 5], [4])):
        q = np.array(qsl, dtype=np.int32)
        c = np.array(ctx, dtype=np.int32)
        st = L.pgqa_plan_mixed(256, 16, 8, 16, c.size, q.ctypes.data, c.ctypes.data, 0, 0, None, 0,
                               ctypes.byref(plan))
        assert st == pg.PGQA_ERR_INVALID_ARG, (qsl, ctx)
    q = np.array([0, 40], dtype=np.int32)
    c = np.array([5000], dtype=np.int32)
    assert L.pgqa_plan_mixed(256, 16, 8, 16, 1, q.ctypes.data, c.ctypes.data, 0, 0, None, 0, ctypes.byref(plan)) == 0
    buf = np.zeros((plan.num_items + plan.num_combine - 1, 8), dtype=np.int32)
    st = L.pgqa_plan_mixed(256, 16, 8, 16, 1, q.ctypes.data, c.ctypes.data, 0, 0, buf.ctypes.data, buf.shape[0],
                           ctypes.byref(plan))
    assert st == pg.PGQA_ERR_INVALID_ARG and b"item buffer" in L.pgqa_last_error()
    for sw, sc in ((48, 0), (0, 96), (8192, 0)):
        assert L.pgqa_plan_mixed(256, 16, 8, 16, 1, q.ctypes.data, c.ctypes.data, sw, sc, None, 0,
                                 ctypes.byref(plan)) == pg.PGQA_ERR_INVALID_ARG

"""GPU parity of the one-launch mixed step (pgqa_plan_mixed on the host, then
pgqa_paged_mixed_attention: decode rows, prefill slices and verify rows in one
attention launch plus one combine) against the fp64 reference, through the C
ABI."""
import numpy as np
import pytest
import torch

import oracle as O
import paged_gqa_decode_head_amd as pg
from paged_gqa_decode_head_amd.workloads import SPECS, Group, StepSpec, make_step

from harness import SCALE, StepRun, bits_of, compact, compare, dev_bf16, dev_i32, f64_of

pytestmark = pytest.mark.gpu

CUS = None


def _note(msg):
    print(msg, flush=True)


def _cus():
    global CUS
    if CUS is None:
        CUS = torch.cuda.get_device_properties(0).multi_processor_count
    return CUS


def _all_segments(w):
    """Every row of the step as one mixed call: decode rows (one token each)
    first, then the chunk segments; q rows are the write's tokens in order."""
    qlens = np.concatenate([np.ones(w.num_decode, dtype=np.int64), np.diff(w.chk_qsl)])
    qsl = np.concatenate([[0], np.cumsum(qlens)]).astype(np.int32)
    ctx = np.concatenate([w.dec_ctx, w.chk_ctx]).astype(np.int32)
    return qsl, ctx


class MixedRun:
    def __init__(self, w, split_wide=0, split_columns=0):
        self.w = w
        s = w.spec
        self.run = StepRun(w)
        self.run.write()
        self.qsl, self.ctx = _all_segments(w)
        self.plan, items = pg.plan_mixed(_cus(), s.block_size, s.num_kv_heads, s.num_q_heads, self.qsl, self.ctx,
                                         split_wide, split_columns)
        self.items = dev_i32(items.reshape(-1, 8)) if items.size else torch.zeros((1, 8), dtype=torch.int32,
                                                                                      device="cuda")
        self.q = self.run.q_out
        self.qsl_d, self.ctx_d, self.bt_d = dev_i32(self.qsl), dev_i32(self.ctx), self.run.bt
        self.max_q = int(np.diff(self.qsl).max()) if len(self.ctx) else 0
        self.max_ctx = int(self.ctx.max()) if len(self.ctx) else 0

    def call(self, out=None, pool=None, bt=None, qsl=None, ctx=None):
        return pg.paged_mixed_attention(pool or self.run.pool, self.q, self.qsl_d if qsl is None else qsl,
                                        self.ctx_d if ctx is None else ctx, self.bt_d if bt is None else bt,
                                        self.max_q, self.max_ctx, SCALE, self.plan, self.items, out=out)

    def oracle(self):
        """fp64 reference on the library's own q_out and cache contents."""
        pk, pv, bt_c = self.run.read_pool()
        return O.chunk_attention(f64_of(self.q), self.qsl, pk, pv, bt_c, self.ctx, SCALE)


def test_mixed_qwen3_step_parity():
    """The mixed Qwen3-1.7B step (8 decode streams, a 512-token slice at offset
    6144, 8 verify rows of 5 tokens) in one attention launch."""
    _note("[mixed] cfg5")
    m = MixedRun(make_step(SPECS["cfg5"]))
    _note(f"  plan {m.plan}")
    out = m.call()
    assert m.run.pool.check_errors() == 0
    ref = m.oracle()
    nd = m.w.num_decode
    compare(out[:nd], ref[:nd], "decode rows")
    compare(out[nd:nd + 512], ref[nd:nd + 512], "prefill slice")
    ma, mr = compare(out[nd + 512:], ref[nd + 512:], "verify rows")
    _note(f"  verify max_abs={ma:.2e} mean_rel={mr:.2e}")
    compare(out, ref, "whole step")


def _spec(name, seed, hq, hkv, bs, segs, decode=()):
    nb = sum(-(-(L + q) // bs) for L, q in segs) + sum(-(-(L + 1) // bs) for L in decode) + 4
    return StepSpec(name, seed, hq, hkv, nb, decode=tuple(Group(1, L, L) for L in decode),
                    chunks=tuple(Group(1, L, L, q) for L, q in segs), block_size=bs)


@pytest.mark.parametrize("seed", range(32))
def test_mixed_random_steps(seed):
    """Seeded random steps: decode rows, wide segments (prefill slices), short
    ones (verify rows, single tokens) and empty ones in one call, random
    prefixes (block boundaries included), head layouts, block sizes and
    splits (planner or forced: many short splits), against the fp64 reference."""
    rng = np.random.default_rng(8300 + seed)
    hq, hkv = [(16, 8), (32, 4), (8, 8), (32, 8), (8, 1), (16, 4)][int(rng.integers(6))]
    bs = int(rng.choice([16, 32, 64, 128, 256]))
    r = hq // hkv
    segs = []
    for _ in range(int(rng.integers(1, 8))):
        kind = int(rng.integers(4))
        q_len = [int(rng.integers(17 // r + 1, 200)), int(rng.integers(2, 16 // r + 2)), 1, 0][kind]
        prefix = int(rng.choice([0, bs - 1, bs, int(rng.integers(1, 1500))]))
        segs.append((prefix, q_len))
    decode = [int(rng.integers(0, 2500)) for _ in range(int(rng.integers(0, 5)))]
    if all(q == 0 for _, q in segs) and not decode:
        segs[0] = (segs[0][0], 1)
    w = make_step(_spec(f"mrand-{seed}", 8400 + seed, hq, hkv, bs, segs, decode))
    gran = max(64, bs)
    sw, sc = [(0, 0), (32, gran), (64, 2 * gran), (0, gran)][seed % 4]
    _note(f"[mrand] seed {seed}: heads {hq}/{hkv} bs {bs} decode {decode} segments {segs} splits {sw}/{sc}")
    m = MixedRun(w, sw, sc)
    out = m.call()
    assert m.run.pool.check_errors() == 0
    compare(out, m.oracle(), f"seed {seed}")


def test_mixed_causal_boundary_probe():
    """A key placed right after a query's position changes neither that query's
    output nor any earlier one (bit-identical), and changes the next query's;
    for a wide segment and a column segment of one call."""
    w = make_step(_spec("mprobe", 8501, 4, 2, 16, [(20, 40), (33, 6)]))
    m = MixedRun(w, 64, 64)
    base = bits_of(m.call())
    for seg, i in ((0, 25), (1, 2)):
        L, q_len = [(20, 40), (33, 6)][seg]
        q0 = int(m.qsl[seg])
        j = L + i + 1
        blk, off = int(w.block_tables[w.num_decode + seg, j // 16]), j % 16
        kb, vb = m.run.pool.read_logical(blocks=[blk])
        k0, v0 = kb.clone(), vb.clone()
        kk = kb.numpy().view(np.uint16).copy()
        vv = vb.numpy().view(np.uint16).copy()
        kk[0, off] = bits_of(m.q[q0 + i + 1, 0::2] * 40)   # each kv head: aligned with query i+1, huge score
        vv[0, off] = O.f64_to_bf16_bits(np.full((2, 128), 50.0))
        m.run.pool.fill_logical(kk.view(np.int16), vv.view(np.int16), blocks=[blk])
        got = bits_of(m.call())
        assert np.array_equal(got[q0:q0 + i + 1], base[q0:q0 + i + 1]), seg
        assert not np.array_equal(got[q0 + i + 1], base[q0 + i + 1]), seg
        m.run.pool.fill_logical(k0, v0, blocks=[blk])


def test_mixed_block_permutation_bit_identical_and_deterministic():
    w = make_step(_spec("mperm", 8502, 16, 8, 16, [(300, 40), (1000, 5), (64, 64)], decode=[700, 33]))
    m = MixedRun(w, 128, 256)
    a = bits_of(m.call())
    assert np.array_equal(a, bits_of(m.call()))
    pk, pv, bt_c = m.run.read_pool()
    rng = np.random.default_rng(3)
    nb = len(m.run.used) + 9
    new_ids = rng.permutation(nb)[: len(m.run.used)]
    pool2 = pg.Pool(nb, 16, 8)
    pool2.fill_logical(pk.view(np.int16), pv.view(np.int16), blocks=new_ids)
    bt2 = np.where(bt_c >= 0, new_ids[np.maximum(bt_c, 0)], -1).astype(np.int32)
    b = bits_of(m.call(pool=pool2, bt=dev_i32(bt2)))
    assert np.array_equal(a, b)


def test_mixed_device_metadata_mismatch_flags_and_zeroes_rows():
    """Items planned for one set of lengths, device metadata that differs for
    one segment: that segment is flagged and its rows zeroed, the others are
    still computed."""
    w = make_step(_spec("mbad", 8503, 16, 8, 16, [(100, 40), (50, 5), (70, 3)], decode=[90]))
    m = MixedRun(w)
    ctx = m.ctx.copy()
    ctx[2] -= 1                                    # segment 2 (5 verify rows): one key less on the device
    out = torch.full_like(m.q, 3.0)
    m.call(out=out, ctx=dev_i32(ctx))
    assert m.run.pool.check_errors() & pg.DEVERR_QUERY
    q0, q1 = int(m.qsl[2]), int(m.qsl[3])
    assert torch.all(out[q0:q1] == 0)
    ref = m.oracle()
    keep = np.r_[0:q0, q1:int(m.qsl[-1])]
    compare(out[keep], ref[keep], "other segments")
    # a wide segment whose offsets moved on the device
    qsl = m.qsl.copy()
    qsl[2] += 1                                   # segment 1 (the 40-token slice) ends one row later
    out = torch.full_like(m.q, 3.0)
    m.call(out=out, qsl=dev_i32(qsl))
    assert m.run.pool.check_errors() & pg.DEVERR_QUERY
    assert torch.all(out[int(m.qsl[1]):int(m.qsl[2])] == 0)
    # a block id outside the pool
    bt = m.bt_d.clone()
    bt[0, 0] = 10_000
    m.call(bt=bt)
    assert m.run.pool.check_errors() & pg.DEVERR_BLOCK_ID


@pytest.mark.parametrize("q_len", [5, 40])
def test_mixed_addressing_probe_one_hot_every_position(q_len):
    """Only key j* matches every query strongly: each query that sees j* must
    return V_j* bit-exactly, for every logical position j*, on a column and a
    wide segment, with one and many splits."""
    bs, hkv, hq = 16, 2, 4
    prefix = 60
    n = prefix + q_len
    nb = 24
    rng = np.random.default_rng(27 + q_len)
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
    qsl_h, ctx_h = np.array([0, q_len], dtype=np.int32), np.array([n], dtype=np.int32)
    qsl, ctx, bt_d = dev_i32(qsl_h), dev_i32(ctx_h), dev_i32(bt)
    plans = []
    for sw, sc in ((32, 64), (4096, 4096)):
        plan, items = pg.plan_mixed(_cus(), bs, hkv, hq, qsl_h, ctx_h, sw, sc)
        plans.append((plan, dev_i32(items)))
    for jstar in range(n):
        kk = np.zeros((nb, bs, hkv, 128), dtype=np.uint16)
        kk[bt[0, jstar // bs], jstar % bs] = hot
        pool.fill_logical(kk.view(np.int16), vk.view(np.int16))
        for plan, items in plans:
            out = bits_of(pg.paged_mixed_attention(pool, q, qsl, ctx, bt_d, q_len, n, SCALE, plan, items))
            for i in range(q_len):
                if jstar <= prefix + i:
                    for h in range(hq):
                        assert np.array_equal(out[i, h], vk[bt[0, jstar // bs], jstar % bs, h // 2]), (jstar, i, h)
    assert pool.check_errors() == 0

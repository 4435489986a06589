"""The C-ABI library builds for gfx950, loads and exports what include/pgqa.h and
include/pgqa_sched.h declare; host-side checks and the split planner work
without a GPU."""
import ctypes
import os
import re

import pytest

import paged_gqa_decode_head_amd as pg

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared_functions():
    src = "".join(open(os.path.join(ROOT, "include", h)).read() for h in ("pgqa.h", "pgqa_sched.h"))
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(pgqa_[a-z_]+)\s*\(", src)))


def test_library_exports_every_declared_symbol():
    L = pg.lib()
    declared = _declared_functions()
    assert len(declared) >= 14
    for name in declared:
        assert hasattr(L, name), name
    assert sorted(pg.exported_symbols()) == declared


def test_library_is_built_for_gfx950():
    data = open(pg.LIB_PATH, "rb").read()
    assert b"gfx950" in data


def test_version_and_status_strings():
    assert re.fullmatch(r"\d+\.\d+\.\d+", pg.version())
    for s in range(7):
        assert pg.lib().pgqa_status_string(s)


def test_pool_bytes():
    assert pg.pool_bytes(32, 16, 8) == 32 * 8 * 2 * 16 * 128 * 2
    assert pg.pool_bytes(7680, 16, 4) == 7680 * 4 * 2 * 16 * 128 * 2
    assert pg.pool_bytes(10, 256, 2) == 10 * 2 * 2 * 256 * 128 * 2
    assert pg.pool_bytes(32, 24, 8) == 0        # block size not a supported power of two
    assert pg.pool_bytes(32, 16, 8, head_dim=64) == 0
    assert pg.pool_bytes(0, 16, 8) == 0


def test_pool_create_rejects_bad_config_before_touching_the_device():
    L = pg.lib()
    h = ctypes.c_void_p()
    cfg = pg.PoolConfig(32, 16, 8, 64, 0)
    assert L.pgqa_pool_create(ctypes.byref(cfg), None, ctypes.byref(h)) == 2   # head_dim 64: unsupported
    assert b"head_dim" in L.pgqa_last_error()
    cfg = pg.PoolConfig(32, 48, 8, 128, 0)
    assert L.pgqa_pool_create(ctypes.byref(cfg), None, ctypes.byref(h)) == 2
    cfg = pg.PoolConfig(0, 16, 8, 128, 0)
    assert L.pgqa_pool_create(ctypes.byref(cfg), None, ctypes.byref(h)) == 1
    assert L.pgqa_pool_create(None, None, ctypes.byref(h)) == 1
    assert L.pgqa_pool_create(ctypes.byref(cfg), None, None) == 1


def test_calls_reject_null_pool():
    L = pg.lib()
    assert L.pgqa_paged_decode_attention(None, None, None, None, 1, 1, 16, 10, 0.1, None, None, 0, None,
                                         None) == 1
    assert L.pgqa_rms_norm_rope_cache_write(None, None, 0, None, 0, None, 0, None, None, None, None, None, 1, 1,
                                            1, 16, 1e-6, 1e6, None, None) == 1
    assert L.pgqa_pool_destroy(None) == 0
    flags = ctypes.c_uint32()
    assert L.pgqa_pool_check_errors(None, None, ctypes.byref(flags)) == 1


@pytest.mark.parametrize("cus", [256, 304, 80])
@pytest.mark.parametrize("bs", [16, 32, 256])
@pytest.mark.parametrize("batch,hkv,ctx", [(1, 8, 32769), (64, 8, 2049), (8, 8, 4097), (64, 4, 1281),
                                            (2, 8, 101), (1, 1, 1), (512, 8, 100000)])
def test_decode_plan_properties(cus, bs, batch, hkv, ctx):
    for r in (1, 2, 8):
        p = pg.plan_decode(cus, bs, batch, hkv, r * hkv, ctx)
        gran = max(bs, 64)
        assert p.split_tokens % gran == 0
        assert 0 < p.split_tokens <= min(4096, 1024 * p.waves_per_split)
        assert p.max_splits == -(-ctx // p.split_tokens)          # covers every key, no empty tail split
        assert p.waves_per_split in (1, 2, 4, 8)
        assert p.load_hint == 0
        if 2 * batch * hkv >= cus:
            assert p.max_splits == -(-ctx // min(4096, 1024 * p.waves_per_split)) or p.max_splits == 1
        elif ctx >= 8192:
            assert batch * hkv * p.max_splits >= cus // 4            # long contexts spread over the chip


def test_plan_rejects_bad_input():
    with pytest.raises(pg.PgqaError):
        pg.plan_decode(0, 16, 1, 8, 16, 100)
    with pytest.raises(pg.PgqaError):
        pg.plan_decode(256, 24, 1, 8, 16, 100)


@pytest.mark.parametrize("cus", [256, 80])
@pytest.mark.parametrize("bs", [16, 64, 256])
@pytest.mark.parametrize("segs,total_q,max_q,ctx", [(8, 40, 5, 4101), (9, 552, 512, 6656), (64, 64, 1, 2049),
                                                     (1, 16, 16, 32784), (3, 9, 3, 700), (1, 1, 1, 1)])
def test_chunk_plan_properties(cus, bs, segs, total_q, max_q, ctx):
    """The chunk planner takes the query-column route (kernel 2) exactly when
    every segment fits 16 MFMA columns (max_q_len x group <= 16); its splits
    then follow the decode kernels' rules, else the chunk kernels' (multiples
    of 32)."""
    for hkv, r in ((8, 1), (8, 2), (4, 4), (4, 8)):
        p = pg.plan_chunk(cus, bs, segs, total_q, hkv, r * hkv, max_q, ctx)
        if max_q * r <= 16:
            assert p.kernel == 2
            assert p.split_tokens % max(bs, 64) == 0 and 0 < p.split_tokens <= 4096
            assert p.max_splits == -(-ctx // p.split_tokens)
        else:
            assert p.kernel == 1
            short = p.short_split_tokens or p.split_tokens
            for sp in (p.split_tokens, short):
                assert sp % 32 == 0 and 0 < sp <= 4096
            assert p.max_splits >= -(-ctx // min(p.split_tokens, short))

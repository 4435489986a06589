"""The Python binding rejects mis-sized or mis-typed tensors before anything
reaches the library (no GPU needed: a stand-in pool on the CPU whose null
handle would make any library call fail with a status, not a ValueError)."""
import types

import pytest
import torch

import paged_gqa_decode_head_amd as pg


def _pool(hkv=8):
    return types.SimpleNamespace(device=torch.device("cpu"), num_kv_heads=hkv, handle=None)


def bf(*s):
    return torch.zeros(s, dtype=torch.bfloat16)


def i32(*s):
    return torch.zeros(s, dtype=torch.int32)


def _decode_args(B=4, hq=16, hkv=8):
    return dict(q=bf(B, hq, 128), context_lens=i32(B), block_tables=i32(B, 9))


@pytest.mark.parametrize("bad", [
    dict(context_lens=i32(3)),                       # fewer lengths than sequences
    dict(context_lens=torch.zeros(4, dtype=torch.int64)),
    dict(block_tables=i32(3, 9)),                    # fewer table rows than sequences
    dict(block_tables=i32(36)),                      # not 2-D
    dict(q=bf(4, 16, 64)),                           # head_dim 64
    dict(out=bf(4, 16, 128)[:, :8]),                 # wrong out shape
    dict(out=torch.zeros(4, 16, 128)),               # fp32 out
])
def test_decode_rejects_mis_sized_inputs(bad):
    args = {**_decode_args(), **bad}
    with pytest.raises((ValueError, TypeError)):
        pg.paged_decode_attention(_pool(), args["q"], args["context_lens"], args["block_tables"], 100, 0.08,
                                  out=args.get("out"))


def test_decode_checks_pass_then_the_library_reports_the_missing_pool():
    a = _decode_args()
    with pytest.raises(pg.PgqaError):
        pg.paged_decode_attention(_pool(), a["q"], a["context_lens"], a["block_tables"], 100, 0.08,
                                  workspace=torch.zeros(256, dtype=torch.uint8),
                                  stream=types.SimpleNamespace(cuda_stream=0))


@pytest.mark.parametrize("bad", [
    dict(k=bf(4, 4, 128)),                           # kv heads of another pool
    dict(v=bf(3, 8, 128)),                           # fewer v rows than sequences
    dict(wq=torch.zeros(128)),                       # fp32 weight read as bf16 otherwise
    dict(wk=bf(64)),
    dict(q_out=bf(4, 16, 64)),
    dict(context_lens=i32(5)),
])
def test_decode_step_rejects_mis_sized_inputs(bad):
    B, hq, hkv = 4, 16, 8
    args = dict(q=bf(B, hq, 128), k=bf(B, hkv, 128), v=bf(B, hkv, 128), wq=bf(128), wk=bf(128),
                context_lens=i32(B), block_tables=i32(B, 9), q_out=None, **{})
    args.update(bad)
    with pytest.raises((ValueError, TypeError)):
        pg.decode_step(_pool(hkv), args["q"], args["k"], args["v"], args["wq"], args["wk"], args["context_lens"],
                       args["block_tables"], 100, 1e-6, 1e6, 0.08, q_out=args["q_out"])
    with pytest.raises((ValueError, TypeError)):
        pg.decode_step_noalloc(_pool(hkv), args["q"], args["k"], args["v"], args["wq"], args["wk"],
                               args["context_lens"], args["block_tables"], 100, 1e-6, 1e6, 0.08, bf(B, hq, 128),
                               q_out=args["q_out"])


@pytest.mark.parametrize("bad", [
    dict(query_start_loc=i32(3)),                    # N + 1 entries needed
    dict(block_tables=i32(2, 9)),                    # fewer table rows than segments
    dict(context_lens=i32(3, 1)),
    dict(q=bf(10, 16, 96)),
    dict(out=bf(9, 16, 128)),
])
def test_chunk_rejects_mis_sized_inputs(bad):
    args = dict(q=bf(10, 16, 128), query_start_loc=i32(4), context_lens=i32(3), block_tables=i32(3, 9), out=None)
    args.update(bad)
    with pytest.raises((ValueError, TypeError)):
        pg.paged_chunk_attention(_pool(), args["q"], args["query_start_loc"], args["context_lens"],
                                 args["block_tables"], 5, 100, 0.08, out=args["out"])


@pytest.mark.parametrize("bad", [
    dict(k=bf(6, 4, 128)),
    dict(positions=i32(5)),
    dict(seq_ids=i32(7)),
    dict(wq=bf(128, 1)),
    dict(q_out=bf(6, 8, 128)),
])
def test_cache_write_rejects_mis_sized_inputs(bad):
    T, hq, hkv = 6, 16, 8
    args = dict(q=bf(T, hq, 128), k=bf(T, hkv, 128), v=bf(T, hkv, 128), wq=bf(128), wk=bf(128),
                positions=i32(T), seq_ids=i32(T), block_tables=i32(2, 9), q_out=None)
    args.update(bad)
    with pytest.raises((ValueError, TypeError)):
        pg.rms_norm_rope_cache_write(_pool(hkv), args["q"], args["k"], args["v"], args["wq"], args["wk"],
                                     args["positions"], args["seq_ids"], args["block_tables"], 1e-6, 1e6,
                                     q_out=args["q_out"])

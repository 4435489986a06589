"""The fused decode step driven from C (tests/c_decode_step.c, built by the
package build with gcc against include/pgqa.h and the HIP runtime): the C
program places the prefix cache through pgqa_pool_layout's strides, runs
pgqa_decode_step and writes out, q_out and the raw pool storage back; here they
are checked against the fp64 oracle (outputs within tolerance; the new
tokens' V and every untouched cache row bit-exact)."""
import math
import os
import subprocess

import numpy as np
import pytest
import torch

import oracle as O
from paged_gqa_decode_head_amd.workloads import Group, StepSpec, make_step

from harness import compare

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
EXE = os.path.join(ROOT, "tests", "bin", "c_decode_step")


def _as_bf16(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16)


@pytest.mark.parametrize("bs", [16, 32])
def test_decode_step_from_c_matches_oracle(tmp_path, bs):
    assert os.path.exists(EXE), "tests/bin/c_decode_step is built by paged_gqa_decode_head_amd.build"
    spec = StepSpec(f"c-abi-{bs}", 977 + bs, 16, 8, 96 * 16 // bs,
                    decode=(Group(1, 0, 0), Group(2, 15, 17), Group(3, 100, 300)), block_size=bs)
    w = make_step(spec)
    s = w.spec
    B, nb = w.num_decode, s.num_blocks
    assert w.num_tokens == B and np.array_equal(w.tok_pos, w.dec_ctx - 1)
    scale = 1.0 / math.sqrt(128)
    files = {"q.bin": w.tok_q, "k.bin": w.tok_k, "v.bin": w.tok_v, "wq.bin": w.wq, "wk.bin": w.wk,
             "ctx.bin": w.dec_ctx.astype(np.int32), "bt.bin": w.block_tables.astype(np.int32),
             "prefix_k.bin": w.prefix_k, "prefix_v.bin": w.prefix_v}
    for name, arr in files.items():
        np.ascontiguousarray(arr).tofile(tmp_path / name)
    args = [EXE, str(tmp_path), str(nb), str(bs), str(s.num_kv_heads), str(s.num_q_heads), str(B),
            str(w.block_tables.shape[1]), str(int(w.dec_ctx.max())), repr(s.eps), repr(s.rope_theta), repr(scale)]
    print("[c-abi]", " ".join(args[2:]), flush=True)
    r = subprocess.run(args, capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, (r.returncode, r.stdout, r.stderr)
    assert "flags 0" in r.stdout

    # oracle: the fused write into a copy of the prefix, then decode over it
    pk, pv = w.prefix_k.copy(), w.prefix_v.copy()
    q_ref, _ = O.fused_norm_rope_write(w.tok_q, w.tok_k, w.tok_v, w.wq, w.wk, w.tok_pos, w.tok_seq,
                                       w.block_tables, s.eps, s.rope_theta, pk, pv)
    out_ref = O.decode_attention(O.bf16_round(q_ref), pk, pv, w.dec_block_tables, w.dec_ctx, scale)
    shape = (B, s.num_q_heads, 128)
    q_out = np.fromfile(tmp_path / "q_out.bin", dtype=np.uint16).reshape(shape)
    out = np.fromfile(tmp_path / "out.bin", dtype=np.uint16).reshape(shape)
    compare(_as_bf16(q_out), q_ref, f"bs={bs} q_out from C")
    compare(_as_bf16(out), out_ref, f"bs={bs} out from C")

    # the pool through the strides the C program read: untouched rows and V bit-exact
    lay = [list(map(int, l.split())) for l in open(tmp_path / "layout.txt").read().split("\n") if l.strip()]
    ks, ko, vs, vo = lay[0][:4], lay[0][4], lay[1][:5], lay[1][5]
    raw = np.fromfile(tmp_path / "pool.bin", dtype=np.uint16)
    b, sl, h, d = np.meshgrid(np.arange(nb), np.arange(bs), np.arange(s.num_kv_heads), np.arange(128), indexing="ij")
    k_got = raw[ko + b * ks[0] + sl * ks[1] + h * ks[2] + d * ks[3]]
    v_got = raw[vo + b * vs[0] + (sl // 16) * vs[1] + (sl % 16) * vs[2] + h * vs[3] + d * vs[4]]
    blk, off = O.slot_of(w.tok_pos, w.tok_seq, w.block_tables, bs)
    new = np.zeros((nb, bs), dtype=bool)
    new[blk, off] = True
    assert np.array_equal(v_got, pv)                                 # V: prefix and new tokens, bit-exact
    assert np.array_equal(k_got[~new], w.prefix_k[~new])             # K rows not written: untouched
    compare(_as_bf16(k_got[blk, off]), O.bf16_bits_to_f64(pk[blk, off]), f"bs={bs} new K rows from C")

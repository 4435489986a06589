"""Seeded synthetic inputs for the paged GQA attention path.

This module only draws random numbers and lays them out; it holds none of the
method's arithmetic (no norm, rotary, slot or attention computation), so both
the GPU path and the fp64 reference may consume what it produces.

Recipe (the same for every workload):
  * generator ``numpy.random.default_rng([714, seed_id, rep])``;
  * per-token q, k, v and every cached prefix key/value: N(0, 1) drawn as
    float32, then rounded to bf16 (round-to-nearest-even, by torch's
    float32 -> bfloat16 conversion);
  * the q_norm and k_norm weights: N(1, 0.1), rounded the same way;
  * context lengths "uniform in [lo, hi]" are integers, both ends included;
  * block tables: one random permutation of the whole pool, dealt to the
    sequences in order, ceil(n / block_size) blocks each; unused table entries
    hold -1;
  * a decode sequence with L cached tokens writes its new token at position L
    and attends to n = L + 1 keys; a chunk of q_len tokens over a cached prefix
    L sits at positions L .. L + q_len - 1 and its segment holds n = L + q_len
    keys.

Everything is held as numpy arrays; bf16 tensors are uint16 bit patterns.  The
cache contents are given in the logical order [num_blocks][block_size][Hkv][D].
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

SEED_BASE = 714


def _bf16_bits(x_f32: np.ndarray) -> np.ndarray:
    import torch

    t = torch.from_numpy(np.ascontiguousarray(x_f32, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


@dataclass(frozen=True)
class Group:
    """``count`` sequences with cached prefix L ~ U[lo, hi] and ``q_len`` new
    tokens each (q_len = 1 is a decode row)."""

    count: int
    lo: int
    hi: int
    q_len: int = 1


@dataclass(frozen=True)
class StepSpec:
    name: str
    seed_id: int
    num_q_heads: int
    num_kv_heads: int
    num_blocks: int
    decode: tuple = ()          # Groups with q_len == 1, served by decode attention
    chunks: tuple = ()          # Groups served by causal chunk attention
    head_dim: int = 128
    block_size: int = 16
    eps: float = 1e-6
    rope_theta: float = 1e6
    prefix_via_write: bool = False  # write the prefix through the fused op too
    description: str = ""


@dataclass
class StepWorkload:
    spec: StepSpec
    block_tables: np.ndarray      # int32 [rows, width], -1 padded
    prefix_k: np.ndarray          # uint16 [num_blocks, bs, Hkv, D] cache contents before the step
    prefix_v: np.ndarray
    tok_q: np.ndarray             # uint16 [T, Hq, D] tokens written this step
    tok_k: np.ndarray             # uint16 [T, Hkv, D]
    tok_v: np.ndarray
    tok_pos: np.ndarray           # int32 [T] absolute positions
    tok_seq: np.ndarray           # int32 [T] block-table rows
    wq: np.ndarray                # uint16 [D]
    wk: np.ndarray
    dec_rows: np.ndarray          # int32 [Bd] block-table rows of the decode sequences (0..Bd-1)
    dec_ctx: np.ndarray           # int32 [Bd] keys attended (n)
    dec_tok: np.ndarray           # int32 [Bd] index of each decode query in the token arrays
    chk_qsl: np.ndarray           # int32 [N+1] query_start_loc over the chunk query rows
    chk_ctx: np.ndarray           # int32 [N]
    chk_tok0: int = 0             # chunk query rows are tokens chk_tok0 .. chk_tok0 + chk_qsl[-1] - 1
    used_blocks: np.ndarray = field(default=None)

    @property
    def num_tokens(self) -> int:
        return int(self.tok_pos.shape[0])

    @property
    def num_decode(self) -> int:
        return int(self.dec_ctx.shape[0])

    @property
    def num_chunks(self) -> int:
        return int(self.chk_ctx.shape[0])

    @property
    def dec_block_tables(self) -> np.ndarray:
        return self.block_tables[: self.num_decode]

    @property
    def chk_block_tables(self) -> np.ndarray:
        return self.block_tables[self.num_decode:]


def _draw_groups(rng, groups):
    out = []
    for g in groups:
        for L in rng.integers(g.lo, g.hi + 1, size=g.count):
            out.append((int(L), int(g.q_len)))
    return out


def make_step(spec: StepSpec, rep: int = 0) -> StepWorkload:
    """Draw one step of synthetic input for ``spec``."""
    if spec.prefix_via_write and spec.chunks:
        raise ValueError("prefix_via_write is only defined for decode-only steps")
    rng = np.random.default_rng([SEED_BASE, spec.seed_id, rep])
    bs, D = spec.block_size, spec.head_dim
    hq, hkv = spec.num_q_heads, spec.num_kv_heads
    dec = _draw_groups(rng, spec.decode)
    chk = _draw_groups(rng, spec.chunks)
    seqs = dec + chk                                   # (prefix L, q_len) per block-table row
    ctx = np.array([L + ql for L, ql in seqs], dtype=np.int64)
    need = -(-ctx // bs)
    if need.sum() > spec.num_blocks:
        raise ValueError(f"{spec.name}: pool of {spec.num_blocks} blocks cannot hold {need.sum()}")
    perm = rng.permutation(spec.num_blocks).astype(np.int32)
    width = int(need.max()) if len(seqs) else 1
    bt = np.full((len(seqs), width), -1, dtype=np.int32)
    cur = 0
    for i, nb in enumerate(need):
        bt[i, :nb] = perm[cur:cur + nb]
        cur += nb
    used = perm[:cur].copy()

    # tokens written this step: decode tokens first, then chunk tokens in row order
    pos, seq = [], []
    for row, (L, ql) in enumerate(seqs):
        start = 0 if spec.prefix_via_write else L
        pos.extend(range(start, L + ql))
        seq.extend([row] * (L + ql - start))
    pos = np.array(pos, dtype=np.int32)
    seq = np.array(seq, dtype=np.int32)
    T = pos.shape[0]
    tok_q = _bf16_bits(rng.standard_normal((T, hq, D), dtype=np.float32))
    tok_k = _bf16_bits(rng.standard_normal((T, hkv, D), dtype=np.float32))
    tok_v = _bf16_bits(rng.standard_normal((T, hkv, D), dtype=np.float32))
    wq = _bf16_bits((1.0 + 0.1 * rng.standard_normal(D)).astype(np.float32))
    wk = _bf16_bits((1.0 + 0.1 * rng.standard_normal(D)).astype(np.float32))

    prefix_k = np.zeros((spec.num_blocks, bs, hkv, D), dtype=np.uint16)
    prefix_v = np.zeros((spec.num_blocks, bs, hkv, D), dtype=np.uint16)
    if not spec.prefix_via_write:
        for row, (L, _) in enumerate(seqs):
            nbp = -(-L // bs)
            if nbp == 0:
                continue
            blks = bt[row, :nbp]
            kk = _bf16_bits(rng.standard_normal((nbp * bs, hkv, D), dtype=np.float32))
            vv = _bf16_bits(rng.standard_normal((nbp * bs, hkv, D), dtype=np.float32))
            kk[L:] = 0
            vv[L:] = 0
            prefix_k[blks] = kk.reshape(nbp, bs, hkv, D)
            prefix_v[blks] = vv.reshape(nbp, bs, hkv, D)

    nd = len(dec)
    # index of each decode row's query = its last written token
    last_tok = np.zeros(len(seqs), dtype=np.int64)
    first_tok = np.zeros(len(seqs), dtype=np.int64)
    for i in range(T):
        last_tok[seq[i]] = i
    for i in range(T - 1, -1, -1):
        first_tok[seq[i]] = i
    dec_tok = last_tok[:nd].astype(np.int32)
    qlens = np.array([ql for _, ql in chk], dtype=np.int64)
    chk_qsl = np.concatenate([[0], np.cumsum(qlens)]).astype(np.int32)
    chk_tok0 = int(first_tok[nd]) if chk else T
    return StepWorkload(
        spec=spec, block_tables=bt, prefix_k=prefix_k, prefix_v=prefix_v,
        tok_q=tok_q, tok_k=tok_k, tok_v=tok_v, tok_pos=pos, tok_seq=seq, wq=wq, wk=wk,
        dec_rows=np.arange(nd, dtype=np.int32), dec_ctx=ctx[:nd].astype(np.int32), dec_tok=dec_tok,
        chk_qsl=chk_qsl, chk_ctx=ctx[nd:].astype(np.int32), chk_tok0=chk_tok0, used_blocks=used,
    )


# ---------------------------------------------------------------------------
# The five Qwen3-shaped workloads: shapes, batch and context draws of each
# ---------------------------------------------------------------------------
SPECS = {
    "cfg1": StepSpec(
        "cfg1", 1, 16, 8, 32, decode=(Group(1, 37, 37), Group(1, 100, 100)), prefix_via_write=True,
        description="tiny single layer, Qwen3-0.6B attention shape (16/8 heads), batch 2, contexts 37 and 100"),
    "cfg2": StepSpec(
        "cfg2", 2, 16, 8, 4096, decode=(Group(8, 512, 4096),),
        description="Qwen3-0.6B decode, batch 8, contexts U[512,4096]"),
    "cfg3a": StepSpec(
        "cfg3a", 31, 16, 8, 3072, decode=(Group(1, 32768, 32768),),
        description="Qwen3-1.7B decode, batch 1, context 32768"),
    "cfg3b": StepSpec(
        "cfg3b", 32, 16, 8, 16384, decode=(Group(64, 1024, 2048),),
        description="Qwen3-1.7B decode, batch 64, contexts U[1024,2048]"),
    "cfg4": StepSpec(
        "cfg4", 4, 32, 4, 64 * 120, decode=(Group(64, 256, 1280),),
        description="Qwen3-30B-A3B attention shape (32/4 heads), batch 64, contexts U[256,1280]"),
    "cfg5": StepSpec(
        "cfg5", 5, 16, 8, 16384,
        decode=(Group(8, 2048, 8192),),
        chunks=(Group(1, 6144, 6144, 512), Group(8, 1024, 4096, 5)),
        description="Qwen3-1.7B mixed step: 8 decode streams U[2048,8192], one 512-token prefill "
                    "slice at offset 6144, 8 verify rows of k+1=5 tokens over U[1024,4096]"),
}

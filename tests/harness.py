"""Test glue: runs a synthetic step through the HIP library and the fp64
reference on the same seeded inputs, and compares them.

Comparison rule: a bf16 result of the library is compared with the unrounded
fp64 reference value; max |diff| <= 2e-2 and sum|diff| / sum|ref| <= 5e-3.
"""
from __future__ import annotations

import math

import numpy as np
import torch

import oracle as O
import paged_gqa_decode_head_amd as pg
from paged_gqa_decode_head_amd.workloads import StepWorkload

MAX_ABS = 2e-2
MEAN_REL = 5e-3
SCALE = 1.0 / math.sqrt(128.0)
SENTINEL = np.uint16(0x7FC1)   # a quiet-NaN bf16 pattern no computed value equals


def dev_bf16(bits: np.ndarray, device="cuda") -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(device).view(torch.bfloat16)


def dev_i32(a: np.ndarray, device="cuda") -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to(device)


def bits_of(t: torch.Tensor) -> np.ndarray:
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def f64_of(t: torch.Tensor) -> np.ndarray:
    return O.bf16_bits_to_f64(bits_of(t))


def compare(got: torch.Tensor, ref: np.ndarray, what: str, max_abs=MAX_ABS, mean_rel=MEAN_REL):
    g = f64_of(got)
    assert g.shape == ref.shape, (what, g.shape, ref.shape)
    assert np.isfinite(g).all(), f"{what}: non-finite output"
    d = np.abs(g - ref)
    ma = float(d.max()) if d.size else 0.0
    denom = float(np.abs(ref).sum())
    mr = float(d.sum() / denom) if denom > 0 else 0.0
    assert ma <= max_abs and mr <= mean_rel, f"{what}: max_abs={ma:.3e} mean_rel={mr:.3e}"
    return ma, mr


def compact(bt: np.ndarray, used: np.ndarray):
    """Renumber the blocks of a table into 0..len(used)-1 (for a compact read-back)."""
    inv = np.full(int(max(used.max(), bt.max())) + 1, -1, dtype=np.int64)
    inv[used] = np.arange(len(used))
    return np.where(bt >= 0, inv[np.maximum(bt, 0)], -1)


class StepRun:
    """One synthetic step on the GPU: pool, inputs, and the library calls."""

    def __init__(self, w: StepWorkload, fill_prefix=True, device="cuda"):
        self.w = w
        s = w.spec
        self.device = torch.device(device)
        self.pool = pg.Pool(s.num_blocks, s.block_size, s.num_kv_heads, device=self.device)
        self.used = w.used_blocks
        if fill_prefix and len(self.used):
            self.pool.fill_logical(w.prefix_k[self.used].view(np.int16), w.prefix_v[self.used].view(np.int16),
                                   blocks=self.used)
        self.q = dev_bf16(w.tok_q)
        self.k = dev_bf16(w.tok_k)
        self.v = dev_bf16(w.tok_v)
        self.wq = dev_bf16(w.wq)
        self.wk = dev_bf16(w.wk)
        self.pos = dev_i32(w.tok_pos)
        self.seq = dev_i32(w.tok_seq)
        self.bt = dev_i32(w.block_tables)
        self.dec_bt = dev_i32(w.dec_block_tables) if w.num_decode else None
        self.dec_ctx = dev_i32(w.dec_ctx)
        self.chk_bt = dev_i32(w.chk_block_tables) if w.num_chunks else None
        self.chk_ctx = dev_i32(w.chk_ctx)
        self.chk_qsl = dev_i32(w.chk_qsl)
        self.q_out = None

    def write(self):
        s = self.w.spec
        self.q_out = pg.rms_norm_rope_cache_write(self.pool, self.q, self.k, self.v, self.wq, self.wk, self.pos,
                                                  self.seq, self.bt, s.eps, s.rope_theta)
        return self.q_out

    def decode_q(self):
        idx = torch.from_numpy(self.w.dec_tok.astype(np.int64)).to(self.device)
        return self.q_out.index_select(0, idx).contiguous()

    def decode(self, plan=None, q=None, out=None):
        q = self.decode_q() if q is None else q
        return pg.paged_decode_attention(self.pool, q, self.dec_ctx, self.dec_bt, int(self.w.dec_ctx.max()), SCALE,
                                         plan=plan, out=out)

    def chunk_q(self):
        t0 = self.w.chk_tok0
        return self.q_out[t0:t0 + int(self.w.chk_qsl[-1])].contiguous()

    def chunk(self, q=None):
        q = self.chunk_q() if q is None else q
        qlens = np.diff(self.w.chk_qsl)
        return pg.paged_chunk_attention(self.pool, q, self.chk_qsl, self.chk_ctx, self.chk_bt, int(qlens.max()),
                                        int(self.w.chk_ctx.max()), SCALE)

    # ---- reference side -------------------------------------------------
    def read_pool(self):
        """GPU cache contents of the used blocks (bits, logical order) and the compacted table."""
        k, v = self.pool.read_logical(blocks=self.used)
        return (k.numpy().view(np.uint16), v.numpy().view(np.uint16),
                compact(self.w.block_tables, self.used))

    def oracle_write(self):
        """fp64 reference of the write call on the same inputs; returns (q_out, k_out, slots)."""
        w = self.w
        s = w.spec
        nb = w.spec.num_blocks
        # the reference cache model only needs the used blocks: compact table
        bt_c = compact(w.block_tables, self.used)
        pk = np.zeros((len(self.used), s.block_size, s.num_kv_heads, 128), dtype=np.uint16)
        pv = np.zeros_like(pk)
        q_ref, k_ref = O.fused_norm_rope_write(w.tok_q, w.tok_k, w.tok_v, w.wq, w.wk, w.tok_pos, w.tok_seq, bt_c,
                                               s.eps, s.rope_theta, pk, pv)
        blk, off = O.slot_of(w.tok_pos, w.tok_seq, bt_c, s.block_size)
        del nb
        return q_ref, k_ref, (blk, off), (pk, pv)

    def oracle_decode_on_gpu_inputs(self, q_gpu: torch.Tensor):
        """Reference decode on the library's own q_out and cache contents (per-call parity)."""
        pk, pv, bt_c = self.read_pool()
        q = f64_of(q_gpu)
        return O.decode_attention(q, pk, pv, bt_c[: self.w.num_decode], self.w.dec_ctx, SCALE)

    def oracle_chunk_on_gpu_inputs(self, q_gpu: torch.Tensor):
        pk, pv, bt_c = self.read_pool()
        q = f64_of(q_gpu)
        return O.chunk_attention(q, self.w.chk_qsl, pk, pv, bt_c[self.w.num_decode:], self.w.chk_ctx, SCALE)


# Decode split kernels: 1 = dot-product (VALU) kernel, 2 = matrix-core (MFMA) kernel.
KERNELS = [1, 2]


def with_kernel(plan, kernel):
    """A copy of a DecodePlan with its split kernel set."""
    return pg.DecodePlan(plan.split_tokens, plan.max_splits, plan.waves_per_split, plan.load_hint, kernel)


def default_plan(w, kernel):
    """The library's plan for the decode rows of step w, with the split kernel set."""
    s = w.spec
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    p = pg.plan_decode(cus, s.block_size, w.num_decode, s.num_kv_heads, s.num_q_heads, int(w.dec_ctx.max()))
    return with_kernel(p, kernel)

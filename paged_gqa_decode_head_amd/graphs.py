"""HIP-graph replay of the decode step at bucketed batch sizes.

Page "[2026春季][T2-1-3]" (InfiniLM issue 498), its change list for paged
graphs: decode graphs are captured only for the batch sizes a scheduler can
reach (every size up to 16, the multiples of 8 above that, and the configured
maximum batch), and any other shape runs eagerly.  Here a step of B
sequences replays the graph of the smallest captured bucket >= B; rows
B .. bucket-1 are padding.

One captured step is, for each layer pool in turn, the norm + rotary + cache
write of one new token per sequence and paged decode attention over the
cache: by default one ``pgqa_decode_step`` launch per layer (the new token sits
at position context_len - 1), or with ``fused=False`` the two calls
``pgqa_rms_norm_rope_cache_write`` (at ``positions``) and
``pgqa_paged_decode_attention``.  Buffers, plans and workspaces are fixed at
capture time: the caller writes a step's inputs into the views ``inputs(B)``
returns and calls ``replay(B)``.  Padding rows attend over zero keys, so their
outputs are zero rows; the fused step writes nothing for them, the two-call
step writes their k/v into slot 0 of a reserved pad block, so no sequence's
cache is touched either way.

This module is host plumbing (torch's graph capture around the library's
launches); every operation of the step runs in libpgqa's kernels.
"""
from __future__ import annotations

from dataclasses import dataclass

from . import (DecodePlan, Pool, bind_cache_write, bind_decode, bind_decode_step, decode_workspace_bytes,
               plan_decode)


def default_buckets(max_batch: int) -> list[int]:
    """1..16, then every multiple of 8 up to max_batch, and max_batch itself."""
    if max_batch < 1:
        raise ValueError("max_batch must be >= 1")
    b = list(range(1, min(16, max_batch) + 1))
    b += list(range(24, max_batch + 1, 8))
    if b[-1] != max_batch:
        b.append(max_batch)
    return b


@dataclass
class StepInputs:
    """Views of the static buffers for a step of B sequences (fill them, then replay)."""
    q: object          # [L, B, Hq, 128] bf16: per layer, the new token's q projection
    k: object          # [L, B, Hkv, 128] bf16
    v: object          # [L, B, Hkv, 128] bf16
    positions: object  # [B] int32: position of the new token (= keys before it); read by the two-call step only
    context_lens: object  # [B] int32: keys attended, the new token included
    block_tables: object  # [B, max_blocks_per_seq] int32


class DecodeGraphs:
    """Captured decode steps over the layer pools ``pools`` for each batch bucket."""

    def __init__(self, pools: list[Pool], num_q_heads: int, max_blocks_per_seq: int, pad_block: int,
                 q_norm_weight, k_norm_weight, eps: float, rope_theta: float, scale: float, max_batch: int,
                 buckets: list[int] | None = None, fused: bool = True):
        import torch

        if not pools:
            raise ValueError("need at least one layer pool")
        p0 = pools[0]
        for p in pools:
            if (p.config.block_size, p.config.num_kv_heads, p.device) != (p0.config.block_size,
                                                                          p0.config.num_kv_heads, p0.device):
                raise ValueError("all layer pools must share block size, kv heads and device")
            if p.config.max_batch_size and max_batch > p.config.max_batch_size:
                raise ValueError(f"max_batch {max_batch} exceeds the pool's max_batch_size")
        if not 0 <= pad_block < p0.config.num_blocks:
            raise ValueError("pad_block must be a block id of the pools")
        self.pools, self.pad_block, self.fused = list(pools), pad_block, bool(fused)
        self.buckets = sorted(set(buckets if buckets is not None else default_buckets(max_batch)))
        if self.buckets[0] < 1 or self.buckets[-1] > max_batch:
            raise ValueError("buckets must lie in 1 .. max_batch")
        L, hq, hkv, bs = len(pools), num_q_heads, p0.config.num_kv_heads, p0.config.block_size
        dev = p0.device
        self.max_batch = max_batch
        self.max_ctx = max_blocks_per_seq * bs
        self._wq, self._wk = q_norm_weight, k_norm_weight
        self._eps, self._theta, self._scale = float(eps), float(rope_theta), float(scale)
        bf16, i32 = torch.bfloat16, torch.int32
        self.q = torch.zeros((L, max_batch, hq, 128), dtype=bf16, device=dev)
        self.k = torch.zeros((L, max_batch, hkv, 128), dtype=bf16, device=dev)
        self.v = torch.zeros((L, max_batch, hkv, 128), dtype=bf16, device=dev)
        self.positions = torch.zeros(max_batch, dtype=i32, device=dev)
        self.seq_ids = torch.arange(max_batch, dtype=i32, device=dev)
        self.context_lens = torch.zeros(max_batch, dtype=i32, device=dev)
        self.block_tables = torch.full((max_batch, max_blocks_per_seq), pad_block, dtype=i32, device=dev)
        self.q_out = torch.zeros((L, max_batch, hq, 128), dtype=bf16, device=dev)
        self.out = torch.zeros((L, max_batch, hq, 128), dtype=bf16, device=dev)
        cus = torch.cuda.get_device_properties(dev).multi_processor_count
        self._graphs = {}
        with torch.cuda.device(dev):
            for B in self.buckets:
                plan = plan_decode(cus, bs, B, hkv, hq, self.max_ctx)
                ws = [torch.zeros(max(256, decode_workspace_bytes(p, B, hq, self.max_ctx, plan)), dtype=torch.uint8,
                                  device=dev) for p in pools]
                side = torch.cuda.Stream()
                side.wait_stream(torch.cuda.current_stream())
                with torch.cuda.stream(side):  # one eager run before capture (all rows are padding here)
                    for c in self._bind(B, plan, ws):
                        c()
                torch.cuda.current_stream().wait_stream(side)
                torch.cuda.synchronize()
                g = torch.cuda.CUDAGraph()
                # relaxed: the calls check their pointers' attributes while the stream
                # captures (a host query that enqueues nothing)
                with torch.cuda.graph(g, capture_error_mode="relaxed"):
                    calls = self._bind(B, plan, ws)  # bound to the capturing stream
                    for c in calls:
                        c()
                self._graphs[B] = (g, calls, plan, ws)

    def _bind(self, B: int, plan: DecodePlan, ws):
        calls = []
        for l, p in enumerate(self.pools):
            if self.fused:
                calls.append(bind_decode_step(p, self.q[l, :B], self.k[l, :B], self.v[l, :B], self._wq, self._wk,
                                              self.context_lens[:B], self.block_tables[:B], self.max_ctx, self._eps,
                                              self._theta, self._scale, self.out[l, :B], plan=plan, workspace=ws[l],
                                              q_out=self.q_out[l, :B]))
                continue
            calls.append(bind_cache_write(p, self.q[l, :B], self.k[l, :B], self.v[l, :B], self._wq, self._wk,
                                          self.positions[:B], self.seq_ids[:B], self.block_tables[:B], self._eps,
                                          self._theta, self.q_out[l, :B]))
            calls.append(bind_decode(p, self.q_out[l, :B], self.context_lens[:B], self.block_tables[:B],
                                     self.max_ctx, self._scale, self.out[l, :B], plan=plan, workspace=ws[l]))
        return calls

    def eager_calls(self, bucket: int):
        """The captured step of `bucket` as pre-bound calls on the current stream
        (same buffers, plan and workspaces), for eager runs of the same work."""
        _, _, plan, ws = self._graphs[bucket]
        return self._bind(bucket, plan, ws)

    def bucket_for(self, batch: int) -> int | None:
        """The smallest captured bucket >= batch, or None (run that step eagerly)."""
        for b in self.buckets:
            if b >= batch:
                return b
        return None

    def plan(self, bucket: int) -> DecodePlan:
        return self._graphs[bucket][2]

    def inputs(self, batch: int) -> StepInputs:
        return StepInputs(self.q[:, :batch], self.k[:, :batch], self.v[:, :batch], self.positions[:batch],
                          self.context_lens[:batch], self.block_tables[:batch])

    def replay(self, batch: int):
        """Run the captured step for the first `batch` rows of the inputs; returns
        (q_out [L, batch, Hq, 128], out [L, batch, Hq, 128]) views."""
        bucket = self.bucket_for(batch)
        if bucket is None:
            raise ValueError(f"no graph for batch {batch} (largest bucket {self.buckets[-1]}); run it eagerly")
        if bucket > batch:  # padding rows: pad block slot 0, no keys
            self.positions[batch:bucket].zero_()
            self.context_lens[batch:bucket].zero_()
            self.block_tables[batch:bucket].fill_(self.pad_block)
        self._graphs[bucket][0].replay()
        return self.q_out[:, :batch], self.out[:, :batch]

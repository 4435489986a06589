#!/usr/bin/env python3
"""Paged GQA decode step benchmark on one MI355X.

A step is one pass of the decode hot path over one batch: per-head RMSNorm +
rotary of the batch's new tokens, their paged K/V cache write, and paged
split-KV GQA decode attention with the log-sum-exp combine, issued as the one
fused launch ``pgqa_decode_step`` (the same step as the two calls cache write +
decode attention, which are timed beside it as ``two_call_step``).  The default
workload is the Qwen3-1.7B decode shape at batch 64 (16 q heads, 8 kv heads,
head_dim 128, block size 16, contexts uniform in [1024, 2048], shuffled block
tables, N(0,1) bf16 inputs).

Consecutive steps use different layers' caches (``--layers`` pools of the same
shape, cycled), as a model's decode step does, so a layer's K/V has been
evicted from the 256 MB Infinity Cache before it is read again.

Prints ONE JSON line.  value = algorithmic bytes of the step / wall-clock step
time of the timed region (synchronised on both sides).  roofline.achieved
divides the same bytes by the kernel's average launch duration: one HIP event
pair on the launch stream around the timed region, over the number of steps
(back-to-back launches, so the launch gaps are included).
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "paged decode attn HBM GB/s (% of peak) + seqs/s, Qwen3-1.7B shapes"
HBM_PEAK_GBS = 8000.0
MFMA_BF16_PEAK_TFLOPS = 2500.0


def decode_alg_bytes(w) -> int:
    """K and V rows of every attended key, q in, out, block-table entries read, context lengths."""
    s = w.spec
    n = w.dec_ctx.astype("int64")
    kv = int(n.sum()) * s.num_kv_heads * 128 * 2 * 2
    qo = 2 * w.num_decode * s.num_q_heads * 128 * 2
    bt = int((-(-n // s.block_size)).sum()) * 4
    return kv + qo + bt + w.num_decode * 4


def step_alg_bytes(w) -> int:
    """The fused step: decode's bytes (every key's K and V row, raw q in, out) plus
    the new tokens' raw k and v in, their normed k and v into the cache, and the
    two weight vectors."""
    s = w.spec
    kv_rows = w.num_decode * s.num_kv_heads * 128 * 2
    return decode_alg_bytes(w) + 2 * kv_rows + 2 * kv_rows + 2 * 128 * 2


def write_alg_bytes(w) -> int:
    """q, k, v in; q_out; k', v into the cache; the two weight vectors; positions, seq ids, table entries."""
    s = w.spec
    T = w.num_tokens
    rows_in = T * (s.num_q_heads + 2 * s.num_kv_heads) * 128 * 2
    rows_out = T * (s.num_q_heads + 2 * s.num_kv_heads) * 128 * 2
    return rows_in + rows_out + 2 * 128 * 2 + T * 12


def chunk_alg(w, qsl, ctx):
    """(flops, KV bytes) of causal chunk attention: 4*D*Hq per visible (query, key)
    pair (QK^T and PV), and the K/V rows of each segment read once."""
    s = w.spec
    pairs = 0
    for i in range(len(ctx)):
        ql, n = int(qsl[i + 1] - qsl[i]), int(ctx[i])
        pairs += ql * (n - ql) + ql * (ql + 1) // 2
    kv = int(ctx.astype("int64").sum()) * s.num_kv_heads * 128 * 2 * 2
    return 4 * 128 * s.num_q_heads * pairs, kv


FLUSH_BYTES = 1 << 30   # 4x the 256 MB Infinity Cache


class CacheFlush:
    """A read of FLUSH_BYTES (torch's sum over a buffer of ones, ordinary cached
    loads) before a timed launch, so that launch finds neither its K/V in the
    Infinity Cache nor its metadata in L2: every row is then an HBM figure, as
    in a model step where the other layers' K/V passes between two uses of one
    layer's cache."""

    def __init__(self, dev):
        import torch

        self.buf = torch.ones(FLUSH_BYTES // 4, dtype=torch.float32, device=dev)
        self.sink = torch.empty((), dtype=torch.float32, device=dev)

    def __call__(self):
        import torch

        torch.sum(self.buf, dim=0, out=self.sink)


def time_calls_cold(calls, iters, flush, warmup=10, stats=None):
    """Median and mean microseconds of each call, each launch preceded by the
    cache flush (HIP events around the launch only, on the current stream);
    stats, if given, receives the p10 and p90."""
    import torch

    for i in range(warmup):
        flush()
        calls[i % len(calls)]()
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(iters)]
    for i in range(iters):
        flush()
        ev[i][0].record()
        calls[i % len(calls)]()
        ev[i][1].record()
    torch.cuda.synchronize()
    ts = sorted(a.elapsed_time(b) * 1e3 for a, b in ev)
    if stats is not None:
        stats["p10_us"] = round(ts[len(ts) // 10], 2)
        stats["p90_us"] = round(ts[(9 * len(ts)) // 10], 2)
    return ts[len(ts) // 2], sum(ts) / len(ts)


def measure_rows(args, dev, names=("cfg2", "cfg3a", "cfg4", "cfg5")):
    """Every hot-path row on its own synthetic workload: decode on each decode
    workload, chunk attention (slice, verify rows, both) on the mixed step.
    Every timed launch follows a 1 GiB cache flush (cold Infinity Cache and L2)."""
    import numpy as np
    import torch

    import paged_gqa_decode_head_amd as pg
    from paged_gqa_decode_head_amd.workloads import SPECS, make_step

    to_bf16 = lambda a: torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(dev).view(torch.bfloat16)
    to_i32 = lambda a: torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to(dev)
    scale = 1.0 / math.sqrt(128)
    cus = torch.cuda.get_device_properties(dev).multi_processor_count
    rows = {"decode": {}, "decode_step": {}, "cache_write": {}, "timing": "median (and p10, p90) of 50 per-launch HIP events after 10 warm-ups, each "
            "launch after a 1 GiB read that evicts the 256 MB Infinity Cache and L2 (cold caches)"}
    flush = CacheFlush(dev)
    time_calls = lambda calls, iters, stats=None: time_calls_cold(calls, iters, flush, stats=stats)  # noqa: E731
    for name in names:
        w = make_step(SPECS[name])
        s = w.spec
        pools = []
        for _ in range(1):
            p = pg.Pool(s.num_blocks, s.block_size, s.num_kv_heads, device=dev)
            p.fill_logical(w.prefix_k[w.used_blocks].view(np.int16), w.prefix_v[w.used_blocks].view(np.int16),
                           blocks=w.used_blocks)
            pools.append(p)
        q, k, v = to_bf16(w.tok_q), to_bf16(w.tok_k), to_bf16(w.tok_v)
        q_out = torch.empty((w.num_tokens, s.num_q_heads, 128), dtype=torch.bfloat16, device=dev)
        writes = [pg.bind_cache_write(p, q, k, v, to_bf16(w.wq), to_bf16(w.wk), to_i32(w.tok_pos), to_i32(w.tok_seq),
                                      to_i32(w.block_tables), s.eps, s.rope_theta, q_out) for p in pools]
        med, _ = time_calls(writes, 20)
        rows["cache_write"][name] = {"tokens": w.num_tokens, "us": round(med, 2),
                                     "alg_bytes": write_alg_bytes(w), "bound": "latency"}
        for wr in writes:
            wr()
        qd = q_out[torch.from_numpy(w.dec_tok.astype(np.int64)).to(dev)].contiguous()
        ctx, bt = to_i32(w.dec_ctx), to_i32(w.dec_block_tables)
        mx = int(w.dec_ctx.max())
        out = torch.empty((w.num_decode, s.num_q_heads, 128), dtype=torch.bfloat16, device=dev)
        plan = pg.plan_decode(cus, s.block_size, w.num_decode, s.num_kv_heads, s.num_q_heads, mx)
        if not args.no_host_lengths:
            plan.set_host_context_lens(w.dec_ctx)
        calls = [pg.bind_decode(p, qd, ctx, bt, mx, scale, out, plan=plan) for p in pools]
        dstats = {}
        med, mean = time_calls(calls, 50, dstats)
        nb = decode_alg_bytes(w)
        # the floor at this size: a plain streaming read of the same byte count,
        # timed the same way (cold caches, events around the launch)
        sbuf = torch.ones(nb // 16 * 4, dtype=torch.int32, device=dev)
        ssink = torch.empty(3 * cus * 256, dtype=torch.int32, device=dev)
        smed, _ = time_calls([pg.bind_stream_read(sbuf, ssink, 3 * cus)], 50)
        del sbuf, ssink
        rows["decode"][name] = {"batch": w.num_decode, "keys": int(w.dec_ctx.sum()), "us": round(med, 2), **dstats,
                                "seqs_per_s": round(w.num_decode / med * 1e6, 1),
                                "alg_bytes": nb, "gbs": round(nb / med / 1e3, 1),
                                "frac_hbm_peak": round(nb / med / 1e3 / HBM_PEAK_GBS, 4),
                                "stream_read_us": round(smed, 2),
                                "frac_of_stream_read": round(smed / med, 4),
                                "plan": {"split_tokens": plan.split_tokens, "max_splits": plan.max_splits,
                                         "waves": plan.waves_per_split,
                                         "kernel": "mfma" if plan.kernel == 2 else "dot"}}
        # the same decode rows as one fused pgqa_decode_step launch (norm + rotary
        # + cache write + decode) on the raw q, k, v of their new tokens
        dsel = torch.from_numpy(w.dec_tok.astype(np.int64)).to(dev)
        qr, kr, vr = q[dsel].contiguous(), k[dsel].contiguous(), v[dsel].contiguous()
        fcalls = [pg.bind_decode_step(p, qr, kr, vr, to_bf16(w.wq), to_bf16(w.wk), ctx, bt, mx, s.eps, s.rope_theta,
                                      scale, out, plan=plan) for p in pools]
        fstats = {}
        fmed, _ = time_calls(fcalls, 50, fstats)
        nbf = step_alg_bytes(w)
        rows["decode_step"][name] = {"batch": w.num_decode, "us": round(fmed, 2), **fstats,
                                     "seqs_per_s": round(w.num_decode / fmed * 1e6, 1), "alg_bytes": nbf,
                                     "gbs": round(nbf / fmed / 1e3, 1),
                                     "frac_hbm_peak": round(nbf / fmed / 1e3 / HBM_PEAK_GBS, 4),
                                     "kernel": "mfma" if plan.kernel == 2 else "dot"}
        if name == "cfg5":
            qc = q_out[w.chk_tok0:].contiguous()
            res = {}
            cases = {"slice+verify": (qc, w.chk_qsl, w.chk_ctx, w.chk_block_tables),
                     "slice": (qc[:512].contiguous(), w.chk_qsl[:2], w.chk_ctx[:1], w.chk_block_tables[:1]),
                     "verify": (qc[512:].contiguous(), w.chk_qsl[1:] - 512, w.chk_ctx[1:], w.chk_block_tables[1:])}
            # the verify rows once more on the chunk kernels (their planner split for such rows)
            cases["verify_chunk_kernels"] = cases["verify"]
            for label, (qq, qs, cx, bb) in cases.items():
                mq, mc = int(np.diff(qs).max()), int(cx.max())
                o2 = torch.empty((qq.shape[0], s.num_q_heads, 128), dtype=torch.bfloat16, device=dev)
                cp = pg.plan_chunk(cus, s.block_size, len(cx), qq.shape[0], s.num_kv_heads, s.num_q_heads, mq, mc)
                if label == "verify_chunk_kernels":
                    cp = pg.ChunkPlan(256, -(-mc // 256), 256, 1)
                calls = [pg.bind_chunk(p, qq, to_i32(qs), to_i32(cx), to_i32(bb), mq, mc, scale, o2, plan=cp)
                         for p in pools]
                cstats = {}
                med, _ = time_calls(calls, 50, cstats)
                flops, kv = chunk_alg(w, qs, cx)
                res[label] = {"us": round(med, 2), **cstats, "tokens_per_s": round(qq.shape[0] / med * 1e6, 1),
                              "tflops": round(flops / med / 1e6, 1),
                              "frac_mfma_bf16_peak": round(flops / med / 1e6 / MFMA_BF16_PEAK_TFLOPS, 4),
                              "kv_gbs": round(kv / med / 1e3, 1), "flops": flops, "kv_bytes": kv,
                              "plan": {"split_tokens": cp.split_tokens, "short_split_tokens": cp.short_split_tokens,
                                       "max_splits": cp.max_splits,
                                       "kernel": "columns" if cp.kernel == 2 else "chunk"}}
            rows["chunk_cfg5"] = res
            # the slice, and the slice with the verify rows, through the one-launch
            # mixed call (host-built work list: the serving path's route for them)
            mres = {}
            for label in ("slice", "slice+verify"):
                qq, qs, cx, bb = cases[label]
                mq, mc = int(np.diff(qs).max()), int(cx.max())
                o2 = torch.empty((qq.shape[0], s.num_q_heads, 128), dtype=torch.bfloat16, device=dev)
                mp, mi = pg.plan_mixed(cus, s.block_size, s.num_kv_heads, s.num_q_heads, qs, cx)
                mi_d = to_i32(mi)
                calls = [pg.bind_mixed(p, qq, to_i32(qs), to_i32(cx), to_i32(bb), mq, mc, scale, o2, mp, mi_d)
                         for p in pools]
                mstats = {}
                med, _ = time_calls(calls, 50, mstats)
                flops, kv = chunk_alg(w, qs, cx)
                mres[label] = {"us": round(med, 2), **mstats, "tokens_per_s": round(qq.shape[0] / med * 1e6, 1),
                               "tflops": round(flops / med / 1e6, 1),
                               "frac_mfma_bf16_peak": round(flops / med / 1e6 / MFMA_BF16_PEAK_TFLOPS, 4),
                               "kv_gbs": round(kv / med / 1e3, 1),
                               "plan": {"split_wide": mp.split_wide, "split_columns": mp.split_columns,
                                        "max_splits": mp.max_splits, "items": mp.num_items}}
            rows["mixed_call_cfg5_chunks"] = mres
            # the whole mixed step's attention as ONE launch (plus one combine)
            # from the host-built work list, against the decode call plus the
            # chunk call it replaces
            qlens = np.concatenate([np.ones(w.num_decode, dtype=np.int64), np.diff(w.chk_qsl)])
            qsl_all = np.concatenate([[0], np.cumsum(qlens)]).astype(np.int32)
            ctx_all = np.concatenate([w.dec_ctx, w.chk_ctx]).astype(np.int32)
            mplan, items = pg.plan_mixed(cus, s.block_size, s.num_kv_heads, s.num_q_heads, qsl_all, ctx_all)
            o_all = torch.empty((w.num_tokens, s.num_q_heads, 128), dtype=torch.bfloat16, device=dev)
            items_d = to_i32(items)
            mq, mc = int(qlens.max()), int(ctx_all.max())
            mcalls = [pg.bind_mixed(p, q_out, to_i32(qsl_all), to_i32(ctx_all), to_i32(w.block_tables), mq, mc, scale,
                                    o_all, mplan, items_d) for p in pools]
            xstats = {}
            med, _ = time_calls(mcalls, 50, xstats)
            flops, kv = chunk_alg(w, qsl_all, ctx_all)
            old_us = rows["decode"][name]["us"] + res["slice+verify"]["us"]
            # the step's write and attention back to back, one event pair
            step_calls = [lambda wr=wr, mc_=mc_: (wr(), mc_()) for wr, mc_ in zip(writes, mcalls)]
            smed, _ = time_calls(step_calls, 30)
            rows["mixed_cfg5"] = {
                "attention_us": round(med, 2), "attention_p10_us": xstats["p10_us"],
                "attention_p90_us": xstats["p90_us"], "tokens_per_s": round(w.num_tokens / med * 1e6, 1),
                "write_plus_attention_us": round(smed, 2),
                "decode_call_plus_chunk_call_us": round(old_us, 2), "speedup_over_two_calls": round(old_us / med, 3),
                "flops": flops, "kv_bytes": kv, "kv_gbs": round(kv / med / 1e3, 1),
                "frac_hbm_peak": round(kv / med / 1e3 / HBM_PEAK_GBS, 4),
                "tflops": round(flops / med / 1e6, 1),
                "plan": {"split_wide": mplan.split_wide, "split_columns": mplan.split_columns,
                         "max_splits": mplan.max_splits, "items": mplan.num_items, "combine_items": mplan.num_combine},
                "launches": "one attention kernel + one combine kernel"}
        del pools
        torch.cuda.empty_cache()
    del flush
    torch.cuda.empty_cache()
    return rows


def measure_graphs(dev, iters=50):
    """Decode step over L layer pools, as the two calls per layer (cache write +
    decode) or the one fused pgqa_decode_step launch per layer ("fused_"),
    issued eagerly through pre-bound calls vs replayed from one captured HIP
    graph:
      *_gpu_us_per_layer   steps issued back to back, events around each step
                           (GPU time, the host runs ahead);
      *_sync_us_per_step   wall clock of one step issued and waited for (the
                           latency a serving loop sees when the next step needs
                           this one's output)."""
    import numpy as np
    import torch

    import paged_gqa_decode_head_amd as pg
    from paged_gqa_decode_head_amd.graphs import DecodeGraphs
    from paged_gqa_decode_head_amd.workloads import SPECS, make_step

    to_bf16 = lambda a: torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(dev).view(torch.bfloat16)
    to_i32 = lambda a: torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to(dev)
    res = {}
    for name, layers in (("cfg1", 28), ("cfg2", 4), ("cfg3b", 4)):
        w = make_step(SPECS[name])
        s = w.spec
        B = w.num_decode
        pools = []
        for _ in range(layers):
            p = pg.Pool(s.num_blocks, s.block_size, s.num_kv_heads, device=dev)
            p.fill_logical(w.prefix_k[w.used_blocks].view(np.int16), w.prefix_v[w.used_blocks].view(np.int16),
                           blocks=w.used_blocks)
            pools.append(p)
        pad = int(np.setdiff1d(np.arange(s.num_blocks), w.used_blocks)[0])
        tok = w.dec_tok
        graphs = {}
        for fused in (False, True):
            g = DecodeGraphs(pools, s.num_q_heads, w.block_tables.shape[1], pad, to_bf16(w.wq), to_bf16(w.wk),
                             s.eps, s.rope_theta, 1.0 / math.sqrt(128), max_batch=B, buckets=[B], fused=fused)
            inp = g.inputs(B)
            for l in range(layers):
                inp.q[l].copy_(to_bf16(w.tok_q[tok]))
                inp.k[l].copy_(to_bf16(w.tok_k[tok]))
                inp.v[l].copy_(to_bf16(w.tok_v[tok]))
            inp.positions.copy_(to_i32(w.tok_pos[tok]))
            inp.context_lens.copy_(to_i32(w.dec_ctx))
            inp.block_tables.copy_(to_i32(w.dec_block_tables))
            graphs[fused] = (g, g.eager_calls(B))  # the captured calls, issued one by one on this stream

        def eager_of(calls):
            def run():
                for c in calls:
                    c()
            return run

        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(iters)]
        out = {"batch": B, "layers": layers}
        runs = (("eager", eager_of(graphs[False][1])), ("graph", lambda: graphs[False][0].replay(B)),
                ("fused_eager", eager_of(graphs[True][1])), ("fused_graph", lambda: graphs[True][0].replay(B)))
        for label, run in runs:
            for _ in range(5):
                run()
            torch.cuda.synchronize()
            for e0, e1 in ev:
                e0.record()
                run()
                e1.record()
            torch.cuda.synchronize()
            ts = sorted(e0.elapsed_time(e1) * 1e3 / layers for e0, e1 in ev)
            out[label + "_gpu_us_per_layer"] = round(ts[len(ts) // 2], 2)
            wall = []
            for _ in range(iters):
                t0 = time.perf_counter()
                run()
                torch.cuda.synchronize()
                wall.append((time.perf_counter() - t0) * 1e6)
            out[label + "_sync_us_per_step"] = round(sorted(wall)[len(wall) // 2], 1)
        res[name] = out
        del graphs, pools
        torch.cuda.empty_cache()
    return res


def measure_block_sizes(dev, sizes=(16, 32, 64, 128, 256)):
    """Decode on the batch-64 step and chunk attention on the mixed step at each
    block size, with the pool's token capacity held fixed."""
    import dataclasses

    import numpy as np
    import torch

    import paged_gqa_decode_head_amd as pg
    from paged_gqa_decode_head_amd.workloads import SPECS, make_step

    to_i32 = lambda a: torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to(dev)
    to_bf16 = lambda a: torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(dev).view(torch.bfloat16)
    scale = 1.0 / math.sqrt(128)
    cus = torch.cuda.get_device_properties(dev).multi_processor_count
    res = {"timing": "median of per-launch HIP events, each launch after a 1 GiB cache flush"}
    flush = CacheFlush(dev)
    time_calls = lambda calls, iters: time_calls_cold(calls, iters, flush)  # noqa: E731
    for bs in sizes:
        row = {}
        for name in ("cfg3b", "cfg5"):
            base = SPECS[name]
            spec = dataclasses.replace(base, block_size=bs, num_blocks=base.num_blocks * base.block_size // bs)
            w = make_step(spec)
            pools = []
            for _ in range(1):
                p = pg.Pool(spec.num_blocks, bs, spec.num_kv_heads, device=dev)
                p.fill_logical(w.prefix_k[w.used_blocks].view(np.int16), w.prefix_v[w.used_blocks].view(np.int16),
                               blocks=w.used_blocks)
                pools.append(p)
            q_out = torch.empty((w.num_tokens, spec.num_q_heads, 128), dtype=torch.bfloat16, device=dev)
            writes = [pg.bind_cache_write(p, to_bf16(w.tok_q), to_bf16(w.tok_k), to_bf16(w.tok_v), to_bf16(w.wq),
                                          to_bf16(w.wk), to_i32(w.tok_pos), to_i32(w.tok_seq),
                                          to_i32(w.block_tables), spec.eps, spec.rope_theta, q_out) for p in pools]
            med, _ = time_calls(writes, 20)
            row[f"{name}_write_us"] = round(med, 2)
            qd = q_out[torch.from_numpy(w.dec_tok.astype(np.int64)).to(dev)].contiguous()
            mx = int(w.dec_ctx.max())
            out = torch.empty((w.num_decode, spec.num_q_heads, 128), dtype=torch.bfloat16, device=dev)
            plan = pg.plan_decode(cus, bs, w.num_decode, spec.num_kv_heads, spec.num_q_heads, mx)
            calls = [pg.bind_decode(p, qd, to_i32(w.dec_ctx), to_i32(w.dec_block_tables), mx, scale, out, plan=plan)
                     for p in pools]
            med, _ = time_calls(calls, 30)
            nb = decode_alg_bytes(w)
            row[f"{name}_decode_us"] = round(med, 2)
            row[f"{name}_decode_frac_hbm_peak"] = round(nb / med / 1e3 / HBM_PEAK_GBS, 4)
            if name == "cfg5":
                qc = q_out[w.chk_tok0:].contiguous()
                qs, cx = w.chk_qsl, w.chk_ctx
                mq, mc = int(np.diff(qs).max()), int(cx.max())
                o2 = torch.empty((qc.shape[0], spec.num_q_heads, 128), dtype=torch.bfloat16, device=dev)
                cp = pg.plan_chunk(cus, bs, len(cx), qc.shape[0], spec.num_kv_heads, spec.num_q_heads, mq, mc)
                calls = [pg.bind_chunk(p, qc, to_i32(qs), to_i32(cx), to_i32(w.chk_block_tables), mq, mc, scale, o2,
                                       plan=cp) for p in pools]
                med, _ = time_calls(calls, 20)
                flops, kv = chunk_alg(w, qs, cx)
                row["cfg5_chunk_us"] = round(med, 2)
                row["cfg5_chunk_frac_mfma_bf16_peak"] = round(flops / med / 1e6 / MFMA_BF16_PEAK_TFLOPS, 4)
            for p in pools:
                assert p.check_errors() == 0
            del pools
            torch.cuda.empty_cache()
        res[str(bs)] = row
    del flush
    torch.cuda.empty_cache()
    return res


def measure_serving(dev, budget=512, prompt_len=6528, streams=8, inject_at=2, tail=3):
    """The decode-stall workload shape: `streams` decode streams (contexts
    U[2048, 8192] already cached) and one prompt of `prompt_len` tokens injected
    at step `inject_at`.  The step planner (host producers) feeds one fused
    write and one attention call per step (the fused decode step when every
    segment is a single token, else the one-launch mixed call from a work list
    built on the host); GPU time per step from events.
    Chunked (token budget `budget`) vs whole-prompt prefill: worst and median
    step time seen by the decode streams, and the prompt's time to its first
    token.  Attention and cache write only: no projections or MLP."""
    import numpy as np
    import torch

    import paged_gqa_decode_head_amd as pg

    rng = np.random.default_rng(606)
    bs, hkv, hq = 16, 8, 16
    width = (8192 + 64 + 8) // bs + 1
    ctx0 = rng.integers(2048, 8193, size=streams)
    nb = int(sum(-(-int(c + 64) // bs) for c in ctx0) + -(-prompt_len // bs) + 64)
    scale = 1.0 / math.sqrt(128)
    cus = torch.cuda.get_device_properties(dev).multi_processor_count
    to_i32 = lambda a: torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to(dev)
    pool = pg.Pool(nb, bs, hkv, device=dev)
    g = torch.Generator(device=dev)
    g.manual_seed(7)
    pool.storage.normal_(generator=g)
    wq = torch.ones(128, dtype=torch.bfloat16, device=dev)
    wk = torch.ones(128, dtype=torch.bfloat16, device=dev)
    qkv_cap = prompt_len + streams * 8
    q_all = torch.randn((qkv_cap, hq, 128), device=dev, generator=g).to(torch.bfloat16)
    k_all = torch.randn((qkv_cap, hkv, 128), device=dev, generator=g).to(torch.bfloat16)
    v_all = torch.randn((qkv_cap, hkv, 128), device=dev, generator=g).to(torch.bfloat16)
    q_buf = torch.empty((qkv_cap, hq, 128), dtype=torch.bfloat16, device=dev)
    o_buf = torch.empty((qkv_cap, hq, 128), dtype=torch.bfloat16, device=dev)
    res = {}
    # a first, untimed pass of the chunked run loads every kernel it uses
    for label, chunked in (("warmup", True), ("chunked", True), ("whole_prompt", False)):
        planner = pg.StepPlanner(budget, streams + 1, chunked, bs, width, streams + 1, np.arange(nb)[::-1])
        for i in range(streams):  # streams whose prefix is already cached (blocks taken directly)
            need = -(-int(ctx0[i]) // bs)
            planner.block_tables[i, :need] = planner.free_list[planner.free_count.value - need:
                                                                planner.free_count.value][::-1]
            planner.free_count.value -= need
            planner.seqs[i] = [int(ctx0[i]), 0, 0, need]
        step_us, decode_gap_us = [], []
        prompt_done_us, t_inject = None, None
        elapsed = 0.0
        step = 0
        while True:
            if step == inject_at:
                planner.seqs[streams] = [0, prompt_len, 0, 0]
                t_inject = elapsed
            plan = planner.plan(token_capacity=qkv_cap)
            segs = plan["segs"]
            T = plan["token_pos"].size
            bt_seg = np.ascontiguousarray(planner.block_tables[segs[:, 0]])
            ctx, qsl = plan["context_lens"], plan["query_start_loc"]
            args = (to_i32(plan["token_pos"]), to_i32(plan["token_seq"]), to_i32(planner.block_tables),
                    to_i32(qsl), to_i32(ctx), to_i32(bt_seg))
            q_out = q_buf[:T]
            out = o_buf[:T]
            if (segs[:, 2] == 1).all():  # host routing: single decode tokens only -> one fused decode step
                calls = [pg.bind_decode_step(pool, q_all[:T], k_all[:T], v_all[:T], wq, wk, args[4], args[5],
                                             int(ctx.max()), 1e-6, 1e6, scale, out, q_out=q_out)]
            else:  # the fused write, then the mixed step's one attention launch from the host-built work list
                mplan, items = pg.plan_mixed(cus, bs, hkv, hq, qsl, ctx)
                calls = [pg.bind_cache_write(pool, q_all[:T], k_all[:T], v_all[:T], wq, wk, args[0], args[1],
                                             args[2], 1e-6, 1e6, q_out),
                         pg.bind_mixed(pool, q_out, args[3], args[4], args[5], int(segs[:, 2].max()),
                                       int(ctx.max()), scale, out, mplan, to_i32(items))]
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for c in calls:
                c()
            e1.record()
            torch.cuda.synchronize()
            us = e0.elapsed_time(e1) * 1e3
            elapsed += us
            step_us.append(round(us, 1))
            planner.commit(segs, None)
            if t_inject is not None and prompt_done_us is None and planner.seqs[streams, 1] == 0 and \
                    planner.seqs[streams, 0] > 0:
                prompt_done_us = elapsed - t_inject
                done_step = step
            step += 1
            if prompt_done_us is not None and step > done_step + tail:
                break
        assert pool.check_errors() == 0
        if label == "warmup":
            continue
        res[label] = {"steps": len(step_us), "worst_step_us": max(step_us),
                      "median_step_us": float(np.median(step_us)), "prompt_ttft_us": round(prompt_done_us, 1),
                      "step_us": step_us}
    res["worst_step_ratio_whole_over_chunked"] = round(res["whole_prompt"]["worst_step_us"] /
                                                       res["chunked"]["worst_step_us"], 2)
    res["config"] = {"streams": streams, "stream_contexts": ctx0.tolist(), "prompt_len": prompt_len,
                     "token_budget": budget, "block_size": bs, "heads": [hq, hkv]}
    return res


def copy_calibration(dev, mib=256, reps=5):
    """A plain streaming kernel of known size (torch.neg: reads and writes `mib`
    MiB per launch, easy to find by name in a counter trace), for scaling the
    FETCH_SIZE / WRITE_SIZE counters."""
    import torch

    src = torch.ones(mib * 2**20 // 2, dtype=torch.bfloat16, device=dev)
    dst = torch.empty_like(src)
    for _ in range(reps):
        torch.neg(src, out=dst)
    torch.cuda.synchronize()
    return {"kernel": "torch.neg", "bytes_read_and_written_each": mib * 2**20, "reps": reps}


def recorded_traffic():
    """HBM bytes per decode launch from the committed counter record, or None if
    the decode kernel's sources changed since the counters were taken."""
    import hashlib

    path = os.path.join(ROOT, "profiles", "decode_cfg3b_traffic.json")
    try:
        rec = json.load(open(path))
        src = b"".join(open(os.path.join(ROOT, "paged_gqa_decode_head_amd", "csrc", f), "rb").read()
                       for f in ("decode.hip", "device_common.hpp", "norm_rope.hpp", "launch.hpp"))
    except OSError:
        return None
    if hashlib.sha256(src).hexdigest() != rec.get("kernel_source_sha256"):
        return None
    return rec["traffic_bytes_per_launch"]


def percentiles(us):
    """median, p10 and p90 of a list of per-launch times (µs)."""
    import numpy as np

    a = np.asarray(us, dtype=np.float64)
    return {"median": round(float(np.median(a)), 3), "p10": round(float(np.percentile(a, 10)), 3),
            "p90": round(float(np.percentile(a, 90)), 3)}


def per_launch_us(call, n, cycle=1):
    """Event pair around each of n launches (after a short warm-up); returns the µs list."""
    import torch

    for i in range(5):
        call(i % cycle)
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]
    for i, (a, b) in enumerate(ev):
        a.record()
        call(i % cycle)
        b.record()
    torch.cuda.synchronize()
    return [a.elapsed_time(b) * 1e3 for a, b in ev]


def stream_read_ceiling(dev, nbytes: int, copies: int = 4):
    """The library's plain streaming-read kernel over nbytes, cycling `copies`
    buffers (so reads come from HBM, not the 256 MB Infinity Cache): the
    achievable read rate of one launch of this size."""
    import torch
    import paged_gqa_decode_head_amd as pg

    nbytes = nbytes // 16 * 16
    bufs = [torch.ones(nbytes // 4, dtype=torch.int32, device=dev) for _ in range(copies)]
    grid = 3 * torch.cuda.get_device_properties(dev).multi_processor_count
    sink = torch.empty(grid * 256, dtype=torch.int32, device=dev)
    calls = [pg.bind_stream_read(b, sink, grid) for b in bufs]
    us = per_launch_us(lambda i: calls[i](), 40, copies)
    pct = percentiles(us)
    del bufs, calls
    torch.cuda.empty_cache()
    return {"kernel": "pgqa_stream_read (16-byte non-temporal loads, grid-stride, 3 workgroups per CU)",
            "bytes": nbytes, "us": pct, "gbs": round(nbytes / pct["median"] / 1e3, 1),
            "frac_hbm_peak": round(nbytes / pct["median"] / 1e3 / HBM_PEAK_GBS, 4)}


# ---------------------------------------------------------------- cpu baseline
# The fp64 oracle timed on the host on the same synthetic steps: one process
# with BLAS at one thread, and a pool of spawned worker processes (created
# before the first GPU call; they import only numpy and the oracle and never
# touch the GPU) over (sequence, kv head) and (segment, kv head, query block)
# units.  The step's arrays reach the workers through shared memory.
CPU_ROWS = ("cfg2", "cfg3a", "cfg3b", "cfg4", "cfg5_decode", "cfg5_slice", "cfg5_verify")
_SHM = {}


def _cpu_worker_init():
    """Worker start-up: one BLAS/OpenMP thread per worker process (the pool is
    the parallelism), set before the worker first imports numpy."""
    for var in ("OMP_NUM_THREADS", "OPENBLAS_NUM_THREADS", "MKL_NUM_THREADS", "BLIS_NUM_THREADS"):
        os.environ[var] = "1"


def _cpu_attach(name, shape, dtype):
    """A numpy view of a shared-memory array (attached once per worker)."""
    import numpy as np
    from multiprocessing import shared_memory

    if name not in _SHM:
        _SHM[name] = shared_memory.SharedMemory(name=name)
    return np.ndarray(shape, dtype=dtype, buffer=_SHM[name].buf)


def _cpu_unit(task):
    """One unit of the oracle's work on the shared arrays: decode attention of
    sequence b over kv head g, or chunk attention of query rows [i0, i1) of
    segment s over kv head g (the rows as a sub-segment that ends at position
    n - q_len + i1, which is how the chunk rule aligns them)."""
    import numpy as np
    import oracle as O

    kind, arrs, scale, r, unit = task
    q = _cpu_attach(*arrs["q"])
    pk = _cpu_attach(*arrs["pk"])
    pv = _cpu_attach(*arrs["pv"])
    bt = _cpu_attach(*arrs["bt"])
    ctx = _cpu_attach(*arrs["ctx"])
    if kind == "decode":
        b, g = unit
        o = O.decode_attention(O.bf16_bits_to_f64(q[b:b + 1, g * r:(g + 1) * r]), pk[:, :, g:g + 1],
                               pv[:, :, g:g + 1], bt[b:b + 1], ctx[b:b + 1], scale)
    else:
        qsl = _cpu_attach(*arrs["qsl"])
        seg, g, i0, i1 = unit
        q0, qlen, n = int(qsl[seg]), int(qsl[seg + 1] - qsl[seg]), int(ctx[seg])
        o = O.chunk_attention(O.bf16_bits_to_f64(q[q0 + i0:q0 + i1, g * r:(g + 1) * r]), np.array([0, i1 - i0]),
                              pk[:, :, g:g + 1], pv[:, :, g:g + 1], bt[seg:seg + 1],
                              np.array([n - qlen + i1]), scale)
    return float(np.abs(o).sum())


def _cpu_step(w, row):
    """(kind, q bits, compact pool K/V, compact block tables, contexts, qsl,
    units, algorithmic bytes, sequences or query tokens) of one row's step."""
    import numpy as np

    s = w.spec
    inv = np.full(s.num_blocks, -1, dtype=np.int64)
    inv[w.used_blocks] = np.arange(len(w.used_blocks))
    bt_c = np.where(w.block_tables >= 0, inv[np.maximum(w.block_tables, 0)], -1)
    pk, pv = w.prefix_k[w.used_blocks], w.prefix_v[w.used_blocks]
    hkv = s.num_kv_heads
    if not row.startswith("cfg5") or row == "cfg5_decode":
        q = w.tok_q[w.dec_tok]
        ctx = w.dec_ctx
        units = [(b, g) for b in range(w.num_decode) for g in range(hkv)]
        work = [int(ctx[b]) for b, _ in units]
        return ("decode", q, pk, pv, bt_c[: w.num_decode], ctx, None, units, decode_alg_bytes(w), w.num_decode,
                None, work)
    qc = w.tok_q[w.chk_tok0:]
    qsl, ctx, bt = w.chk_qsl, w.chk_ctx, bt_c[w.num_decode:]
    segs = [0] if row == "cfg5_slice" else list(range(1, len(ctx)))
    units, work = [], []
    for seg in segs:
        ql, n = int(qsl[seg + 1] - qsl[seg]), int(ctx[seg])
        for g in range(hkv):
            for i0 in range(0, ql, 32):
                i1 = min(ql, i0 + 32)
                units.append((seg, g, i0, i1))
                work.append(sum(n - ql + i + 1 for i in range(i0, i1)))   # visible (query, key) pairs
    sel = np.array(segs)
    flops, kv = chunk_alg(w, np.concatenate([[0], np.cumsum(np.diff(qsl)[sel])]), ctx[sel])
    tokens = int(np.diff(qsl)[sel].sum())
    return ("chunk", qc, pk, pv, bt, ctx, qsl, units, kv, tokens, flops, work)


def cpu_baseline(pool, pool_size, seconds_per_row: float, sample=None):
    """The oracle on every row's step, one process (BLAS at one thread) and the
    worker pool; rates from the same algorithmic bytes as the GPU rows."""
    import numpy as np
    from multiprocessing import shared_memory

    import oracle as O
    from paged_gqa_decode_head_amd.workloads import SPECS, make_step

    try:
        from threadpoolctl import threadpool_limits
    except ImportError:
        threadpool_limits = None
    scale = 1.0 / math.sqrt(128)
    out = {}
    for row in CPU_ROWS:
        w = make_step(SPECS[row.split("_")[0]])
        st = _cpu_step(w, row)
        kind, q, pk, pv, bt, ctx, qsl, units, nbytes, count = st[:10]
        shms, arrs = [], {}
        for key, a in (("q", q), ("pk", pk), ("pv", pv), ("bt", bt.astype(np.int64)), ("ctx", ctx.astype(np.int64)),
                       ("qsl", None if qsl is None else qsl.astype(np.int64))):
            if a is None:
                continue
            a = np.ascontiguousarray(a)
            m = shared_memory.SharedMemory(create=True, size=max(a.nbytes, 1))
            np.ndarray(a.shape, dtype=a.dtype, buffer=m.buf)[...] = a
            shms.append(m)
            arrs[key] = (m.name, a.shape, a.dtype.str)
        work = st[11]
        r = w.spec.num_q_heads // w.spec.num_kv_heads
        tasks = [(kind, arrs, scale, r, u) for u in units]
        res = {"units": len(units), "alg_bytes": int(nbytes)}
        if kind == "chunk":
            res["flops"] = int(st[10])
        for mode in ("single_thread", "pool"):
            ctxm = threadpool_limits(limits=1) if threadpool_limits is not None else None
            if ctxm is not None:
                ctxm.__enter__()
            try:
                if mode == "pool":
                    # whole steps: one timed, repeated while that took under the row's budget
                    run = lambda: pool.map(_cpu_unit, tasks, chunksize=max(1, len(tasks) // (4 * pool_size)))
                    t0 = time.perf_counter()
                    run()
                    el, reps = time.perf_counter() - t0, 1
                    more = min(50, int(seconds_per_row / max(el, 1e-3)))
                    if more > 0:
                        t0 = time.perf_counter()
                        for _ in range(more):
                            run()
                        el, reps = (time.perf_counter() - t0) / more, more
                    sampled = 1.0
                else:
                    # units in a strided order until the budget is spent; the
                    # step's time is extrapolated by the share of its (query,
                    # key) pairs done (units of one step differ only in length)
                    order = [i for k in range(7) for i in range(k, len(tasks), 7)]
                    done_work, reps, t0 = 0, 0, time.perf_counter()
                    for i in order:
                        _cpu_unit(tasks[i])
                        done_work += work[i]
                        reps += 1
                        if time.perf_counter() - t0 >= seconds_per_row:
                            break
                    sampled = done_work / sum(work)
                    el = (time.perf_counter() - t0) / sampled
            finally:
                if ctxm is not None:
                    ctxm.__exit__(None, None, None)
            d = {"s_per_step": round(el, 5), "gbs": round(nbytes / el / 1e9, 3),
                 "cores": 1 if mode == "single_thread" else pool_size,
                 "steps_timed" if mode == "pool" else "units_timed": reps,
                 "share_of_step_timed": round(min(sampled, 1.0) if mode != "pool" else float(reps), 4)}
            if kind == "decode":
                d["seqs_per_s"] = round(count / el, 1)
            else:
                d["tokens_per_s"] = round(count / el, 1)
                d["gflops"] = round(st[10] / el / 1e9, 2)
            res[mode] = d
        for m in shms:
            m.close()
            m.unlink()
        out[row] = res
    parity = None
    if sample is not None:
        rows = sample["rows"]
        ref = O.decode_attention(O.bf16_bits_to_f64(sample["q_bits"])[rows], sample["k_bits"], sample["v_bits"],
                                 sample["block_tables"][rows], sample["ctx"][rows], sample["scale"])
        got = O.bf16_bits_to_f64(sample["out_bits"])[rows]
        d = np.abs(got - ref)
        parity = {"rows": rows, "max_abs": float(d.max()), "mean_rel": float(d.sum() / np.abs(ref).sum())}
    head = out["cfg3b"]["pool"]
    return {
        "value": head["gbs"], "unit": "GB/s", "seqs_per_s": head["seqs_per_s"], "cores": pool_size,
        "host_cpus": os.cpu_count(), "affinity_cpus": len(os.sched_getaffinity(0)), "kind": "oracle",
        "sample": "the whole batch-64 Qwen3-1.7B decode step (64 sequences x 8 kv heads), repeated, fp64 numpy "
                  f"oracle in a pool of {pool_size} spawned processes over (sequence, kv head) units; every other "
                  "row's step in 'rows' the same way, and in one process with BLAS at one thread on a strided "
                  "sample of the step's units (share_of_step_timed), extrapolated by (query, key) pairs",
        "rows": out,
        "parity_sample": parity,
    }


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="cfg3b")
    ap.add_argument("--layers", type=int, default=4)
    ap.add_argument("--split-tokens", type=int, default=0, help="override the planner's split length")
    ap.add_argument("--waves", type=int, default=0, help="override the planner's waves per split")
    ap.add_argument("--cpu-seconds", type=float, default=2.0, help="host time budget per cpu_baseline row and mode")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--main-only", action="store_true", help="skip the per-row measurements of the other workloads")
    ap.add_argument("--only", choices=["cfg2", "cfg3a", "cfg4", "cfg5", "chunk"], default=None,
                    help="profiling aid: run only one workload's rows and print them (cfg5 or chunk: the mixed "
                         "workload, chunk attention included)")
    ap.add_argument("--calibrate-copy", action="store_true", help="also run a 256 MiB plain copy (counter scaling)")
    ap.add_argument("--no-host-lengths", action="store_true",
                    help="do not pass the host-side context lengths to the decode plans (natural unit order)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py: the benchmark runs on one GPU only (asked for --gpus {args.gpus}); the decode path "
              "shards by sequence or kv head with no exchange, which this benchmark does not exercise",
              file=sys.stderr)
        sys.exit(2)

    # The oracle's worker processes are spawned before anything touches the GPU.
    cpu_pool, cpu_pool_size = None, 0
    if not args.no_cpu_baseline and args.only is None:
        import multiprocessing as mp

        cpu_pool_size = max(1, min(16, len(os.sched_getaffinity(0))))
        cpu_pool = mp.get_context("spawn").Pool(cpu_pool_size, initializer=_cpu_worker_init)

    import numpy as np
    import torch

    import paged_gqa_decode_head_amd as pg
    from paged_gqa_decode_head_amd.workloads import SPECS, make_step

    torch.cuda.set_device(0)
    dev = torch.device("cuda", 0)
    if args.only is not None:
        # profiling aid: only one workload's rows (its write, decode and, for the
        # mixed workload, chunk calls)
        print(json.dumps({"rows": measure_rows(args, dev, ("cfg5",) if args.only == "chunk" else (args.only,))}),
              flush=True)
        if args.calibrate_copy:
            copy_calibration(dev)
        return
    w = make_step(SPECS[args.workload])
    s = w.spec
    to_bf16 = lambda a: torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(dev).view(torch.bfloat16)
    to_i32 = lambda a: torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to(dev)

    pools = []
    for _ in range(args.layers):
        p = pg.Pool(s.num_blocks, s.block_size, s.num_kv_heads, device=dev)
        p.fill_logical(w.prefix_k[w.used_blocks].view(np.int16), w.prefix_v[w.used_blocks].view(np.int16),
                       blocks=w.used_blocks)
        pools.append(p)
    q, k, v = to_bf16(w.tok_q), to_bf16(w.tok_k), to_bf16(w.tok_v)
    wq, wk = to_bf16(w.wq), to_bf16(w.wk)
    pos, seq, bt = to_i32(w.tok_pos), to_i32(w.tok_seq), to_i32(w.block_tables)
    ctx = to_i32(w.dec_ctx)
    max_ctx = int(w.dec_ctx.max())
    scale = 1.0 / math.sqrt(128)
    q_out = torch.empty((w.num_tokens, s.num_q_heads, 128), dtype=torch.bfloat16, device=dev)
    out = torch.empty((w.num_decode, s.num_q_heads, 128), dtype=torch.bfloat16, device=dev)
    props = torch.cuda.get_device_properties(dev)
    plan = pg.plan_decode(props.multi_processor_count, s.block_size, w.num_decode, s.num_kv_heads, s.num_q_heads,
                          max_ctx)
    if args.split_tokens:
        plan.split_tokens = args.split_tokens
        plan.max_splits = -(-max_ctx // args.split_tokens)
    if args.waves:
        plan.waves_per_split = args.waves
    ws = torch.zeros(pg.decode_workspace_bytes(pools[0], w.num_decode, s.num_q_heads, max_ctx, plan),
                     dtype=torch.uint8, device=dev)
    # the serving loop's host-side lengths, for the length-balanced unit order
    # (the same plan without them is timed beside it)
    plan_nohint = pg.DecodePlan(plan.split_tokens, plan.max_splits, plan.waves_per_split, plan.load_hint,
                                plan.kernel)
    if not args.no_host_lengths:
        plan.set_host_context_lens(w.dec_ctx)
    assert w.num_tokens == w.num_decode and np.array_equal(w.dec_tok, np.arange(w.num_decode))
    assert np.array_equal(w.tok_pos, w.dec_ctx - 1)
    fused = [pg.bind_decode_step(p, q, k, v, wq, wk, ctx, bt, max_ctx, s.eps, s.rope_theta, scale, out, plan=plan,
                                 workspace=ws) for p in pools]
    two = [(pg.bind_cache_write(p, q, k, v, wq, wk, pos, seq, bt, s.eps, s.rope_theta, q_out),
            pg.bind_decode(p, q_out, ctx, bt, max_ctx, scale, out, plan=plan, workspace=ws)) for p in pools]
    fused_nohint = [pg.bind_decode_step(p, q, k, v, wq, wk, ctx, bt, max_ctx, s.eps, s.rope_theta, scale, out,
                                        plan=plan_nohint, workspace=ws) for p in pools]

    def timed(issue):
        """Warmup, then exactly args.steps steps between two synchronisations,
        with one HIP event pair on the launch stream bracketing the region.
        Returns (wall ms per step, event ms per step)."""
        for i in range(args.warmup):
            issue(i)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        t0 = time.perf_counter()
        e0.record()
        for i in range(args.steps):
            issue(i)
        e1.record()
        torch.cuda.synchronize()
        return (time.perf_counter() - t0) * 1e3 / args.steps, e0.elapsed_time(e1) / args.steps

    def issue_fused(i):
        fused[i % args.layers]()

    def issue_two(i):
        wr, dc = two[i % args.layers]
        wr()
        dc()

    ms_two, _ = timed(issue_two)
    ms_step, step_ms = timed(issue_fused)
    ms_nohint, nohint_ms = timed(lambda i: fused_nohint[i % args.layers]())
    # the two-call step's split between its launches: events around each call, in a loop of its own
    ev_two = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    for i, e in enumerate(ev_two):
        wr, dc = two[i % args.layers]
        e[0].record()
        wr()
        e[1].record()
        dc()
        e[2].record()
    torch.cuda.synchronize()
    for p in pools:
        assert p.check_errors() == 0

    write_ms = sum(e[0].elapsed_time(e[1]) for e in ev_two) / args.steps
    decode_ms = sum(e[1].elapsed_time(e[2]) for e in ev_two) / args.steps
    dec_bytes = decode_alg_bytes(w)
    wr_bytes = write_alg_bytes(w)
    step_bytes = step_alg_bytes(w)
    gbs = step_bytes / (ms_step * 1e-3) / 1e9
    launch_gbs = step_bytes / (step_ms * 1e-3) / 1e9
    two_bytes = dec_bytes + wr_bytes

    # One fused step's outputs for the sampled parity check of the cpu_baseline
    # leg (q_out requested so the reference sees the q the kernel used).
    sample = None
    fused_pool = pools[0]
    if not args.no_cpu_baseline:
        pg.decode_step(fused_pool, q, k, v, wq, wk, ctx, bt, max_ctx, s.eps, s.rope_theta, scale, plan=plan,
                       workspace=ws, out=out, q_out=q_out)
        torch.cuda.synchronize()
        k_all, v_all = fused_pool.read_logical(blocks=w.used_blocks)
        inv = np.full(s.num_blocks, -1, dtype=np.int64)
        inv[w.used_blocks] = np.arange(len(w.used_blocks))
        sample = {"rows": [0, w.num_decode // 2, w.num_decode - 1],
                  "q_bits": q_out.view(torch.int16).cpu().numpy().view(np.uint16),
                  "out_bits": out.view(torch.int16).cpu().numpy().view(np.uint16),
                  "k_bits": k_all.numpy().view(np.uint16), "v_bits": v_all.numpy().view(np.uint16),
                  "block_tables": np.where(w.block_tables >= 0, inv[np.maximum(w.block_tables, 0)], -1),
                  "ctx": w.dec_ctx, "scale": scale}

    launch_dist = percentiles(per_launch_us(lambda i: fused[i % args.layers](), args.steps, args.layers))
    ceiling = stream_read_ceiling(dev, step_bytes) if not args.main_only else None

    result = {
        "metric": METRIC,
        "value": round(gbs, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": f"{args.workload}: {s.description}",
            "batch": w.num_decode, "num_q_heads": s.num_q_heads, "num_kv_heads": s.num_kv_heads,
            "head_dim": 128, "block_size": s.block_size, "context_tokens": int(w.dec_ctx.sum()),
            "layers_cycled": args.layers,
            "plan": {"split_tokens": plan.split_tokens, "max_splits": plan.max_splits,
                     "waves_per_split": plan.waves_per_split,
                     "kernel": "mfma" if plan.kernel == 2 else "dot",
                     "host_context_lens": bool(plan.host_context_lens)},
        },
        "pct_of_hbm_peak": round(100 * gbs / HBM_PEAK_GBS, 2),
        "seqs_per_s": round(w.num_decode / (ms_step * 1e-3), 1),
        "tokens_per_s": round(w.num_decode / (ms_step * 1e-3), 1),
        "step_alg_bytes": step_bytes,
        "step_us_events": round(step_ms * 1e3, 3),
        "roofline": {
            "kernel": "decode_kernel<2, 4, true, true> (fused decode step: norm + rotary + cache write + decode)",
            "bound": "hbm", "achieved": round(launch_gbs, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(launch_gbs / HBM_PEAK_GBS, 4),
            "traffic": recorded_traffic() if args.workload == "cfg3b" else None,
            "alg_bytes_per_launch": step_bytes, "avg_launch_us": round(step_ms * 1e3, 3),
            "launch_us_events_each": launch_dist,
            "frac_of_stream_read": round(launch_gbs / ceiling["gbs"], 4) if ceiling else None,
        },
        "stream_read_ceiling": ceiling,
        "without_host_lengths": {
            "what": "the same fused step with plan.host_context_lens unset (natural unit order)",
            "ms_per_step": round(ms_nohint, 5), "us_events": round(nohint_ms * 1e3, 3),
            "frac_hbm_peak": round(step_bytes / (nohint_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
        },
        "two_call_step": {
            "calls": "pgqa_rms_norm_rope_cache_write + pgqa_paged_decode_attention",
            "ms_per_step": round(ms_two, 5), "alg_bytes": two_bytes,
            "value_gbs": round(two_bytes / (ms_two * 1e-3) / 1e9, 2),
            "write_us": round(write_ms * 1e3, 3), "decode_us": round(decode_ms * 1e3, 3),
            "decode_gbs": round(dec_bytes / (decode_ms * 1e-3) / 1e9, 2),
        },
    }
    if args.calibrate_copy:
        result["copy_calibration"] = copy_calibration(dev)
    if not args.main_only:
        del pools, fused, two, fused_pool, fused_nohint
        torch.cuda.empty_cache()
        result["rows"] = measure_rows(args, dev)
        result["rows"]["decode_graph"] = measure_graphs(dev)
        result["rows"]["block_size"] = measure_block_sizes(dev)
        result["rows"]["serving_decode_stall"] = measure_serving(dev)
    if cpu_pool is not None:
        result["cpu_baseline"] = cpu_baseline(cpu_pool, cpu_pool_size, args.cpu_seconds, sample)
        cpu_pool.close()
        cpu_pool.join()
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()

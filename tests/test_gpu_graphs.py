"""HIP-graph capture and replay of the decode step (cache write + decode over
two layer pools) at bucketed batch sizes, checked bit for bit against the same
calls made eagerly with the same plan, replay after replay, with eager work
and synchronisations in between; the graph path is also checked against the
fp64 reference once."""
import numpy as np
import pytest
import torch

import oracle as O
import paged_gqa_decode_head_amd as pg
from paged_gqa_decode_head_amd.graphs import DecodeGraphs

from harness import SCALE, bits_of, compare, dev_bf16, dev_i32

pytestmark = pytest.mark.gpu

NB, BS, MAXB, MBS = 64, 16, 4, 8   # pool blocks, block size, max batch, blocks/seq
EPS, THETA = 1e-6, 1e6


def _bf16(rng, shape):
    return torch.from_numpy(rng.standard_normal(shape)).to(torch.bfloat16).to("cuda")


def _pools(rng, n, hkv):
    k = torch.from_numpy(rng.standard_normal((NB, BS, hkv, 128))).to(torch.bfloat16)
    v = torch.from_numpy(rng.standard_normal((NB, BS, hkv, 128))).to(torch.bfloat16)
    out = []
    for _ in range(n):
        p = pg.Pool(NB, BS, hkv)
        p.fill_logical(k.view(torch.int16).numpy(), v.view(torch.int16).numpy())
        out.append(p)
    return out


@pytest.mark.parametrize("fused", [True, False])
@pytest.mark.parametrize("hq,hkv", [(16, 8), (32, 4)])  # the dot-product and the matrix-core split kernel
def test_decode_graph_replays_match_eager_calls(fused, hq, hkv):
    """Graphs of the fused step (one launch per layer) or of the two calls,
    against the two eager calls: the fused step is bit-identical to them."""
    rng = np.random.default_rng(31)
    L = 2
    state = rng.bit_generator.state
    pools_g = _pools(rng, L, hkv)
    rng.bit_generator.state = state
    pools_e = _pools(rng, L, hkv)
    wq = torch.from_numpy(1 + 0.1 * rng.standard_normal(128)).to(torch.bfloat16).cuda()
    wk = torch.from_numpy(1 + 0.1 * rng.standard_normal(128)).to(torch.bfloat16).cuda()
    pad = NB - 1
    graphs = DecodeGraphs(pools_g, hq, MBS, pad, wq, wk, EPS, THETA, SCALE, MAXB, buckets=[1, 2, 4], fused=fused)
    assert graphs.bucket_for(3) == 4 and graphs.bucket_for(5) is None
    perm = rng.permutation(NB - 1)  # block ids for the sequences; the pad block is never dealt
    for step, B in enumerate([3, 4, 1, 3, 2]):
        print(f"[graph] fused={fused} heads {hq}/{hkv} step {step} batch {B}", flush=True)
        bucket = graphs.bucket_for(B)
        ctx = rng.integers(1, MBS * BS + 1, size=B).astype(np.int32)
        bt = np.full((B, MBS), -1, dtype=np.int32)
        for i in range(B):
            nblk = -(-int(ctx[i]) // BS)
            bt[i, :nblk] = perm[i * MBS: i * MBS + nblk]
        pos = ctx - 1
        q, k, v = _bf16(rng, (L, B, hq, 128)), _bf16(rng, (L, B, hkv, 128)), _bf16(rng, (L, B, hkv, 128))
        ctx_d, bt_d, pos_d = dev_i32(ctx), dev_i32(bt), dev_i32(pos)
        seq_d = dev_i32(np.arange(B))
        # eager calls with the bucket's plan
        qo_e, out_e = [], []
        for l in range(L):
            qo = pg.rms_norm_rope_cache_write(pools_e[l], q[l].contiguous(), k[l].contiguous(), v[l].contiguous(),
                                              wq, wk, pos_d, seq_d, bt_d, EPS, THETA)
            qo_e.append(qo)
            out_e.append(pg.paged_decode_attention(pools_e[l], qo, ctx_d, bt_d, graphs.max_ctx, SCALE,
                                                   plan=graphs.plan(bucket)))
        # graph replay
        inp = graphs.inputs(B)
        inp.q.copy_(q)
        inp.k.copy_(k)
        inp.v.copy_(v)
        inp.positions.copy_(pos_d)
        inp.context_lens.copy_(ctx_d)
        inp.block_tables.copy_(bt_d)
        qo_g, out_g = graphs.replay(B)
        # unrelated eager work and a synchronisation between replays
        x = torch.randn(256, 256, device="cuda")
        (x @ x).sum().item()
        torch.cuda.synchronize()
        for l in range(L):
            assert np.array_equal(bits_of(qo_g[l]), bits_of(qo_e[l])), (step, l, "q_out")
            assert np.array_equal(bits_of(out_g[l]), bits_of(out_e[l])), (step, l, "out")
        if step == 0:  # the graph path against the fp64 reference (layer 0)
            kk, vv = pools_g[0].read_logical()
            ref = O.decode_attention(O.bf16_bits_to_f64(bits_of(qo_g[0])), kk.numpy().view(np.uint16),
                                     vv.numpy().view(np.uint16), bt, ctx, SCALE)
            compare(out_g[0], ref, "graph replay vs fp64")
    # the caches agree everywhere but in the pad block
    for l in range(L):
        kg, vg = pools_g[l].read_logical()
        ke, ve = pools_e[l].read_logical()
        keep = np.arange(NB) != pad
        assert np.array_equal(kg.numpy()[keep], ke.numpy()[keep])
        assert np.array_equal(vg.numpy()[keep], ve.numpy()[keep])
        assert pools_g[l].check_errors() == 0 and pools_e[l].check_errors() == 0

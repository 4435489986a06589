"""Pins of the fp64 reference against things other than itself.

Each test checks the reference against a closed form, an invariant, a library
routine (torch, transformers' Qwen3 modules) or brute force, chosen so that a
plausible mistake (a dropped term, a wrong sign, a swapped index, a wrong
alignment) fails at least one of them.  No GPU is used here.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "closed_forms.json")


def _golden():
    with open(GOLDEN) as f:
        return json.load(f)


# ---------------------------------------------------------------- bf16 format
def test_bf16_round_matches_torch_on_fp32_values():
    rng = np.random.default_rng(0)
    x = np.concatenate([
        rng.standard_normal(20000).astype(np.float32),
        (rng.standard_normal(2000) * 1e-39).astype(np.float32),   # bf16 subnormal range
        (rng.standard_normal(2000) * 3e38).astype(np.float32),    # near overflow
        np.array([0.0, -0.0, np.inf, -np.inf], dtype=np.float32),
    ])
    # exact ties: the low 16 bits are 0x8000; even and odd upper halves
    ties = (np.arange(0x3F80, 0x3F90, dtype=np.uint32) << 16) | 0x8000
    x = np.concatenate([x, ties.view(np.float32)])
    ref = torch.from_numpy(x).to(torch.bfloat16).to(torch.float64).numpy()
    got = O.bf16_round(x.astype(np.float64))
    assert np.array_equal(got, ref)
    bits = O.f64_to_bf16_bits(x.astype(np.float64))
    assert np.array_equal(O.bf16_bits_to_f64(bits), ref)


def test_bf16_ties_go_to_even():
    # 1 + 2**-8 is halfway between 1 and 1 + 2**-7: the even neighbour is 1
    assert O.bf16_round(np.array([1 + 2.0 ** -8]))[0] == 1.0
    # 1 + 3 * 2**-8 is halfway between 1 + 2**-7 (odd) and 1 + 2**-6 (even)
    assert O.bf16_round(np.array([1 + 3 * 2.0 ** -8]))[0] == 1 + 2.0 ** -6


# ---------------------------------------------------------------- a1 RMSNorm
def test_rms_norm_unit_rms_before_weight():
    rng = np.random.default_rng(1)
    x = rng.standard_normal((7, 3, 128)) * rng.uniform(0.01, 100, size=(7, 3, 1))
    y = O.rms_norm(x, np.ones(128), eps=0.0)
    assert np.allclose(np.sqrt(np.mean(y * y, axis=-1)), 1.0, rtol=0, atol=1e-14)
    # with eps the RMS is sqrt(ms / (ms + eps))
    ms = np.mean(x * x, axis=-1)
    y = O.rms_norm(x, np.ones(128), eps=1e-6)
    assert np.allclose(np.sqrt(np.mean(y * y, axis=-1)), np.sqrt(ms / (ms + 1e-6)), rtol=1e-14)


def test_rms_norm_scale_invariant_without_eps():
    rng = np.random.default_rng(2)
    x = rng.standard_normal((5, 128))
    w = 1 + 0.1 * rng.standard_normal(128)
    assert np.allclose(O.rms_norm(x, w, 0.0), O.rms_norm(37.5 * x, w, 0.0), rtol=1e-14, atol=0)


def test_rms_norm_closed_forms():
    for case in _golden()["rms_norm"]:
        D = case["head_dim"]
        w = np.linspace(0.5, 1.5, D)
        if "nonzero" in case:
            x = np.zeros(D)
            for i, v in case["nonzero"].items():
                x[int(i)] = v
            y = O.rms_norm(x[None], w, case["eps"])[0]
            assert y[0] == pytest.approx(case["y0_over_w0"] * w[0], rel=1e-15)
            assert np.all(y[1:] == 0)
        else:
            x = np.full(D, case["constant"])
            y = O.rms_norm(x[None], w, case["eps"])[0]
            assert np.allclose(y, case["y_over_w"] * w, rtol=1e-15, atol=0)


def test_rms_norm_matches_torch_and_qwen3_module():
    from transformers.models.qwen3.modeling_qwen3 import Qwen3RMSNorm

    rng = np.random.default_rng(3)
    x = rng.standard_normal((9, 16, 128))
    w = 1 + 0.1 * rng.standard_normal(128)
    ref = torch.nn.functional.rms_norm(torch.from_numpy(x), (128,), torch.from_numpy(w), eps=1e-6)
    assert np.allclose(O.rms_norm(x, w, 1e-6), ref.numpy(), rtol=1e-13, atol=1e-13)
    # the model's own module (computes in fp32 internally): plain weight, eps inside the root
    m = Qwen3RMSNorm(128, eps=1e-6).double()
    with torch.no_grad():
        m.weight.copy_(torch.from_numpy(w))
        ref2 = m(torch.from_numpy(x)).numpy()
    assert np.allclose(O.rms_norm(x, w, 1e-6), ref2, rtol=2e-6, atol=2e-6)


# ---------------------------------------------------------------- a2 RoPE
def test_rope_closed_forms():
    for case in _golden()["rope"]:
        D, i, p = case["head_dim"], case["pair"], case["position"]
        y = np.zeros((1, 1, D))
        y[0, 0, i] = 1.0                       # unit vector in the first half of pair i
        out = O.rope_neox(y, np.array([p]), case["theta"])[0, 0]
        assert out[i] == pytest.approx(case["cos"], abs=1e-15)
        assert out[i + D // 2] == pytest.approx(case["sin"], abs=1e-15)
        y = np.zeros((1, 1, D))
        y[0, 0, i + D // 2] = 1.0              # unit vector in the second half
        out = O.rope_neox(y, np.array([p]), case["theta"])[0, 0]
        assert out[i] == pytest.approx(-case["sin"], abs=1e-15)
        assert out[i + D // 2] == pytest.approx(case["cos"], abs=1e-15)
        others = np.delete(out, [i, i + D // 2])
        assert np.all(others == 0)


def test_rope_invariants():
    rng = np.random.default_rng(4)
    T, H, D = 11, 3, 128
    y = rng.standard_normal((T, H, D))
    pos = rng.integers(0, 40000, size=T)
    r = O.rope_neox(y, pos, 1e6)
    # pair norms preserved
    n0 = y[..., :64] ** 2 + y[..., 64:] ** 2
    n1 = r[..., :64] ** 2 + r[..., 64:] ** 2
    assert np.allclose(n0, n1, rtol=1e-12)
    # position 0 is the identity
    assert np.array_equal(O.rope_neox(y, np.zeros(T, dtype=np.int64), 1e6), y)
    # R(a) R(b) = R(a + b)
    a = rng.integers(0, 20000, size=T)
    b = rng.integers(0, 20000, size=T)
    assert np.allclose(O.rope_neox(O.rope_neox(y, a, 1e6), b, 1e6), O.rope_neox(y, a + b, 1e6), atol=1e-9)
    # <R(p) q, R(p') k> depends only on p - p'
    q = rng.standard_normal((1, 1, D))
    k = rng.standard_normal((1, 1, D))
    d1 = np.sum(O.rope_neox(q, np.array([900]), 1e6) * O.rope_neox(k, np.array([400]), 1e6))
    d2 = np.sum(O.rope_neox(q, np.array([30500]), 1e6) * O.rope_neox(k, np.array([30000]), 1e6))
    assert d1 == pytest.approx(d2, rel=1e-9)


def test_rope_matches_qwen3_rotary():
    from transformers import Qwen3Config
    from transformers.models.qwen3.modeling_qwen3 import Qwen3RotaryEmbedding, apply_rotary_pos_emb

    cfg = Qwen3Config(head_dim=128, hidden_size=2048, num_attention_heads=16, num_key_value_heads=8,
                      rope_theta=1e6)
    if getattr(cfg, "rope_parameters", None) is not None:
        cfg.rope_parameters["rope_theta"] = 1e6
    inv, _ = Qwen3RotaryEmbedding.compute_default_rope_parameters(cfg)
    assert np.allclose(O.rope_inv_freq(128, 1e6), inv.double().numpy(), rtol=1e-6, atol=0)
    # pairing and sign convention: HF rotates (x1, x2) -> (x1 c - x2 s, x2 c + x1 s)
    rng = np.random.default_rng(5)
    T, H = 6, 4
    y = rng.standard_normal((T, H, 128))
    pos = np.array([0, 1, 7, 100, 2049, 32768])
    ang = pos[:, None].astype(np.float64) * O.rope_inv_freq(128, 1e6)[None, :]
    emb = np.concatenate([ang, ang], axis=-1)
    cos = torch.from_numpy(np.cos(emb))[None]                 # [1, T, D]
    sin = torch.from_numpy(np.sin(emb))[None]
    yt = torch.from_numpy(y).permute(1, 0, 2)[None]           # [1, H, T, D]
    ref, _ = apply_rotary_pos_emb(yt, yt, cos, sin, unsqueeze_dim=1)
    ref = ref[0].permute(1, 0, 2).numpy()
    assert np.allclose(O.rope_neox(y, pos, 1e6), ref, rtol=0, atol=1e-12)


# ---------------------------------------------------------------- a3 slots
def _walk_slots(block_tables, lens, bs):
    """(seq, pos) -> (block, offset) by walking each table row slot by slot."""
    m = {}
    for s, n in enumerate(lens):
        p = 0
        for blk in block_tables[s]:
            for off in range(bs):
                if p == n:
                    break
                m[(s, p)] = (int(blk), off)
                p += 1
    return m


@pytest.mark.parametrize("bs", [16, 32, 256])
def test_slot_of_matches_walk(bs):
    rng = np.random.default_rng(6)
    lens = [1, bs - 1, bs, bs + 1, 5 * bs + 3]
    need = [-(-n // bs) for n in lens]
    perm = rng.permutation(sum(need) + 7)
    bt = np.full((len(lens), max(need)), -1, dtype=np.int64)
    c = 0
    for i, k in enumerate(need):
        bt[i, :k] = perm[c:c + k]
        c += k
    walk = _walk_slots(bt, lens, bs)
    seqs = np.array([s for s, _ in walk])
    poss = np.array([p for _, p in walk])
    blk, off = O.slot_of(poss, seqs, bt, bs)
    assert [(int(b), int(o)) for b, o in zip(blk, off)] == [walk[k] for k in walk]


def test_fused_write_touches_exactly_the_token_slots():
    rng = np.random.default_rng(7)
    nb, bs, hkv, hq, D = 12, 16, 2, 4, 128
    sentinel = np.uint16(0x7FC1)
    pk = np.full((nb, bs, hkv, D), sentinel, dtype=np.uint16)
    pv = pk.copy()
    bt = rng.permutation(nb)[:10].reshape(2, 5)
    pos = np.array([0, 15, 16, 47, 3, 79], dtype=np.int64)
    seq = np.array([0, 0, 0, 0, 1, 1], dtype=np.int64)
    T = len(pos)
    bits = lambda *s: O.f64_to_bf16_bits(rng.standard_normal(s))
    q, k, v = bits(T, hq, D), bits(T, hkv, D), bits(T, hkv, D)
    wq, wk = bits(D), bits(D)
    O.fused_norm_rope_write(q, k, v, wq, wk, pos, seq, bt, 1e-6, 1e6, pk, pv)
    changed = {tuple(i) for i in np.argwhere(np.any(pk != sentinel, axis=(2, 3)))}
    walk = _walk_slots(bt, [80, 80], bs)
    expect = {walk[(int(s), int(p))] for s, p in zip(seq, pos)}
    assert changed == expect
    for t in range(T):
        b, o = walk[(int(seq[t]), int(pos[t]))]
        assert np.array_equal(pv[b, o], v[t])
    assert np.all((pv != sentinel).any(axis=(2, 3)) == (pk != sentinel).any(axis=(2, 3)))


# ---------------------------------------------------------------- a4-a6 attention
def _pool_from_dense(Kd, Vd, bs, rng, extra_blocks=3):
    """Scatter dense per-sequence K/V [S][n, Hkv, D] into a shuffled paged pool."""
    hkv, D = Kd[0].shape[1], Kd[0].shape[2]
    need = [-(-k.shape[0] // bs) for k in Kd]
    nb = sum(need) + extra_blocks
    perm = rng.permutation(nb)
    pk = np.zeros((nb, bs, hkv, D), dtype=np.uint16)
    pv = np.zeros_like(pk)
    bt = np.full((len(Kd), max(need)), -1, dtype=np.int64)
    c = 0
    for s, (k, v) in enumerate(zip(Kd, Vd)):
        bt[s, :need[s]] = perm[c:c + need[s]]
        c += need[s]
        for j in range(k.shape[0]):
            pk[bt[s, j // bs], j % bs] = O.f64_to_bf16_bits(k[j])
            pv[bt[s, j // bs], j % bs] = O.f64_to_bf16_bits(v[j])
    return pk, pv, bt


def _bf(x):
    return O.bf16_round(x)


def test_single_key_returns_v():
    rng = np.random.default_rng(8)
    hq, hkv, D, bs = 4, 2, 128, 16
    Kd = [_bf(rng.standard_normal((1, hkv, D)))]
    Vd = [_bf(rng.standard_normal((1, hkv, D)))]
    pk, pv, bt = _pool_from_dense(Kd, Vd, bs, rng)
    q = rng.standard_normal((1, hq, D)) * 10
    o = O.decode_attention(q, pk, pv, bt, [1], 1 / math.sqrt(D))
    for h in range(hq):
        assert np.array_equal(o[0, h], Vd[0][0, h // 2])


def test_identical_keys_give_mean_of_v():
    rng = np.random.default_rng(9)
    hq, hkv, D, bs, n = 4, 2, 128, 16, 37
    k1 = _bf(rng.standard_normal((1, hkv, D)))
    Kd = [np.repeat(k1, n, axis=0)]
    Vd = [_bf(rng.standard_normal((n, hkv, D)))]
    pk, pv, bt = _pool_from_dense(Kd, Vd, bs, rng)
    q = rng.standard_normal((1, hq, D))
    o = O.decode_attention(q, pk, pv, bt, [n], 1 / math.sqrt(D))
    for h in range(hq):
        assert np.allclose(o[0, h], Vd[0][:, h // 2].mean(axis=0), rtol=1e-13, atol=1e-14)


def test_two_key_softmax_closed_form():
    D = 128
    scale = 1 / math.sqrt(D)
    q = np.zeros(D)
    q[5] = 1.0
    K = np.zeros((2, D))
    K[1, 5] = math.log(3) / scale          # scores (0, ln 3)
    V = np.array([[1.0] * D, [5.0] * D])
    w = _golden()["attention"][0]["weights"]
    assert np.allclose(O.attend(q, K, V, scale), w[0] * V[0] + w[1] * V[1], rtol=1e-14)


def _sdpa(q, K, V, mask):
    """torch fp64 scaled_dot_product_attention with GQA; q [Hq,Lq,D], K/V [Hkv,Lk,D]."""
    return torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q)[None], torch.from_numpy(K)[None], torch.from_numpy(V)[None],
        attn_mask=None if mask is None else torch.from_numpy(mask), enable_gqa=True)[0].numpy()


@pytest.mark.parametrize("hq,hkv", [(16, 8), (32, 4), (4, 4)])
def test_decode_matches_sdpa_brute_force(hq, hkv):
    rng = np.random.default_rng(10 + hq)
    D, bs = 128, 16
    lens = [1, 15, 16, 17, 50]
    Kd = [_bf(rng.standard_normal((n, hkv, D))) for n in lens]
    Vd = [_bf(rng.standard_normal((n, hkv, D))) for n in lens]
    pk, pv, bt = _pool_from_dense(Kd, Vd, bs, rng)
    q = rng.standard_normal((len(lens), hq, D))
    o = O.decode_attention(q, pk, pv, bt, lens, 1 / math.sqrt(D))
    for b, n in enumerate(lens):
        ref = _sdpa(q[b][:, None, :], Kd[b].transpose(1, 0, 2), Vd[b].transpose(1, 0, 2), None)[:, 0]
        assert np.allclose(o[b], ref, rtol=1e-12, atol=1e-12)


def test_chunk_matches_sdpa_with_explicit_bottom_right_mask():
    rng = np.random.default_rng(11)
    hq, hkv, D, bs = 8, 2, 128, 16
    segs = [(0, 7), (20, 5), (33, 1), (3, 40)]          # (cached prefix, q_len)
    lens = [L + ql for L, ql in segs]
    Kd = [_bf(rng.standard_normal((n, hkv, D))) for n in lens]
    Vd = [_bf(rng.standard_normal((n, hkv, D))) for n in lens]
    pk, pv, bt = _pool_from_dense(Kd, Vd, bs, rng)
    qsl = np.concatenate([[0], np.cumsum([ql for _, ql in segs])])
    q = rng.standard_normal((qsl[-1], hq, D))
    o = O.chunk_attention(q, qsl, pk, pv, bt, lens, 1 / math.sqrt(D))
    for s, (L, ql) in enumerate(segs):
        n = L + ql
        # query i may see key j iff j <= L + i  (mask built from the tril of an n x n matrix)
        mask = np.tril(np.ones((n, n), dtype=bool))[L:]
        ref = _sdpa(q[qsl[s]:qsl[s + 1]].transpose(1, 0, 2), Kd[s].transpose(1, 0, 2),
                    Vd[s].transpose(1, 0, 2), mask)
        assert np.allclose(o[qsl[s]:qsl[s + 1]], ref.transpose(1, 0, 2), rtol=1e-12, atol=1e-12)


def test_chunk_without_prefix_is_textbook_causal():
    rng = np.random.default_rng(12)
    hq, hkv, D, bs, n = 4, 2, 128, 16, 45
    Kd = [_bf(rng.standard_normal((n, hkv, D)))]
    Vd = [_bf(rng.standard_normal((n, hkv, D)))]
    pk, pv, bt = _pool_from_dense(Kd, Vd, bs, rng)
    q = rng.standard_normal((n, hq, D))
    o = O.chunk_attention(q, [0, n], pk, pv, bt, [n], 1 / math.sqrt(D))
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q.transpose(1, 0, 2))[None], torch.from_numpy(Kd[0].transpose(1, 0, 2))[None],
        torch.from_numpy(Vd[0].transpose(1, 0, 2))[None], is_causal=True, enable_gqa=True)[0].numpy()
    assert np.allclose(o, ref.transpose(1, 0, 2), rtol=1e-12, atol=1e-12)


def test_chunk_query_equals_decode_at_its_position():
    """Query i of a chunk is a decode query whose context ends at its own position."""
    rng = np.random.default_rng(13)
    hq, hkv, D, bs, L, ql = 4, 2, 128, 16, 29, 6
    n = L + ql
    Kd = [_bf(rng.standard_normal((n, hkv, D)))]
    Vd = [_bf(rng.standard_normal((n, hkv, D)))]
    pk, pv, bt = _pool_from_dense(Kd, Vd, bs, rng)
    q = rng.standard_normal((ql, hq, D))
    o = O.chunk_attention(q, [0, ql], pk, pv, bt, [n], 1 / math.sqrt(D))
    for i in range(ql):
        d = O.decode_attention(q[i:i + 1], pk, pv, bt[:1], [L + i + 1], 1 / math.sqrt(D))
        assert np.array_equal(o[i], d[0])


def test_chunk_ignores_future_keys():
    rng = np.random.default_rng(14)
    hq, hkv, D, bs, L, ql = 2, 1, 128, 16, 10, 4
    n = L + ql
    Kd = [_bf(rng.standard_normal((n, hkv, D)))]
    Vd = [_bf(rng.standard_normal((n, hkv, D)))]
    q = rng.standard_normal((ql, hq, D))
    pk, pv, bt = _pool_from_dense(Kd, Vd, bs, np.random.default_rng(0))
    o = O.chunk_attention(q, [0, ql], pk, pv, bt, [n], 1 / math.sqrt(D))
    # make the key right after query 0 huge and aligned with q: query 0 must not change
    K2 = [Kd[0].copy()]
    K2[0][L + 1] = _bf(q[0, 0] * 50)[None]
    V2 = [Vd[0].copy()]
    V2[0][L + 1] = 100.0
    pk2, pv2, bt2 = _pool_from_dense(K2, V2, bs, np.random.default_rng(0))
    o2 = O.chunk_attention(q, [0, ql], pk2, pv2, bt2, [n], 1 / math.sqrt(D))
    assert np.array_equal(o[0], o2[0])
    assert not np.allclose(o[1], o2[1])


def test_split_combine_equals_unsplit():
    rng = np.random.default_rng(15)
    n, D = 300, 128
    K = rng.standard_normal((n, D))
    V = rng.standard_normal((n, D))
    q = rng.standard_normal(D) * 2
    ref = O.attend(q, K, V, 1 / math.sqrt(D))
    for bounds in ([0, n], [0, 1, n], [0, 100, 100, 200, n], [0, 0, 0, n, n], [0, 17, 64, 65, 299, n]):
        got = O.split_attention(q, K, V, 1 / math.sqrt(D), bounds)
        assert np.allclose(got, ref, rtol=1e-12, atol=1e-13), bounds
    for _ in range(20):
        cuts = np.sort(rng.integers(0, n + 1, size=rng.integers(1, 12)))
        bounds = np.concatenate([[0], cuts, [n]])
        assert np.allclose(O.split_attention(q, K, V, 1 / math.sqrt(D), bounds), ref, rtol=1e-12, atol=1e-13)


def test_outputs_invariant_under_block_permutation():
    rng = np.random.default_rng(16)
    hq, hkv, D, bs = 4, 2, 128, 16
    lens = [70, 33]
    Kd = [_bf(rng.standard_normal((n, hkv, D))) for n in lens]
    Vd = [_bf(rng.standard_normal((n, hkv, D))) for n in lens]
    pk, pv, bt = _pool_from_dense(Kd, Vd, bs, np.random.default_rng(1))
    pk2, pv2, bt2 = _pool_from_dense(Kd, Vd, bs, np.random.default_rng(2))
    assert not np.array_equal(bt, bt2)
    q = rng.standard_normal((2, hq, D))
    a = O.decode_attention(q, pk, pv, bt, lens, 1 / math.sqrt(D))
    b = O.decode_attention(q, pk2, pv2, bt2, lens, 1 / math.sqrt(D))
    assert np.array_equal(a, b)


def test_empty_context_gives_zero_row():
    pk = np.zeros((2, 16, 1, 128), dtype=np.uint16)
    o = O.decode_attention(np.ones((1, 2, 128)), pk, pk, np.array([[0]]), [0], 0.1)
    assert np.all(o == 0)


# ---------------------------------------------------------------- a1+a2+a3 composed
def _fused_case_rows(case, key):
    D = case["head_dim"]
    row = np.zeros(D)
    for i, v in case[key].items():
        row[int(i)] = v
    return row


def test_fused_write_closed_forms():
    """Norm before rotary, each row with its own weight: hand-derived values."""
    for case in _golden()["fused_write"]:
        D = case["head_dim"]
        x = _fused_case_rows(case, "x_nonzero")
        wq = np.ones(D)
        wk = np.ones(D)
        for i, v in case["w_nonzero"].items():
            wq[int(i)] = v
        for i, v in case["k_w_nonzero"].items():
            wk[int(i)] = v
        bits = O.f64_to_bf16_bits
        assert np.array_equal(O.bf16_bits_to_f64(bits(x)), x)      # exactly representable
        pk = np.zeros((2, 16, 1, D), dtype=np.uint16)
        pv = pk.copy()
        q_out, k_out = O.fused_norm_rope_write(
            bits(x)[None, None], bits(x)[None, None], bits(x)[None, None], bits(wq), bits(wk),
            np.array([case["position"]]), np.array([0]), np.array([[1]]), case["eps"], case["theta"],
            pk, pv)
        for name, got in (("q_out_nonzero", q_out[0, 0]), ("k_out_nonzero", k_out[0, 0])):
            want = _fused_case_rows(case, name)
            # dims outside pair 0 stay exactly 0; pair 0 matches the closed form
            assert np.allclose(got, want, rtol=1e-14, atol=1e-14), name
        assert np.array_equal(pk[1, 1, 0], bits(k_out[0, 0]))


def _qwen3_attention(hq, hkv, D, wq, wk):
    """A Qwen3 attention layer whose projections select slices of the hidden row.

    hidden = [q | k | v] (hq*D + 2*hkv*D values), so the layer's q, k and v are
    exactly the given rows, and o_proj returns the attention output unchanged in
    the first hq*D dims.  Everything else is the model's own code path: its
    q_norm/k_norm modules, then its rotary helper, then its cache update and
    eager attention.
    """
    from transformers import Qwen3Config
    from transformers.models.qwen3.modeling_qwen3 import Qwen3Attention

    hidden = hq * D + 2 * hkv * D
    cfg = Qwen3Config(hidden_size=hidden, num_attention_heads=hq, num_key_value_heads=hkv,
                      head_dim=D, rms_norm_eps=1e-6, attention_bias=False, attention_dropout=0.0)
    cfg._attn_implementation = "eager"
    layer = Qwen3Attention(cfg, layer_idx=0).double().eval()
    eye = torch.eye(hidden, dtype=torch.float64)
    with torch.no_grad():
        layer.q_proj.weight.copy_(eye[: hq * D])
        layer.k_proj.weight.copy_(eye[hq * D: (hq + hkv) * D])
        layer.v_proj.weight.copy_(eye[(hq + hkv) * D:])
        layer.o_proj.weight.copy_(eye[:, : hq * D])
        layer.q_norm.weight.copy_(torch.from_numpy(wq))
        layer.k_norm.weight.copy_(torch.from_numpy(wk))
    return layer


@pytest.mark.parametrize("hq,hkv,start", [(16, 8, 0), (32, 4, 1500)])
def test_fused_write_matches_qwen3_attention_layer(hq, hkv, start):
    """q_out/k_out and the attention built on them against the model's own layer.

    The layer's cache holds its k after norm and rotary; its output depends on
    q after norm and rotary.  Different q and k weights catch a swapped weight;
    weights far from 1 in both halves of each rotary pair catch a weight
    applied after the rotation.
    """
    from transformers.cache_utils import DynamicCache

    rng = np.random.default_rng(17 + hq)
    D, T, eps, theta = 128, 12, 1e-6, 1e6
    bits = O.f64_to_bf16_bits
    q = bits(rng.standard_normal((T, hq, D)))
    k = bits(rng.standard_normal((T, hkv, D)))
    v = bits(rng.standard_normal((T, hkv, D)))
    wq = bits(1 + 0.3 * rng.standard_normal(D))
    wk = bits(1 + 0.3 * rng.standard_normal(D))
    pos = np.arange(start, start + T)
    # the oracle: one fused write of the T tokens into a small shuffled pool
    bs = 16
    nb = -(-(start + T) // bs) + 2
    bt = rng.permutation(nb)[None, : -(-(start + T) // bs)]
    pk = np.zeros((nb, bs, hkv, D), dtype=np.uint16)
    pv = pk.copy()
    q_out, k_out = O.fused_norm_rope_write(q, k, v, wq, wk, pos, np.zeros(T, dtype=np.int64), bt,
                                           eps, theta, pk, pv)
    # the model: fp64 rotary tables from fp64 angles (the frequency itself is
    # pinned against the model's in test_rope_matches_qwen3_rotary)
    f64 = O.bf16_bits_to_f64
    layer = _qwen3_attention(hq, hkv, D, f64(wq), f64(wk))
    ang = pos[:, None].astype(np.float64) * O.rope_inv_freq(D, theta)[None, :]
    emb = np.concatenate([ang, ang], axis=-1)
    cos, sin = torch.from_numpy(np.cos(emb))[None], torch.from_numpy(np.sin(emb))[None]
    x = np.concatenate([f64(q).reshape(T, -1), f64(k).reshape(T, -1), f64(v).reshape(T, -1)], axis=1)
    mask = torch.full((T, T), -math.inf, dtype=torch.float64).triu(1)[None, None]
    cache = DynamicCache()
    with torch.no_grad():
        out, _ = layer(torch.from_numpy(x)[None], (cos, sin), mask, past_key_values=cache)
    model_k = cache.layers[0].keys[0].permute(1, 0, 2).numpy()        # [T, hkv, D]
    # Qwen3RMSNorm normalises in fp32, hence the 1e-5 bound
    assert np.allclose(k_out, model_k, rtol=0, atol=2e-5)
    # the attention of every token over the tokens up to itself, from the oracle's
    # unrounded q_out / k_out (the model's cache keeps k unrounded too)
    r = hq // hkv
    ref = np.zeros((T, hq, D))
    for t in range(T):
        for h in range(hq):
            ref[t, h] = O.attend(q_out[t, h], k_out[: t + 1, h // r], f64(v)[: t + 1, h // r],
                                 1 / math.sqrt(D))
    got = out[0, :, : hq * D].reshape(T, hq, D).numpy()
    assert np.allclose(got, ref, rtol=0, atol=2e-5)
    # and q_out itself from the model's q_norm module and rotary helper
    from transformers.models.qwen3.modeling_qwen3 import apply_rotary_pos_emb
    with torch.no_grad():
        qn = layer.q_norm(torch.from_numpy(f64(q))).permute(1, 0, 2)[None]
        qr, _ = apply_rotary_pos_emb(qn, qn, cos, sin, unsqueeze_dim=1)
    assert np.allclose(q_out, qr[0].permute(1, 0, 2).numpy(), rtol=0, atol=2e-5)

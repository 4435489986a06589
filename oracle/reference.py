"""fp64 reference definition of the paged GQA attention hot path.

TEST INFRASTRUCTURE ONLY: used by ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py``; never by the product path.

Sources (web pages, cited by title and section):
  [P1] "perf: Qwen3 offline inference — hybrid attention backend, fused
       rms_norm_rope, chunked prefill + prompt-lookup spec decoding"
       (InfiniLM pull request 585).
  [P2] "Ascend qwen3.6 optimizate baseline" (vllm-plugin-FL pull request 301).
  [P3] "[2026春季][T2-1-3]" (InfiniLM issue 498).

What the pages fix and what is a reading of them:
  * [P1] Summary item 2: q and k get a per-head RMSNorm followed by rotary
    embedding, fused, and the model is full-rotary.  The norm formula, the
    weight semantics (plain ``* w``), eps inside the square root and the
    neox pairing (i, i + D/2) with inverse frequency theta**(-2i/D) are the
    standard Qwen3 definitions; the pages do not print them (plain reading).
  * [P1] Summary item 1: keys and values live in a block-table addressed
    paged cache; pure decode runs a split-KV kernel over it, prefill and mixed
    batches run a varlen kernel over the same cache.  Attention itself is the
    textbook softmax(scale * q k^T) v with scale = 1/sqrt(D) (plain reading);
    query head h reads kv head floor(h / r), r = Hq / Hkv (contiguous groups).
  * [P1] Summary item 4: chunked-prefill slices and fixed b x (k+1) verify
    shapes are causal query chunks over that cache; a chunk of q_len tokens whose
    segment holds n keys (itself included) is bottom-right aligned: its i-th
    query sits at position n - q_len + i and sees keys 0 .. that position.
  * The split-KV form (per-split max, sum and unnormalised accumulator, then
    a log-sum-exp combine) is an exact rearrangement of the softmax; it is
    kept here only so that the combine can be checked against the unsplit form.

Conventions of this module:
  * All arithmetic is float64.  bf16 tensors are carried as uint16 bit patterns
    (the storage format) and widened exactly with ``bf16_bits_to_f64``.
  * The oracle's own cache model is the logical layout
    ``K[num_blocks][block_size][Hkv][D]`` (the "BSHD" cache of [P1] Summary
    item 1), independent of whatever physical layout the GPU library uses.
  * A sequence with zero visible keys yields a zero output row (the softmax over
    an empty set is undefined; zero is the convention taken here, and the library
    does the same).
"""
from __future__ import annotations

import numpy as np

__all__ = [
    "bf16_round",
    "bf16_bits_to_f64",
    "f64_to_bf16_bits",
    "rms_norm",
    "rope_inv_freq",
    "rope_neox",
    "slot_of",
    "fused_norm_rope_write",
    "gather_kv",
    "attend",
    "decode_attention",
    "chunk_attention",
    "split_partials",
    "combine_partials",
    "split_attention",
]


# --------------------------------------------------------------------------
# bf16 storage format
# --------------------------------------------------------------------------
_BF16_MAX = float.fromhex("0x1.fe00000000000p+127")  # (2 - 2**-7) * 2**127
_BF16_MIN_NORMAL = 2.0 ** -126
_BF16_SUBNORMAL_QUANTUM = 2.0 ** -133


def bf16_round(x) -> np.ndarray:
    """Round float64 values to the nearest bf16 value, ties to even.

    bf16 keeps 8 significant bits (1 implicit + 7 stored) and fp32's exponent
    range.  A normal x = m * 2**e with m in [0.5, 1) is rounded on the grid
    2**(e-8); below the smallest normal the grid is the subnormal quantum
    2**-133.  Results beyond the largest finite bf16 become +-inf.  ``np.rint``
    rounds half to even, which is the IEEE default rounding.
    """
    x = np.asarray(x, dtype=np.float64)
    out = np.array(x, copy=True)
    finite = np.isfinite(x)
    ax = np.abs(x)
    normal = finite & (ax >= _BF16_MIN_NORMAL)
    m, e = np.frexp(x[normal])
    out[normal] = np.ldexp(np.rint(m * 256.0), e - 8)
    sub = finite & (ax < _BF16_MIN_NORMAL)
    out[sub] = np.rint(x[sub] / _BF16_SUBNORMAL_QUANTUM) * _BF16_SUBNORMAL_QUANTUM
    over = finite & (np.abs(out) > _BF16_MAX)
    out[over] = np.copysign(np.inf, x[over])
    return out


def bf16_bits_to_f64(bits) -> np.ndarray:
    """Widen bf16 bit patterns (uint16) to float64, exactly.

    A bf16 value is the upper half of an IEEE fp32 word, so placing the 16 bits
    in the high half of a uint32 and reading it as fp32 gives the value.
    """
    b = np.asarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def f64_to_bf16_bits(x) -> np.ndarray:
    """Encode float64 values as bf16 bit patterns (rounding ties to even)."""
    r = bf16_round(x).astype(np.float32)  # exact: every bf16 value is an fp32 value
    return (r.view(np.uint32) >> 16).astype(np.uint16)


# --------------------------------------------------------------------------
# a1: per-head RMSNorm   ([P1] Summary item 2; Platform status: CPU impl exists)
# --------------------------------------------------------------------------
def rms_norm(x: np.ndarray, w: np.ndarray, eps: float) -> np.ndarray:
    """y = x / sqrt(mean_d x_d**2 + eps) * w over the last (head_dim) axis.

    ``w`` has shape [D] and is shared by every head of the tensor.
    """
    x = np.asarray(x, dtype=np.float64)
    ms = np.mean(x * x, axis=-1, keepdims=True)
    return x / np.sqrt(ms + eps) * np.asarray(w, dtype=np.float64)


# --------------------------------------------------------------------------
# a2: neox rotary embedding, full rotary   ([P1] Summary item 2)
# --------------------------------------------------------------------------
def rope_inv_freq(head_dim: int, theta: float) -> np.ndarray:
    """f_i = theta ** (-2 i / D) for i in [0, D/2)."""
    i = np.arange(head_dim // 2, dtype=np.float64)
    return np.power(float(theta), -2.0 * i / head_dim)


def rope_neox(y: np.ndarray, positions: np.ndarray, theta: float) -> np.ndarray:
    """Rotate each pair (i, i + D/2) of y[t, h, :] by the angle p_t * f_i.

    y' _i       = y_i cos a - y_{i+D/2} sin a
    y' _{i+D/2} = y_{i+D/2} cos a + y_i sin a
    """
    y = np.asarray(y, dtype=np.float64)
    d = y.shape[-1]
    half = d // 2
    ang = np.asarray(positions, dtype=np.float64)[:, None] * rope_inv_freq(d, theta)[None, :]
    c = np.cos(ang)[:, None, :]
    s = np.sin(ang)[:, None, :]
    lo, hi = y[..., :half], y[..., half:]
    return np.concatenate([lo * c - hi * s, hi * c + lo * s], axis=-1)


# --------------------------------------------------------------------------
# a3: paged cache slot of a token   ([P1] Summary item 1; [P3] Summary,
#     PagedKVCacheConfig(num_blocks, block_size, max_batch_size))
# --------------------------------------------------------------------------
def slot_of(positions, seq_ids, block_tables, block_size: int):
    """(physical block, offset in block) of each token: the logical block
    floor(p / bs) of the token's sequence is looked up in its block-table row."""
    p = np.asarray(positions, dtype=np.int64)
    s = np.asarray(seq_ids, dtype=np.int64)
    bt = np.asarray(block_tables, dtype=np.int64)
    return bt[s, p // block_size], p % block_size


def fused_norm_rope_write(q_bits, k_bits, v_bits, wq_bits, wk_bits, positions, seq_ids,
                          block_tables, eps, theta, pool_k, pool_v):
    """One call of the fused op: RMSNorm then RoPE on q and k, cache write.

    Inputs are bf16 bit arrays q [T,Hq,D], k/v [T,Hkv,D], weights [D]; the
    cache model ``pool_k``/``pool_v`` is uint16 [num_blocks, bs, Hkv, D] and is
    updated in place with the bf16 (ties-to-even) rounding of k' and v, because
    the cache stores bf16.

    Returns (q_out, k_out) as *unrounded* float64 [T,Hq,D] and [T,Hkv,D], so a
    bf16 result can be compared with the exact value.
    """
    q = bf16_bits_to_f64(q_bits)
    k = bf16_bits_to_f64(k_bits)
    wq = bf16_bits_to_f64(wq_bits)
    wk = bf16_bits_to_f64(wk_bits)
    q_out = rope_neox(rms_norm(q, wq, eps), positions, theta)
    k_out = rope_neox(rms_norm(k, wk, eps), positions, theta)
    bs = pool_k.shape[1]
    blk, off = slot_of(positions, seq_ids, block_tables, bs)
    pool_k[blk, off] = f64_to_bf16_bits(k_out)
    pool_v[blk, off] = np.asarray(v_bits, dtype=np.uint16)
    return q_out, k_out


# --------------------------------------------------------------------------
# a4-a6: attention over the paged cache
# --------------------------------------------------------------------------
def gather_kv(pool_k, pool_v, bt_row, n: int, g: int):
    """Keys/values 0..n-1 of one sequence and kv head g, as float64 [n, D].

    Logical key j lives at block bt_row[j // bs], offset j % bs.
    """
    bs = pool_k.shape[1]
    j = np.arange(n)
    blk = np.asarray(bt_row, dtype=np.int64)[j // bs]
    off = j % bs
    return bf16_bits_to_f64(pool_k[blk, off, g]), bf16_bits_to_f64(pool_v[blk, off, g])


def attend(q: np.ndarray, K: np.ndarray, V: np.ndarray, scale: float) -> np.ndarray:
    """Textbook attention of one query vector over n keys: softmax(scale q.K) V."""
    if K.shape[0] == 0:
        return np.zeros(V.shape[1], dtype=np.float64)
    z = scale * (K @ q)
    w = np.exp(z - z.max())
    return (w / w.sum()) @ V


def decode_attention(q, pool_k, pool_v, block_tables, context_lens, scale):
    """Paged GQA decode: one query token per sequence, attending to all of its
    n_b cached keys (the token just written included).

    q: float64 [B, Hq, D]; returns float64 [B, Hq, D].
    """
    q = np.asarray(q, dtype=np.float64)
    B, Hq, D = q.shape
    hkv = pool_k.shape[2]
    r = Hq // hkv
    out = np.zeros((B, Hq, D), dtype=np.float64)
    for b in range(B):
        n = int(context_lens[b])
        for g in range(hkv):
            K, V = gather_kv(pool_k, pool_v, block_tables[b], n, g)
            for h in range(g * r, (g + 1) * r):
                out[b, h] = attend(q[b, h], K, V, scale)
    return out


def chunk_attention(q, query_start_loc, pool_k, pool_v, block_tables, context_lens, scale):
    """Causal query chunks over the paged cache (chunked-prefill slices and
    b x (k+1) verify rows).

    Segment s owns query rows query_start_loc[s] .. query_start_loc[s+1]-1 of
    q [Tq, Hq, D] and n_s = context_lens[s] keys in its block-table row, its own
    tokens included.  Its i-th query is at position p = n_s - q_len_s + i and
    attends to keys 0..p.
    """
    q = np.asarray(q, dtype=np.float64)
    _, Hq, D = q.shape
    hkv = pool_k.shape[2]
    r = Hq // hkv
    out = np.zeros_like(q)
    qsl = np.asarray(query_start_loc, dtype=np.int64)
    for s in range(len(qsl) - 1):
        q0, q1 = int(qsl[s]), int(qsl[s + 1])
        qlen, n = q1 - q0, int(context_lens[s])
        for g in range(hkv):
            K, V = gather_kv(pool_k, pool_v, block_tables[s], n, g)
            for i in range(qlen):
                p = n - qlen + i
                for h in range(g * r, (g + 1) * r):
                    out[q0 + i, h] = attend(q[q0 + i, h], K[: p + 1], V[: p + 1], scale)
    return out


# --------------------------------------------------------------------------
# Split-KV form and log-sum-exp combine ([P1] Summary item 1, "split-KV")
# --------------------------------------------------------------------------
def split_partials(q, K, V, scale, bounds):
    """Partial results of one query over the key ranges [bounds[k], bounds[k+1]).

    For each range: m = max z, l = sum exp(z - m), a = sum exp(z - m) V and
    lse = m + ln l.  An empty range has lse = -inf, l = 0 and a = 0.
    """
    parts = []
    for k in range(len(bounds) - 1):
        lo, hi = int(bounds[k]), int(bounds[k + 1])
        if hi <= lo:
            parts.append((-np.inf, 0.0, np.zeros(V.shape[1]), -np.inf))
            continue
        z = scale * (K[lo:hi] @ q)
        m = z.max()
        e = np.exp(z - m)
        l = e.sum()
        parts.append((m, l, e @ V[lo:hi], m + np.log(l)))
    return parts


def combine_partials(parts):
    """o = sum_k exp(lse_k - lse) a_k / l_k with lse = M + ln sum_k exp(lse_k - M),
    M = max_k lse_k; ranges with lse_k = -inf carry weight 0."""
    lses = np.array([p[3] for p in parts], dtype=np.float64)
    if not np.isfinite(lses).any():
        return np.zeros_like(parts[0][2])
    M = lses.max()
    lse = M + np.log(np.sum(np.exp(lses - M)))
    o = np.zeros_like(parts[0][2])
    for m, l, a, lk in parts:
        if np.isfinite(lk):
            o = o + np.exp(lk - lse) * (a / l)
    return o


def split_attention(q, K, V, scale, bounds):
    """Attention of one query evaluated in split form."""
    return combine_partials(split_partials(q, K, V, scale, bounds))

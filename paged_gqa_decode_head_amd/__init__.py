"""Paged GQA attention hot path for MI355X (gfx950): Python binding of libpgqa.

The C ABI (include/pgqa.h) does the work; this module only marshals torch
tensors (device memory) and the current HIP stream into it.  There is no
fallback: if ``libpgqa.so`` is missing or fails to load, every entry point
raises.  Build it with ``python -m paged_gqa_decode_head_amd.build``.

Entry points (same names as the C ABI, without the ``pgqa_`` prefix):
  Pool(...)                         pgqa_pool_create / pgqa_pool_destroy / pgqa_pool_layout
  rms_norm_rope_cache_write(...)    pgqa_rms_norm_rope_cache_write
  paged_decode_attention(...)       pgqa_paged_decode_attention
  paged_chunk_attention(...)        pgqa_paged_chunk_attention
  plan_decode(...)                  pgqa_plan_decode
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libpgqa.so")

PGQA_OK = 0
PGQA_ERR_INVALID_ARG = 1
STATUS_NAMES = {
    0: "PGQA_OK", 1: "PGQA_ERR_INVALID_ARG", 2: "PGQA_ERR_UNSUPPORTED", 3: "PGQA_ERR_POINTER_KIND",
    4: "PGQA_ERR_WORKSPACE", 5: "PGQA_ERR_HIP", 6: "PGQA_ERR_DEVICE",
}
DEVERR_SEQ_ID, DEVERR_POSITION, DEVERR_BLOCK_ID, DEVERR_CONTEXT, DEVERR_QUERY = 0x1, 0x2, 0x4, 0x8, 0x10


class PgqaError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{STATUS_NAMES.get(status, status)}: {message}")
        self.status = status


class PoolConfig(ctypes.Structure):
    _fields_ = [("num_blocks", ctypes.c_int32), ("block_size", ctypes.c_int32),
                ("num_kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("max_batch_size", ctypes.c_int32)]


class DecodePlan(ctypes.Structure):
    _fields_ = [("split_tokens", ctypes.c_int32), ("max_splits", ctypes.c_int32),
                ("waves_per_split", ctypes.c_int32), ("load_hint", ctypes.c_int32), ("kernel", ctypes.c_int32),
                ("host_context_lens", ctypes.c_void_p)]

    def set_host_context_lens(self, lens):
        """Attach a host copy of the call's context lengths (kept alive with the
        plan); None detaches it."""
        import numpy as np

        if lens is None:
            self._host_lens = None
            self.host_context_lens = None
            return self
        self._host_lens = np.ascontiguousarray(lens, dtype=np.int32)
        self.host_context_lens = self._host_lens.ctypes.data
        return self

    def __repr__(self):
        return (f"DecodePlan(split_tokens={self.split_tokens}, max_splits={self.max_splits}, "
                f"waves_per_split={self.waves_per_split}, load_hint={self.load_hint}, kernel={self.kernel}, "
                f"host_context_lens={'set' if self.host_context_lens else 'None'})")


class ChunkPlan(ctypes.Structure):
    _fields_ = [("split_tokens", ctypes.c_int32), ("max_splits", ctypes.c_int32),
                ("short_split_tokens", ctypes.c_int32), ("kernel", ctypes.c_int32)]

    def __repr__(self):
        return (f"ChunkPlan(split_tokens={self.split_tokens}, max_splits={self.max_splits}, "
                f"short_split_tokens={self.short_split_tokens})")


class MixedPlan(ctypes.Structure):
    _fields_ = [("split_wide", ctypes.c_int32), ("split_columns", ctypes.c_int32), ("max_splits", ctypes.c_int32),
                ("num_items", ctypes.c_int32), ("num_combine", ctypes.c_int32)]

    def __repr__(self):
        return (f"MixedPlan(split_wide={self.split_wide}, split_columns={self.split_columns}, "
                f"max_splits={self.max_splits}, num_items={self.num_items}, num_combine={self.num_combine})")


MIXED_ITEM_INTS = 8   # PGQA_MIXED_ITEM_INTS


class SchedConfig(ctypes.Structure):
    _fields_ = [("token_budget", ctypes.c_int32), ("max_segments", ctypes.c_int32),
                ("chunked_prefill", ctypes.c_int32), ("block_size", ctypes.c_int32),
                ("max_blocks_per_seq", ctypes.c_int32)]


SEG_DECODE, SEG_VERIFY, SEG_PREFILL = 0, 1, 2

_lib = None

_P, _I32, _I64, _SZ, _F32, _F64 = (ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t,
                                   ctypes.c_float, ctypes.c_double)
_SIGNATURES = {
    "pgqa_version": ([], ctypes.c_char_p),
    "pgqa_stream_read": ([_P, _SZ, _P, _SZ, _I32, _P], ctypes.c_int),
    "pgqa_last_error": ([], ctypes.c_char_p),
    "pgqa_status_string": ([ctypes.c_int], ctypes.c_char_p),
    "pgqa_pool_bytes": ([ctypes.POINTER(PoolConfig)], _SZ),
    "pgqa_pool_create": ([ctypes.POINTER(PoolConfig), _P, ctypes.POINTER(_P)], ctypes.c_int),
    "pgqa_pool_destroy": ([_P], ctypes.c_int),
    "pgqa_pool_layout": ([_P, ctypes.POINTER(_I64), ctypes.POINTER(_I64), ctypes.POINTER(_I64),
                          ctypes.POINTER(_I64)], ctypes.c_int),
    "pgqa_pool_check_errors": ([_P, _P, ctypes.POINTER(ctypes.c_uint32)], ctypes.c_int),
    "pgqa_rms_norm_rope_cache_write": ([_P, _P, _I64, _P, _I64, _P, _I64, _P, _P, _P, _P, _P, _I32, _I32,
                                        _I32, _I32, _F32, _F64, _P, _P], ctypes.c_int),
    "pgqa_plan_decode": ([_I32, _I32, _I32, _I32, _I32, _I32, ctypes.POINTER(DecodePlan)], ctypes.c_int),
    "pgqa_decode_workspace_bytes": ([_P, _I32, _I32, _I32, ctypes.POINTER(DecodePlan)], _SZ),
    "pgqa_paged_decode_attention": ([_P, _P, _P, _P, _I32, _I32, _I32, _I32, _F32, ctypes.POINTER(DecodePlan),
                                     _P, _SZ, _P, _P], ctypes.c_int),
    "pgqa_decode_step": ([_P, _P, _I64, _P, _I64, _P, _I64, _P, _P, _F32, _F64, _P, _P, _I32, _I32, _I32, _I32,
                          _F32, ctypes.POINTER(DecodePlan), _P, _SZ, _P, _P, _P], ctypes.c_int),
    "pgqa_decode_step_noalloc": ([_P, _P, _I64, _P, _I64, _P, _I64, _P, _P, _F32, _F64, _P, _P, _I32, _I32, _I32,
                                  _I32, _F32, ctypes.POINTER(DecodePlan), _P, _P, _P], ctypes.c_int),
    "pgqa_plan_chunk": ([_I32, _I32, _I32, _I32, _I32, _I32, _I32, _I32, ctypes.POINTER(ChunkPlan)],
                        ctypes.c_int),
    "pgqa_chunk_workspace_bytes": ([_P, _I32, _I32, _I32, _I32, _I32, ctypes.POINTER(ChunkPlan)], _SZ),
    "pgqa_paged_chunk_attention": ([_P, _P, _P, _P, _P, _I32, _I32, _I32, _I32, _I32, _I32, _F32,
                                    ctypes.POINTER(ChunkPlan), _P, _SZ, _P, _P], ctypes.c_int),
    "pgqa_plan_mixed": ([_I32, _I32, _I32, _I32, _I32, _P, _P, _I32, _I32, _P, _I64, ctypes.POINTER(MixedPlan)],
                        ctypes.c_int),
    "pgqa_mixed_workspace_bytes": ([ctypes.POINTER(MixedPlan), _I32, _I32], _SZ),
    "pgqa_paged_mixed_attention": ([_P, _P, _P, _P, _P, _I32, _I32, _I32, _I32, _I32, _I32, _F32,
                                    ctypes.POINTER(MixedPlan), _P, _P, _SZ, _P, _P], ctypes.c_int),
    # host producers (include/pgqa_sched.h)
    "pgqa_prompt_lookup": ([_P, _I32, _I32, _I32, _I32, _P], _I32),
    "pgqa_accept_greedy": ([_P, _I32, _P, _P], _I32),
    "pgqa_sched_plan_step": ([ctypes.POINTER(SchedConfig), _P, _I32, _P, _P, ctypes.POINTER(_I32), _P, _P, _P, _P,
                              _P, _I32, ctypes.POINTER(_I32), ctypes.POINTER(_I32)], ctypes.c_int),
    "pgqa_sched_commit": ([_P, _I32, _P, _I32, _P], ctypes.c_int),
    "pgqa_sched_release": ([ctypes.POINTER(SchedConfig), _P, _I32, _I32, _P, _P, ctypes.POINTER(_I32), _I32],
                           ctypes.c_int),
}


def lib() -> ctypes.CDLL:
    """The loaded libpgqa (raises if it is not built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it with `python -m paged_gqa_decode_head_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        for name, (args, res) in _SIGNATURES.items():
            fn = getattr(L, name)
            fn.argtypes = args
            fn.restype = res
        _lib = L
    return _lib


def exported_symbols():
    return list(_SIGNATURES)


def _check(status: int):
    if status != PGQA_OK:
        raise PgqaError(status, lib().pgqa_last_error().decode())


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    import torch

    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _require(t, name, dtype=None, device=None, contiguous=True):
    import torch

    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, the pool on {device}")
    if contiguous and not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _shape(t, name, *dims):
    """t has shape dims (None = any extent); ValueError otherwise."""
    if t.dim() != len(dims) or any(d is not None and t.shape[i] != d for i, d in enumerate(dims)):
        want = "[" + ", ".join("*" if d is None else str(d) for d in dims) + "]"
        raise ValueError(f"{name} has shape {list(t.shape)}, expected {want}")


def _check_decode_inputs(pool, q, context_lens, block_tables, out, fused=None):
    """Shapes and dtypes of a decode call (or, with fused = (k, v, wq, wk, q_out),
    a fused decode step) before anything reaches the library."""
    import torch

    _require(context_lens, "context_lens", torch.int32, pool.device)
    _require(block_tables, "block_tables", torch.int32, pool.device)
    B, hq = q.shape[0], q.shape[1]
    if q.dim() != 3 or q.shape[2] != 128:
        raise ValueError(f"q has shape {list(q.shape)}, expected [batch, num_q_heads, 128]")
    _shape(context_lens, "context_lens", B)
    if block_tables.dim() != 2 or block_tables.shape[0] < B or block_tables.shape[1] < 1:
        raise ValueError(f"block_tables has shape {list(block_tables.shape)}, expected [>= {B}, >= 1]")
    if out is not None:
        _require(out, "out", torch.bfloat16, pool.device)
        _shape(out, "out", B, hq, 128)
    if fused is not None:
        k, v, wq, wk, q_out = fused
        hkv = pool.num_kv_heads
        for name, t in (("k", k), ("v", v)):
            if t.shape[0] < B or (t.dim() == 3 and tuple(t.shape[1:]) != (hkv, 128)) or \
                    (t.dim() == 2 and t.shape[1] < hkv * 128) or t.dim() not in (2, 3):
                raise ValueError(f"{name} has shape {list(t.shape)}, expected [{B}, {hkv}, 128] rows")
        for name, t in (("q_norm_weight", wq), ("k_norm_weight", wk)):
            _require(t, name, torch.bfloat16, pool.device)
            _shape(t, name, 128)
        if q_out is not None:
            _require(q_out, "q_out", torch.bfloat16, pool.device)
            _shape(q_out, "q_out", B, hq, 128)


def _check_write_inputs(pool, q, k, v, q_norm_weight, k_norm_weight, positions, seq_ids, block_tables, q_out):
    import torch

    for name, t in (("q", q), ("k", k), ("v", v)):
        _require(t, name, torch.bfloat16, pool.device, contiguous=False)
        if t.dim() != 3 or t.shape[2] != 128 or t.stride(2) != 1 or t.stride(1) != 128:
            raise ValueError(f"{name} must be [T, heads, 128] with dense heads and dims")
    T = q.shape[0]
    for name, t in (("k", k), ("v", v)):
        _shape(t, name, T, pool.num_kv_heads, 128)
    for name, t in (("q_norm_weight", q_norm_weight), ("k_norm_weight", k_norm_weight)):
        _require(t, name, torch.bfloat16, pool.device)
        _shape(t, name, 128)
    for name, t in (("positions", positions), ("seq_ids", seq_ids), ("block_tables", block_tables)):
        _require(t, name, torch.int32, pool.device)
    _shape(positions, "positions", T)
    _shape(seq_ids, "seq_ids", T)
    if block_tables.dim() != 2 or block_tables.shape[0] < 1 or block_tables.shape[1] < 1:
        raise ValueError(f"block_tables has shape {list(block_tables.shape)}, expected [num_seqs, width]")
    _require(q_out, "q_out", torch.bfloat16, pool.device)
    _shape(q_out, "q_out", T, q.shape[1], 128)


def _check_chunk_inputs(pool, q, query_start_loc, context_lens, block_tables, out):
    import torch

    for name, t in (("query_start_loc", query_start_loc), ("context_lens", context_lens),
                    ("block_tables", block_tables)):
        _require(t, name, torch.int32, pool.device)
    if q.dim() != 3 or q.shape[2] != 128:
        raise ValueError(f"q has shape {list(q.shape)}, expected [total_q, num_q_heads, 128]")
    N = context_lens.shape[0] if context_lens.dim() == 1 else -1
    if N < 0:
        raise ValueError(f"context_lens has shape {list(context_lens.shape)}, expected [num_segments]")
    _shape(query_start_loc, "query_start_loc", N + 1)
    if block_tables.dim() != 2 or block_tables.shape[0] < N or block_tables.shape[1] < 1:
        raise ValueError(f"block_tables has shape {list(block_tables.shape)}, expected [>= {N}, >= 1]")
    if out is not None:
        _require(out, "out", torch.bfloat16, pool.device)
        _shape(out, "out", q.shape[0], q.shape[1], 128)


def version() -> str:
    return lib().pgqa_version().decode()


def pool_bytes(num_blocks, block_size, num_kv_heads, head_dim=128, max_batch_size=0) -> int:
    cfg = PoolConfig(num_blocks, block_size, num_kv_heads, head_dim, max_batch_size)
    return int(lib().pgqa_pool_bytes(ctypes.byref(cfg)))


class Pool:
    """A paged K/V pool: torch owns the storage, libpgqa owns its layout."""

    def __init__(self, num_blocks: int, block_size: int, num_kv_heads: int, head_dim: int = 128,
                 max_batch_size: int = 0, device=None):
        import torch

        self.config = PoolConfig(num_blocks, block_size, num_kv_heads, head_dim, max_batch_size)
        nbytes = int(lib().pgqa_pool_bytes(ctypes.byref(self.config)))
        if nbytes == 0:
            _check(lib().pgqa_pool_create(ctypes.byref(self.config), None, ctypes.byref(_P())))
        dev = torch.device("cuda") if device is None else torch.device(device)
        if dev.index is None:
            dev = torch.device(dev.type, torch.cuda.current_device())
        self.device = dev
        with torch.cuda.device(self.device):
            self.storage = torch.empty(nbytes // 2, dtype=torch.bfloat16, device=self.device)
            h = _P()
            _check(lib().pgqa_pool_create(ctypes.byref(self.config), _ptr(self.storage), ctypes.byref(h)))
        self.handle = h
        self.num_blocks, self.block_size, self.num_kv_heads = num_blocks, block_size, num_kv_heads
        self.head_dim = head_dim
        ks, vs = (_I64 * 4)(), (_I64 * 5)()
        ko, vo = _I64(), _I64()
        _check(lib().pgqa_pool_layout(self.handle, ks, ctypes.byref(ko), vs, ctypes.byref(vo)))
        self.k_strides, self.k_offset = tuple(ks), ko.value
        self.v_strides, self.v_offset = tuple(vs), vo.value
        self._ws = {}

    def k_view(self):
        """K cache as a strided bf16 view [num_blocks, block_size, num_kv_heads, head_dim]."""
        shape = (self.num_blocks, self.block_size, self.num_kv_heads, self.head_dim)
        return self.storage.as_strided(shape, self.k_strides, self.k_offset)

    def v_view(self):
        """V cache as a strided bf16 view [num_blocks, block_size / 16, 16, num_kv_heads, head_dim]
        (the slot index split as slot = 16 * piece + j; reshape a copy to get [.., block_size, ..])."""
        shape = (self.num_blocks, self.block_size // 16, 16, self.num_kv_heads, self.head_dim)
        return self.storage.as_strided(shape, self.v_strides, self.v_offset)

    def fill_logical(self, k, v, blocks=None):
        """Copy logical [n, block_size, Hkv, 128] K/V (bf16, or int16/uint16 bit
        patterns) into the cache: all blocks, or the listed physical ``blocks``."""
        import torch

        def as_bf16(x):
            x = torch.as_tensor(x)
            if x.dtype in (torch.int16, torch.uint16):
                x = x.view(torch.int16).view(torch.bfloat16)
            return x.to(self.device)

        kv, vv = self.k_view(), self.v_view()
        pieces = lambda x: x.reshape(x.shape[0], self.block_size // 16, 16, *x.shape[2:])
        if blocks is None:
            kv.copy_(as_bf16(k))
            vv.copy_(pieces(as_bf16(v)))
        else:
            idx = torch.as_tensor(blocks, dtype=torch.long, device=self.device)
            kv[idx] = as_bf16(k)
            vv[idx] = pieces(as_bf16(v))

    def read_logical(self, blocks=None):
        """(K, V) as CPU int16 bit patterns [n, block_size, Hkv, 128] in logical order."""
        import torch

        kv, vv = self.k_view(), self.v_view()
        if blocks is not None:
            idx = torch.as_tensor(blocks, dtype=torch.long, device=self.device)
            kv, vv = kv[idx], vv[idx]
        vv = vv.contiguous().reshape(vv.shape[0], self.block_size, *vv.shape[3:])
        return (kv.contiguous().view(torch.int16).cpu(), vv.view(torch.int16).cpu())

    def check_errors(self, stream=None) -> int:
        """Synchronise the stream and return (and clear) the device error bits."""
        flags = ctypes.c_uint32(0)
        st = lib().pgqa_pool_check_errors(self.handle, _stream(stream), ctypes.byref(flags))
        if st not in (PGQA_OK, 6):
            _check(st)
        return int(flags.value)

    def workspace(self, nbytes: int, key: str):
        """A zero-filled device workspace of at least nbytes, cached per purpose."""
        import torch

        ws = self._ws.get(key)
        if ws is None or ws.numel() < nbytes:
            ws = torch.zeros(max(nbytes, 256), dtype=torch.uint8, device=self.device)
            self._ws[key] = ws
        return ws

    def close(self):
        if getattr(self, "handle", None):
            _check(lib().pgqa_pool_destroy(self.handle))
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def rms_norm_rope_cache_write(pool: Pool, q, k, v, q_norm_weight, k_norm_weight, positions, seq_ids,
                              block_tables, eps: float, rope_theta: float, q_out=None, stream=None):
    """Fused per-head RMSNorm + neox RoPE of q/k and paged K/V write; returns q_out.

    q [T, Hq, 128], k/v [T, Hkv, 128] bf16 (token rows may be strided: the
    head and dim axes must be dense), weights [128] bf16, positions/seq_ids [T]
    int32, block_tables [num_seqs, width] int32.
    """
    import torch

    T, hq = q.shape[0], q.shape[1]
    if q_out is None:
        q_out = torch.empty((T, hq, 128), dtype=torch.bfloat16, device=pool.device)
    _check_write_inputs(pool, q, k, v, q_norm_weight, k_norm_weight, positions, seq_ids, block_tables, q_out)
    _check(lib().pgqa_rms_norm_rope_cache_write(
        pool.handle, _ptr(q), q.stride(0), _ptr(k), k.stride(0), _ptr(v), v.stride(0),
        _ptr(q_norm_weight), _ptr(k_norm_weight), _ptr(positions), _ptr(seq_ids), _ptr(block_tables),
        block_tables.shape[1], block_tables.shape[0], T, hq, float(eps), float(rope_theta), _ptr(q_out),
        _stream(stream)))
    return q_out


def plan_decode(num_cus, block_size, batch, num_kv_heads, num_q_heads, max_context_len) -> DecodePlan:
    p = DecodePlan()
    _check(lib().pgqa_plan_decode(num_cus, block_size, batch, num_kv_heads, num_q_heads, max_context_len,
                                  ctypes.byref(p)))
    return p


def decode_workspace_bytes(pool: Pool, batch, num_q_heads, max_context_len, plan: DecodePlan = None) -> int:
    return int(lib().pgqa_decode_workspace_bytes(pool.handle, batch, num_q_heads, max_context_len,
                                                 None if plan is None else ctypes.byref(plan)))


def paged_decode_attention(pool: Pool, q, context_lens, block_tables, max_context_len: int, scale: float,
                           plan: DecodePlan = None, workspace=None, out=None, stream=None):
    """Paged split-KV GQA decode attention; returns out [B, Hq, 128] bf16.

    ``max_context_len`` is a host-side upper bound of ``context_lens`` (no
    device read).  ``workspace`` (uint8, zero-filled once) defaults to a
    per-pool cached buffer.
    """
    import torch

    _require(q, "q", torch.bfloat16, pool.device)
    _check_decode_inputs(pool, q, context_lens, block_tables, out)
    B, hq = q.shape[0], q.shape[1]
    if out is None:
        out = torch.empty((B, hq, 128), dtype=torch.bfloat16, device=pool.device)
    pp = None if plan is None else ctypes.byref(plan)
    need = int(lib().pgqa_decode_workspace_bytes(pool.handle, B, hq, max_context_len, pp))
    if workspace is None:
        workspace = pool.workspace(need, "decode")
    _check(lib().pgqa_paged_decode_attention(
        pool.handle, _ptr(q), _ptr(context_lens), _ptr(block_tables), block_tables.shape[1], B, hq,
        int(max_context_len), float(scale), pp, _ptr(workspace), workspace.numel() * workspace.element_size(),
        _ptr(out), _stream(stream)))
    return out


def decode_step(pool: Pool, q, k, v, q_norm_weight, k_norm_weight, context_lens, block_tables, max_context_len: int,
                eps: float, rope_theta: float, scale: float, plan: DecodePlan = None, workspace=None, out=None,
                q_out=None, stream=None):
    """Fused decode step: norm + rotary of each sequence's new token (at position
    context_lens[b] - 1), its cache write, and decode attention; returns out
    [B, Hq, 128] bf16.  q/k/v: [B, H, 128] bf16 (or row-strided 2-D views)."""
    import torch

    for name, t in (("q", q), ("k", k), ("v", v)):
        _require(t, name, torch.bfloat16, pool.device, contiguous=False)
        if t.stride(-1) != 1 or (t.dim() == 3 and t.stride(1) != 128):
            raise ValueError(f"{name}: heads must be contiguous 128-element rows")
    _check_decode_inputs(pool, q, context_lens, block_tables, out, (k, v, q_norm_weight, k_norm_weight, q_out))
    B, hq = q.shape[0], q.shape[1]
    if out is None:
        out = torch.empty((B, hq, 128), dtype=torch.bfloat16, device=pool.device)
    pp = None if plan is None else ctypes.byref(plan)
    need = int(lib().pgqa_decode_workspace_bytes(pool.handle, B, hq, max_context_len, pp))
    if workspace is None:
        workspace = pool.workspace(need, "decode")
    _check(lib().pgqa_decode_step(
        pool.handle, _ptr(q), q.stride(0), _ptr(k), k.stride(0), _ptr(v), v.stride(0), _ptr(q_norm_weight),
        _ptr(k_norm_weight), float(eps), float(rope_theta), _ptr(context_lens), _ptr(block_tables),
        block_tables.shape[1], B, hq, int(max_context_len), float(scale), pp, _ptr(workspace),
        workspace.numel() * workspace.element_size(), None if q_out is None else _ptr(q_out), _ptr(out),
        _stream(stream)))
    return out


NOALLOC_SCRATCH_BYTES = 8 << 20   # PGQA_NOALLOC_SCRATCH_BYTES


def decode_step_noalloc(pool: Pool, q, k, v, q_norm_weight, k_norm_weight, context_lens, block_tables,
                        max_context_len: int, eps: float, rope_theta: float, scale: float, out,
                        plan: DecodePlan = None, q_out=None, stream=None):
    """pgqa_decode_step_noalloc: the fused decode step with its split partials in
    the library's fixed per-GPU scratch; ``out`` (and ``q_out``) are the caller's,
    nothing is allocated.  Calls that overlap on one GPU race on the scratch."""
    import torch

    for name, t in (("q", q), ("k", k), ("v", v)):
        _require(t, name, torch.bfloat16, pool.device, contiguous=False)
        if t.stride(-1) != 1 or (t.dim() == 3 and t.stride(1) != 128):
            raise ValueError(f"{name}: heads must be contiguous 128-element rows")
    _check_decode_inputs(pool, q, context_lens, block_tables, out, (k, v, q_norm_weight, k_norm_weight, q_out))
    pp = None if plan is None else ctypes.byref(plan)
    _check(lib().pgqa_decode_step_noalloc(
        pool.handle, _ptr(q), q.stride(0), _ptr(k), k.stride(0), _ptr(v), v.stride(0), _ptr(q_norm_weight),
        _ptr(k_norm_weight), float(eps), float(rope_theta), _ptr(context_lens), _ptr(block_tables),
        block_tables.shape[1], q.shape[0], q.shape[1], int(max_context_len), float(scale), pp,
        None if q_out is None else _ptr(q_out), _ptr(out), _stream(stream)))
    return out


def plan_chunk(num_cus, block_size, num_segments, total_q, num_kv_heads, num_q_heads, max_q_len,
               max_context_len) -> ChunkPlan:
    p = ChunkPlan()
    _check(lib().pgqa_plan_chunk(num_cus, block_size, num_segments, total_q, num_kv_heads, num_q_heads,
                                 max_q_len, max_context_len, ctypes.byref(p)))
    return p


def chunk_workspace_bytes(pool: Pool, num_segments, total_q, num_q_heads, max_q_len, max_context_len,
                          plan: ChunkPlan = None) -> int:
    return int(lib().pgqa_chunk_workspace_bytes(pool.handle, num_segments, total_q, num_q_heads, max_q_len,
                                                max_context_len, None if plan is None else ctypes.byref(plan)))


def paged_chunk_attention(pool: Pool, q, query_start_loc, context_lens, block_tables, max_q_len: int,
                          max_context_len: int, scale: float, plan: ChunkPlan = None, workspace=None, out=None,
                          stream=None):
    """Causal chunk attention over the paged cache; returns out [total_q, Hq, 128] bf16.

    Segment s owns query rows query_start_loc[s] .. query_start_loc[s+1]-1 and
    context_lens[s] keys (its own tokens included, already in the cache).
    """
    import torch

    _require(q, "q", torch.bfloat16, pool.device)
    _check_chunk_inputs(pool, q, query_start_loc, context_lens, block_tables, out)
    Tq, hq = q.shape[0], q.shape[1]
    N = context_lens.shape[0]
    if out is None:
        out = torch.empty((Tq, hq, 128), dtype=torch.bfloat16, device=pool.device)
    pp = None if plan is None else ctypes.byref(plan)
    need = int(lib().pgqa_chunk_workspace_bytes(pool.handle, N, Tq, hq, int(max_q_len), int(max_context_len), pp))
    if workspace is None:
        workspace = pool.workspace(need, "chunk")
    _check(lib().pgqa_paged_chunk_attention(
        pool.handle, _ptr(q), _ptr(query_start_loc), _ptr(context_lens), _ptr(block_tables), block_tables.shape[1],
        N, Tq, hq, int(max_q_len), int(max_context_len), float(scale), pp, _ptr(workspace),
        workspace.numel() * workspace.element_size(), _ptr(out), _stream(stream)))
    return out

def plan_mixed(num_cus, block_size, num_kv_heads, num_q_heads, query_start_loc, context_lens, split_wide=0,
               split_columns=0):
    """pgqa_plan_mixed on host copies of the step's metadata: (MixedPlan, int32
    numpy array [num_items + num_combine, MIXED_ITEM_INTS])."""
    import numpy as np

    qsl = np.ascontiguousarray(query_start_loc, dtype=np.int32)
    ctx = np.ascontiguousarray(context_lens, dtype=np.int32)
    if qsl.ndim != 1 or ctx.ndim != 1 or qsl.size != ctx.size + 1:
        raise ValueError("query_start_loc must hold len(context_lens) + 1 entries")
    plan = MixedPlan()
    _check(lib().pgqa_plan_mixed(num_cus, block_size, num_kv_heads, num_q_heads, ctx.size, _np_ptr(qsl),
                                 _np_ptr(ctx), split_wide, split_columns, None, 0, ctypes.byref(plan)))
    items = np.zeros((plan.num_items + plan.num_combine, MIXED_ITEM_INTS), dtype=np.int32)
    if items.size:
        _check(lib().pgqa_plan_mixed(num_cus, block_size, num_kv_heads, num_q_heads, ctx.size, _np_ptr(qsl),
                                     _np_ptr(ctx), split_wide, split_columns, _np_ptr(items), items.shape[0],
                                     ctypes.byref(plan)))
    return plan, items


def mixed_workspace_bytes(plan: MixedPlan, total_q: int, num_q_heads: int) -> int:
    return int(lib().pgqa_mixed_workspace_bytes(ctypes.byref(plan), total_q, num_q_heads))


def _mixed_args(pool, q, query_start_loc, context_lens, block_tables, max_q_len, max_context_len, scale, plan,
                items, workspace, out, stream):
    import torch

    _require(q, "q", torch.bfloat16, pool.device)
    _check_chunk_inputs(pool, q, query_start_loc, context_lens, block_tables, out)
    _require(items, "items", torch.int32, pool.device)
    if items.dim() != 2 or items.shape[1] != MIXED_ITEM_INTS or items.shape[0] < plan.num_items + plan.num_combine:
        raise ValueError(f"items has shape {list(items.shape)}, the plan needs "
                         f"[{plan.num_items + plan.num_combine}, {MIXED_ITEM_INTS}]")
    Tq, hq = q.shape[0], q.shape[1]
    need = mixed_workspace_bytes(plan, Tq, hq)
    if workspace is None:
        workspace = pool.workspace(need, "mixed")
    args = (pool.handle, _ptr(q), _ptr(query_start_loc), _ptr(context_lens), _ptr(block_tables),
            block_tables.shape[1], context_lens.shape[0], Tq, hq, int(max_q_len), int(max_context_len), float(scale),
            ctypes.byref(plan), _ptr(items), _ptr(workspace), workspace.numel() * workspace.element_size(), _ptr(out),
            _stream(stream))
    return args, workspace


def paged_mixed_attention(pool: Pool, q, query_start_loc, context_lens, block_tables, max_q_len: int,
                          max_context_len: int, scale: float, plan: MixedPlan, items, workspace=None, out=None,
                          stream=None):
    """One attention launch (plus one combine) for a mixed step from the work
    list of plan_mixed (``items``: its device copy, int32 [n, 8]); returns out
    [total_q, Hq, 128] bf16.  Same semantics as paged_chunk_attention."""
    import torch

    if out is None:
        out = torch.empty((q.shape[0], q.shape[1], 128), dtype=torch.bfloat16, device=pool.device)
    args, _ = _mixed_args(pool, q, query_start_loc, context_lens, block_tables, max_q_len, max_context_len, scale,
                          plan, items, workspace, out, stream)
    _check(lib().pgqa_paged_mixed_attention(*args))
    return out


def bind_mixed(pool: Pool, q, query_start_loc, context_lens, block_tables, max_q_len: int, max_context_len: int,
               scale: float, out, plan: MixedPlan, items, workspace=None, stream=None) -> "BoundCall":
    args, workspace = _mixed_args(pool, q, query_start_loc, context_lens, block_tables, max_q_len, max_context_len,
                                  scale, plan, items, workspace, out, stream)
    keep = (q, query_start_loc, context_lens, block_tables, out, items, workspace, plan)
    return BoundCall(lib().pgqa_paged_mixed_attention, args, keep)


def bind_stream_read(src, sink, grid: int = 0, stream=None) -> "BoundCall":
    """pgqa_stream_read over all of ``src`` (a device tensor of a multiple of 16
    bytes); ``sink`` must hold grid * 256 uint32 words (grid 0: three per CU)."""
    nbytes = src.numel() * src.element_size()
    keep = (src, sink)
    args = (_ptr(src), nbytes, _ptr(sink), sink.numel() * sink.element_size(), int(grid), _stream(stream))
    return BoundCall(lib().pgqa_stream_read, args, keep)


class BoundCall:
    """A C-ABI call with its arguments marshalled once; calling it re-issues the
    same launch (same tensors, same stream) without per-call Python work."""

    def __init__(self, fn, args, keep):
        self._fn, self._args, self._keep = fn, args, keep

    def __call__(self):
        st = self._fn(*self._args)
        if st != PGQA_OK:
            _check(st)


def bind_cache_write(pool: Pool, q, k, v, q_norm_weight, k_norm_weight, positions, seq_ids, block_tables,
                     eps: float, rope_theta: float, q_out, stream=None) -> BoundCall:
    _check_write_inputs(pool, q, k, v, q_norm_weight, k_norm_weight, positions, seq_ids, block_tables, q_out)
    keep = (q, k, v, q_norm_weight, k_norm_weight, positions, seq_ids, block_tables, q_out)
    args = (pool.handle, _ptr(q), q.stride(0), _ptr(k), k.stride(0), _ptr(v), v.stride(0), _ptr(q_norm_weight),
            _ptr(k_norm_weight), _ptr(positions), _ptr(seq_ids), _ptr(block_tables), block_tables.shape[1],
            block_tables.shape[0], q.shape[0], q.shape[1], float(eps), float(rope_theta), _ptr(q_out),
            _stream(stream))
    return BoundCall(lib().pgqa_rms_norm_rope_cache_write, args, keep)


def bind_decode(pool: Pool, q, context_lens, block_tables, max_context_len: int, scale: float, out,
                plan: DecodePlan = None, workspace=None, stream=None) -> BoundCall:
    import torch

    _require(q, "q", torch.bfloat16, pool.device)
    _check_decode_inputs(pool, q, context_lens, block_tables, out)
    B, hq = q.shape[0], q.shape[1]
    pp = None if plan is None else ctypes.byref(plan)
    need = int(lib().pgqa_decode_workspace_bytes(pool.handle, B, hq, max_context_len, pp))
    if workspace is None:
        workspace = pool.workspace(need, "decode")
    keep = (q, context_lens, block_tables, out, workspace, plan)
    args = (pool.handle, _ptr(q), _ptr(context_lens), _ptr(block_tables), block_tables.shape[1], B, hq,
            int(max_context_len), float(scale), pp, _ptr(workspace), workspace.numel() * workspace.element_size(),
            _ptr(out), _stream(stream))
    return BoundCall(lib().pgqa_paged_decode_attention, args, keep)


def bind_decode_step(pool: Pool, q, k, v, q_norm_weight, k_norm_weight, context_lens, block_tables,
                     max_context_len: int, eps: float, rope_theta: float, scale: float, out, plan: DecodePlan = None,
                     workspace=None, q_out=None, stream=None) -> BoundCall:
    import torch

    for name, t in (("q", q), ("k", k), ("v", v)):
        _require(t, name, torch.bfloat16, pool.device, contiguous=False)
        if t.stride(-1) != 1 or (t.dim() == 3 and t.stride(1) != 128):
            raise ValueError(f"{name}: heads must be contiguous 128-element rows")
    _check_decode_inputs(pool, q, context_lens, block_tables, out, (k, v, q_norm_weight, k_norm_weight, q_out))
    B, hq = q.shape[0], q.shape[1]
    pp = None if plan is None else ctypes.byref(plan)
    need = int(lib().pgqa_decode_workspace_bytes(pool.handle, B, hq, max_context_len, pp))
    if workspace is None:
        workspace = pool.workspace(need, "decode")
    keep = (q, k, v, q_norm_weight, k_norm_weight, context_lens, block_tables, out, workspace, plan, q_out)
    args = (pool.handle, _ptr(q), q.stride(0), _ptr(k), k.stride(0), _ptr(v), v.stride(0), _ptr(q_norm_weight),
            _ptr(k_norm_weight), float(eps), float(rope_theta), _ptr(context_lens), _ptr(block_tables),
            block_tables.shape[1], B, hq, int(max_context_len), float(scale), pp, _ptr(workspace),
            workspace.numel() * workspace.element_size(), None if q_out is None else _ptr(q_out), _ptr(out),
            _stream(stream))
    return BoundCall(lib().pgqa_decode_step, args, keep)


def bind_chunk(pool: Pool, q, query_start_loc, context_lens, block_tables, max_q_len: int, max_context_len: int,
               scale: float, out, plan: ChunkPlan = None, workspace=None, stream=None) -> BoundCall:
    import torch

    _require(q, "q", torch.bfloat16, pool.device)
    _check_chunk_inputs(pool, q, query_start_loc, context_lens, block_tables, out)
    Tq, hq = q.shape[0], q.shape[1]
    N = context_lens.shape[0]
    pp = None if plan is None else ctypes.byref(plan)
    need = int(lib().pgqa_chunk_workspace_bytes(pool.handle, N, Tq, hq, int(max_q_len), int(max_context_len), pp))
    if workspace is None:
        workspace = pool.workspace(need, "chunk")
    keep = (q, query_start_loc, context_lens, block_tables, out, workspace, plan)
    args = (pool.handle, _ptr(q), _ptr(query_start_loc), _ptr(context_lens), _ptr(block_tables),
            block_tables.shape[1], N, Tq, hq, int(max_q_len), int(max_context_len), float(scale), pp,
            _ptr(workspace), workspace.numel() * workspace.element_size(), _ptr(out), _stream(stream))
    return BoundCall(lib().pgqa_paged_chunk_attention, args, keep)


# ---------------------------------------------------------------- host producers
def _np_ptr(a):
    return ctypes.c_void_p(a.ctypes.data) if a is not None and a.size else None


def _i32_array(x, name):
    import numpy as np

    a = np.ascontiguousarray(x, dtype=np.int32)
    if a.ndim != 1:
        raise ValueError(f"{name} must be 1-D")
    return a


def prompt_lookup(tokens, min_ngram: int, max_ngram: int, k: int):
    """Draft of up to k tokens for a token history (pgqa_prompt_lookup); int32 array."""
    import numpy as np

    t = _i32_array(tokens, "tokens")
    draft = np.zeros(max(k, 1), dtype=np.int32)
    n = lib().pgqa_prompt_lookup(_np_ptr(t), t.size, min_ngram, max_ngram, k, _np_ptr(draft))
    if n < 0:
        raise PgqaError(PGQA_ERR_INVALID_ARG, lib().pgqa_last_error().decode())
    return draft[:n]


def accept_greedy(draft, target):
    """Accepted draft prefix plus the target's next token (pgqa_accept_greedy); int32 array."""
    import numpy as np

    d, t = _i32_array(draft, "draft"), _i32_array(target, "target")
    if t.size != d.size + 1:
        raise ValueError("target needs len(draft) + 1 tokens")
    out = np.zeros(d.size + 1, dtype=np.int32)
    n = lib().pgqa_accept_greedy(_np_ptr(d), d.size, _np_ptr(t), _np_ptr(out))
    if n < 0:
        raise PgqaError(PGQA_ERR_INVALID_ARG, lib().pgqa_last_error().decode())
    return out[:n]


class StepPlanner:
    """Chunked-prefill step planner over host state (pgqa_sched_*).

    seqs: int32 [N, 4] rows (cached, prompt_left, num_draft, num_blocks);
    block_tables: int32 [N, max_blocks_per_seq]; free_list: int32 stack of free
    block ids (top = last of the first free_count entries)."""

    def __init__(self, token_budget: int, max_segments: int, chunked_prefill: bool, block_size: int,
                 max_blocks_per_seq: int, num_seqs: int, free_blocks):
        import numpy as np

        self.config = SchedConfig(token_budget, max_segments, int(bool(chunked_prefill)), block_size,
                                  max_blocks_per_seq)
        self.seqs = np.zeros((num_seqs, 4), dtype=np.int32)
        self.block_tables = np.full((num_seqs, max_blocks_per_seq), -1, dtype=np.int32)
        fb = np.ascontiguousarray(free_blocks, dtype=np.int32)
        self.free_list = fb.copy()
        self.free_count = ctypes.c_int32(fb.size)

    def plan(self, token_capacity: int):
        """One step: dict of segs [S, 4] (seq, kind, q_len, context_len), query_start_loc [S+1],
        context_lens [S], token_pos [T], token_seq [T]."""
        import numpy as np

        ms = self.config.max_segments
        segs = np.zeros((ms, 4), dtype=np.int32)
        qsl = np.zeros(ms + 1, dtype=np.int32)
        ctx = np.zeros(ms, dtype=np.int32)
        pos = np.zeros(max(token_capacity, 1), dtype=np.int32)
        sq = np.zeros(max(token_capacity, 1), dtype=np.int32)
        nseg, ntok = ctypes.c_int32(0), ctypes.c_int32(0)
        _check(lib().pgqa_sched_plan_step(ctypes.byref(self.config), _np_ptr(self.seqs), self.seqs.shape[0],
                                          _np_ptr(self.block_tables), _np_ptr(self.free_list),
                                          ctypes.byref(self.free_count), _np_ptr(segs), _np_ptr(qsl), _np_ptr(ctx),
                                          _np_ptr(pos), _np_ptr(sq), token_capacity, ctypes.byref(nseg),
                                          ctypes.byref(ntok)))
        S, T = nseg.value, ntok.value
        return {"segs": segs[:S].copy(), "query_start_loc": qsl[:S + 1].copy(), "context_lens": ctx[:S].copy(),
                "token_pos": pos[:T].copy(), "token_seq": sq[:T].copy()}

    def commit(self, segs, accepted=None):
        import numpy as np

        segs = np.ascontiguousarray(segs, dtype=np.int32)
        acc = None if accepted is None else np.ascontiguousarray(accepted, dtype=np.int32)
        _check(lib().pgqa_sched_commit(_np_ptr(self.seqs), self.seqs.shape[0], _np_ptr(segs), segs.shape[0],
                                       _np_ptr(acc)))

    def release(self, seq: int):
        _check(lib().pgqa_sched_release(ctypes.byref(self.config), _np_ptr(self.seqs), self.seqs.shape[0], seq,
                                        _np_ptr(self.block_tables), _np_ptr(self.free_list),
                                        ctypes.byref(self.free_count), self.free_list.size))


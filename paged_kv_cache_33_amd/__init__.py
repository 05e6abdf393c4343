"""Paged KV-cache decode attention for AMD MI355X (gfx950).

A thin Python binding over libpagedkv's C ABI (include/pagedkv.h), with the
same names.  It only marshals arguments: it checks that each torch tensor is a
contiguous device buffer of the size the C call documents, then passes raw
pointers and the stream.  Every step of the computation runs in the HIP
kernels; if the library is missing, every call raises.

PyTorch is used for device memory and streams only.
"""
from __future__ import annotations

import ctypes as C
from typing import Optional, Union

import torch

import numpy as np

from . import _lib
from ._lib import KVPoolDesc, NoBlocks, PagedKVError  # noqa: F401

__all__ = [
    "KVPool",
    "PagedKVError",
    "kv_pool_bytes",
    "kv_pool_create",
    "kv_slot_mapping",
    "reshape_and_cache",
    "kv_cache_append",
    "kv_cache_append_chunk",
    "paged_attention_workspace_bytes",
    "paged_attention_decode",
    "kv_decode_step",
    "paged_attention_reduce",
    "paged_attention_decode_noalloc",
    "paged_attention_multi",
    "kv_decode_kernel_kind",
    "kv_copy_blocks",
    "kv_read_tiles",
    "BlockManager",
    "NoBlocks",
    "library_path",
]

BLOCK_SIZE = 16


def library_path() -> str:
    return _lib.LIB_PATH


def _dtype_code(dtype) -> int:
    if dtype in ("bf16", torch.bfloat16, _lib.KV_BF16):
        return _lib.KV_BF16
    if dtype in ("f32", torch.float32, _lib.KV_F32):
        return _lib.KV_F32
    if dtype in ("fp8", "fp8_e4m3", torch.float8_e4m3fn, _lib.KV_FP8_E4M3):
        return _lib.KV_FP8_E4M3
    if dtype in ("int8", torch.int8, _lib.KV_INT8):
        return _lib.KV_INT8
    raise ValueError(f"unsupported dtype {dtype!r}")


def _elem_size(code: int) -> int:
    """Bytes of one cache element."""
    return {_lib.KV_BF16: 2, _lib.KV_F32: 4, _lib.KV_FP8_E4M3: 1, _lib.KV_INT8: 1}[code]


def _act_code(code: int) -> int:
    """Element type of query, output and cache-write rows for a cache type."""
    return _lib.KV_BF16 if code in (_lib.KV_FP8_E4M3, _lib.KV_INT8) else code


def _stream_handle(stream) -> int:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, torch.cuda.Stream):
        return stream.cuda_stream
    return int(stream)


def _buf(t: torch.Tensor, name: str, nbytes: Optional[int] = None,
         elem_size: Optional[int] = None, dtype: Optional[torch.dtype] = None) -> int:
    """Pointer of a contiguous device tensor, after checking what the C call reads."""
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must live on the GPU (got {t.device})")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype} (got {t.dtype})")
    if elem_size is not None and t.element_size() != elem_size:
        raise ValueError(f"{name} must have {elem_size}-byte elements (got {t.element_size()})")
    have = t.numel() * t.element_size()
    if nbytes is not None and have != nbytes:
        raise ValueError(f"{name} holds {have} bytes, the call reads/writes {nbytes}")
    return t.data_ptr()


def kv_pool_bytes(num_blocks: int, num_kv_heads: int, head_dim: int, dtype) -> int:
    """Bytes of ONE cache (K or V) of this geometry (0 if unsupported)."""
    desc = KVPoolDesc(num_blocks, BLOCK_SIZE, num_kv_heads, head_dim, _dtype_code(dtype), 1.0, 1.0)
    return int(_lib.load().kv_pool_bytes(C.byref(desc)))


class KVPool:
    """A K cache and a V cache in the documented block layout, owned by torch.

    dtype "fp8" holds E4M3 codes; k_scale / v_scale are its per-tensor scales
    (ignored for bf16 / f32 / int8 pools).  dtype "int8" holds int8 codes and,
    after them in each buffer, one float32 scale per (block, head, slot) row."""

    def __init__(self, k_cache: torch.Tensor, v_cache: torch.Tensor, num_blocks: int,
                 num_kv_heads: int, head_dim: int, dtype, k_scale: float = 1.0,
                 v_scale: float = 1.0):
        lib = _lib.load()
        self.dtype_code = _dtype_code(dtype)
        self.num_blocks = int(num_blocks)
        self.num_kv_heads = int(num_kv_heads)
        self.head_dim = int(head_dim)
        self.k_scale = float(k_scale)
        self.v_scale = float(v_scale)
        self.desc = KVPoolDesc(self.num_blocks, BLOCK_SIZE, self.num_kv_heads, self.head_dim,
                               self.dtype_code, self.k_scale, self.v_scale)
        need = int(lib.kv_pool_bytes(C.byref(self.desc)))
        if need == 0:
            _lib.check(lib.kv_pool_create(C.byref(self.desc), None, None, C.byref(C.c_void_p())))
        kp = _buf(k_cache, "k_cache", need)
        vp = _buf(v_cache, "v_cache", need)
        handle = C.c_void_p()
        _lib.check(lib.kv_pool_create(C.byref(self.desc), kp, vp, C.byref(handle)))
        self.k_cache = k_cache
        self.v_cache = v_cache
        self._handle = handle

    @classmethod
    def allocate(cls, num_blocks: int, num_kv_heads: int, head_dim: int, dtype,
                 device="cuda", k_scale: float = 1.0, v_scale: float = 1.0) -> "KVPool":
        code = _dtype_code(dtype)
        tdt = {_lib.KV_BF16: torch.bfloat16, _lib.KV_F32: torch.float32,
               _lib.KV_FP8_E4M3: torch.uint8, _lib.KV_INT8: torch.uint8}[code]
        # elements, plus an int8 pool's row scales (kv_pool_bytes counts both)
        n = kv_pool_bytes(num_blocks, num_kv_heads, head_dim, dtype) // _elem_size(code)
        k = torch.empty(n, dtype=tdt, device=device)
        v = torch.empty(n, dtype=tdt, device=device)
        return cls(k, v, num_blocks, num_kv_heads, head_dim, dtype, k_scale, v_scale)

    @property
    def handle(self) -> C.c_void_p:
        if self._handle is None:
            raise RuntimeError("pool is closed")
        return self._handle

    @property
    def elem_size(self) -> int:
        """Bytes of one cache element."""
        return _elem_size(self.dtype_code)

    @property
    def act_code(self) -> int:
        return _act_code(self.dtype_code)

    @property
    def act_size(self) -> int:
        """Bytes of one query / output / cache-write row element."""
        return _elem_size(self.act_code)

    def close(self) -> None:
        if getattr(self, "_handle", None) is not None:
            _lib.load().kv_pool_destroy(self._handle)
            self._handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def kv_pool_create(k_cache, v_cache, num_blocks, num_kv_heads, head_dim, dtype,
                   k_scale: float = 1.0, v_scale: float = 1.0) -> KVPool:
    return KVPool(k_cache, v_cache, num_blocks, num_kv_heads, head_dim, dtype, k_scale, v_scale)


def kv_slot_mapping(block_tables: torch.Tensor, context_lens: torch.Tensor,
                    slot_mapping: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """Slot of each sequence's newest token, computed on the GPU (int64 [B])."""
    if block_tables.dim() != 2:
        raise ValueError("block_tables must be [B, max_nb]")
    B, max_nb = block_tables.shape
    tp = _buf(block_tables, "block_tables", dtype=torch.int32)
    cp = _buf(context_lens, "context_lens", 4 * B, dtype=torch.int32)
    if slot_mapping is None:
        slot_mapping = torch.empty(B, dtype=torch.int64, device=block_tables.device)
    sp = _buf(slot_mapping, "slot_mapping", 8 * B, dtype=torch.int64)
    _lib.check(_lib.load().kv_slot_mapping(tp, max_nb, cp, B, sp, _stream_handle(stream)))
    return slot_mapping


def reshape_and_cache(pool: KVPool, key: torch.Tensor, value: torch.Tensor,
                      slot_mapping: torch.Tensor, stream=None) -> None:
    """Write token i's K/V rows ([N, H_kv, d]) into slot slot_mapping[i]."""
    N = int(slot_mapping.numel())
    row = pool.num_kv_heads * pool.head_dim * pool.act_size
    kp = _buf(key, "key", N * row, elem_size=pool.act_size)
    vp = _buf(value, "value", N * row, elem_size=pool.act_size)
    sp = _buf(slot_mapping, "slot_mapping", 8 * N, dtype=torch.int64)
    _lib.check(_lib.load().reshape_and_cache(pool.handle, kp, vp, sp, N, _stream_handle(stream)))


def kv_cache_append(pool: KVPool, key: torch.Tensor, value: torch.Tensor,
                    block_tables: torch.Tensor, context_lens: torch.Tensor,
                    slot_mapping: Optional[torch.Tensor] = None, stream=None) -> None:
    """Append one token per sequence (rows [B, H_kv, d]) at position ctx - 1:
    slot mapping and cache write in one launch; see pagedkv.h."""
    if block_tables.dim() != 2:
        raise ValueError("block_tables must be [B, max_nb]")
    B, max_nb = block_tables.shape
    row = B * pool.num_kv_heads * pool.head_dim * pool.act_size
    kp = _buf(key, "key", row, elem_size=pool.act_size)
    vp = _buf(value, "value", row, elem_size=pool.act_size)
    tp = _buf(block_tables, "block_tables", dtype=torch.int32)
    cp = _buf(context_lens, "context_lens", 4 * B, dtype=torch.int32)
    sp = None if slot_mapping is None else _buf(slot_mapping, "slot_mapping", 8 * B,
                                                dtype=torch.int64)
    _lib.check(_lib.load().kv_cache_append(pool.handle, kp, vp, tp, max_nb, cp, B, sp,
                                           _stream_handle(stream)))


def kv_cache_append_chunk(pool: KVPool, key: torch.Tensor, value: torch.Tensor,
                          query_start: torch.Tensor, max_query_len: int,
                          block_tables: torch.Tensor, context_lens: torch.Tensor,
                          slot_mapping: Optional[torch.Tensor] = None, stream=None) -> None:
    """Append the n_b = query_start[b+1] - query_start[b] newest tokens of each
    sequence (rows [num_rows, H_kv, d]) at positions ctx - n_b .. ctx - 1; see
    pagedkv.h."""
    if block_tables.dim() != 2:
        raise ValueError("block_tables must be [B, max_nb]")
    B, max_nb = block_tables.shape
    if key.dim() != 3:
        raise ValueError("key must be [num_rows, H_kv, head_dim]")
    T = int(key.shape[0])
    row = T * pool.num_kv_heads * pool.head_dim * pool.act_size
    kp = _buf(key, "key", row, elem_size=pool.act_size)
    vp = _buf(value, "value", row, elem_size=pool.act_size)
    qsp = _buf(query_start, "query_start", 4 * (B + 1), dtype=torch.int32)
    tp = _buf(block_tables, "block_tables", dtype=torch.int32)
    cp = _buf(context_lens, "context_lens", 4 * B, dtype=torch.int32)
    sp = None if slot_mapping is None else _buf(slot_mapping, "slot_mapping", 8 * T,
                                                dtype=torch.int64)
    _lib.check(_lib.load().kv_cache_append_chunk(pool.handle, kp, vp, T, qsp, int(max_query_len),
                                                 tp, max_nb, cp, B, sp, _stream_handle(stream)))


def paged_attention_multi(pool: KVPool, out: torch.Tensor, query: torch.Tensor,
                          query_start: torch.Tensor, max_query_len: int,
                          block_tables: torch.Tensor, context_lens: torch.Tensor, scale: float,
                          stream=None, window: int = 0) -> None:
    """Attention of several new query rows per sequence ([num_rows, H, d], bf16),
    causal within each sequence's rows (and within a sliding window of `window`
    positions when > 0); see pagedkv.h."""
    if query.dim() != 3 or query.shape[2] != pool.head_dim:
        raise ValueError("query must be [num_rows, H, head_dim]")
    T, H, d = query.shape
    if block_tables.dim() != 2:
        raise ValueError("block_tables must be [B, max_nb]")
    B, max_nb = block_tables.shape
    qp = _buf(query, "query", T * H * d * 2, elem_size=2)
    op = _buf(out, "out", T * H * d * 2, elem_size=2)
    qsp = _buf(query_start, "query_start", 4 * (B + 1), dtype=torch.int32)
    tp = _buf(block_tables, "block_tables", dtype=torch.int32)
    cp = _buf(context_lens, "context_lens", 4 * B, dtype=torch.int32)
    _lib.check(_lib.load().paged_attention_multi(
        pool.handle, op, qp, T, qsp, int(max_query_len), tp, max_nb, cp, B, H, float(scale),
        int(window), _stream_handle(stream)))


def paged_attention_workspace_bytes(B: int, H: int, head_dim: int, max_context_len: int,
                                    partition_size: int) -> int:
    return int(_lib.load().paged_attention_workspace_bytes(B, H, head_dim, max_context_len,
                                                           partition_size))


def paged_attention_decode(pool: KVPool, out: torch.Tensor, query: torch.Tensor,
                           block_tables: torch.Tensor, context_lens: torch.Tensor,
                           max_context_len: int, scale: float, partition_size: int = 0,
                           workspace: Optional[torch.Tensor] = None, stream=None,
                           window: int = 0) -> None:
    """Decode attention for one new query per sequence; see pagedkv.h.  window
    > 0 calls paged_attention_decode_window (the last `window` tokens only)."""
    if query.dim() != 3 or query.shape[2] != pool.head_dim:
        raise ValueError("query must be [B, H, head_dim]")
    B, H, d = query.shape
    if block_tables.dim() != 2 or block_tables.shape[0] != B:
        raise ValueError("block_tables must be [B, max_nb]")
    max_nb = int(block_tables.shape[1])
    es = pool.act_size
    qp = _buf(query, "query", B * H * d * es, elem_size=es)
    op = _buf(out, "out", B * H * d * es, elem_size=es)
    tp = _buf(block_tables, "block_tables", dtype=torch.int32)
    cp = _buf(context_lens, "context_lens", 4 * B, dtype=torch.int32)
    wp, wbytes = None, 0
    if partition_size:
        if workspace is None:
            raise ValueError("split mode (partition_size > 0) needs a workspace")
        wp = _buf(workspace, "workspace")
        wbytes = workspace.numel() * workspace.element_size()
    lib = _lib.load()
    if window:
        _lib.check(lib.paged_attention_decode_window(
            pool.handle, op, qp, tp, max_nb, cp, B, H, int(max_context_len), float(scale),
            int(window), int(partition_size), wp, wbytes, _stream_handle(stream)))
    else:
        _lib.check(lib.paged_attention_decode(
            pool.handle, op, qp, tp, max_nb, cp, B, H, int(max_context_len), float(scale),
            int(partition_size), wp, wbytes, _stream_handle(stream)))


def kv_decode_step(pool: KVPool, out: torch.Tensor, query: torch.Tensor, key: torch.Tensor,
                   value: torch.Tensor, block_tables: torch.Tensor, context_lens: torch.Tensor,
                   max_context_len: int, scale: float, partition_size: int = 0,
                   workspace: Optional[torch.Tensor] = None,
                   slot_mapping: Optional[torch.Tensor] = None, stream=None,
                   window: int = 0) -> None:
    """One decode step in one launch: the cache write of the newest rows (key,
    value [B, H_kv, d]) and the attention, which takes the newest position from
    those rows; see pagedkv.h."""
    if query.dim() != 3 or query.shape[2] != pool.head_dim:
        raise ValueError("query must be [B, H, head_dim]")
    B, H, d = query.shape
    if block_tables.dim() != 2 or block_tables.shape[0] != B:
        raise ValueError("block_tables must be [B, max_nb]")
    es = pool.act_size
    row = B * pool.num_kv_heads * d * es
    qp = _buf(query, "query", B * H * d * es, elem_size=es)
    op = _buf(out, "out", B * H * d * es, elem_size=es)
    kp = _buf(key, "key", row, elem_size=es)
    vp = _buf(value, "value", row, elem_size=es)
    tp = _buf(block_tables, "block_tables", dtype=torch.int32)
    cp = _buf(context_lens, "context_lens", 4 * B, dtype=torch.int32)
    sp = None if slot_mapping is None else _buf(slot_mapping, "slot_mapping", 8 * B,
                                                dtype=torch.int64)
    wp, wbytes = None, 0
    if partition_size:
        if workspace is None:
            raise ValueError("split mode (partition_size > 0) needs a workspace")
        wp = _buf(workspace, "workspace")
        wbytes = workspace.numel() * workspace.element_size()
    _lib.check(_lib.load().kv_decode_step(
        pool.handle, op, qp, kp, vp, tp, int(block_tables.shape[1]), cp, B, H,
        int(max_context_len), float(scale), int(window), int(partition_size), wp, wbytes, sp,
        _stream_handle(stream)))


def paged_attention_decode_noalloc(pool: KVPool, out: torch.Tensor, query: torch.Tensor,
                                   block_tables: torch.Tensor, context_lens: torch.Tensor,
                                   max_context_len: int, scale: float, partition_size: int = 0,
                                   stream=None) -> None:
    """Split decode and merge with the partials in the library's scratch (no
    workspace, nothing allocated); see pagedkv.h."""
    if query.dim() != 3 or query.shape[2] != pool.head_dim:
        raise ValueError("query must be [B, H, head_dim]")
    B, H, d = query.shape
    if block_tables.dim() != 2 or block_tables.shape[0] != B:
        raise ValueError("block_tables must be [B, max_nb]")
    es = pool.act_size
    qp = _buf(query, "query", B * H * d * es, elem_size=es)
    op = _buf(out, "out", B * H * d * es, elem_size=es)
    tp = _buf(block_tables, "block_tables", dtype=torch.int32)
    cp = _buf(context_lens, "context_lens", 4 * B, dtype=torch.int32)
    _lib.check(_lib.load().paged_attention_decode_noalloc(
        pool.handle, op, qp, tp, int(block_tables.shape[1]), cp, B, H, int(max_context_len),
        float(scale), int(partition_size), _stream_handle(stream)))


def paged_attention_reduce(out: torch.Tensor, workspace: torch.Tensor, context_lens: torch.Tensor,
                           max_context_len: int, partition_size: int, dtype, stream=None,
                           window: int = 0) -> None:
    """Merge the split partials of paged_attention_decode into out [B, H, d];
    dtype is the output's (an fp8 pool's activation type, bf16, is accepted as
    "fp8" too)."""
    if out.dim() != 3:
        raise ValueError("out must be [B, H, head_dim]")
    B, H, d = out.shape
    code = _act_code(_dtype_code(dtype))
    op = _buf(out, "out", B * H * d * _elem_size(code), elem_size=_elem_size(code))
    need = paged_attention_workspace_bytes(B, H, d, max_context_len, partition_size)
    wp = _buf(workspace, "workspace")
    if workspace.numel() * workspace.element_size() < need:
        raise ValueError(f"workspace must hold at least {need} bytes")
    cp = _buf(context_lens, "context_lens", 4 * B, dtype=torch.int32)
    lib = _lib.load()
    if window:
        _lib.check(lib.paged_attention_reduce_window(
            op, wp, cp, B, H, d, int(max_context_len), int(window), int(partition_size), code,
            _stream_handle(stream)))
    else:
        _lib.check(lib.paged_attention_reduce(
            op, wp, cp, B, H, d, int(max_context_len), int(partition_size), code,
            _stream_handle(stream)))


def kv_decode_kernel_kind(pool: KVPool, H: int) -> int:
    """0 = vector-ALU decode kernel, 1 = matrix-core kernel, < 0 unsupported."""
    return int(_lib.load().kv_decode_kernel_kind(pool.handle, H))


def kv_copy_blocks(pool: KVPool, src: torch.Tensor, dst: torch.Tensor, stream=None) -> None:
    """Copy whole blocks src[i] -> dst[i] of both caches on the GPU (device int32 [n])."""
    n = int(src.numel())
    sp = _buf(src, "src", 4 * n, dtype=torch.int32)
    dp = _buf(dst, "dst", 4 * n, dtype=torch.int32)
    _lib.check(_lib.load().kv_copy_blocks(pool.handle, sp, dp, n, _stream_handle(stream)))


def kv_read_tiles(pool: KVPool, tiles: torch.Tensor, sink: torch.Tensor, stream=None) -> None:
    """Read the listed K/V tiles (device int32 tile indices p * H_kv + h) once,
    with no arithmetic: the bandwidth ceiling of that access pattern.  One
    work-group per element of sink (device int32/uint32 [groups]); each stores
    the XOR of the 32-bit words it read."""
    n = int(tiles.numel())
    tp = _buf(tiles, "tiles", 4 * n, dtype=torch.int32)
    groups = int(sink.numel())
    sp = _buf(sink, "sink", 4 * groups, elem_size=4)
    _lib.check(_lib.load().kv_read_tiles(pool.handle, tp, n, sp, groups, _stream_handle(stream)))


class BlockManager:
    """The C ABI's host block manager (kv_bm_*): tables, counts, free queue,
    prefix cache, fork and copy-on-write for a pool of num_blocks blocks."""

    def __init__(self, num_blocks: int):
        lib = _lib.load()
        h = C.c_void_p()
        _lib.check(lib.kv_bm_create(int(num_blocks), C.byref(h)))
        self._h = h
        self.num_blocks = int(num_blocks)

    def close(self) -> None:
        if getattr(self, "_h", None) is not None:
            _lib.load().kv_bm_destroy(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def admit(self, seq: int, prompt, salt: str = "") -> int:
        """Build seq's table for a prompt (token ids); return the tokens found cached."""
        toks = np.ascontiguousarray(np.asarray(prompt, dtype=np.int32))
        sb = salt.encode("utf-8")
        hits = C.c_int32()
        _lib.check(_lib.load().kv_bm_admit(self._h, int(seq), toks.ctypes.data if toks.size else None,
                                           int(toks.size), sb, len(sb), C.byref(hits)))
        return int(hits.value)

    def append(self, seq: int, token: int):
        """Write one token; return (slot, (src, dst) of a copy-on-write or None)."""
        slot, cs, cd = C.c_int64(), C.c_int32(), C.c_int32()
        _lib.check(_lib.load().kv_bm_append(self._h, int(seq), int(token), C.byref(slot),
                                            C.byref(cs), C.byref(cd)))
        return int(slot.value), (None if cs.value < 0 else (int(cs.value), int(cd.value)))

    def append_batch(self, seqs, tokens):
        """Append tokens[b] to seqs[b] in order; return (slots int64 [B], copy
        pairs int32 [n, 2] to make first)."""
        ids = np.ascontiguousarray(np.asarray(seqs, dtype=np.int64))
        toks = np.ascontiguousarray(np.asarray(tokens, dtype=np.int32))
        if ids.shape != toks.shape:
            raise ValueError("one token per sequence")
        B = ids.size
        slots = np.empty(B, dtype=np.int64)
        cs = np.empty(max(B, 1), dtype=np.int32)
        cd = np.empty(max(B, 1), dtype=np.int32)
        n, done = C.c_int32(), C.c_int32()
        _lib.check(_lib.load().kv_bm_append_batch(self._h, ids.ctypes.data, toks.ctypes.data, B,
                                                  slots.ctypes.data, cs.ctypes.data,
                                                  cd.ctypes.data, C.byref(n), C.byref(done)))
        return slots, np.stack([cs[:n.value], cd[:n.value]], axis=1)

    def fork(self, seq: int, child: int) -> None:
        _lib.check(_lib.load().kv_bm_fork(self._h, int(seq), int(child)))

    def release(self, seq: int) -> None:
        _lib.check(_lib.load().kv_bm_release(self._h, int(seq)))

    def num_free(self) -> int:
        return int(_lib.load().kv_bm_num_free(self._h))

    def table(self, seq: int):
        nb, nt = C.c_int32(), C.c_int32()
        lib = _lib.load()
        _lib.check(lib.kv_bm_table(self._h, int(seq), None, 0, C.byref(nb), C.byref(nt)))
        out = np.zeros(max(nb.value, 1), dtype=np.int32)
        _lib.check(lib.kv_bm_table(self._h, int(seq), out.ctypes.data, out.size, C.byref(nb),
                                   C.byref(nt)))
        return out[:nb.value].tolist()

    def num_tokens(self, seq: int) -> int:
        nb, nt = C.c_int32(), C.c_int32()
        _lib.check(_lib.load().kv_bm_table(self._h, int(seq), None, 0, C.byref(nb), C.byref(nt)))
        return int(nt.value)

    def batch_tables(self, seqs, max_nb: int):
        """Host int32 tables [B, max_nb] (-1 past each table) and lengths [B]."""
        ids = np.ascontiguousarray(np.asarray(seqs, dtype=np.int64))
        B = ids.size
        tables = np.empty((B, max_nb), dtype=np.int32)
        lens = np.empty(B, dtype=np.int32)
        _lib.check(_lib.load().kv_bm_batch_tables(self._h, ids.ctypes.data, B, int(max_nb),
                                                  tables.ctypes.data, lens.ctypes.data))
        return tables, lens
